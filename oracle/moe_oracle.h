/*
 * moe_oracle.h -- CPU oracle for the routed FP8 (E4M3, 128x128 block-scaled)
 * mixture-of-experts expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, sequential-order C
 * implementation used to check the GPU library.  Only the test suite, the
 * package smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or helper with the GPU library, and the
 * GPU library never calls it.
 *
 * What it follows (page titles and sections of the source pages):
 *  - Netra Kernel README, capability table: FP8 E4M3 weights with explicit
 *    block scales; Netra Kernel README (kernel laboratory), supported-targets
 *    table: E4M3 with 128x128 block scales on gfx950.
 *  - Netra Kernel README, "Build the exact c64 M768 MoE prefill pair": the
 *    routed MoE stage order -- routing, gate/up, SiLU and quantisation,
 *    down-partial, then a separate route reducer with its own reduction order.
 *  - Netra compiler architecture, compatibility-engine paragraph: gate/up
 *    results are FP32, activations are FP8 with FP32 activation-scale tensors.
 *  - Inferact amd-kernels README, atomics rule: partial results are summed in
 *    a fixed order, never with atomic adds.
 *  - Inferact amd-kernels README, reference convention: the reference states
 *    where each rounding happens, the scale layout and the accumulate type.
 *
 * Rounding points (each one is a documented reading where the pages are
 * silent; the list lives in the design notes of the repository):
 *  - E4M3 is the OCP "FN" variant: bias 7, max finite 448, no infinities,
 *    codes 0x7F/0xFF are NaN.  Decode is an explicit 256-entry table.
 *  - encode(v): nearest E4M3 value, ties to the even code, |v| > 448 clamps
 *    to +-448 (saturating), the sign of zero is kept, NaN -> 0x7F.
 *  - Block scale s = amax / 448 (fp32 division); code = encode(fp32(v / s));
 *    amax == 0 gives s = 0 and all-zero codes.  Weights: one scale per
 *    128x128 block, layout [batch][N/128][K/128].  Activations: one scale per
 *    token (or route) per 128 columns, layout [rows][K/128].
 *  - Router: fp32 softmax over E logits (max-subtracted expf, sum in
 *    ascending expert order, divide), top-k chosen on the fp32 logits with
 *    ties to the lower expert index (IEEE compare, so -0 == +0), rank order =
 *    selection order, weights renormalised over the k picks (sum in rank
 *    order, divide).
 *  - Block GEMM: per 128-wide K block, fp32 sum of exact E4M3*E4M3 products
 *    in ascending k; then acc += blk * (s_act * s_w), scale product rounded
 *    first, blocks in ascending order.  Output fp32.
 *  - SiLU-mul: v = (a / (1 + expf(-a))) * u in fp32, gate rows [0, i) and up
 *    rows [i, 2i) of w13; then the 1x128 requantisation above.
 *  - Combine: out[t] = bf16_rne( sum_r w[t,r] * y[t*k + r] ), fp32 multiply
 *    then add, r ascending (rank order), starting from 0.
 *  Compiled with -ffp-contract=off and no fast-math so every operation above
 *  rounds exactly once, in the written order.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- formats -------------------------------------------------------- */
float    oracle_e4m3_decode(uint8_t code);
/* the table itself, for exhaustive checks */
const float* oracle_e4m3_table(void);
/* RNE + saturating encoder by bisection over the table */
uint8_t  oracle_e4m3_encode(float v);
/* same contract by exhaustive linear search over all finite codes (slow) */
uint8_t  oracle_e4m3_encode_linear(float v);
void     oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out);
uint16_t oracle_bf16_encode(float v);
float    oracle_bf16_decode(uint16_t b);

/* ---- threads (results do not depend on the count) ------------------- */
void oracle_set_threads(int n);
int  oracle_get_threads(void);

/* ---- weight preparation: per 128x128 block of each [N,K] matrix ----- */
/* w: fp32 [batch][N][K] -> q: e4m3 [batch][N][K], s: fp32 [batch][N/128][K/128] */
void oracle_quant_weight_block128(const float* w, int64_t batch, int N, int K,
                                  uint8_t* q, float* s);

/* ---- the steps of the layer ----------------------------------------- */
/* logits fp32 [M][E] -> ids int32 [M][k] (rank order), w fp32 [M][k] */
void oracle_router(const float* logits, int M, int E, int k, int32_t* ids, float* w);

/* rows of bf16 bits [M][K] -> q e4m3 [M][K], s fp32 [M][K/128] */
void oracle_act_quant(const uint16_t* x, int M, int K, uint8_t* q, float* s);

/* ids int32 [R] with values in [0,E) -> counts [E], offsets [E+1],
 * sorted [R] = route ids grouped by expert ascending, route id ascending
 * inside each expert (stable counting sort). */
void oracle_group(const int32_t* ids, int R, int E,
                  int32_t* counts, int32_t* offsets, int32_t* sorted);

/* Block-scaled FP8 GEMM for a set of rows:
 *   for r < R: out[r][n] = sum_kb ( sum_kk A[arow[r]][kb*128+kk] * W[wsel[r]][n][kb*128+kk] )
 *                                 * (As[arow[r]][kb] * Ws[wsel[r]][n/128][kb])
 * A e4m3 [*][K], As fp32 [*][K/128], W e4m3 [*][N][K], Ws fp32 [*][N/128][K/128],
 * out fp32 [R][N]. */
void oracle_block_gemm(const uint8_t* A, const float* As, const int32_t* arow,
                       const uint8_t* W, const float* Ws, const int32_t* wsel,
                       int R, int N, int K, float* out);

/* g fp32 [R][2I] -> a2 e4m3 [R][I], a2s fp32 [R][I/128] */
void oracle_silu_mul_quant(const float* g, int R, int I, uint8_t* a2, float* a2s);

/* y fp32 [M*k][H], w fp32 [M][k] -> out bf16 bits [M][H] */
void oracle_combine(const float* y, const float* w, int M, int k, int H, uint16_t* out);

/* BF16 routing (Netra Kernel README capability table: BF16 routing among the
 * gfx950 operation families): router logits from bf16 hidden rows x [M][K]
 * and a bf16 router weight wr [E][K]: logits[t][e] = fp32( sum over j of
 * x[t][j] * wr[e][j] ), every product exact, the sum in float64 in ascending
 * j, one rounding to fp32.  The ids and weights then come from
 * oracle_router on these logits. */
void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int M, int K, int E, float* logits);

/* Front end before the layer (normalisation and quantisation fusion of the
 * Netra Kernel README directory map, gfx950 norm family): RMSNorm of bf16
 * rows, rounded to bf16, then the 1x128 quantisation of oracle_act_quant.
 * Per row: ss = sum of x^2 in float64 (every square is exact), r =
 * fp32(1 / sqrt(ss / K + eps)) with the sum, division, square root and
 * reciprocal in float64 and one rounding to fp32 at the end; y[c] =
 * bf16_rne(fp32(fp32(x[c] * r) * gamma[c])).  gamma is the fp32 norm weight
 * (1 + w for a zero-centred weight w).
 * x bf16 bits [M][K], gamma fp32 [K] -> y bf16 bits [M][K], q e4m3 [M][K],
 * s fp32 [M][K/128]. */
void oracle_rmsnorm_act_quant(const uint16_t* x, const float* gamma, float eps, int M, int K,
                              uint16_t* y, uint8_t* q, float* s);

/* Intermediates of one forward, all optional (NULL = not wanted). */
typedef struct {
    int32_t* ids;      /* [M*k]      */
    float*   topk_w;   /* [M*k]      */
    uint8_t* xq;       /* [M*h]      */
    float*   xs;       /* [M*h/128]  */
    int32_t* counts;   /* [E]        */
    int32_t* offsets;  /* [E+1]      */
    int32_t* sorted;   /* [M*k]      */
    float*   g;        /* [M*k*2i]   */
    uint8_t* a2;       /* [M*k*i]    */
    float*   a2s;      /* [M*k*i/128]*/
    float*   y;        /* [M*k*h]    */
} oracle_intermediates;

/* Whole layer.  x bf16 bits [M][h]; logits fp32 [M][E];
 * w13 e4m3 [E][2i][h] (rows [0,i) gate, [i,2i) up); s13 fp32 [E][2i/128][h/128];
 * w2 e4m3 [E][h][i]; s2 fp32 [E][h/128][i/128]; out bf16 bits [M][h].
 * Returns 0, or -1 on an unsupported shape (h or i not a multiple of 128,
 * k outside [1, E], M < 0).  Allocates its own temporaries. */
int oracle_moe_forward(const uint16_t* x, const float* logits,
                       const uint8_t* w13, const float* s13,
                       const uint8_t* w2, const float* s2,
                       uint16_t* out, int M, int h, int i, int E, int k,
                       oracle_intermediates* dbg);

/* MXFP4 weight variant (Inferact amd-kernels README, naming section: the
 * MoE kernel moe/mxfp4_h6144_i768_e128_top4; Netra Kernel README, targets
 * table: MXFP4 checkpoints, and its real-checkpoint checks against staged
 * FP64 dequantised-MXFP4 references).  Weights are OCP MX FP4: E2M1
 * elements with one E8M0 power-of-two scale per 32 consecutive K elements.
 * Activations stay E4M3 with 1x128 fp32 scales, as in the FP8 layer.
 *  - E2M1 decode: explicit 16-entry table; encode: nearest value, ties to
 *    the code with mantissa bit 0, saturating to +-6, sign of zero kept.
 *  - E8M0 decode: 2^(code - 127).
 *  - Quantisation per 1x32 block: e = floor(log2(amax)) - 2, clamped to
 *    [-127, 127]; scale code e + 127; element codes E2M1(w * 2^-e); an
 *    all-zero block has scale code 0 and zero codes.
 *  - GEMMs: every term E2M1 * 2^(s - 127) * E4M3 * activation scale is
 *    exact in float64; they are summed in float64 in ascending K and the sum
 *    is rounded once to fp32 (gate/up results and down partials are fp32).
 *  - Everything else (routing, activation quantisation, SiLU-mul
 *    requantisation, rank-order combine) as in oracle_moe_forward. */
float oracle_e2m1_decode(uint8_t code);
uint8_t oracle_e2m1_encode(float v);
double oracle_e8m0_decode(uint8_t code);
/* w fp32 [rows][K] -> codes [rows][K/2] (element 2j low nibble of byte j),
 * scales E8M0 [rows][K/32].  K % 32 == 0. */
void oracle_mxfp4_quantize(const float* w, int64_t rows, int K, uint8_t* codes, uint8_t* scales);
/* Whole layer with MXFP4 weights: w13 [E][2i][h/2] + e13 [E][2i][h/32];
 * w2 [E][h][i/2] + e2 [E][h][i/32].  Other arguments and intermediates as in
 * oracle_moe_forward (counts, offsets and sorted are not filled). */
int oracle_moe_forward_mxfp4(const uint16_t* x, const float* logits,
                             const uint8_t* w13, const uint8_t* e13,
                             const uint8_t* w2, const uint8_t* e2,
                             uint16_t* out, int M, int h, int i, int E, int k,
                             oracle_intermediates* dbg);

#ifdef __cplusplus
}
#endif
#endif
