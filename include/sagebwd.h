/*
 * sagebwd.h -- C ABI of the MI355X (gfx950) SageBwd trainable INT8 attention.
 *
 * What is computed (SageBwd: A Trainable Low-bit Attention, abstract; the
 * SageAttention3 summary page, sections "Approach" and "Measured effects"):
 * softmax attention forward and backward in which six of the seven matmuls
 * run on INT8 operands with 32-bit integer accumulation -- forward Q K^T and
 * P~ V, backward Q K^T (recomputed), P^T dO, dS K and dS^T Q -- while the
 * seventh, dO V^T, runs in FP16 with FP32 accumulation.  Operands are
 * prepared with K-smoothing (subtract the per-head token mean of K; softmax
 * ignores the resulting per-row shift) and optional Q-smoothing, then
 * quantized symmetrically per block of 64 tokens x 64 channels with scale
 * absmax/127.  P~ in [0,1] uses the fixed scale 1/127 against its tile-row
 * maximum; P and dS in the backward use one absmax/127 scale per 64x64 tile.
 * The forward/backward structure (online softmax, log-sum-exp, Delta =
 * rowsum(dO*O)) is FlashAttention-2's, listed under "Builds on" on the
 * SageBwd page.
 *
 * Layout and types (every call):
 *   Q, K, V, O, dO, dQ, dK, dV : bfloat16, contiguous [B, H, N, D], D = 64
 *                                innermost, 16-byte aligned device pointers.
 *   LSE                        : float32 [B, H, N], natural log of the row sum
 *                                of exp(score) with score = q.k / 8 (the
 *                                un-smoothed scores), device pointer.
 *   softmax scale              : fixed 1/sqrt(64) = 1/8.
 *   causal                     : keep key j <= query i (top-left aligned).
 *
 * Ownership: the caller owns every buffer, including the workspace, whose
 * size the *_workspace_size calls give (256-byte aligned device memory).
 * The library allocates nothing, keeps no global state, never synchronizes
 * the host, and enqueues all work on ``stream`` (a hipStream_t; NULL means
 * the default stream).  Outputs are overwritten, never accumulated into, and
 * must not alias inputs or the workspace.  Calls on distinct streams with
 * distinct workspaces may run concurrently.
 *
 * Errors: 0 on success, a negative SAGEBWD_ERR_* code otherwise.  Argument
 * checks (null pointers, sizes, flags, alignment, workspace size) happen
 * before any HIP call, so a failing call launches nothing.  A launch failure
 * reported by the HIP runtime returns SAGEBWD_ERR_HIP.  Not checked:
 * finiteness of the inputs, and |dO|, |V| <= 65504 (they are converted to
 * FP16 for dO V^T).
 */
#ifndef SAGEBWD_H
#define SAGEBWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sagebwd_params {
    int32_t B;          /* batch, >= 1 */
    int32_t H;          /* heads, >= 1 */
    int32_t N;          /* tokens (queries = keys), 1 <= N <= 2^18 */
    int32_t D;          /* head dimension, must be 64 */
    int32_t causal;     /* 0 or 1 */
    int32_t smooth_q;   /* 0 or 1: subtract the per-head token mean of Q */
    int32_t smooth_k;   /* 0 or 1: subtract the per-head token mean of K */
    int32_t int8_dp;    /* 0 or 1: backward only.  1 = the all-INT8 ablation of the
                           SageAttention3 summary's table of measured effects:
                           dO V^T also from per-block INT8 codes of dO and V
                           (i32 accumulation, scaled by s_dO s_V) instead of
                           FP16.  0 (the method) keeps it in FP16. */
    int32_t qk_norm;    /* 0 or 1: QK-norm fused in (SageBwd abstract, insight
                           (i): necessary for stable training at many tokens
                           per step).  Every token row x of Q and of K becomes
                           x_n = bf16(fp32(x r)), r = 1/sqrt(mean_c x^2 + 1e-6)
                           (float64, rounded once to float32), before smoothing
                           and quantization, so attention (and LSE) use the
                           normalized scores; the backward returns dQ, dK
                           with respect to the Q, K passed in, through
                           dx = r (dx_n - x_n mean_c(dx_n x_n)).  Forward and
                           backward must be called with the same value. */
    int32_t mxfp8;      /* 0 or 1: the FP8 quantization that the SageBwd page
                           compares with INT8 (and finds less accurate), in
                           the form MI355X's scaled FP8 matrix instructions
                           take: every quantized operand (Q, K, V, dO, P, dS)
                           as OCP FP8 E4M3 codes with one power-of-two (E8M0)
                           scale per 32x32 block, 2^e with e the least integer
                           such that 448 2^e >= the block's absmax, clamped to
                           [-126, 127]; the forward's P~ = exp(S - running row
                           max) coded as E4M3(256 P~).  Smoothing, QK-norm,
                           the FP16 dO V^T and the outputs are as in the INT8
                           mode.  Not with int8_dp (SAGEBWD_ERR_UNSUPPORTED).
                           Forward and backward must be called with the same
                           value. */
    int32_t fp4;        /* 0 or 1: forward only (inference).  The FP4 attention of
                           the SageAttention3 summary ("Approach": FP4
                           microscaling on both matmuls) in MI355X's MXFP4
                           form: E2M1 codes with one power-of-two (E8M0) scale
                           per 32 values of the contraction index, 2^e with e
                           the least integer such that 6 2^e >= the block's
                           absmax, clamped to [-126, 127]; Q and K per token
                           and 32 consecutive channels; V and P~ per channel
                           (per query) and the 32 keys of one key class
                           (key % 8) / 4 of a 64-key tile; P~ = exp(S - running
                           row max); the Q-smoothing bias from the float
                           centred K.  Not with mxfp8 or int8_dp; the
                           backward entry points, the backward kernels of
                           sagebwd_debug_tile and sagebwd_prepare with dO
                           return SAGEBWD_ERR_UNSUPPORTED. */
} sagebwd_params;

#define SAGEBWD_OK               0
#define SAGEBWD_ERR_INVALID_ARG (-1)   /* null pointer, size < 1, flag not 0/1, misaligned */
#define SAGEBWD_ERR_UNSUPPORTED (-2)   /* D != 64, N or B*H beyond the supported range, a mode
                                          combination or an entry point the modes do not have */
#define SAGEBWD_ERR_WORKSPACE   (-3)   /* ws_bytes smaller than the required size */
#define SAGEBWD_ERR_HIP         (-4)   /* the HIP runtime reported a launch error */
#define SAGEBWD_ERR_SCRATCH     (-5)   /* sagebwd_fwd_noalloc: the problem's workspace exceeds
                                          SAGEBWD_NOALLOC_SCRATCH_BYTES */

/* Workspace bytes needed by sagebwd_fwd / sagebwd_bwd for these params;
 * 0 if the params are invalid.  Both grow linearly with B*H*N (about 5.2
 * bytes per element of Q for the forward and 10.3 for the backward: codes,
 * block scales, per-token rows and FP16 copies); nothing of size N^2 is kept
 * (e.g. B=1, H=32, N=16384 causal: 174 MB and 346 MB). */
size_t sagebwd_fwd_workspace_size(const sagebwd_params* p);
size_t sagebwd_bwd_workspace_size(const sagebwd_params* p);

/* Forward.  Reads Q, K, V; writes O [B,H,N,64] bf16 and LSE [B,H,N] fp32. */
int sagebwd_fwd(const sagebwd_params* p,
                const void* Q, const void* K, const void* V,
                void* O, float* LSE,
                void* ws, size_t ws_bytes, void* stream);

/* Backward.  Reads Q, K, V, the forward's O and LSE, and dO (all as above,
 * with the same params as the forward call); writes dQ, dK, dV
 * [B,H,N,64] bf16.
 *
 * fwd_ws (nullable): the workspace of a completed sagebwd_fwd call with the
 * same params and the same Q, K, V, still unmodified, and its size
 * fwd_ws_bytes (at least sagebwd_fwd_workspace_size).  The backward then
 * reads the forward's smoothing means, Q and K codes (both operand
 * layouts), block scales, LSE correction and Q-smoothing bias from it
 * instead of re-quantizing; it only reads fwd_ws.  With fwd_ws NULL it
 * re-quantizes Q, K, V into ws.  The results are bit-identical either way
 * (the quantization is deterministic).  The library cannot check that
 * fwd_ws holds that forward's data; any other content gives wrong results.
 * ws is always a backward workspace (sagebwd_bwd_workspace_size bytes). */
int sagebwd_bwd(const sagebwd_params* p,
                const void* Q, const void* K, const void* V,
                const void* O, const float* LSE, const void* dO,
                void* dQ, void* dK, void* dV,
                const void* fwd_ws, size_t fwd_ws_bytes,
                void* ws, size_t ws_bytes, void* stream);

/* Stages.  sagebwd_fwd runs FWD_PREPARE then FWD_ATTN; sagebwd_bwd runs
 * BWD_PREPARE then BWD_ATTN, all on the same stream.  The stage calls run one
 * stage each, for callers that schedule or time them separately; a stage
 * reads what the earlier stages of its pass wrote into ``ws`` (same params,
 * inputs and workspace), and the full sequence is exactly the pass.
 * BWD_ATTN is BWD_DKDV then BWD_DQ; the two are independent of each other
 * (each recomputes the scores, P and dS it needs from the preparation's
 * output) and may run in either order.
 *   FWD_PREPARE  smoothing means; Q, K, V block quantization
 *   FWD_ATTN     the fused forward kernel (INT8 QK^T and P~V)
 *   BWD_PREPARE  (without fwd_ws) means and quantization again; then
 *                -Delta, log2 LSE, dO codes, FP16 copies of dO and V
 *                (int8_dp: also row-layout dO codes, V codes and scales)
 *   BWD_DKDV     dK and dV (INT8 QK^T, P^T dO, dS^T Q; FP16 dO V^T)
 *   BWD_DQ       dQ (INT8 QK^T and dS K; FP16 dO V^T): the same scores, P,
 *                dS, tile scales and dS codes as BWD_DKDV, bit for bit
 *   BWD_ATTN     BWD_DKDV then BWD_DQ */
#define SAGEBWD_STAGE_FWD_PREPARE 0
#define SAGEBWD_STAGE_FWD_ATTN    1
#define SAGEBWD_STAGE_BWD_PREPARE 2
#define SAGEBWD_STAGE_BWD_DKDV    3
#define SAGEBWD_STAGE_BWD_DQ      4
#define SAGEBWD_STAGE_BWD_ATTN    5
int sagebwd_fwd_stage(const sagebwd_params* p, int stage,
                      const void* Q, const void* K, const void* V,
                      void* O, float* LSE,
                      void* ws, size_t ws_bytes, void* stream);
int sagebwd_bwd_stage(const sagebwd_params* p, int stage,
                      const void* Q, const void* K, const void* V,
                      const void* O, const float* LSE, const void* dO,
                      void* dQ, void* dK, void* dV,
                      const void* fwd_ws, size_t fwd_ws_bytes,
                      void* ws, size_t ws_bytes, void* stream);

/* Forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It is sagebwd_fwd with its workspace taken from a
 * buffer compiled into the library: a static device array of
 * SAGEBWD_NOALLOC_SCRATCH_BYTES (256 MiB) that every GPU the library runs on
 * holds until the process ends.  The call allocates nothing: on its first use
 * on a device it looks the array's address up once (hipGetSymbolAddress) and
 * keeps it.  Inputs and outputs are the caller's, as for sagebwd_fwd.
 * Returns SAGEBWD_ERR_SCRATCH, before any HIP call, when
 * sagebwd_fwd_workspace_size(p) exceeds the buffer (e.g. B=1, H=32, N=16384
 * needs 174 MB and fits; B=1, H=32, N=32768 does not).  The buffer is shared
 * by every call on a GPU and keeps the last call's contents (the forward
 * overwrites everything it reads), so calls that overlap on one GPU (on
 * different streams, or from different threads) race; calls in stream order
 * do not.  A backward cannot reuse this forward's quantization (pass
 * fwd_ws = NULL to sagebwd_bwd). */
#define SAGEBWD_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int sagebwd_fwd_noalloc(const sagebwd_params* p,
                        const void* Q, const void* K, const void* V,
                        void* O, float* LSE, void* stream);

/* Static description of a status code. */
const char* sagebwd_status_string(int status);

/* ---- inspection entry points (used by the bit-exact tests) ---------------
 *
 * sagebwd_prepare runs only the preparation kernels of sagebwd_bwd
 * (smoothing means, block quantization of Q, K, V and dO, Delta and the
 * backward's log2-domain LSE) into a backward-sized workspace, so the codes,
 * scales and means can be read back and compared bit for bit.  O and LSE may
 * be NULL together with dO (then only Q, K, V are prepared).
 *
 * sagebwd_ws_region returns the byte offset and size of one region of that
 * workspace; the region ids and their layouts are:
 *   0  MU_Q   float32 [BH][64]       Q token means (0 if !smooth_q)
 *   1  MU_K   float32 [BH][64]       K token means (0 if !smooth_k)
 *   2  Q_R    int8  [BH][T][4096]    Q codes, "row operand" layout
 *   3  K_R    int8  [BH][T][4096]    K codes, row operand layout
 *   4  V_T    int8  [BH][T][4096]    V codes, "transposed operand" layout
 *   5  Q_T    int8  [BH][T][4096]    Q codes, transposed operand layout
 *   6  K_T    int8  [BH][T][4096]    K codes, transposed operand layout
 *   7  DO_T   int8  [BH][T][4096]    dO codes, transposed operand layout
 *   8  S_Q    float32 [BH][T]        block scales (likewise 9 S_K, 10 S_V, 11 S_DO)
 *   12 CORR   float32 [BH][Np]       q_raw . mu_K / 8 per query (0 past N)
 *   13 BIAS   float32 [BH][Np]       Q-smoothing key bias mu_Q . K^_j times log2(e)/8
 *   14 NDELTA float32 [BH][Np]       -rowsum(dO * O)
 *   15 LSE2   float32 [BH][Np]       (LSE - CORR) * log2(e); +inf past N
 *   16 DO16   fp16 [BH][Np][64]      dO in FP16, natural layout
 *   17 V16    fp16 [BH][Np][64]      V in FP16, natural layout
 *   18 DO_R   int8  [BH][T][4096]    dO codes, row operand layout (int8_dp only)
 *   19 V_R    int8  [BH][T][4096]    V codes, row operand layout (int8_dp only)
 *   20 RQ     float32 [BH][Np]       QK-norm factor r of each Q token (qk_norm only; 0 past N)
 *   21 RK     float32 [BH][Np]       likewise for K
 * with T = ceil(N/64), Np = 64 T.  With mxfp8 the code regions hold E4M3
 * code bytes in the same layouts, and each 4-byte block scale (regions 8-11)
 * holds the four biased exponents e + 127 of the block's 32x32 sub-blocks,
 * byte 2*(r/32) + c/32 (token half, channel half).  With fp4 the
 * regions Q_R, K_R and V_T hold FP4 blocks in their 4096-byte slots: 2048
 * bytes of E2M1 codes (two per byte, the first in the low nibble), then 128
 * exponent bytes e + 127.  Q_R, K_R: 16-byte chunk th*64 + 32h + m holds the
 * channels 32h..32h+31 of token 32th + m; the exponent of (token r, channel
 * half h) is byte 2048 + 2r + h.  V_T: chunk db*64 + 32h + m holds channel
 * 32db + m at the keys of class h, value 16kb + j at key
 * 32kb + 8(j/4) + 4h + j%4; the exponent of (channel c, class h) is byte
 * 2048 + 2c + h.  Regions 5-11 are unused; BIAS holds mu_Q . K~_j times
 * log2(e)/8 with K~ the centred float K.  Regions a pass does not use have size 0.  Within a 4096-byte block of 64 tokens x
 * 64 channels, element (token r, channel c) sits at byte
 *   row operand:         ((r/32*2 + c/32)*64 + 32*((c%32)/16) + r%32)*16 + c%16
 *   transposed operand:  ((c/32*2 + r/32)*64 + 32*((r%8)/4) + c%32)*16
 *                          + 4*((r%32)/8) + r%4
 * so that one 16-byte load per lane feeds a 32x32x32 INT8 MFMA operand.
 * Returns SAGEBWD_ERR_INVALID_ARG for an unknown region id. */
/* sagebwd_debug_tile runs one pass of one attention kernel through its
 * debug instantiation, which also writes the values of a single 64x64 tile
 * (head ``bh`` = b*H + h, query block ``qblock``, key block ``kblock``) to
 * ``dump`` (SAGEBWD_DUMP_BYTES bytes, row-major blocks):
 *   kernel 0 (forward, writes O and LSE; ws of at least the forward size):
 *     A i32[q][k] at 0, 127*P^ f32[q][k] at 16384, P~ codes u8[q][k] at 32768,
 *     P~ V i32[q][c] at 36864
 *   kernel 1 (dK/dV; runs the backward preparation first; writes dK, dV):
 *     A at 0, P f32[q][k] at 16384, P codes u8[q][k] at 32768,
 *     P^T dO i32[k][c] at 36864, dS f32[q][k] at 53248, dS codes u8[q][k] at
 *     69632, dS^T Q i32[k][c] at 73728, s_P and s_dS f32 at 90112
 *   kernel 2 (dQ; runs the backward preparation and the dK/dV kernel first;
 *     writes dK, dV, dQ): A at 0, dS f32[q][k] at 53248, its dS codes
 *     u8[q][k] at 32768, dS K i32[q][c] at 36864, s_dS f32 at 90112
 * (q, k: query and key within the blocks; c: channel), so that the INT8
 * codes, block scales and integer tile products can be re-derived exactly
 * from the kernel's own pre-quantization values.  With mxfp8 = 1 the MXFP8
 * kernels dump their tile instead (no integer products exist there: the FP8
 * MFMA accumulates in float32):
 *   kernel 0: the FP8 product S f32[q][k] at 0, P~ f32[q][k] at 16384, P~
 *     E4M3 codes u8[q][k] at 32768, the log2-domain scores z f32[q][k] at
 *     53248, the running row maxima after this tile f32[q] at 90112
 *   kernel 1: S at 0, P at 16384, P codes at 32768, dS f32[q][k] at 53248,
 *     dS codes u8[q][k] at 69632, the E8M0 exponents (unbiased, int32) of P
 *     at 90112 and of dS at 90128, each indexed 2 * (key half) + query half
 *   kernel 2: S at 0, dS at 53248, dS codes at 32768, dS exponents at 90128
 * and with fp4 = 1 (kernel 0 only; SAGEBWD_ERR_UNSUPPORTED otherwise) the FP4
 * forward: S, P~, z and the running maxima as the MXFP8 forward, the E2M1
 * code nibbles u8[q][k] at 32768 and the P~ block exponents int32[q][key
 * class (k % 8) / 4] at 36864.  Tiles above the causal diagonal are never
 * computed and are rejected (SAGEBWD_ERR_INVALID_ARG). */
#define SAGEBWD_DUMP_BYTES 90368
int sagebwd_debug_tile(const sagebwd_params* p, int kernel, int bh, int qblock, int kblock,
                       const void* Q, const void* K, const void* V, void* O, float* LSE, const void* dO,
                       void* dQ, void* dK, void* dV, void* dump, size_t dump_bytes,
                       void* ws, size_t ws_bytes, void* stream);

int sagebwd_prepare(const sagebwd_params* p,
                    const void* Q, const void* K, const void* V,
                    const void* O, const float* LSE, const void* dO,
                    void* ws, size_t ws_bytes, void* stream);
int sagebwd_ws_region(const sagebwd_params* p, int region, size_t* offset, size_t* bytes);

/* sagebwd_check_block_scale checks the quantizers' block-scale arithmetic
 * (the absmax/127 scale and its inverse of every INT8 block; SageBwd
 * abstract): for every float32 a = m 2^e, e in [e_lo, e_hi], and all 2^23
 * mantissas m, it compares the kernels' fast quotients a/127 and 127/a with
 * the compiled IEEE float32 divisions on the GPU, and adds the numbers of
 * mismatches to counts[0] (a/127) and counts[1] (127/a), a device array of
 * two uint64 that the caller zeroes.  With out_s and out_inv (device arrays
 * of 2^23 floats each, or both NULL) it also writes the two fast quotients
 * of every mantissa of exponent e_lo, for a check on the host.  Requires
 * -126 <= e_lo <= e_hi <= 127 (SAGEBWD_ERR_INVALID_ARG otherwise).  The
 * kernels use these quotients for absmax >= 2^-100 only. */
int sagebwd_check_block_scale(int e_lo, int e_hi, unsigned long long* counts, float* out_s, float* out_inv,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGEBWD_H */
