// Preparation kernels: K/Q smoothing means, per-block INT8 quantization of
// Q, K, V into the MFMA operand layouts, and the backward's per-row
// preprocessing (Delta, log2-domain LSE, dO codes, FP16 copies of dO and V).
//
// SageBwd (abstract, insight iv): K-smoothing subtracts the token mean of K
// per head, which shifts every score row by a constant that softmax ignores;
// Q-smoothing is optional.  Quantization is symmetric INT8 with one
// absmax/127 scale per block of 64 tokens x 64 channels.  These kernels are
// bound by HBM bandwidth: every input element is read once and one code byte
// (plus, for the backward, one FP16 copy) is written.
#include "prep.h"

namespace sagebwd {

// ---------------------------------------------------------------- QK-norm
// Factor r = 1/sqrt(mean_c x^2 + 1e-6) of every token row of Q (tensor 0)
// and K (tensor 1), in float64 and rounded once to float32 (SageBwd abstract,
// insight (i): QK-norm); every later kernel reads x_n = bf16(fp32(x r)).  The
// squares of bf16 values are exact in float64; the order of their sum moves
// it by a few float64 ulps at most, far below what changes the float32 r
// except within ~1e-16 of one of its rounding boundaries.  0 past N.
__global__ __launch_bounds__(256) void k_rownorm(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                 float* __restrict__ rq, float* __restrict__ rk, int N, int T) {
    const int t = blockIdx.x, bh = blockIdx.y, tensor = blockIdx.z;
    const int r = threadIdx.x / 4, g = threadIdx.x % 4;
    const int tok = t * BLK + r;
    const bool valid = tok < N;
    double ss = 0.0;
    if (valid) {
        const uint16_t* src = (tensor == 0 ? q : k) + ((size_t)bh * N + tok) * HD + 16 * g;
        const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 8);
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double a = bf16_to_f32(w[j] & 0xFFFFu), b = bf16_to_f32(w[j] >> 16);
            ss = __builtin_fma(a, a, ss);
            ss = __builtin_fma(b, b, ss);
        }
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (g == 0) {
        const float rr = valid ? (float)(1.0 / __builtin_sqrt(ss * (1.0 / HD) + QK_NORM_EPS)) : 0.0f;
        (tensor == 0 ? rq : rk)[(size_t)bh * T * BLK + tok] = rr;
    }
}

// ---------------------------------------------------------------- means
// Partial float64 column sums of K (tensor 0) and Q (tensor 1) over chunks
// of SUM_CHUNK tokens.  The order of additions is fixed; for bf16 inputs
// every partial sum is exact in practice (the oracle checks the condition),
// so the final mean does not depend on the order at all.
__global__ __launch_bounds__(256) void k_colsum(const uint16_t* __restrict__ q,
                                                const uint16_t* __restrict__ k,
                                                const float* __restrict__ rq, const float* __restrict__ rk,
                                                double* __restrict__ sums, int N, int nchunk,
                                                int do_q, int do_k) {
    const int chunk = blockIdx.x, bh = blockIdx.y, tensor = blockIdx.z;
    if ((tensor == 0 && !do_k) || (tensor == 1 && !do_q)) return;
    const uint16_t* src = (tensor == 0 ? k : q) + (size_t)bh * N * HD;
    const float* rn = tensor == 0 ? rk : rq;      // QK-norm factors, or null
    const size_t rbase = (size_t)bh * ((N + BLK - 1) / BLK) * BLK;
    const int g = threadIdx.x % 8;            // 8 channels per thread
    const int tr = threadIdx.x / 8;           // 32 token rows
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int t0 = chunk * SUM_CHUNK;
    // all of this thread's rows in flight at once, then the sums in row order
    constexpr int ROWS = SUM_CHUNK / 32;
    uint4 u[ROWS];
    float rr[ROWS];
#pragma unroll
    for (int s = 0; s < ROWS; ++s) {
        const int tok = t0 + tr + 32 * s;
        u[s] = tok < N ? *(const uint4*)(src + (size_t)tok * HD + 8 * g) : make_uint4(0, 0, 0, 0);
        rr[s] = (rn && tok < N) ? rn[rbase + tok] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < ROWS; ++s) {
        if (t0 + tr + 32 * s >= N) continue;   // past the last token: nothing added (not even +0)
        const uint32_t w[4] = {u[s].x, u[s].y, u[s].z, u[s].w};
        if (rn) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] += (double)qk_normed(w[j] & 0xFFFFu, rr[s]);
                acc[2 * j + 1] += (double)qk_normed(w[j] >> 16, rr[s]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] += (double)bf16_to_f32(w[j] & 0xFFFFu);
                acc[2 * j + 1] += (double)bf16_to_f32(w[j] >> 16);
            }
        }
    }
    __shared__ double part[32][HD];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[tr][8 * g + j] = acc[j];
    __syncthreads();
    if (threadIdx.x < HD) {
        double s = 0.0;
        for (int r = 0; r < 32; ++r) s += part[r][threadIdx.x];
        sums[(((size_t)bh * 2 + tensor) * nchunk + chunk) * HD + threadIdx.x] = s;
    }
}

// mu = fp32(fp64(sum) / N); zero when the tensor is not smoothed.
__global__ __launch_bounds__(128) void k_means(const double* __restrict__ sums, float* __restrict__ mu_q,
                                               float* __restrict__ mu_k, int N, int nchunk, int do_q,
                                               int do_k) {
    const int bh = blockIdx.x, tensor = threadIdx.x / HD, c = threadIdx.x % HD;
    const int on = tensor == 0 ? do_k : do_q;
    float m = 0.0f;
    if (on) {
        double s = 0.0;
        const double* p = sums + ((size_t)bh * 2 + tensor) * nchunk * HD + c;
        // sixteen partial sums in flight at a time, added in chunk order
        constexpr int BATCH = 16;
        for (int i0 = 0; i0 < nchunk; i0 += BATCH) {
            double v[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) v[j] = i0 + j < nchunk ? p[(size_t)(i0 + j) * HD] : 0.0;
#pragma unroll
            for (int j = 0; j < BATCH; ++j)
                if (i0 + j < nchunk) s += v[j];
        }
        m = (float)(s / (double)N);
    }
    (tensor == 0 ? mu_k : mu_q)[(size_t)bh * HD + c] = m;
}

// ---------------------------------------------------------------- quantize
// One workgroup per 64-token block of one tensor.  Thread (r = tid/4,
// g = tid%4) owns token r, channels 16g..16g+15.
__device__ __forceinline__ float block_absmax_256(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return a;
}

// Write the 4 KB code block held in LDS (codes[token][channel]) in the
// transposed operand layout: thread tid builds 16-byte chunk tid.
__device__ __forceinline__ void store_transposed(const int8_t (*codes)[HD], int8_t* dst) {
    const int tid = threadIdx.x;
    const int db = tid / 128, ks = (tid / 64) % 2, lane = tid % 64, h = lane / 32;
    const int c = 32 * db + lane % 32;
    uint32_t w[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 32 * ks + 8 * q4 + 4 * h + j;
            x |= (uint32_t)(uint8_t)codes[r][c] << (8 * j);
        }
        w[q4] = x;
    }
    *(uint4*)(dst + tid * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

// MXFP8: the absmax of this thread's 32 x 32 block (tokens 32 (r/32).., channels
// 32 (g/2)..) over the 4 waves of the workgroup: lanes of one wave share a
// block when they differ only in lane bits 0 (g % 2) and 2..5 (token).
__device__ __forceinline__ float mx_block_absmax(float v, float (*red)[2]) {
#pragma unroll
    for (int o : {1, 4, 8, 16, 32}) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x / 64, cb = (threadIdx.x % 4) / 2;
    if ((threadIdx.x & 61) == 0) red[w][cb] = v;       // lanes 0 and 2 of each wave
    __syncthreads();
    const int tb = threadIdx.x / 128;
    return fmaxf(red[2 * tb][cb], red[2 * tb + 1][cb]);
}

// tensor 0 = Q, 1 = K, 2 = V.  MX: E4M3 codes and E8M0 scales instead of INT8
// codes and absmax/127 scales (same code layouts; the scale slot of a 64x64
// block holds its four exponent bytes + 127, byte 2 (token half) + channel half).
template <bool MX>
__global__ __launch_bounds__(256) void k_quantize(QuantArgs a) {
    const int t = blockIdx.x, bh = blockIdx.y, tensor = blockIdx.z;
    const int r = threadIdx.x / 4, g = threadIdx.x % 4;
    const int tok = t * BLK + r;
    const bool valid = tok < a.N;
    const uint16_t* src = (tensor == 0 ? a.q : tensor == 1 ? a.k : a.v) + ((size_t)bh * a.N + tok) * HD + 16 * g;
    const float* mu = tensor == 0 ? a.mu_q : tensor == 1 ? a.mu_k : nullptr;
    float raw[16], x[16];
    uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
    if (valid) {
        u0 = *(const uint4*)src;
        u1 = *(const uint4*)(src + 8);
    }
    // this thread's 16 channels of the centring mean and of the mean its side
    // output needs (Q: mu_K for the LSE correction; K: mu_Q for the score
    // bias), loaded as vectors together with the tokens (loads of single
    // elements behind the pointer tests were waited for one after another)
    float mc[16], mo[16];
    const float* mo_src = tensor == 0 ? (a.smooth_k ? a.mu_k : nullptr) : tensor == 1 ? a.mu_q : nullptr;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        const float4 c4 = mu ? ((const float4*)(mu + (size_t)bh * HD + 16 * g))[j4] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 o4 = mo_src ? ((const float4*)(mo_src + (size_t)bh * HD + 16 * g))[j4] : make_float4(0.f, 0.f, 0.f, 0.f);
        mc[4 * j4 + 0] = c4.x;
        mc[4 * j4 + 1] = c4.y;
        mc[4 * j4 + 2] = c4.z;
        mc[4 * j4 + 3] = c4.w;
        mo[4 * j4 + 0] = o4.x;
        mo[4 * j4 + 1] = o4.y;
        mo[4 * j4 + 2] = o4.z;
        mo[4 * j4 + 3] = o4.w;
    }
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    const float* rn = tensor == 0 ? a.rq : tensor == 1 ? a.rk : nullptr;   // QK-norm: x_n = bf16(fp32(x r))
    if (rn) {
        const float rr = valid ? rn[(size_t)bh * a.T * BLK + tok] : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            raw[2 * j] = qk_normed(w[j] & 0xFFFFu, rr);
            raw[2 * j + 1] = qk_normed(w[j] >> 16, rr);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            raw[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
            raw[2 * j + 1] = bf16_to_f32(w[j] >> 16);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        x[j] = mu ? raw[j] - mc[j] : raw[j];
        if (!valid) x[j] = 0.0f;
        amax = fmaxf(amax, fabsf(x[j]));
    }
    __shared__ float red[4];
    __shared__ float red_mx[4][2];
    __shared__ int8_t codes[BLK][HD];
    const size_t blk = (size_t)bh * a.T + t;
    float* scale_out = tensor == 0 ? a.sq : tensor == 1 ? a.sk : a.sv;
    uint32_t cw[4] = {0, 0, 0, 0};
    float mu_dot = 0.0f;   // K only: sum_c mu_q[c] * code[c] (dequantized code for MX)
    float s;
    if (MX) {
        const int e = mx_exponent(mx_block_absmax(amax, red_mx));
        const float sc = pow2f(e);
        if (r % 32 == 0 && g % 2 == 0) ((uint8_t*)scale_out)[blk * 4 + 2 * (r / 32) + g / 2] = (uint8_t)(e + 127);
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) cw[j4] = fp8_quad(x[4 * j4], x[4 * j4 + 1], x[4 * j4 + 2], x[4 * j4 + 3], sc);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int byte = (cw[j / 4] >> (8 * (j % 4))) & 0xFF;
            codes[r][16 * g + j] = (int8_t)byte;
            if (tensor == 1) mu_dot = __builtin_fmaf(mo[j], fp8_value(cw[j / 4], j % 4), mu_dot);
        }
        s = sc;
    } else {
        const float a_blk = block_absmax_256(amax, red);
        float inv;
        block_scale(a_blk, s, inv);
        if (threadIdx.x == 0) scale_out[blk] = s;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int cq = code_int(x[j], inv);
            codes[r][16 * g + j] = (int8_t)cq;
            cw[j / 4] |= (uint32_t)(uint8_t)cq << (8 * (j % 4));
            if (tensor == 1) mu_dot = __builtin_fmaf(mo[j], (float)cq, mu_dot);
        }
    }
    int8_t* rdst = tensor == 0 ? a.q_r : tensor == 1 ? a.k_r : nullptr;
    if (rdst) *(uint4*)(rdst + blk * 4096 + row_operand_offset(r, 16 * g)) = make_uint4(cw[0], cw[1], cw[2], cw[3]);

    // per-token side outputs
    if (tensor == 0) {
        float cd = 0.0f;
        if (a.smooth_k) {
#pragma unroll
            for (int j = 0; j < 16; ++j) cd = __builtin_fmaf(raw[j], mo[j], cd);
        }
        cd += __shfl_xor(cd, 1, 64);
        cd += __shfl_xor(cd, 2, 64);
        if (g == 0) a.corr[(size_t)bh * a.T * BLK + tok] = valid ? cd * 0.125f : 0.0f;
    } else if (tensor == 1) {
        // MX: the two channel halves of a token have their own scale, so each
        // thread scales its partial sum before the reduction
        if (MX) mu_dot *= s;
        mu_dot += __shfl_xor(mu_dot, 1, 64);
        mu_dot += __shfl_xor(mu_dot, 2, 64);
        const float bias = MX ? mu_dot * SCORE_SCALE_LOG2 : mu_dot * s * SCORE_SCALE_LOG2;
        if (g == 0) a.bias[(size_t)bh * a.T * BLK + tok] = (valid && a.smooth_q) ? bias : 0.0f;
    }

    int8_t* tdst = tensor == 0 ? a.q_t : tensor == 1 ? a.k_t : a.v_t;
    if (tdst) {
        __syncthreads();
        store_transposed(codes, tdst + blk * 4096);
    }
}

// ---------------------------------------------------------------- FP4
// E2M1 codes with one E8M0 exponent per 32 values of the contraction index,
// in blocks of 2048 code bytes + 128 exponent bytes (in the 4096-byte slots of
// the code regions).  Q and K (row FP4 layout): 16-byte chunk th*64 + 32h + m
// holds the 32 channels 32h.. of token 32th + m, value i in nibble i; the
// exponent of (token r, channel half h) is byte 2048 + 2r + h.  V (class
// layout): chunk db*64 + 32h + m holds channel c = 32db + m at the 32 keys of
// key class h = (key % 8) / 4, value 16kb + j at key 32kb + 8(j/4) + 4h + j%4
// (the keys one half-wave holds in the accumulator layout of the scores);
// the exponent of (channel c, class h) is byte 2048 + 2c + h.  One workgroup
// per 64-token block of one tensor (tensor 0 = Q, 1 = K, 2 = V).
__global__ __launch_bounds__(256) void k_quantize_fp4(QuantArgs a) {
    const int t = blockIdx.x, bh = blockIdx.y, tensor = blockIdx.z;
    const int r = threadIdx.x / 4, g = threadIdx.x % 4;
    const int tok = t * BLK + r;
    const bool valid = tok < a.N;
    const uint16_t* src = (tensor == 0 ? a.q : tensor == 1 ? a.k : a.v) + ((size_t)bh * a.N + tok) * HD + 16 * g;
    const float* mu = tensor == 0 ? a.mu_q : tensor == 1 ? a.mu_k : nullptr;
    float raw[16], x[16];
    uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
    if (valid) {
        u0 = *(const uint4*)src;
        u1 = *(const uint4*)(src + 8);
    }
    // this thread's 16 channels of the centring mean and of the mean its side
    // output needs (Q: mu_K for the LSE correction; K: mu_Q for the score
    // bias), loaded as vectors together with the tokens (loads of single
    // elements behind the pointer tests were waited for one after another)
    float mc[16], mo[16];
    const float* mo_src = tensor == 0 ? (a.smooth_k ? a.mu_k : nullptr) : tensor == 1 ? a.mu_q : nullptr;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        const float4 c4 = mu ? ((const float4*)(mu + (size_t)bh * HD + 16 * g))[j4] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 o4 = mo_src ? ((const float4*)(mo_src + (size_t)bh * HD + 16 * g))[j4] : make_float4(0.f, 0.f, 0.f, 0.f);
        mc[4 * j4 + 0] = c4.x;
        mc[4 * j4 + 1] = c4.y;
        mc[4 * j4 + 2] = c4.z;
        mc[4 * j4 + 3] = c4.w;
        mo[4 * j4 + 0] = o4.x;
        mo[4 * j4 + 1] = o4.y;
        mo[4 * j4 + 2] = o4.z;
        mo[4 * j4 + 3] = o4.w;
    }
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    const float* rn = tensor == 0 ? a.rq : tensor == 1 ? a.rk : nullptr;
    if (rn) {
        const float rr = valid ? rn[(size_t)bh * a.T * BLK + tok] : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            raw[2 * j] = qk_normed(w[j] & 0xFFFFu, rr);
            raw[2 * j + 1] = qk_normed(w[j] >> 16, rr);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            raw[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
            raw[2 * j + 1] = bf16_to_f32(w[j] >> 16);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        x[j] = mu ? raw[j] - mc[j] : raw[j];
        if (!valid) x[j] = 0.0f;
        amax = fmaxf(amax, fabsf(x[j]));
    }
    const size_t blk = (size_t)bh * a.T + t;
    if (tensor < 2) {
        // block (token r, channel half g / 2): this thread and its neighbour
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        const int e = fp4_exponent(amax);
        const float sc = pow2f(e);
        uint8_t* dst = (uint8_t*)(tensor == 0 ? a.q_r : a.k_r) + blk * 4096;
        const uint32_t c0 = fp4_oct(x, sc), c1 = fp4_oct(x + 8, sc);
        const int h = g / 2;
        *(uint2*)(dst + ((r / 32) * 64 + 32 * h + r % 32) * 16 + 8 * (g % 2)) = make_uint2(c0, c1);
        if (g % 2 == 0) dst[FP4_EXP_OFF + 2 * r + h] = (uint8_t)(e + 127);
        if (tensor == 0) {
            float cd = 0.0f;
            if (a.smooth_k) {
#pragma unroll
                for (int j = 0; j < 16; ++j) cd = __builtin_fmaf(raw[j], mo[j], cd);
            }
            cd += __shfl_xor(cd, 1, 64);
            cd += __shfl_xor(cd, 2, 64);
            if (g == 0) a.corr[(size_t)bh * a.T * BLK + tok] = valid ? cd * 0.125f : 0.0f;
        } else {
            // Q-smoothing bias from the centred float K (not its 4-bit codes)
            float mu_dot = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) mu_dot = __builtin_fmaf(mo[j], x[j], mu_dot);
            mu_dot += __shfl_xor(mu_dot, 1, 64);
            mu_dot += __shfl_xor(mu_dot, 2, 64);
            if (g == 0) a.bias[(size_t)bh * a.T * BLK + tok] = (valid && a.smooth_q) ? mu_dot * SCORE_SCALE_LOG2 : 0.0f;
        }
        return;
    }
    // V: stage the block, then thread (c, h, kb) codes 16 keys of channel c
    __shared__ float vs[BLK][HD + 1];
    __shared__ float red[2][2][HD];   // [kb][h][c] partial maxima
#pragma unroll
    for (int j = 0; j < 16; ++j) vs[r][16 * g + j] = x[j];
    __syncthreads();
    const int c = threadIdx.x % HD, h = (threadIdx.x / HD) % 2, kb = threadIdx.x / 128;
    float y[16];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        y[j] = vs[32 * kb + 8 * (j / 4) + 4 * h + j % 4][c];
        m = fmaxf(m, fabsf(y[j]));
    }
    red[kb][h][c] = m;
    __syncthreads();
    const int e = fp4_exponent(fmaxf(red[0][h][c], red[1][h][c]));
    const float sc = pow2f(e);
    uint8_t* dst = (uint8_t*)a.v_t + blk * 4096;
    const uint32_t c0 = fp4_oct(y, sc), c1 = fp4_oct(y + 8, sc);
    *(uint2*)(dst + ((c / 32) * 64 + 32 * h + c % 32) * 16 + 8 * kb) = make_uint2(c0, c1);
    if (kb == 0) dst[FP4_EXP_OFF + 2 * c + h] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------- backward prep
// One workgroup per 64-token block: -Delta = -rowsum(dO*O) (fp32), the
// log2-domain LSE of the smoothed scores, dO codes (transposed operand
// layout) and scale, FP16 copies of dO and V.  Rows past N are zeroed (their
// LSE is +inf so every P of such a row is 0).  For the all-INT8 ablation also
// the dO codes in the row-operand layout and the V codes (the same quantizer
// as the forward's, V not centred) with their block scales.
template <bool MX>
__global__ __launch_bounds__(256) void k_bwd_pre(BwdPreArgs a) {
    const int t = blockIdx.x, bh = blockIdx.y;
    const int r = threadIdx.x / 4, g = threadIdx.x % 4;
    const int tok = t * BLK + r;
    const bool valid = tok < a.N;
    const size_t in_off = ((size_t)bh * a.N + tok) * HD + 16 * g;
    float dov[16], ov[16], vv[16];
    uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0, o0 = d0, o1 = d0, v0 = d0, v1 = d0;
    if (valid) {
        d0 = *(const uint4*)(a.dout + in_off);
        d1 = *(const uint4*)(a.dout + in_off + 8);
        o0 = *(const uint4*)(a.o + in_off);
        o1 = *(const uint4*)(a.o + in_off + 8);
        v0 = *(const uint4*)(a.v + in_off);
        v1 = *(const uint4*)(a.v + in_off + 8);
    }
    const uint32_t dw[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    const uint32_t ow[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
    const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float delta = 0.0f, amax = 0.0f, vmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        dov[2 * j] = bf16_to_f32(dw[j] & 0xFFFFu);
        dov[2 * j + 1] = bf16_to_f32(dw[j] >> 16);
        ov[2 * j] = bf16_to_f32(ow[j] & 0xFFFFu);
        ov[2 * j + 1] = bf16_to_f32(ow[j] >> 16);
        vv[2 * j] = bf16_to_f32(vw[j] & 0xFFFFu);
        vv[2 * j + 1] = bf16_to_f32(vw[j] >> 16);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        delta = __builtin_fmaf(dov[j], ov[j], delta);
        amax = fmaxf(amax, fabsf(dov[j]));
        vmax = fmaxf(vmax, fabsf(vv[j]));
    }
    delta += __shfl_xor(delta, 1, 64);
    delta += __shfl_xor(delta, 2, 64);
    const size_t row = (size_t)bh * a.T * BLK + tok;
    if (g == 0) {
        a.delta[row] = valid ? -delta : 0.0f;
        a.lse2[row] = valid ? (a.lse[(size_t)bh * a.N + tok] - a.corr[row]) * LOG2E : __builtin_inff();
    }
    // FP16 copies (natural layout [Np][64])
    {
        uint32_t hw[8], vh[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            _Float16 a0 = (_Float16)dov[2 * j], a1 = (_Float16)dov[2 * j + 1];
            _Float16 b0 = (_Float16)vv[2 * j], b1 = (_Float16)vv[2 * j + 1];
            hw[j] = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
            vh[j] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        }
        uint4* dd = (uint4*)(a.do16 + row * HD + 16 * g);
        dd[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dd[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        uint4* vd = (uint4*)(a.v16 + row * HD + 16 * g);
        vd[0] = make_uint4(vh[0], vh[1], vh[2], vh[3]);
        vd[1] = make_uint4(vh[4], vh[5], vh[6], vh[7]);
    }
    // dO codes
    __shared__ float red[4];
    __shared__ float red_mx[4][2];
    __shared__ int8_t codes[BLK][HD];
    const size_t blk = (size_t)bh * a.T + t;
    uint32_t cw[4] = {0, 0, 0, 0};
    if (MX) {
        const int e = mx_exponent(mx_block_absmax(amax, red_mx));
        const float sc = pow2f(e);
        if (r % 32 == 0 && g % 2 == 0) ((uint8_t*)a.sdo)[blk * 4 + 2 * (r / 32) + g / 2] = (uint8_t)(e + 127);
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) cw[j4] = fp8_quad(dov[4 * j4], dov[4 * j4 + 1], dov[4 * j4 + 2], dov[4 * j4 + 3], sc);
#pragma unroll
        for (int j = 0; j < 16; ++j) codes[r][16 * g + j] = (int8_t)((cw[j / 4] >> (8 * (j % 4))) & 0xFF);
    } else {
        const float a_blk = block_absmax_256(amax, red);
        float s, inv;
        block_scale(a_blk, s, inv);
        if (threadIdx.x == 0) a.sdo[blk] = s;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int cq = code_int(dov[j], inv);
            codes[r][16 * g + j] = (int8_t)cq;
            cw[j / 4] |= (uint32_t)(uint8_t)cq << (8 * (j % 4));
        }
    }
    if (a.do_r) *(uint4*)(a.do_r + blk * 4096 + row_operand_offset(r, 16 * g)) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    __syncthreads();
    store_transposed(codes, a.do_t + blk * 4096);
    if (a.v_r) {
        __shared__ float red_v[4];
        float sv, invv;
        block_scale(block_absmax_256(vmax, red_v), sv, invv);
        if (threadIdx.x == 0) a.sv[blk] = sv;
        uint32_t vw4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 16; ++j) vw4[j / 4] |= (uint32_t)(uint8_t)code_int(vv[j], invv) << (8 * (j % 4));
        *(uint4*)(a.v_r + blk * 4096 + row_operand_offset(r, 16 * g)) = make_uint4(vw4[0], vw4[1], vw4[2], vw4[3]);
    }
}

// ---------------------------------------------------------------- launchers
int launch_means(const MeansArgs& m, hipStream_t st) {
    const int nchunk = (m.N + SUM_CHUNK - 1) / SUM_CHUNK;
    if (m.smooth_q || m.smooth_k) {
        hipLaunchKernelGGL(k_colsum, dim3(nchunk, m.BH, 2), dim3(256), 0, st, m.q, m.k, m.rq, m.rk, m.sums, m.N,
                           nchunk, m.smooth_q, m.smooth_k);
    }
    hipLaunchKernelGGL(k_means, dim3(m.BH), dim3(128), 0, st, m.sums, m.mu_q, m.mu_k, m.N, nchunk, m.smooth_q,
                       m.smooth_k);
    return 0;
}

int launch_rownorm(const uint16_t* q, const uint16_t* k, float* rq, float* rk, int N, int T, int BH, hipStream_t st) {
    hipLaunchKernelGGL(k_rownorm, dim3(T, BH, 2), dim3(256), 0, st, q, k, rq, rk, N, T);
    return 0;
}

int launch_quantize(const QuantArgs& a, int BH, int ntensors, int fmt, hipStream_t st) {
    if (fmt == FMT_FP4) hipLaunchKernelGGL(k_quantize_fp4, dim3(a.T, BH, ntensors), dim3(256), 0, st, a);
    else if (fmt == FMT_MXFP8) hipLaunchKernelGGL(k_quantize<true>, dim3(a.T, BH, ntensors), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_quantize<false>, dim3(a.T, BH, ntensors), dim3(256), 0, st, a);
    return 0;
}

int launch_bwd_pre(const BwdPreArgs& a, int BH, bool mx, hipStream_t st) {
    if (mx) hipLaunchKernelGGL(k_bwd_pre<true>, dim3(a.T, BH), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_bwd_pre<false>, dim3(a.T, BH), dim3(256), 0, st, a);
    return 0;
}

}  // namespace sagebwd
