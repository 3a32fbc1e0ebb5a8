// Exhaustive check of the block-scale arithmetic of the quantizers: the fast
// correctly rounded quotients a/127 (quot127) and 127/a (div127) against the
// compiled IEEE float32 divisions, for every float32 a = m 2^e with e in a
// given range and all 2^23 mantissas m.  The absmax/127 scale of every INT8
// block (SageBwd abstract: INT8 with absmax/127 per block) is one of these
// quotients, so this covers every value the kernels can form.
#include "sagebwd.h"

#include "common.h"

namespace sagebwd {

constexpr int CHECK_PER_THREAD = 16;

// One workgroup of 256 threads checks 4096 consecutive mantissas of one
// exponent; mismatch counts are summed in LDS and added to the two global
// counters by one thread (a vector atomic in a lane-divergent branch).
__global__ __launch_bounds__(256) void k_check_block_scale(int e_lo, unsigned long long* counts, float* out_s,
                                                           float* out_inv) {
    const int e = e_lo + (int)(blockIdx.x >> 11);               // 2^23 / 4096 = 2048 workgroups per exponent
    const uint32_t m0 = (blockIdx.x & 2047u) * 4096u + threadIdx.x;
    uint32_t bad_s = 0, bad_inv = 0;
#pragma unroll
    for (int j = 0; j < CHECK_PER_THREAD; ++j) {
        const uint32_t m = m0 + 256u * j;
        const float a = __uint_as_float(((uint32_t)(e + 127) << 23) | m);
        const float s = quot127(a), inv = div127(a);
        bad_s += s != a / 127.0f;
        bad_inv += inv != 127.0f / a;
        if (out_s && e == e_lo) {
            out_s[m] = s;
            out_inv[m] = inv;
        }
    }
    __shared__ uint32_t red[2][256];
    red[0][threadIdx.x] = bad_s;
    red[1][threadIdx.x] = bad_inv;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            red[0][threadIdx.x] += red[0][threadIdx.x + w];
            red[1][threadIdx.x] += red[1][threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0 && (red[0][0] | red[1][0])) {
        atomicAdd(&counts[0], (unsigned long long)red[0][0]);
        atomicAdd(&counts[1], (unsigned long long)red[1][0]);
    }
}

}  // namespace sagebwd

extern "C" int sagebwd_check_block_scale(int e_lo, int e_hi, unsigned long long* counts, float* out_s,
                                         float* out_inv, void* stream) {
    if (e_lo < -126 || e_hi > 127 || e_lo > e_hi || !counts) return SAGEBWD_ERR_INVALID_ARG;
    if ((out_s == nullptr) != (out_inv == nullptr)) return SAGEBWD_ERR_INVALID_ARG;
    const unsigned nblocks = (unsigned)(e_hi - e_lo + 1) * 2048u;
    hipLaunchKernelGGL(sagebwd::k_check_block_scale, dim3(nblocks), dim3(256), 0, (hipStream_t)stream, e_lo, counts,
                       out_s, out_inv);
    return hipGetLastError() == hipSuccess ? SAGEBWD_OK : SAGEBWD_ERR_HIP;
}
