// Fused forward: S^T = K Q^T on INT8 MFMA (i32 accumulation), dequantize,
// online softmax in registers, P~ codes with the fixed scale 1/127 against
// the tile-row maximum, O^T += V^T P~^T on INT8 MFMA, then O and LSE.
//
// SageBwd (abstract): the two forward matmuls are among the six INT8 ones.
// The tile loop and the online softmax (running max, running sum, rescaling)
// follow FlashAttention-2 (under "Builds on" on the SageBwd page).
//
// Work split: one wave owns 64 query rows (one quantization block of Q) and
// walks the key blocks; 4 waves per workgroup, each independent.  Computing
// S^T instead of S puts one query per lane column, so every softmax row
// statistic lives in one lane (plus its partner in the other half-wave), and
// the P~ codes leave the accumulator already in the B-operand layout of the
// V^T P~^T product.  K and V code tiles are loaded from L2 straight into
// registers (16 bytes per lane per 32x32 operand).
#include "attn.h"

namespace sagebwd {

template <bool CAUSAL, bool SMOOTHQ>
__global__ __launch_bounds__(256) void k_fwd(FwdArgs a) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, h = lane / 32, l32 = lane % 32;
    const int bh = blockIdx.y;
    const int iq = (a.ngroups - 1 - blockIdx.x) * 4 + wave;   // longest causal rows first
    if (iq >= a.T) return;
    const size_t bt = (size_t)bh * a.T;
    const size_t np = (size_t)a.T * BLK;

    v4i qop[2][2];
    {
        const v4i* src = (const v4i*)(a.q_r + (bt + iq) * 4096);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) qop[qb][ks] = src[(qb * 2 + ks) * 64 + lane];
    }
    const float sQ = a.sq[bt + iq];

    float M[2] = {-__builtin_inff(), -__builtin_inff()};
    float L[2] = {0.0f, 0.0f};          // per half-wave partial sums of 127 * P^
    v16f O[2][2];                        // [qb][db]: lane = query, registers = channels
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < 2; ++db) O[qb][db] = v16f{};

    const int t_end = CAUSAL ? iq : a.T - 1;
    const bool ragged = (a.N % BLK) != 0;
    for (int t = 0; t <= t_end; ++t) {
        v4i kop[2][2], vop[2][2];
        {
            const v4i* ks_ = (const v4i*)(a.k_r + (bt + t) * 4096);
            const v4i* vs_ = (const v4i*)(a.v_t + (bt + t) * 4096);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    kop[x][ks] = ks_[(x * 2 + ks) * 64 + lane];
                    vop[x][ks] = vs_[(x * 2 + ks) * 64 + lane];
                }
        }
        const float sc = tile_scale(sQ, a.sk[bt + t]);
        const float sv = a.sv[bt + t];

        v16i s[2][2];   // [kb][qb]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                s[kb][qb] = mfma_i8(kop[kb][0], qop[qb][0], v16i{});
                s[kb][qb] = mfma_i8(kop[kb][1], qop[qb][1], s[kb][qb]);
            }

        float z[2][2][16];
        float bias[2][16];
        if (SMOOTHQ) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const float4 b4 = *(const float4*)(a.bias + bh * np + t * BLK + 32 * kb + 8 * r4 + 4 * h);
                    bias[kb][4 * r4 + 0] = b4.x;
                    bias[kb][4 * r4 + 1] = b4.y;
                    bias[kb][4 * r4 + 2] = b4.z;
                    bias[kb][4 * r4 + 3] = b4.w;
                }
        }
        const bool need_mask = (CAUSAL && t == iq) || (ragged && t == a.T - 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float af = (float)s[kb][qb][r];
                    z[kb][qb][r] = SMOOTHQ ? __builtin_fmaf(af, sc, bias[kb][r]) : af * sc;
                }
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = t * BLK + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                        const int q = iq * BLK + 32 * qb + l32;
                        if (key >= a.N || (CAUSAL && key > q)) z[kb][qb][r] = -__builtin_inff();
                    }
        }

        v4i pc[2][2];   // [qb][kb] B operand of V^T P~^T (k = keys of step kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, z[kb][qb][r]);
            mx = fmaxf(mx, half_swap(mx));
            const bool live = mx > -__builtin_inff();
            const float mref = live ? mx - LOG2_127 : 0.0f;
            float ls = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                uint32_t bits[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = __builtin_amdgcn_exp2f(z[kb][qb][r] - mref);   // 127 * P^
                    ls += v;
                    bits[r] = round_bits(v);
                }
                pc[qb][kb] = v4i{(int)pack4(bits[0], bits[1], bits[2], bits[3]),
                                 (int)pack4(bits[4], bits[5], bits[6], bits[7]),
                                 (int)pack4(bits[8], bits[9], bits[10], bits[11]),
                                 (int)pack4(bits[12], bits[13], bits[14], bits[15])};
            }
            // online update (tile weight exp2(mx - M) folds in the V scale)
            const float m_new = live ? fmaxf(M[qb], mx) : M[qb];
            const float alpha = M[qb] > -__builtin_inff() ? __builtin_amdgcn_exp2f(M[qb] - m_new) : 0.0f;
            const float e = live ? __builtin_amdgcn_exp2f(mx - m_new) : 0.0f;
            L[qb] = __builtin_fmaf(L[qb], alpha, e * ls);
            M[qb] = m_new;
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) O[qb][db][r] *= alpha;
            }
            const float w = e * sv;
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                v16i pv = mfma_i8(vop[db][0], pc[qb][0], v16i{});
                pv = mfma_i8(vop[db][1], pc[qb][1], pv);
#pragma unroll
                for (int r = 0; r < 16; ++r) O[qb][db][r] = __builtin_fmaf((float)pv[r], w, O[qb][db][r]);
            }
        }
    }

    // epilogue: O / L in bf16, LSE in natural log of the un-smoothed scores
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float Lt = L[qb] + half_swap(L[qb]);
        const int q = iq * BLK + 32 * qb + l32;
        if (q < a.N) {
            const float inv_l = 1.0f / Lt;
            uint16_t* orow = a.o + ((size_t)bh * a.N + q) * HD;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = 32 * db + 8 * r4 + 4 * h;
                    const uint32_t w0 = f32_to_bf16_rne(O[qb][db][4 * r4 + 0] * inv_l) |
                                        (f32_to_bf16_rne(O[qb][db][4 * r4 + 1] * inv_l) << 16);
                    const uint32_t w1 = f32_to_bf16_rne(O[qb][db][4 * r4 + 2] * inv_l) |
                                        (f32_to_bf16_rne(O[qb][db][4 * r4 + 3] * inv_l) << 16);
                    *(uint2*)(orow + d) = make_uint2(w0, w1);
                }
            if (h == 0) {
                const float lse2 = M[qb] + log2f(Lt) - LOG2_127;   // log2 of the row sum
                a.lse[(size_t)bh * a.N + q] = lse2 * LN2 + a.corr[bh * np + q];
            }
        }
    }
}

int launch_fwd(const FwdArgs& a, int BH, bool causal, bool smooth_q, hipStream_t st) {
    dim3 grid(a.ngroups, BH), block(256);
    if (causal) {
        if (smooth_q) hipLaunchKernelGGL((k_fwd<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fwd<true, false>), grid, block, 0, st, a);
    } else {
        if (smooth_q) hipLaunchKernelGGL((k_fwd<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fwd<false, false>), grid, block, 0, st, a);
    }
    return 0;
}

}  // namespace sagebwd
