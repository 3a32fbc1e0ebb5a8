// Backward: recompute S on INT8 MFMA, P = exp(S - LSE), P codes per 64x64
// tile, dV = P^T dO on INT8 MFMA, dP = dO V^T on FP16 MFMA, dS = P*(dP-Delta),
// dS codes per 64x64 tile, dK = dS^T Q and dQ = dS K on INT8 MFMA.
//
// SageBwd (abstract): five of the six INT8 matmuls are in the backward, and
// the score gradient dS is where quantization error mainly arises; the
// SageAttention3 summary ("Approach", ablation table, "Surprising findings")
// keeps dO V^T in FP16 because quantizing it hurts dQ.  The gradient formulas
// are FlashAttention-2's (under "Builds on").
//
// Two kernels, no atomics:
//   k_bwd_dkdv  one wave per key block, loops over query blocks; computes S
//               (lane = key), so P and dS codes leave the accumulator as the
//               A operand of P^T dO and dS^T Q (contraction over queries).
//   k_bwd_dq    one wave per query block, loops over key blocks; computes
//               S^T (lane = query), so dS^T codes feed K^T dS^T directly.
// Both evaluate P and dS with the same float32 operations on bit-identical
// operands (the FP16 MFMA gives the same bits for dO V^T and V dO^T), so the
// dS tile, its scale and its codes are identical in the two kernels.
#include "attn.h"

namespace sagebwd {

__device__ __forceinline__ int dot4_sum(int packed) {
    return __builtin_amdgcn_sdot4(packed, 0x01010101, 0, false);
}

template <bool CAUSAL, bool SMOOTHQ>
__global__ __launch_bounds__(256) void k_bwd_dkdv(BwdArgs a) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, h = lane / 32, l32 = lane % 32;
    const int bh = blockIdx.y;
    const int t = blockIdx.x * 4 + wave;                     // key block (longest causal first)
    if (t >= a.T) return;
    const size_t bt = (size_t)bh * a.T;
    const size_t np = (size_t)a.T * BLK;
    const size_t rowbase = bh * np;

    v4i kop[2][2];                                           // B operand of Q K^T: lane = key
    {
        const v4i* src = (const v4i*)(a.k_r + (bt + t) * 4096);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) kop[kb][ks] = src[(kb * 2 + ks) * 64 + lane];
    }
    v8h vh[2][4];                                            // B operand of dO V^T: lane = key
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            vh[kb][ks] = *(const v8h*)(a.v16 + (rowbase + t * BLK + 32 * kb + l32) * HD + 16 * ks + 8 * h);
    float kbias[2] = {0.0f, 0.0f};
    if (SMOOTHQ) {
        kbias[0] = a.bias[rowbase + t * BLK + l32];
        kbias[1] = a.bias[rowbase + t * BLK + 32 + l32];
    }
    const float sK = a.sk[bt + t];

    v16f dk[2][2], dv[2][2];                                 // [kb][db]: lane = channel, regs = keys
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            dk[kb][db] = v16f{};
            dv[kb][db] = v16f{};
        }
    float gsum[2] = {0.0f, 0.0f};                            // sum_i s_dS colsum(dS codes), per half

    const bool ragged_keys = (t == a.T - 1) && (a.N % BLK) != 0;
    for (int i = CAUSAL ? t : 0; i < a.T; ++i) {
        v4i qop[2][2];                                       // A operand: lane = query
        {
            const v4i* src = (const v4i*)(a.q_r + (bt + i) * 4096);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) qop[qb][ks] = src[(qb * 2 + ks) * 64 + lane];
        }
        const float sQ = a.sq[bt + i];
        const float sc = tile_scale(sQ, sK);
        v16i s[2][2];                                        // [qb][kb]: lane = key, regs = queries
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[qb][kb] = mfma_i8(qop[qb][0], kop[kb][0], v16i{});
                s[qb][kb] = mfma_i8(qop[qb][1], kop[kb][1], s[qb][kb]);
            }
        float p[2][2][16];
        float pmax = 0.0f;
        const bool diag = CAUSAL && i == t;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 l4 = *(const float4*)(a.lse2 + rowbase + i * BLK + 32 * qb + 8 * r4 + 4 * h);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * r4 + j;
                        float pv = bwd_prob<SMOOTHQ>(s[qb][kb][r], sc, kbias[kb], lv[j]);
                        if (diag || ragged_keys) {
                            const int key = t * BLK + 32 * kb + l32;
                            const int q = i * BLK + 32 * qb + 8 * r4 + 4 * h + j;
                            if (key >= a.N || (CAUSAL && key > q)) pv = 0.0f;
                        }
                        p[qb][kb][r] = pv;
                        pmax = fmaxf(pmax, pv);
                    }
            }
        pmax = wave_max(pmax);
        float sP, invP;
        block_scale(pmax, sP, invP);

        // dV += s_P s_dO (P codes^T dO codes)
        {
            v4i pc[2][2];                                    // [kb][qs]: A operand, k = queries
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) {
                    uint32_t w[4];
#pragma unroll
                    for (int d4 = 0; d4 < 4; ++d4)
                        w[d4] = pack4(code_bits(p[qs][kb][4 * d4 + 0], invP), code_bits(p[qs][kb][4 * d4 + 1], invP),
                                      code_bits(p[qs][kb][4 * d4 + 2], invP), code_bits(p[qs][kb][4 * d4 + 3], invP));
                    pc[kb][qs] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
                }
            const v4i* dsrc = (const v4i*)(a.do_t + (bt + i) * 4096);
            const float wv = sP * a.sdo[bt + i];
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const v4i d0 = dsrc[(db * 2 + 0) * 64 + lane], d1 = dsrc[(db * 2 + 1) * 64 + lane];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    v16i acc = mfma_i8(pc[kb][0], d0, v16i{});
                    acc = mfma_i8(pc[kb][1], d1, acc);
#pragma unroll
                    for (int r = 0; r < 16; ++r) dv[kb][db][r] = __builtin_fmaf((float)acc[r], wv, dv[kb][db][r]);
                }
            }
        }

        // dP = dO V^T (FP16), dS = P * (dP - Delta), in place of P
        float dsmax = 0.0f;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            v8h doh[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                doh[ks] = *(const v8h*)(a.do16 + (rowbase + i * BLK + 32 * qb + l32) * HD + 16 * ks + 8 * h);
            float dl[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 d4 = *(const float4*)(a.delta + rowbase + i * BLK + 32 * qb + 8 * r4 + 4 * h);
                dl[4 * r4 + 0] = d4.x;
                dl[4 * r4 + 1] = d4.y;
                dl[4 * r4 + 2] = d4.z;
                dl[4 * r4 + 3] = d4.w;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                v16f dp = mfma_f16(doh[0], vh[kb][0], v16f{});
                dp = mfma_f16(doh[1], vh[kb][1], dp);
                dp = mfma_f16(doh[2], vh[kb][2], dp);
                dp = mfma_f16(doh[3], vh[kb][3], dp);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float ds = p[qb][kb][r] * (dp[r] - dl[r]);
                    p[qb][kb][r] = ds;
                    dsmax = fmaxf(dsmax, fabsf(ds));
                }
            }
        }
        dsmax = wave_max(dsmax);
        float sdS, invdS;
        block_scale(dsmax, sdS, invdS);

        // dK += s_dS s_Q (dS codes^T Q codes) [+ colsum term for Q-smoothing]
        {
            v4i dc[2][2];                                    // [kb][qs]
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) {
                    uint32_t w[4];
#pragma unroll
                    for (int d4 = 0; d4 < 4; ++d4)
                        w[d4] = pack4(code_bits(p[qs][kb][4 * d4 + 0], invdS), code_bits(p[qs][kb][4 * d4 + 1], invdS),
                                      code_bits(p[qs][kb][4 * d4 + 2], invdS), code_bits(p[qs][kb][4 * d4 + 3], invdS));
                    dc[kb][qs] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
                }
            if (SMOOTHQ) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    int cs = 0;
#pragma unroll
                    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
                        for (int d4 = 0; d4 < 4; ++d4) cs += dot4_sum(dc[kb][qs][d4]);
                    gsum[kb] = __builtin_fmaf((float)cs, sdS, gsum[kb]);
                }
            }
            const v4i* qsrc = (const v4i*)(a.q_t + (bt + i) * 4096);
            const float wk = sdS * sQ;
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const v4i q0 = qsrc[(db * 2 + 0) * 64 + lane], q1 = qsrc[(db * 2 + 1) * 64 + lane];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    v16i acc = mfma_i8(dc[kb][0], q0, v16i{});
                    acc = mfma_i8(dc[kb][1], q1, acc);
#pragma unroll
                    for (int r = 0; r < 16; ++r) dk[kb][db][r] = __builtin_fmaf((float)acc[r], wk, dk[kb][db][r]);
                }
            }
        }
    }

    // epilogue: dK (x 1/8, plus g_j mu_q) and dV in bf16; lane = channel, regs = keys
    float gfull[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) gfull[kb] = gsum[kb] + half_swap(gsum[kb]);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int d = 32 * db + l32;
        const float muq = SMOOTHQ ? a.mu_q[(size_t)bh * HD + d] : 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kr = 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                const int key = t * BLK + kr;
                float gk = 0.0f;
                if (SMOOTHQ) gk = __shfl(gfull[kb], 8 * (r / 4) + 4 * h + (r % 4), 64);
                if (key < a.N) {
                    const float dkv = (SMOOTHQ ? __builtin_fmaf(gk, muq, dk[kb][db][r]) : dk[kb][db][r]) * 0.125f;
                    a.dk[((size_t)bh * a.N + key) * HD + d] = (uint16_t)f32_to_bf16_rne(dkv);
                    a.dv[((size_t)bh * a.N + key) * HD + d] = (uint16_t)f32_to_bf16_rne(dv[kb][db][r]);
                }
            }
    }
}

template <bool CAUSAL, bool SMOOTHQ>
__global__ __launch_bounds__(256) void k_bwd_dq(BwdArgs a) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, h = lane / 32, l32 = lane % 32;
    const int bh = blockIdx.y;
    const int iq = (a.ngroups - 1 - blockIdx.x) * 4 + wave;   // longest causal rows first
    if (iq >= a.T) return;
    const size_t bt = (size_t)bh * a.T;
    const size_t np = (size_t)a.T * BLK;
    const size_t rowbase = bh * np;

    v4i qop[2][2];                                            // B operand of K Q^T: lane = query
    {
        const v4i* src = (const v4i*)(a.q_r + (bt + iq) * 4096);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) qop[qb][ks] = src[(qb * 2 + ks) * 64 + lane];
    }
    v8h doh[2][4];                                            // B operand of V dO^T: lane = query
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            doh[qb][ks] = *(const v8h*)(a.do16 + (rowbase + iq * BLK + 32 * qb + l32) * HD + 16 * ks + 8 * h);
    float lq[2], dlq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        lq[qb] = a.lse2[rowbase + iq * BLK + 32 * qb + l32];
        dlq[qb] = a.delta[rowbase + iq * BLK + 32 * qb + l32];
    }
    const float sQ = a.sq[bt + iq];

    v16f dq[2][2];                                            // [db][qb]: lane = query, regs = channels
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dq[db][qb] = v16f{};

    const int t_end = CAUSAL ? iq : a.T - 1;
    for (int t = 0; t <= t_end; ++t) {
        v4i kop[2][2];                                        // A operand: lane = key
        {
            const v4i* src = (const v4i*)(a.k_r + (bt + t) * 4096);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) kop[kb][ks] = src[(kb * 2 + ks) * 64 + lane];
        }
        const float sK = a.sk[bt + t];
        const float sc = tile_scale(sQ, sK);
        v16i s[2][2];                                         // [kb][qb]: lane = query, regs = keys
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                s[kb][qb] = mfma_i8(kop[kb][0], qop[qb][0], v16i{});
                s[kb][qb] = mfma_i8(kop[kb][1], qop[qb][1], s[kb][qb]);
            }
        float bias[2][16];
        if (SMOOTHQ) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const float4 b4 = *(const float4*)(a.bias + rowbase + t * BLK + 32 * kb + 8 * r4 + 4 * h);
                    bias[kb][4 * r4 + 0] = b4.x;
                    bias[kb][4 * r4 + 1] = b4.y;
                    bias[kb][4 * r4 + 2] = b4.z;
                    bias[kb][4 * r4 + 3] = b4.w;
                }
        }
        const bool need_mask = (CAUSAL && t == iq) || (t == a.T - 1 && (a.N % BLK) != 0);
        float ds[2][2][16];                                   // [kb][qb]
        float dsmax = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            v8h vh[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                vh[ks] = *(const v8h*)(a.v16 + (rowbase + t * BLK + 32 * kb + l32) * HD + 16 * ks + 8 * h);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                v16f dp = mfma_f16(vh[0], doh[qb][0], v16f{});
                dp = mfma_f16(vh[1], doh[qb][1], dp);
                dp = mfma_f16(vh[2], doh[qb][2], dp);
                dp = mfma_f16(vh[3], doh[qb][3], dp);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pv = bwd_prob<SMOOTHQ>(s[kb][qb][r], sc, SMOOTHQ ? bias[kb][r] : 0.0f, lq[qb]);
                    if (need_mask) {
                        const int key = t * BLK + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                        const int q = iq * BLK + 32 * qb + l32;
                        if (key >= a.N || (CAUSAL && key > q)) pv = 0.0f;
                    }
                    const float d = pv * (dp[r] - dlq[qb]);
                    ds[kb][qb][r] = d;
                    dsmax = fmaxf(dsmax, fabsf(d));
                }
            }
        }
        dsmax = wave_max(dsmax);
        float sdS, invdS;
        block_scale(dsmax, sdS, invdS);
        v4i dc[2][2];                                         // [qb][ks]: B operand, k = keys
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint32_t w[4];
#pragma unroll
                for (int d4 = 0; d4 < 4; ++d4)
                    w[d4] = pack4(code_bits(ds[ks][qb][4 * d4 + 0], invdS), code_bits(ds[ks][qb][4 * d4 + 1], invdS),
                                  code_bits(ds[ks][qb][4 * d4 + 2], invdS), code_bits(ds[ks][qb][4 * d4 + 3], invdS));
                dc[qb][ks] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            }
        const v4i* ksrc = (const v4i*)(a.k_t + (bt + t) * 4096);
        const float wq = sdS * sK;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            const v4i k0 = ksrc[(db * 2 + 0) * 64 + lane], k1 = ksrc[(db * 2 + 1) * 64 + lane];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                v16i acc = mfma_i8(k0, dc[qb][0], v16i{});
                acc = mfma_i8(k1, dc[qb][1], acc);
#pragma unroll
                for (int r = 0; r < 16; ++r) dq[db][qb][r] = __builtin_fmaf((float)acc[r], wq, dq[db][qb][r]);
            }
        }
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = iq * BLK + 32 * qb + l32;
        if (q < a.N) {
            uint16_t* row = a.dq + ((size_t)bh * a.N + q) * HD;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = 32 * db + 8 * r4 + 4 * h;
                    const uint32_t w0 = f32_to_bf16_rne(dq[db][qb][4 * r4 + 0] * 0.125f) |
                                        (f32_to_bf16_rne(dq[db][qb][4 * r4 + 1] * 0.125f) << 16);
                    const uint32_t w1 = f32_to_bf16_rne(dq[db][qb][4 * r4 + 2] * 0.125f) |
                                        (f32_to_bf16_rne(dq[db][qb][4 * r4 + 3] * 0.125f) << 16);
                    *(uint2*)(row + d) = make_uint2(w0, w1);
                }
        }
    }
}

int launch_bwd_dkdv(const BwdArgs& a, int BH, bool causal, bool smooth_q, hipStream_t st) {
    dim3 grid(a.ngroups, BH), block(256);
    if (causal) {
        if (smooth_q) hipLaunchKernelGGL((k_bwd_dkdv<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dkdv<true, false>), grid, block, 0, st, a);
    } else {
        if (smooth_q) hipLaunchKernelGGL((k_bwd_dkdv<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dkdv<false, false>), grid, block, 0, st, a);
    }
    return 0;
}

int launch_bwd_dq(const BwdArgs& a, int BH, bool causal, bool smooth_q, hipStream_t st) {
    dim3 grid(a.ngroups, BH), block(256);
    if (causal) {
        if (smooth_q) hipLaunchKernelGGL((k_bwd_dq<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dq<true, false>), grid, block, 0, st, a);
    } else {
        if (smooth_q) hipLaunchKernelGGL((k_bwd_dq<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dq<false, false>), grid, block, 0, st, a);
    }
    return 0;
}

}  // namespace sagebwd
