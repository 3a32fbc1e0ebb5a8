// Fused forward: S^T = K Q^T on INT8 MFMA (i32 accumulation), dequantize,
// online softmax in registers, P~ codes with the fixed scale 1/127 against
// the tile-row maximum, O^T += V^T P~^T on INT8 MFMA, then O and LSE.
//
// SageBwd (abstract): both forward matmuls are among the six INT8 ones.  The
// tile loop and the online softmax (running max, running sum, rescaling)
// follow FlashAttention-2 (under "Builds on" on the SageBwd page).
//
// Work split (gfx950): a workgroup of 4 waves owns 128 query rows (two
// quantization blocks of Q); each wave owns 32 of them.  The K and V code
// tiles of each 64-key step go global -> LDS once per workgroup by DMA
// (buffer loads into LDS, no registers held), double buffered and fetched one
// step ahead, and every wave reads its MFMA operands from there (16 bytes per
// lane per 32x32 operand).  Computing S^T rather than S puts one query per
// lane column, so every softmax row statistic lives in one lane and its
// partner in the other half-wave, and the P~ codes leave the accumulator
// already in the B-operand layout of V^T P~^T.  The causal kernels are held
// to 128 registers per wave (four waves per SIMD), the non-causal ones to 168
// (three: the MXFP8 and FP4 ones spill a few registers there and still run
// 15 % faster than at two waves).  Causal grids start
// the longest query groups of all heads first; non-causal ones deal the
// workgroups of one head to one XCD when the head count allows (its K/V
// codes then stay in that XCD's L2).
#include "attn.h"

namespace sagebwd {

constexpr int FWD_WAVES = 4;

constexpr float RESCALE_THRESHOLD = 8.0f;   // log2 units; O and L may grow by up to 2^8

struct FwdSmem {
    v4i k[2][256];       // K row-operand code tile, 2 buffers
    v4i v[2][256];       // V transposed-operand code tile
    float bias[2][64];   // Q-smoothing key bias (log2 domain)
};

// Maximum of a lane's 32 scores: one chain the compiler turns into v_max3_f32
// (15 of them and one v_max_f32), starting from the first score.
__device__ __forceinline__ float row_max32(const float (&z)[2][16]) {
    float m = __builtin_fmaxf(z[0][0], z[0][1]);
#pragma unroll
    for (int i = 2; i < 32; ++i) m = __builtin_fmaxf(m, z[i / 16][i % 16]);
    return m;
}

// max of two row maxima that come out of a lane swap (bit patterns of
// non-NaN floats): the median of (x, y, +inf) is max(x, y) and, unlike
// fmaxf on values the compiler cannot prove canonical, needs no quieting.
// (+inf goes through an empty asm so the compiler does not turn the median
// back into a maximum that it would then quiet; the asm has no side effects
// and is hoisted out of the loops.)
__device__ __forceinline__ float max2_swapped(uint32_t x, uint32_t y) {
    float inf = __builtin_inff();
    asm("" : "+v"(inf));
    return __builtin_amdgcn_fmed3f(__uint_as_float(x), __uint_as_float(y), inf);
}

// Workgroup -> (head, query group).  Consecutive workgroup ids are dealt to
// the 8 XCDs in turn.  Causal (longest_first): the longest group of every
// head, then the next longest of every head, and so on, so that the longest
// work starts first across the whole grid (head bh stays on XCD bh % 8 when
// the head count is a multiple of 8); dispatching head by head left some of
// the longest groups to start near the end.  Otherwise all groups of a head
// go to the same XCD when the head count allows.
__device__ __forceinline__ void map_group(int ngroups, int BH, int& bh, int& g, bool longest_first = false) {
    const int L = blockIdx.x;
    if (longest_first) {
        bh = L % BH;
        g = ngroups - 1 - L / BH;
    } else if ((BH & 7) == 0) {
        const int xcd = L & 7, s = L >> 3;
        bh = (s / ngroups) * 8 + xcd;
        g = ngroups - 1 - (s % ngroups);
    } else {
        bh = L / ngroups;
        g = ngroups - 1 - (L % ngroups);
    }
}

// One 64-key step of one wave: scores, tile-row max, P~ codes, online update
// and the P~V product.  MASK is set only for the causal diagonal tile and the
// ragged last tile, so the common path carries no per-element selects.
template <bool CAUSAL, bool SMOOTHQ, bool MASK, bool DUMP>
__device__ __forceinline__ void fwd_tile(const FwdSmem& sm, int buf, const v4i (&qop)[2], float sc, float sv,
                                         int t, int q, int N, int lane, int h, float& M, float& L, v16f (&O)[2],
                                         uint8_t* dp, int qloc) {
    v16i s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma_i8(sm.k[buf][(kb * 2 + 0) * 64 + lane], qop[0], v16i{});
        s[kb] = mfma_i8(sm.k[buf][(kb * 2 + 1) * 64 + lane], qop[1], s[kb]);
    }
    if (DUMP && dp) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<int>(dp, dumpoff::A)[qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] = s[kb][r];
    }
    float z[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float bias[16];
        if (SMOOTHQ) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 b4 = *(const float4*)&sm.bias[buf][32 * kb + 8 * r4 + 4 * h];
                bias[4 * r4 + 0] = b4.x;
                bias[4 * r4 + 1] = b4.y;
                bias[4 * r4 + 2] = b4.z;
                bias[4 * r4 + 3] = b4.w;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float af = (float)s[kb][r];
            z[kb][r] = SMOOTHQ ? __builtin_fmaf(af, sc, bias[r]) : af;
            if (MASK) {
                const int key = t * BLK + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                if (key >= N || (CAUSAL && key > q)) z[kb][r] = -__builtin_inff();
            }
        }
    }
    float mx = row_max32(z);
    {
        // after the swap the two registers hold, in every lane, this lane's
        // value and its partner's (lane l ^ 32): their maximum is the row's
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = max2_swapped(sw[0], sw[1]);
    }
    // tile-row max in log2 units; the code is rne(127 * exp2(score - max))
    const float mt = SMOOTHQ ? mx : mx * sc;
    const float off = LOG2_127 - mt;
    const bool row_live = !MASK || mx > -__builtin_inff();
    v4i pc[2];
    uint32_t csum = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        uint32_t w4[4];
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
            uint32_t pk4 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float zz = z[kb][4 * d4 + j];
                float v = __builtin_amdgcn_exp2f(SMOOTHQ ? zz + off : __builtin_fmaf(zz, sc, off));
                if (MASK && !(zz > -__builtin_inff())) v = 0.0f;
                pk4 = __builtin_amdgcn_cvt_pk_u8_f32(v, j, pk4);
                if (DUMP && dp) {
                    const int kk = 32 * kb + 8 * d4 + 4 * h + j;
                    dump_at<float>(dp, dumpoff::F1)[qloc * 64 + kk] = v;
                    dp[dumpoff::C1 + qloc * 64 + kk] = (uint8_t)(pk4 >> (8 * j));
                }
            }
            w4[d4] = pk4;
            csum = __builtin_amdgcn_udot4(pk4, 0x01010101u, csum, false);
        }
        pc[kb] = v4i{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
    }
    // online update with a lazily raised reference max
    if (row_live && mt > M + RESCALE_THRESHOLD) {
        const float alpha = M > -__builtin_inff() ? __builtin_amdgcn_exp2f(M - mt) : 0.0f;
        M = mt;
        L *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    const float e = row_live ? __builtin_amdgcn_exp2f(mt - M) : 0.0f;
    L = __builtin_fmaf(e, (float)csum, L);
    const float wv = e * sv;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        v16i pvacc = mfma_i8(sm.v[buf][(db * 2 + 0) * 64 + lane], pc[0], v16i{});
        pvacc = mfma_i8(sm.v[buf][(db * 2 + 1) * 64 + lane], pc[1], pvacc);
        if (DUMP && dp) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<int>(dp, dumpoff::ACC1)[qloc * 64 + 32 * db + 8 * (r / 4) + 4 * h + (r % 4)] = pvacc[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] = __builtin_fmaf((float)pvacc[r], wv, O[db][r]);
    }
}

template <bool CAUSAL, bool SMOOTHQ, bool DUMP>
__global__ __launch_bounds__(256, CAUSAL ? 4 : 3) void k_fwd(FwdArgs a) {
    __shared__ FwdSmem sm;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    int bh, g;
    map_group(a.ngroups, a.BH, bh, g, CAUSAL);
    const int T = a.T;
    const int qblk = 2 * g + wave / 2, qhalf = wave % 2;
    const bool live = qblk < T;
    const int t_last_wg = CAUSAL ? min(2 * g + 1, T - 1) : T - 1;
    const int t_last = CAUSAL ? qblk : T - 1;
    const bool ragged = (a.N & (BLK - 1)) != 0;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const v4i* kg = (const v4i*)(a.k_r + bt * 4096);
    const v4i* vg = (const v4i*)(a.v_t + bt * 4096);
    const float* bg = a.bias + bh * np;

    v4i qop[2] = {v4i{}, v4i{}};
    float sQ = 0.0f;
    if (live) {
        const v4i* src = (const v4i*)(a.q_r + (bt + qblk) * 4096);
        qop[0] = src[(qhalf * 2 + 0) * 64 + lane];
        qop[1] = src[(qhalf * 2 + 1) * 64 + lane];
        sQ = a.sq[bt + qblk];
    }
    const int q = qblk * BLK + 32 * qhalf + l32;
    uint8_t* dp_sel = (DUMP && bh == a.dump_bh && qblk == a.dump_i) ? a.dump : nullptr;

    // key block t's K and V code blocks (and key bias) -> LDS buffer b by DMA
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const rsrc_t r_k = raw_rsrc(kg, (uint32_t)T * 4096u), r_v = raw_rsrc(vg, (uint32_t)T * 4096u);
    const rsrc_t r_b = raw_rsrc(bg, (uint32_t)T * 256u);
    const uint32_t off16 = 16u * (uint32_t)tid;
    auto fetch = [&](int t, int b) {
        bdma16_to_lds(r_k, off16, (uint32_t)t * 4096u, &sm.k[b][64 * wave_u]);
        bdma16_to_lds(r_v, off16, (uint32_t)t * 4096u, &sm.v[b][64 * wave_u]);
        if (SMOOTHQ && wave_u == 0 && lane < 16)
            bdma16_to_lds(r_b, 16u * (uint32_t)lane, (uint32_t)t * 256u, &sm.bias[b][0]);
    };
    fetch(0, 0);
    wait_vmem();
    lds_barrier();

    float M = -__builtin_inff();   // reference max (log2), raised lazily
    float L = 0.0f;                // sum over tiles of exp2(m_t - M) * (code sum of this half-wave)
    v16f O[2] = {v16f{}, v16f{}};  // [db]: lane = query, registers = channels

    auto step = [&](int t, auto maybe_masked) {
        const int buf = t & 1;
        const bool more = t < t_last_wg;
        // buffer buf ^ 1 was last read in step t - 1, which every wave has
        // finished; the copy is waited for before this step's barrier
        if (more) fetch(t + 1, buf ^ 1);
        if (live && t <= t_last) {
            const float sc = tile_scale(sQ, a.sk[bt + t]);
            const float sv = a.sv[bt + t];
            uint8_t* dp = (DUMP && t == a.dump_t) ? dp_sel : nullptr;
            if (decltype(maybe_masked)::value && ((CAUSAL && t == qblk) || (ragged && t == T - 1)))
                fwd_tile<CAUSAL, SMOOTHQ, true, DUMP>(sm, buf, qop, sc, sv, t, q, a.N, lane, h, M, L, O, dp,
                                                      32 * qhalf + l32);
            else
                fwd_tile<CAUSAL, SMOOTHQ, false, DUMP>(sm, buf, qop, sc, sv, t, q, a.N, lane, h, M, L, O, dp,
                                                       32 * qhalf + l32);
        }
        wait_vmem();
        lds_barrier();
    };
    // Only the last two steps can hold a masked tile (the causal diagonal
    // and the ragged last key block come last), so they run in a loop of
    // their own: the main loop then carries one form of the tile and the
    // compiler keeps O in the same registers across it (with both forms in
    // the loop it copied O between them on every step).
    const int t_tail = t_last_wg > 1 ? t_last_wg - 1 : 0;
    int t = 0;
    for (; t < t_tail; ++t) step(t, Flag<false>{});
    for (; t <= t_last_wg; ++t) step(t, Flag<true>{});

    // epilogue: O / L in bf16; LSE in natural log of the un-smoothed scores
    if (live && q < a.N) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(L), __float_as_uint(L), false, false);
        const float Lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv_l = 1.0f / Lt;
        uint16_t* orow = a.o + ((size_t)bh * a.N + q) * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * h;
                const uint32_t w0 = f32_to_bf16_rne(O[db][4 * r4 + 0] * inv_l) |
                                    (f32_to_bf16_rne(O[db][4 * r4 + 1] * inv_l) << 16);
                const uint32_t w1 = f32_to_bf16_rne(O[db][4 * r4 + 2] * inv_l) |
                                    (f32_to_bf16_rne(O[db][4 * r4 + 3] * inv_l) << 16);
                *(uint2*)(orow + d) = make_uint2(w0, w1);
            }
        if (h == 0) {
            const float lse2 = M + log2f(Lt) - LOG2_127;   // log2 of the row sum of exp2(score)
            a.lse[(size_t)bh * a.N + q] = lse2 * LN2 + a.corr[bh * np + q];
        }
    }
}

// ---------------------------------------------------------------- MXFP8
// The same work split with OCP E4M3 codes and E8M0 block exponents (one per
// 32 tokens x 32 channels) on the scaled FP8 MFMA, which applies the block
// scales inside the instruction: S^T = K Q^T arrives dequantized in float32,
// so no per-tile dequantization multiply remains.  P~ = exp(S - M_t) against
// the running row maximum M_t is coded as E4M3(256 P~) (scale 2^-8 on the
// P~ side of V^T P~^T).  O and the row sum l accumulate in the MFMA
// accumulators themselves (l as the product of an all-ones A operand with
// P~^T, every row of which is the same sum) and are rescaled whenever M_t
// rises.

template <bool CAUSAL, bool SMOOTHQ, bool MASK, bool DUMP>
__device__ __forceinline__ void fwd_tile_mx(const FwdSmem& sm, int buf, v8i qop, int sq_e, uint32_t sk_w,
                                            uint32_t sv_w, int t, int q, int N, int lane, int h, float& M,
                                            v16f (&O)[2], v16f& Lacc, v8i ones, int e_one, int e_pt, uint8_t* dp,
                                            int qloc) {
    v16f s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma_fp8(cat8(sm.k[buf][(kb * 2 + 0) * 64 + lane], sm.k[buf][(kb * 2 + 1) * 64 + lane]), qop,
                         v16f{}, ebyte(sk_w, 2 * kb + h), sq_e);
    if (DUMP && dp) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<float>(dp, dumpoff::A)[qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] = s[kb][r];
    }
    float z[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float bias[16];
        if (SMOOTHQ) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 b4 = *(const float4*)&sm.bias[buf][32 * kb + 8 * r4 + 4 * h];
                bias[4 * r4 + 0] = b4.x;
                bias[4 * r4 + 1] = b4.y;
                bias[4 * r4 + 2] = b4.z;
                bias[4 * r4 + 3] = b4.w;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // log2-domain scores
            z[kb][r] = SMOOTHQ ? __builtin_fmaf(s[kb][r], SCORE_SCALE_LOG2, bias[r]) : s[kb][r] * SCORE_SCALE_LOG2;
            if (MASK) {
                const int key = t * BLK + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                if (key >= N || (CAUSAL && key > q)) z[kb][r] = -__builtin_inff();
            }
        }
    }
    if (DUMP && dp) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<float>(dp, dumpoff::F2)[qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] = z[kb][r];
    }
    float mx = row_max32(z);
    {
        // after the swap the two registers hold, in every lane, this lane's
        // value and its partner's (lane l ^ 32): their maximum is the row's
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = max2_swapped(sw[0], sw[1]);
    }
    // running maximum (log2 units); O and l follow it.  The rescale runs for
    // the whole wave when any of its rows rises (factor 1 for the others), so
    // the accumulators are never updated under a partial execution mask.
    const float mt = mx;
    const bool rise = mt > M;
    if (__builtin_amdgcn_ballot_w64(rise)) {
        const float alpha = !rise ? 1.0f : M > -__builtin_inff() ? __builtin_amdgcn_exp2f(M - mt) : 0.0f;
        M = rise ? mt : M;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
        Lacc[0] *= alpha;   // only register 0 of the row-sum accumulator is read
    }
    const float off = -M;
    if (DUMP && dp && h == 0) dump_at<float>(dp, dumpoff::SC)[qloc] = M;
    v8i pc;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float zz = z[kb][4 * d4 + j];
                v[j] = __builtin_amdgcn_exp2f(zz + off);
                if (MASK && !(zz > -__builtin_inff())) v[j] = 0.0f;
            }
            pc[4 * kb + d4] = (int)fp8_quad(v[0], v[1], v[2], v[3], 0x1p-8f);
            if (DUMP && dp) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = 32 * kb + 8 * d4 + 4 * h + j;
                    dump_at<float>(dp, dumpoff::F1)[qloc * 64 + kk] = v[j];
                    dp[dumpoff::C1 + qloc * 64 + kk] = (uint8_t)((uint32_t)pc[4 * kb + d4] >> (8 * j));
                }
            }
        }
#pragma unroll
    for (int db = 0; db < 2; ++db)
        O[db] = mfma_fp8(cat8(sm.v[buf][(db * 2 + 0) * 64 + lane], sm.v[buf][(db * 2 + 1) * 64 + lane]), pc, O[db],
                         ebyte(sv_w, 2 * h + db), e_pt);
    Lacc = mfma_fp8(ones, pc, Lacc, e_one, e_pt);
}

template <bool CAUSAL, bool SMOOTHQ, bool DUMP>
__global__ __launch_bounds__(256, CAUSAL ? 4 : 3) void k_fwd_mx(FwdArgs a) {
    __shared__ FwdSmem sm;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    int bh, g;
    map_group(a.ngroups, a.BH, bh, g, CAUSAL);
    const int T = a.T;
    const int qblk = 2 * g + wave / 2, qhalf = wave % 2;
    const bool live = qblk < T;
    const int t_last_wg = CAUSAL ? min(2 * g + 1, T - 1) : T - 1;
    const int t_last = CAUSAL ? qblk : T - 1;
    const bool ragged = (a.N & (BLK - 1)) != 0;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const v4i* kg = (const v4i*)(a.k_r + bt * 4096);
    const v4i* vg = (const v4i*)(a.v_t + bt * 4096);
    const float* bg = a.bias + bh * np;
    const uint32_t* skw = (const uint32_t*)a.sk + bt;
    const uint32_t* svw = (const uint32_t*)a.sv + bt;

    // Q codes of this wave's 32 queries (B operand), the exponent of their
    // 32-channel block h
    v8i qop = v8i{};
    int sq_e = E8M0_ONE;
    if (live) {
        const v4i* src = (const v4i*)(a.q_r + (bt + qblk) * 4096);
        qop = cat8(src[(qhalf * 2 + 0) * 64 + lane], src[(qhalf * 2 + 1) * 64 + lane]);
        sq_e = ebyte(((const uint32_t*)a.sq)[bt + qblk], 2 * qhalf + h);
    }
    const int e_one = opaque(E8M0_ONE), e_pt = opaque(E8M0_ONE - 8);
    const v8i ones = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                         0x38383838};
    const int q = qblk * BLK + 32 * qhalf + l32;
    uint8_t* dp_sel = (DUMP && bh == a.dump_bh && qblk == a.dump_i) ? a.dump : nullptr;

    // key block t's K and V code blocks (and key bias) -> LDS buffer b by DMA
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const rsrc_t r_k = raw_rsrc(kg, (uint32_t)T * 4096u), r_v = raw_rsrc(vg, (uint32_t)T * 4096u);
    const rsrc_t r_b = raw_rsrc(bg, (uint32_t)T * 256u);
    const uint32_t off16 = 16u * (uint32_t)tid;
    auto fetch = [&](int t, int b) {
        bdma16_to_lds(r_k, off16, (uint32_t)t * 4096u, &sm.k[b][64 * wave_u]);
        bdma16_to_lds(r_v, off16, (uint32_t)t * 4096u, &sm.v[b][64 * wave_u]);
        if (SMOOTHQ && wave_u == 0 && lane < 16)
            bdma16_to_lds(r_b, 16u * (uint32_t)lane, (uint32_t)t * 256u, &sm.bias[b][0]);
    };
    fetch(0, 0);
    wait_vmem();
    lds_barrier();

    float M = -__builtin_inff();   // running row maximum (log2)
    v16f O[2] = {v16f{}, v16f{}};  // [db]: lane = query, registers = channels
    v16f Lacc = v16f{};            // register 0: the row sum of the dequantized P~

    auto step = [&](int t, auto maybe_masked) {
        const int buf = t & 1;
        const bool more = t < t_last_wg;
        // buffer buf ^ 1 was last read in step t - 1, which every wave has
        // finished; the copy is waited for before this step's barrier
        if (more) fetch(t + 1, buf ^ 1);
        if (live && t <= t_last) {
            const uint32_t sk_w = skw[t], sv_w = svw[t];
            uint8_t* dp = (DUMP && t == a.dump_t) ? dp_sel : nullptr;
            if (decltype(maybe_masked)::value && ((CAUSAL && t == qblk) || (ragged && t == T - 1)))
                fwd_tile_mx<CAUSAL, SMOOTHQ, true, DUMP>(sm, buf, qop, sq_e, sk_w, sv_w, t, q, a.N, lane, h, M, O,
                                                         Lacc, ones, e_one, e_pt, dp, 32 * qhalf + l32);
            else
                fwd_tile_mx<CAUSAL, SMOOTHQ, false, DUMP>(sm, buf, qop, sq_e, sk_w, sv_w, t, q, a.N, lane, h, M, O,
                                                          Lacc, ones, e_one, e_pt, dp, 32 * qhalf + l32);
        }
        wait_vmem();
        lds_barrier();
    };
    // Only the last two steps can hold a masked tile (the causal diagonal
    // and the ragged last key block come last), so they run in a loop of
    // their own: the main loop then carries one form of the tile and the
    // compiler keeps O in the same registers across it (with both forms in
    // the loop it copied O between them on every step).
    const int t_tail = t_last_wg > 1 ? t_last_wg - 1 : 0;
    int t = 0;
    for (; t < t_tail; ++t) step(t, Flag<false>{});
    for (; t <= t_last_wg; ++t) step(t, Flag<true>{});

    if (live && q < a.N) {
        const float Lt = Lacc[0];
        const float inv_l = 1.0f / Lt;
        uint16_t* orow = a.o + ((size_t)bh * a.N + q) * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * h;
                const uint32_t w0 = f32_to_bf16_rne(O[db][4 * r4 + 0] * inv_l) |
                                    (f32_to_bf16_rne(O[db][4 * r4 + 1] * inv_l) << 16);
                const uint32_t w1 = f32_to_bf16_rne(O[db][4 * r4 + 2] * inv_l) |
                                    (f32_to_bf16_rne(O[db][4 * r4 + 3] * inv_l) << 16);
                *(uint2*)(orow + d) = make_uint2(w0, w1);
            }
        if (h == 0) a.lse[(size_t)bh * a.N + q] = (M + log2f(Lt)) * LN2 + a.corr[bh * np + q];
    }
}

// ---------------------------------------------------------------- FP4
// Inference forward on E2M1 codes with one E8M0 exponent per 32 values of the
// contraction index (FP4 blocks of 2048 code bytes + 128 exponent bytes, the
// layouts of the FP4 quantizer), the same work split and online softmax as
// the MXFP8 forward.  A half-wave of the score product holds, for its query,
// the 32 keys of one key class of the tile, which is exactly one FP4 block of
// P~ (and the matching V block): the block maximum and exponent are in-lane.

struct FwdFp4Smem {
    v4i k[2][136];       // K FP4 block: 128 code chunks + 8 chunks of exponents
    v4i v[2][136];       // V FP4 block (class layout)
    float bias[2][64];
};

template <bool CAUSAL, bool SMOOTHQ, bool MASK, bool DUMP>
__device__ __forceinline__ void fwd_tile_fp4(const FwdFp4Smem& sm, int buf, v4i qop, int sq_e, int t, int q, int N,
                                             int lane, int h, int l32, float& M, v16f (&O)[2], v16f& Lacc,
                                             int e_one, uint8_t* dp, int qloc) {
    const uint8_t* kx = (const uint8_t*)sm.k[buf] + FP4_EXP_OFF;
    const uint8_t* vx = (const uint8_t*)sm.v[buf] + FP4_EXP_OFF;
    v16f s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma_fp4(sm.k[buf][kb * 64 + lane], qop, v16f{}, kx[2 * (32 * kb + l32) + h], sq_e);
    if (DUMP && dp) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<float>(dp, dumpoff::A)[qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] = s[kb][r];
    }
    float z[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float bias[16];
        if (SMOOTHQ) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 b4 = *(const float4*)&sm.bias[buf][32 * kb + 8 * r4 + 4 * h];
                bias[4 * r4 + 0] = b4.x;
                bias[4 * r4 + 1] = b4.y;
                bias[4 * r4 + 2] = b4.z;
                bias[4 * r4 + 3] = b4.w;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // log2-domain scores
            z[kb][r] = SMOOTHQ ? __builtin_fmaf(s[kb][r], SCORE_SCALE_LOG2, bias[r]) : s[kb][r] * SCORE_SCALE_LOG2;
            if (MASK) {
                const int key = t * BLK + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                if (key >= N || (CAUSAL && key > q)) z[kb][r] = -__builtin_inff();
            }
        }
    }
    if (DUMP && dp) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<float>(dp, dumpoff::F2)[qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] = z[kb][r];
    }
    float mx = row_max32(z);
    {
        // after the swap the two registers hold, in every lane, this lane's
        // value and its partner's (lane l ^ 32): their maximum is the row's
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = max2_swapped(sw[0], sw[1]);
    }
    const float mt = mx;
    const bool rise = mt > M;
    if (__builtin_amdgcn_ballot_w64(rise)) {
        const float alpha = !rise ? 1.0f : M > -__builtin_inff() ? __builtin_amdgcn_exp2f(M - mt) : 0.0f;
        M = rise ? mt : M;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
        Lacc[0] *= alpha;   // only register 0 of the row-sum accumulator is read
    }
    const float off = -M;
    float p[32];   // value 16 kb + r of this lane's P~ block
    uint32_t pm = 0;   // P~ >= 0: its maximum is the maximum of the bit patterns
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float zz = z[kb][r];
            float v = __builtin_amdgcn_exp2f(zz + off);
            if (MASK && !(zz > -__builtin_inff())) v = 0.0f;
            p[16 * kb + r] = v;
        }
#pragma unroll
    for (int i = 0; i < 32; ++i) pm = max(pm, __float_as_uint(p[i]));
    const int pe = fp4_exponent(__uint_as_float(pm));
    const float psc = pow2f(pe);
    const v4i pc = v4i{(int)fp4_oct(p, psc), (int)fp4_oct(p + 8, psc), (int)fp4_oct(p + 16, psc),
                       (int)fp4_oct(p + 24, psc)};
    if (DUMP && dp) {
        // P~ and its code nibble per [query][key]; the block exponent per
        // [query][key class]; the running maximum per query
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int kk = 32 * (i / 16) + 8 * ((i % 16) / 4) + 4 * h + (i % 4);
            dump_at<float>(dp, dumpoff::F1)[qloc * 64 + kk] = p[i];
            dp[dumpoff::C1 + qloc * 64 + kk] = (uint8_t)(((uint32_t)pc[i / 8] >> (4 * (i % 8))) & 0xFu);
        }
        dump_at<int>(dp, dumpoff::ACC1)[qloc * 2 + h] = pe;
        if (h == 0) dump_at<float>(dp, dumpoff::SC)[qloc] = M;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
        O[db] = mfma_fp4(sm.v[buf][db * 64 + lane], pc, O[db], vx[2 * (32 * db + l32) + h], pe + 127);
    const v4i ones = v4i{(int)E2M1_ONES, (int)E2M1_ONES, (int)E2M1_ONES, (int)E2M1_ONES};
    Lacc = mfma_fp4(ones, pc, Lacc, e_one, pe + 127);
}

template <bool CAUSAL, bool SMOOTHQ, bool DUMP>
__global__ __launch_bounds__(256, CAUSAL ? 4 : 3) void k_fwd_fp4(FwdArgs a) {
    __shared__ FwdFp4Smem sm;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    int bh, g;
    map_group(a.ngroups, a.BH, bh, g, CAUSAL);
    const int T = a.T;
    const int qblk = 2 * g + wave / 2, qhalf = wave % 2;
    const bool live = qblk < T;
    const int t_last_wg = CAUSAL ? min(2 * g + 1, T - 1) : T - 1;
    const int t_last = CAUSAL ? qblk : T - 1;
    const bool ragged = (a.N & (BLK - 1)) != 0;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const v4i* kg = (const v4i*)(a.k_r + bt * 4096);   // 256 chunks per 4096-byte slot, 136 used
    const v4i* vg = (const v4i*)(a.v_t + bt * 4096);
    const float* bg = a.bias + bh * np;

    v4i qop = v4i{};
    int sq_e = E8M0_ONE;
    if (live) {
        const uint8_t* qb = (const uint8_t*)a.q_r + (bt + qblk) * 4096;
        qop = ((const v4i*)qb)[qhalf * 64 + lane];
        sq_e = qb[FP4_EXP_OFF + 2 * (32 * qhalf + l32) + h];
    }
    const int e_one = opaque(E8M0_ONE);
    const int q = qblk * BLK + 32 * qhalf + l32;
    uint8_t* dp_sel = (DUMP && bh == a.dump_bh && qblk == a.dump_i) ? a.dump : nullptr;

    // key block t's K and V FP4 blocks (136 chunks of 16 bytes: waves 0 and
    // 1 and lanes 0-7 of wave 2) and key bias -> LDS buffer b by DMA
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const rsrc_t r_k = raw_rsrc(kg, (uint32_t)T * 4096u), r_v = raw_rsrc(vg, (uint32_t)T * 4096u);
    const rsrc_t r_b = raw_rsrc(bg, (uint32_t)T * 256u);
    const uint32_t off16 = 16u * (uint32_t)tid;
    auto fetch = [&](int t, int b) {
        if (wave_u < 2 || (wave_u == 2 && lane < 8)) {
            bdma16_to_lds(r_k, off16, (uint32_t)t * 4096u, &sm.k[b][64 * wave_u]);
            bdma16_to_lds(r_v, off16, (uint32_t)t * 4096u, &sm.v[b][64 * wave_u]);
        }
        if (SMOOTHQ && wave_u == 3 && lane < 16)
            bdma16_to_lds(r_b, 16u * (uint32_t)lane, (uint32_t)t * 256u, &sm.bias[b][0]);
    };
    fetch(0, 0);
    wait_vmem();
    lds_barrier();

    float M = -__builtin_inff();
    v16f O[2] = {v16f{}, v16f{}};
    v16f Lacc = v16f{};

    auto step = [&](int t, auto maybe_masked) {
        const int buf = t & 1;
        const bool more = t < t_last_wg;
        // buffer buf ^ 1 was last read in step t - 1, which every wave has
        // finished; the copy is waited for before this step's barrier
        if (more) fetch(t + 1, buf ^ 1);
        if (live && t <= t_last) {
            uint8_t* dp = (DUMP && t == a.dump_t) ? dp_sel : nullptr;
            if (decltype(maybe_masked)::value && ((CAUSAL && t == qblk) || (ragged && t == T - 1)))
                fwd_tile_fp4<CAUSAL, SMOOTHQ, true, DUMP>(sm, buf, qop, sq_e, t, q, a.N, lane, h, l32, M, O, Lacc,
                                                          e_one, dp, 32 * qhalf + l32);
            else
                fwd_tile_fp4<CAUSAL, SMOOTHQ, false, DUMP>(sm, buf, qop, sq_e, t, q, a.N, lane, h, l32, M, O, Lacc,
                                                           e_one, dp, 32 * qhalf + l32);
        }
        wait_vmem();
        lds_barrier();
    };
    // Only the last two steps can hold a masked tile (the causal diagonal
    // and the ragged last key block come last), so they run in a loop of
    // their own: the main loop then carries one form of the tile and the
    // compiler keeps O in the same registers across it (with both forms in
    // the loop it copied O between them on every step).
    const int t_tail = t_last_wg > 1 ? t_last_wg - 1 : 0;
    int t = 0;
    for (; t < t_tail; ++t) step(t, Flag<false>{});
    for (; t <= t_last_wg; ++t) step(t, Flag<true>{});

    if (live && q < a.N) {
        const float Lt = Lacc[0];
        const float inv_l = 1.0f / Lt;
        uint16_t* orow = a.o + ((size_t)bh * a.N + q) * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * h;
                const uint32_t w0 = f32_to_bf16_rne(O[db][4 * r4 + 0] * inv_l) |
                                    (f32_to_bf16_rne(O[db][4 * r4 + 1] * inv_l) << 16);
                const uint32_t w1 = f32_to_bf16_rne(O[db][4 * r4 + 2] * inv_l) |
                                    (f32_to_bf16_rne(O[db][4 * r4 + 3] * inv_l) << 16);
                *(uint2*)(orow + d) = make_uint2(w0, w1);
            }
        if (h == 0) a.lse[(size_t)bh * a.N + q] = (M + log2f(Lt)) * LN2 + a.corr[bh * np + q];
    }
}

int launch_fwd(const FwdArgs& a, int BH, bool causal, bool smooth_q, int fmt, hipStream_t st, bool dump) {
    dim3 grid(a.ngroups * BH), block(64 * FWD_WAVES);
    if (fmt == FMT_FP4) {
#define SAGEBWD_FWD_FP4(C, S)                                                                    \
    do {                                                                                         \
        if (dump) hipLaunchKernelGGL((k_fwd_fp4<C, S, true>), grid, block, 0, st, a);            \
        else hipLaunchKernelGGL((k_fwd_fp4<C, S, false>), grid, block, 0, st, a);                \
    } while (0)
        if (causal) {
            if (smooth_q) SAGEBWD_FWD_FP4(true, true);
            else SAGEBWD_FWD_FP4(true, false);
        } else {
            if (smooth_q) SAGEBWD_FWD_FP4(false, true);
            else SAGEBWD_FWD_FP4(false, false);
        }
#undef SAGEBWD_FWD_FP4
        return 0;
    }
    if (fmt == FMT_MXFP8) {
#define SAGEBWD_FWD_MX(C, S)                                                                     \
    do {                                                                                         \
        if (dump) hipLaunchKernelGGL((k_fwd_mx<C, S, true>), grid, block, 0, st, a);             \
        else hipLaunchKernelGGL((k_fwd_mx<C, S, false>), grid, block, 0, st, a);                 \
    } while (0)
        if (causal) {
            if (smooth_q) SAGEBWD_FWD_MX(true, true);
            else SAGEBWD_FWD_MX(true, false);
        } else {
            if (smooth_q) SAGEBWD_FWD_MX(false, true);
            else SAGEBWD_FWD_MX(false, false);
        }
#undef SAGEBWD_FWD_MX
        return 0;
    }
#define SAGEBWD_FWD(C, S)                                                                        \
    do {                                                                                         \
        if (dump) hipLaunchKernelGGL((k_fwd<C, S, true>), grid, block, 0, st, a);                \
        else hipLaunchKernelGGL((k_fwd<C, S, false>), grid, block, 0, st, a);                    \
    } while (0)
    if (causal) {
        if (smooth_q) SAGEBWD_FWD(true, true);
        else SAGEBWD_FWD(true, false);
    } else {
        if (smooth_q) SAGEBWD_FWD(false, true);
        else SAGEBWD_FWD(false, false);
    }
#undef SAGEBWD_FWD
    return 0;
}

}  // namespace sagebwd
