// Backward: recompute S on INT8 MFMA, P = exp(S - LSE), P codes per 64x64
// tile, dV = P^T dO on INT8 MFMA, dP = dO V^T on FP16 MFMA, dS = P*(dP-Delta),
// dS codes per 64x64 tile, dK = dS^T Q and dQ = dS K on INT8 MFMA.
//
// SageBwd (abstract): five of the six INT8 matmuls are in the backward, and
// the score gradient dS is where quantization error mainly arises; the
// SageAttention3 summary ("Approach", the ablation table, "Surprising
// findings") keeps dO V^T in FP16 because quantizing it hurts dQ.  The
// gradient formulas are FlashAttention-2's (under "Builds on").
//
// Two kernels, no atomics, bitwise repeatable:
//   k_bwd_dkdv  a workgroup of 4 waves owns two 64-key blocks (each wave 32
//               keys) and walks the query blocks.  It computes S (lane = key),
//               so P and dS codes leave the accumulator as the A operand of
//               P^T dO and dS^T Q (contraction over queries).  It also stores
//               every tile's dS codes and scale in the workspace.
//   k_bwd_dq    each wave owns one 64-query block and streams its stored dS
//               codes: dQ = sum_t s_dS s_K (dS codes K codes), with no
//               recomputation of S, P or dS; the four waves of a workgroup
//               share each key block's K^T codes through LDS.
// A 64x64 quantization tile of P or dS is held by a pair of waves, which
// exchange their partial maxima through LDS.  The streamed operand tiles go
// through double-buffered LDS, fetched one step ahead; FP16 rows are stored
// with their 16-byte chunks XOR-swizzled by row so column reads do not
// collide on LDS banks.
#include "attn.h"

namespace sagebwd {

constexpr int BWD_WAVES = 4;

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 32 lanes of this lane's half of the wave (its pair of 16-lane
// rows), returned in each of them with the same bits: DPP within each row,
// then the row pair through v_permlane16_swap (both lanes add the two row
// sums in the same order).
__device__ __forceinline__ float half_sum32(float v) {
    v += dppf<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dppf<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dppf<0x141>(v);   // row_half_mirror
    v += dppf<0x140>(v);   // row_mirror
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Maximum over the 64 lanes of a wave of non-negative floats, returned as a
// uniform value.  Non-negative floats order like their bit patterns, so the
// reduction runs on unsigned integers: DPP within each 16-lane row, then two
// DPP row broadcasts that leave the maximum in lane 63, read once.
__device__ __forceinline__ float wave_max64(float f) {
    uint32_t v = __float_as_uint(f);
    v = umax(v, dppu<0xB1>(v));    // quad_perm [1,0,3,2]
    v = umax(v, dppu<0x4E>(v));    // quad_perm [2,3,0,1]
    v = umax(v, dppu<0x141>(v));   // row_half_mirror
    v = umax(v, dppu<0x140>(v));   // row_mirror
    // every lane of a row holds the row's maximum; row_bcast:15 folds row 0
    // into row 1 and row 2 into row 3, row_bcast:31 row 1 into rows 2 and 3,
    // so lane 63 ends with the wave's maximum (rows outside the row mask keep
    // their own value)
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return __uint_as_float(__builtin_amdgcn_readlane(v, 63));
}

// Four signed codes rne(x * inv) packed into one dword.
__device__ __forceinline__ int pack_codes(float x0, float x1, float x2, float x3, float inv) {
    return (int)pack4(code_bits(x0, inv), code_bits(x1, inv), code_bits(x2, inv), code_bits(x3, inv));
}

// FP16 rows of 8 chunks of 16 bytes in LDS: chunk c of row r sits at slot
// c ^ ((r / 2) % 8), so any 16 consecutive rows read at one chunk cover all
// 64 banks (with c ^ (r % 8), rows r and r + 8 would collide).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Global -> LDS copies that bypass the registers (global_load_lds): every
// lane of the wave moves 16 (4) bytes from its own global address to
// lds_wave_base + 16 (4) * lane.  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16_to_lds(const void* g, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void* g, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}
// Wait for this wave's outstanding vector-memory loads (LDS DMA included).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then s_barrier (a compiler memory barrier too).  Unlike
// __syncthreads() it does not wait for this wave's global stores; the DMA
// into LDS is waited for explicitly before it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// Workgroup -> (head, group) as in the forward: causal grids deal the
// longest group of every head first (longest_first), others keep the groups
// of a head on one XCD when the head count allows.  first_small selects which
// groups are longest (smallest index first for the key-block kernel, whose
// causal work is largest at small key blocks).
__device__ __forceinline__ void map_group_bwd(int ngroups, int BH, bool first_small, int& bh, int& g,
                                              bool longest_first = false) {
    const int L = blockIdx.x;
    int s_in_head;
    if (longest_first) {
        // every head's largest group first, then the next: the longest
        // causal work starts earliest; head bh still runs on XCD bh % 8
        bh = L % BH;
        s_in_head = L / BH;
    } else if ((BH & 7) == 0) {
        const int xcd = L & 7, s = L >> 3;
        bh = (s / ngroups) * 8 + xcd;
        s_in_head = s % ngroups;
    } else {
        bh = L / ngroups;
        s_in_head = L % ngroups;
    }
    g = first_small ? s_in_head : ngroups - 1 - s_in_head;
}

// ------------------------------------------------------------------ dK, dV

struct DkdvSmem {
    v4i q_r[2][256];     // Q row-operand codes (A operand of Q K^T)
    v4i q_t[2][256];     // Q transposed codes (B operand of dS^T Q)
    v4i do_t[2][256];    // dO transposed codes (B operand of P^T dO)
    v8h do16[2][512];    // dO in FP16, [64 rows][8 chunks], swizzled (A operand of dO V^T)
    float lse2[2][128];  // [0, 64): log2-domain LSE, [64, 128): -Delta of the query block
    float qs[2][4];      // [0]: Q block scale, [1]: dO block scale
    float red[2][4];     // partial tile maxima of P [0] and dS [1], per wave
};

// P for one 64-query x 32-key half tile in the S layout (lane = key,
// registers = queries): P = exp2(sc A + (bias_j - lse2_i)), log2 domain.  The
// outer difference bias_j - lse2_i is the rank-2 product [-lse2 | 1] [1 | bias]^T,
// formed on the FP32 MFMA (32x32x2: lane l carries A[l%32][l/32] and
// B[l/32][l%32]) in the accumulator layout of the score product, so each score
// costs one FMA before its exp.  MASK only on the causal diagonal tile and the
// ragged last key block, so the common path carries no per-element selects
// (a masked P is a select after its exp, not a branch around it).
// dP - Delta (the same layout) is formed here too: it does not depend on P, so
// its MFMAs are scheduled one by one between groups of the score arithmetic
// instead of stalling the wave later.
template <bool CAUSAL, bool MASK, bool INT8DP>
__device__ __forceinline__ void dkdv_probs(const DkdvSmem& sm, int buf, const v4i (&kop)[2], float sc, float brow,
                                           int i, int key, int N, int lane, int h, float (&p)[2][16],
                                           v16f (&dpd)[2], const v8h (&vh)[4], const v4i (&vop)[2], float sV,
                                           uint8_t* dp = nullptr) {
    // all operands first (the LSE row is read by every lane, so no divergent
    // branch splits the reads from the MFMAs), then both query halves' MFMAs
    v4i qa[2][2];
    float lv[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        qa[qb][0] = sm.q_r[buf][(qb * 2 + 0) * 64 + lane];
        qa[qb][1] = sm.q_r[buf][(qb * 2 + 1) * 64 + lane];
        lv[qb] = sm.lse2[buf][32 * qb + lane % 32];
        asm volatile("" : "+v"(lv[qb]));
    }
    v16i s[2];
    v16f corr[2];
    s[0] = mfma_i8(qa[0][0], kop[0], v16i{});
    s[1] = mfma_i8(qa[1][0], kop[0], v16i{});
    s[0] = mfma_i8(qa[0][1], kop[1], s[0]);
    s[1] = mfma_i8(qa[1][1], kop[1], s[1]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
        corr[qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(h == 0 ? -lv[qb] : 1.0f, brow, v16f{}, 0, 0, 0);
    if (!INT8DP) __builtin_amdgcn_sched_barrier(0);   // score MFMAs issue before everything below
    // dP - Delta = dO V^T + (-Delta) on the FP16 MFMA with -Delta as the
    // accumulator input (all-INT8: s_dO s_V (dO codes V codes^T) + (-Delta))
    const int l32 = lane % 32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = 32 * qb + l32;
        v16f nd;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float4 d4 = *(const float4*)&sm.lse2[buf][64 + 32 * qb + 8 * r4 + 4 * h];
            nd[4 * r4 + 0] = d4.x;
            nd[4 * r4 + 1] = d4.y;
            nd[4 * r4 + 2] = d4.z;
            nd[4 * r4 + 3] = d4.w;
        }
        if (INT8DP) {
            const v4i* dor = (const v4i*)sm.do16[buf];
            v16i ai = mfma_i8(dor[(qb * 2 + 0) * 64 + lane], vop[0], v16i{});
            ai = mfma_i8(dor[(qb * 2 + 1) * 64 + lane], vop[1], ai);
            const float wdp = sm.qs[buf][1] * sV;
#pragma unroll
            for (int r = 0; r < 16; ++r) dpd[qb][r] = __builtin_fmaf((float)ai[r], wdp, nd[r]);
        } else {
            v16f d = mfma_f16(sm.do16[buf][swz(row, 0 + h)], vh[0], nd);
            d = mfma_f16(sm.do16[buf][swz(row, 2 + h)], vh[1], d);
            d = mfma_f16(sm.do16[buf][swz(row, 4 + h)], vh[2], d);
            dpd[qb] = mfma_f16(sm.do16[buf][swz(row, 6 + h)], vh[3], d);
        }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if (dp) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<int>(dp, dumpoff::A)[(32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] = s[qb][r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[qb][r], sc, corr[qb][r]));
            if (MASK) {
                // a select, not a branch around each exp
                asm volatile("" : "+v"(pv));
                const int q = i * BLK + 32 * qb + 8 * (r / 4) + 4 * h + (r % 4);
                pv = (key >= N || (CAUSAL && key > q)) ? 0.0f : pv;
            }
            p[qb][r] = pv;
        }
    }
    if (!INT8DP) {
        // the score MFMAs first, then each dP MFMA between groups of exps
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
        }
    }
}

template <bool CAUSAL, bool SMOOTHQ, bool INT8DP, bool DUMP>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv(BwdArgs a) {
    __shared__ DkdvSmem sm;
    const int tid = threadIdx.x, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: per-wave values live in SGPRs
    int bh, g;
    map_group_bwd(a.ngroups, a.BH, true, bh, g, CAUSAL);
    const int T = a.T;
    const int kvb = 2 * g + wave / 2, kh = wave % 2;
    const bool live = kvb < T;
    const int key = kvb * BLK + 32 * kh + l32;                // this lane's key (S layout)
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const size_t rowbase = bh * np;

    // persistent operands of this wave's 32 keys: K codes, and V in FP16 (or,
    // for the all-INT8 dO V^T, V codes and the V block scale)
    v4i kop[2] = {v4i{}, v4i{}}, vop[2] = {v4i{}, v4i{}};
    v8h vh[4];
    float kbias = 0.0f, sK = 0.0f, sV = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vh[ks] = v8h{};
    if (live) {
        const v4i* src = (const v4i*)(a.k_r + (bt + kvb) * 4096);
        kop[0] = src[(kh * 2 + 0) * 64 + lane];
        kop[1] = src[(kh * 2 + 1) * 64 + lane];
        if (INT8DP) {
            const v4i* vs = (const v4i*)(a.v_r + (bt + kvb) * 4096);
            vop[0] = vs[(kh * 2 + 0) * 64 + lane];
            vop[1] = vs[(kh * 2 + 1) * 64 + lane];
            sV = a.sv[bt + kvb];
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) vh[ks] = *(const v8h*)(a.v16 + (rowbase + key) * HD + 16 * ks + 8 * h);
        }
        if (SMOOTHQ) kbias = a.bias[rowbase + key];
        sK = a.sk[bt + kvb];
    }
    const float brow = h == 0 ? 1.0f : kbias;   // B operand of the rank-2 score correction

    const int i0 = CAUSAL ? min(2 * g, T - 1) : 0;
    // query block i -> LDS buffer b by DMA; LDS slot s of the FP16 dO tile
    // holds global chunk (s / 8, (s % 8) ^ (s / 16 % 8)), the swizzled layout
    // (the all-INT8 dO V^T stages the dO row-operand codes there instead)
    const v4i* qrg = (const v4i*)(a.q_r + bt * 4096);
    const v4i* qtg = (const v4i*)(a.q_t + bt * 4096);
    const v4i* dtg = (const v4i*)(a.do_t + bt * 4096);
    auto fetch = [&](int i, int b) {
        dma16_to_lds(qrg + (size_t)i * 256 + tid, &sm.q_r[b][64 * wave]);
        dma16_to_lds(qtg + (size_t)i * 256 + tid, &sm.q_t[b][64 * wave]);
        dma16_to_lds(dtg + (size_t)i * 256 + tid, &sm.do_t[b][64 * wave]);
        if (INT8DP) {
            dma16_to_lds((const v4i*)(a.do_r + bt * 4096) + (size_t)i * 256 + tid, (v4i*)sm.do16[b] + 64 * wave);
        } else {
            const v4i* hs = (const v4i*)(a.do16 + (rowbase + (size_t)i * BLK) * HD);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int s = 256 * j + tid, row = s / 8;
                dma16_to_lds(hs + row * 8 + ((s % 8) ^ ((row >> 1) & 7)), (v4i*)sm.do16[b] + 256 * j + 64 * wave);
            }
        }
        if (wave == 0 && lane < 32)
            dma16_to_lds((lane < 16 ? a.lse2 : a.delta) + rowbase + (size_t)i * BLK + 4 * (lane % 16), &sm.lse2[b][0]);
        if (wave == 1 && lane < 2) dma4_to_lds((lane == 0 ? a.sq : a.sdo) + bt + i, &sm.qs[b][0]);
    };

    v16f dk[2] = {v16f{}, v16f{}}, dv[2] = {v16f{}, v16f{}};   // [db]: lane = channel, regs = keys
    float gsum = 0.0f;                                          // sum_i s_dS colsum(dS codes), this half

    // the dS codes of the previous query block: stored just after the next
    // block's DMA has been waited for, so that the stores complete during
    // the following compute instead of delaying that wait
    v4i dc_prev[2] = {v4i{}, v4i{}};
    float sds_prev = 0.0f;
    size_t tix_prev = 0;
    bool have_prev = false;
    auto store_prev = [&]() {
        // streaming stores: the codes are read once, by the dQ kernel
        v4i* dst = (v4i*)(a.ds_codes + tix_prev * 4096) + kh * 128 + lane;
        __builtin_nontemporal_store(dc_prev[0], dst);
        __builtin_nontemporal_store(dc_prev[1], dst + 64);
        if (lane == 0) a.ds_scale[tix_prev] = sds_prev;   // both waves of the tile write the same value
    };

    fetch(i0, 0);
    wait_vmem();
    lds_barrier();
    const bool ragged_keys = (kvb == T - 1) && (a.N & (BLK - 1)) != 0;
    for (int i = i0; i < T; ++i) {
        const int buf = (i - i0) & 1;
        const bool more = i + 1 < T;
        const bool active = live && (!CAUSAL || i >= kvb);
        const bool masked = (CAUSAL && i == kvb) || ragged_keys;
        float p[2][16];                      // [qb]: lane = key, regs = queries
        const float sQ = sm.qs[buf][0];
        const float sc = tile_scale(sQ, sK);
        uint8_t* dp = (DUMP && bh == a.dump_bh && kvb == a.dump_t && i == a.dump_i) ? a.dump : nullptr;
        v16f dpe[2];
        if (active) {
            if (masked)
                dkdv_probs<CAUSAL, true, INT8DP>(sm, buf, kop, sc, brow, i, key, a.N, lane, h, p, dpe, vh, vop, sV,
                                                 DUMP ? dp : nullptr);
            else
                dkdv_probs<CAUSAL, false, INT8DP>(sm, buf, kop, sc, brow, i, key, a.N, lane, h, p, dpe, vh, vop, sV,
                                                  DUMP ? dp : nullptr);
            if (DUMP && dp) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<float>(dp, dumpoff::F1)[(32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] = p[qb][r];
            }
            // P >= 0: its maximum is the maximum of the bit patterns
            uint32_t pm0 = 0, pm1 = 0;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                pm0 = umax(pm0, umax(__float_as_uint(p[0][r]), __float_as_uint(p[0][r + 1])));
                pm1 = umax(pm1, umax(__float_as_uint(p[1][r]), __float_as_uint(p[1][r + 1])));
            }
            const float pm = wave_max64(__uint_as_float(umax(pm0, pm1)));
            if (lane == 0) sm.red[0][wave] = pm;
        }
        // the next query block goes to the other buffer by DMA
        if (more) fetch(i + 1, buf ^ 1);
        wait_vmem();
        lds_barrier();
        if (have_prev) store_prev();
        have_prev = false;
        float dsm = 0.0f;
        if (active) {
            float sP, invP;
            // both partial maxima are >= 0: the larger is the larger bit pattern
            block_scale(__uint_as_float(umax(__float_as_uint(sm.red[0][wave]), __float_as_uint(sm.red[0][wave ^ 1]))),
                        sP, invP);
            // dV += s_P s_dO (P codes^T dO codes)
            v4i pc[2];
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
                pc[qs] = v4i{pack_codes(p[qs][0], p[qs][1], p[qs][2], p[qs][3], invP),
                             pack_codes(p[qs][4], p[qs][5], p[qs][6], p[qs][7], invP),
                             pack_codes(p[qs][8], p[qs][9], p[qs][10], p[qs][11], invP),
                             pack_codes(p[qs][12], p[qs][13], p[qs][14], p[qs][15], invP)};
            if (DUMP && dp) {
                if (lane == 0 && kh == 0) dump_at<float>(dp, dumpoff::SC)[0] = sP;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dp[dumpoff::C1 + (32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] =
                            (uint8_t)code_bits(p[qb][r], invP);
            }
            const float wv = sP * sm.qs[buf][1];
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                v16i acc = mfma_i8(pc[0], sm.do_t[buf][(db * 2 + 0) * 64 + lane], v16i{});
                acc = mfma_i8(pc[1], sm.do_t[buf][(db * 2 + 1) * 64 + lane], acc);
                if (DUMP && dp) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<int>(dp, dumpoff::ACC1)[(32 * kh + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + 32 * db + l32] = acc[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dv[db][r] = __builtin_fmaf((float)acc[r], wv, dv[db][r]);
            }
            // dS = P * (dP - Delta) in place of P
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) p[qb][r] = p[qb][r] * dpe[qb][r];
            {
                float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    m0 = max_abs2f(m0, p[0][r], p[0][r + 1]);
                    m1 = max_abs2f(m1, p[1][r], p[1][r + 1]);
                }
                dsm = wave_max64(max3f(m0, m1, m1));
            }
            if (lane == 0) sm.red[1][wave] = dsm;
            if (DUMP && dp) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<float>(dp, dumpoff::F2)[(32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] = p[qb][r];
            }
        }
        lds_barrier();
        if (active) {
            float sdS, invdS;
            block_scale(__uint_as_float(umax(__float_as_uint(sm.red[1][wave]), __float_as_uint(sm.red[1][wave ^ 1]))),
                        sdS, invdS);
            if (DUMP && dp) {
                if (lane == 0 && kh == 0) dump_at<float>(dp, dumpoff::SC)[1] = sdS;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dp[dumpoff::C2 + (32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] =
                            (uint8_t)code_bits(p[qb][r], invdS);
            }
            v4i dc[2];
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
                dc[qs] = v4i{pack_codes(p[qs][0], p[qs][1], p[qs][2], p[qs][3], invdS),
                             pack_codes(p[qs][4], p[qs][5], p[qs][6], p[qs][7], invdS),
                             pack_codes(p[qs][8], p[qs][9], p[qs][10], p[qs][11], invdS),
                             pack_codes(p[qs][12], p[qs][13], p[qs][14], p[qs][15], invdS)};
            // hand the tile's codes and scale to the dQ kernel: 16-byte chunk
            // (kh * 2 + qs) * 64 + lane of the tile holds this lane's key with
            // the 16 queries of dc[qs] (the A-operand layout of dS^T Q)
            dc_prev[0] = dc[0];
            dc_prev[1] = dc[1];
            sds_prev = sdS;
            tix_prev = (size_t)bh * a.ntiles + ds_tile_index(CAUSAL, i, kvb, T);
            have_prev = true;
            if (SMOOTHQ) {
                int cs = 0;
#pragma unroll
                for (int qs = 0; qs < 2; ++qs)
#pragma unroll
                    for (int d4 = 0; d4 < 4; ++d4) cs = __builtin_amdgcn_sdot4(dc[qs][d4], 0x01010101, cs, false);
                gsum = __builtin_fmaf((float)cs, sdS, gsum);
            }
            const float wk = sdS * sQ;
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                v16i acc = mfma_i8(dc[0], sm.q_t[buf][(db * 2 + 0) * 64 + lane], v16i{});
                acc = mfma_i8(dc[1], sm.q_t[buf][(db * 2 + 1) * 64 + lane], acc);
                if (DUMP && dp) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<int>(dp, dumpoff::ACC2)[(32 * kh + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + 32 * db + l32] = acc[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dk[db][r] = __builtin_fmaf((float)acc[r], wk, dk[db][r]);
            }
        }
        lds_barrier();
    }
    if (have_prev) store_prev();

    // epilogue: dK (x 1/8, plus colsum(dS) mu_q for Q-smoothing) and dV in bf16;
    // lane = channel, registers = keys of this wave's half block
    if (!live) return;
    float gfull = 0.0f;
    if (SMOOTHQ) {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(gsum), __float_as_uint(gsum), false, false);
        gfull = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const float muq = SMOOTHQ ? a.mu_q[(size_t)bh * HD + 32 * db + l32] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float gk = SMOOTHQ ? __shfl(gfull, 8 * (r / 4) + 4 * h + (r % 4), 64) : 0.0f;
            dk[db][r] = (SMOOTHQ ? __builtin_fmaf(gk, muq, dk[db][r]) : dk[db][r]) * 0.125f;
        }
    }
    if (a.rk) {
        // QK-norm: dK = r (dK_n - K_n mean_c(dK_n K_n)).  A key's 64 channels
        // are two registers in each of the 32 lanes of this half.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = kvb * BLK + 32 * kh + 8 * (r / 4) + 4 * h + (r % 4);
            const bool ok = kk < a.N;
            const float rr = ok ? a.rk[rowbase + kk] : 0.0f;
            const uint16_t* krow = a.k_in + ((size_t)bh * a.N + (ok ? kk : 0)) * HD;
            const float kn0 = ok ? qk_normed(krow[l32], rr) : 0.0f;
            const float kn1 = ok ? qk_normed(krow[32 + l32], rr) : 0.0f;
            const float mean = half_sum32(__builtin_fmaf(dk[1][r], kn1, dk[0][r] * kn0)) * (1.0f / HD);
            dk[0][r] = rr * __builtin_fmaf(-kn0, mean, dk[0][r]);
            dk[1][r] = rr * __builtin_fmaf(-kn1, mean, dk[1][r]);
        }
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int d = 32 * db + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = kvb * BLK + 32 * kh + 8 * (r / 4) + 4 * h + (r % 4);
            if (kk < a.N) {
                a.dk[((size_t)bh * a.N + kk) * HD + d] = (uint16_t)f32_to_bf16_rne(dk[db][r]);
                a.dv[((size_t)bh * a.N + kk) * HD + d] = (uint16_t)f32_to_bf16_rne(dv[db][r]);
            }
        }
    }
}

// ------------------------------------------------------------------ dQ

// dQ from the dS codes and scales the key-block kernel stored: for each key
// block t, dQ_i += s_dS(i,t) s_K,t (dS codes(i,t) K codes_t), so nothing is
// recomputed.  The stored codes hold, per lane, one key and 16 queries (the
// layout in which the key-block kernel contracts over queries); dQ contracts
// over keys, so each 32x32 code block is first transposed on the MFMA
// itself, as the product with an INT8 identity matrix: D = A I puts query n
// in lane n and keys 8(r/4) + 4h + r%4 in register r, exact small integers
// whose low bytes are the codes in the B-operand layout of K^T dS^T.
//
// Each wave owns one 64-query block: per key block it streams the 4 KB dS
// code tile of its block (HBM, read once, prefetched DQ_DEPTH key blocks
// ahead) and reads the 4 KB K^T code block of the key block, which every
// query block of the head needs.  The K^T reads from L2, not the dS stream,
// bounded an earlier form with 32 queries per wave and one K^T read per wave;
// here each K^T block serves 64 queries, and the four waves of a workgroup
// (four consecutive query blocks, so nearly the same key-block range) share
// one copy staged through LDS, loaded a quarter per wave.

constexpr int DQ_DEPTH = 3;
constexpr int DQ_BLOCKS_PER_WG = 4;   // one query block per wave

struct DqStep {
    v4i ds[2][2];  // [qs][kh]: dS codes of query half qs, key half kh (A operand, lane = key)
    v4i kq;        // this wave's quarter of the K^T code block (INT8 kernel)
    float sds, sk; // s_dS(i, t) and s_K,t (MXFP8 kernel: their exponent words)
};

// Vector loads the compiler does not track (inline assembly): the INT8 dQ
// kernel waits for them itself with dq_wait, which names the registers of a
// ring slot as operands so that no use of them can move above the wait.
// (The compiler's own wait counts lose precision around the prefetch loop and
// fall back to waiting for every load in flight.)
__device__ __forceinline__ v4i gload_nt(const v4i* p) {
    v4i r;
    asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(r) : "v"(p));
    return r;
}
__device__ __forceinline__ v4i gload(const v4i* p) {
    v4i r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p));
    return r;
}
__device__ __forceinline__ float gload1(const float* p) {
    float r;
    asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p));
    return r;
}
// Wait until at most N of this wave's vector loads are outstanding.
template <int N>
__device__ __forceinline__ void dq_wait(DqStep& s) {
    asm volatile("s_waitcnt vmcnt(%7)"
                 : "+v"(s.ds[0][0]), "+v"(s.ds[0][1]), "+v"(s.ds[1][0]), "+v"(s.ds[1][1]), "+v"(s.kq), "+v"(s.sds),
                   "+v"(s.sk)
                 : "n"(N));
}

// dQ (x 1/8) in bf16; with QK-norm dQ = r (dQ_n - Q_n mean_c(dQ_n Q_n)), the
// other 32 channels of this lane's query being in the other half of the wave.
__device__ __forceinline__ void dq_epilogue(const BwdArgs& a, v16f (&dq)[2], int bh, int q, int h, size_t rowbase) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[db][r] *= 0.125f;
    const bool qok = q < a.N;
    if (a.rq) {
        const float rr = qok ? a.rq[rowbase + q] : 0.0f;
        const uint16_t* qrow = a.q_in + ((size_t)bh * a.N + (qok ? q : 0)) * HD;
        float qn[2][16];
        float part = 0.0f;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const uint2 u = qok ? *(const uint2*)(qrow + 32 * db + 8 * r4 + 4 * h) : make_uint2(0, 0);
                qn[db][4 * r4 + 0] = qk_normed(u.x & 0xFFFFu, rr);
                qn[db][4 * r4 + 1] = qk_normed(u.x >> 16, rr);
                qn[db][4 * r4 + 2] = qk_normed(u.y & 0xFFFFu, rr);
                qn[db][4 * r4 + 3] = qk_normed(u.y >> 16, rr);
#pragma unroll
                for (int j = 0; j < 4; ++j) part = __builtin_fmaf(dq[db][4 * r4 + j], qn[db][4 * r4 + j], part);
            }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        const float mean = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * (1.0f / HD);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) dq[db][r] = rr * __builtin_fmaf(-qn[db][r], mean, dq[db][r]);
    }
    if (qok) {
        uint16_t* row = a.dq + ((size_t)bh * a.N + q) * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * h;
                const uint32_t w0 = f32_to_bf16_rne(dq[db][4 * r4 + 0]) | (f32_to_bf16_rne(dq[db][4 * r4 + 1]) << 16);
                const uint32_t w1 = f32_to_bf16_rne(dq[db][4 * r4 + 2]) | (f32_to_bf16_rne(dq[db][4 * r4 + 3]) << 16);
                *(uint2*)(row + d) = make_uint2(w0, w1);
            }
    }
}

template <bool CAUSAL, bool DUMP>
__global__ __launch_bounds__(256, 2) void k_bwd_dq(BwdArgs a) {
    // the wave index as a uniform value, so everything per wave (block,
    // range, scale loads, the step guard) stays scalar
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, h = lane / 32,
              l32 = lane % 32;
    const int T = a.T;
    int bh, g;
    map_group_bwd((T + DQ_BLOCKS_PER_WG - 1) / DQ_BLOCKS_PER_WG, a.BH, false, bh, g, CAUSAL);
    const int qblk_wg_last = DQ_BLOCKS_PER_WG * g + DQ_BLOCKS_PER_WG - 1;
    const int qblk = min(DQ_BLOCKS_PER_WG * g + wave, T - 1);   // waves past T only help stage K^T
    const bool live = DQ_BLOCKS_PER_WG * g + wave < T;
    const int t_end = !live ? 0 : CAUSAL ? qblk + 1 : T;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const size_t rowbase = bh * np;
    const size_t tile0 = (size_t)bh * a.ntiles + ds_tile_index(CAUSAL, qblk, 0, T);
    const v4i* dsg = (const v4i*)(a.ds_codes + tile0 * 4096) + lane;
    const float* dss = a.ds_scale + tile0;
    const v4i* ktg_wave = (const v4i*)(a.k_t + bt * 4096) + 64 * wave + lane;
    const float* skg = a.sk + bt;

    // INT8 identity as the B operand: column n = l32 has its one at k
    // position n, which lies in half (n % 8) / 4, byte 4 (n / 8) + n % 4
    v4i eye = v4i{0, 0, 0, 0};
    if (h == (l32 % 8) / 4) eye[l32 / 8] = 1 << (8 * (l32 % 4));

    const int wg_end = CAUSAL ? min(qblk_wg_last, T - 1) + 1 : T;   // steps of the workgroup's longest wave
    // chunk (kh * 2 + qs) * 64 + lane of a tile: key 32 kh + l32, 16 queries of
    // half qs.  Every step loads (past the wave's own range it re-reads its
    // last tile), so the wait counts before each use are fixed.
    auto load = [&](int t, DqStep& s) {   // seven untracked loads per slot
        const int td = min(t, max(t_end - 1, 0));
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) s.ds[qs][kh] = gload_nt(dsg + (size_t)td * 256 + (kh * 2 + qs) * 64);
        s.kq = gload(ktg_wave + (size_t)min(t, wg_end - 1) * 256);
        s.sds = gload1(dss + td);
        s.sk = gload1(skg + td);
    };
    v16f dq[2][2] = {{v16f{}, v16f{}}, {v16f{}, v16f{}}};   // [qs][db]: lane = query, regs = channels
    auto step = [&](int t, const DqStep& s, const v4i* kts) {
        v4i kt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) kt[j] = kts[j * 64 + lane];
        const float wq = s.sds * s.sk;
        const bool dump_here = DUMP && bh == a.dump_bh && qblk == a.dump_i && t == a.dump_t;
        if (dump_here && lane == 0) dump_at<float>(a.dump, dumpoff::SC)[0] = s.sds;
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            v4i dc[2];
            v16i tr[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                tr[kh] = mfma_i8(s.ds[qs][kh], eye, v16i{});
                dc[kh] = v4i{(int)pack4(tr[kh][0], tr[kh][1], tr[kh][2], tr[kh][3]),
                             (int)pack4(tr[kh][4], tr[kh][5], tr[kh][6], tr[kh][7]),
                             (int)pack4(tr[kh][8], tr[kh][9], tr[kh][10], tr[kh][11]),
                             (int)pack4(tr[kh][12], tr[kh][13], tr[kh][14], tr[kh][15])};
            }
            if (dump_here) {
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        a.dump[dumpoff::C1 + (32 * qs + l32) * 64 + 32 * kh + 8 * (r / 4) + 4 * h + (r % 4)] =
                            (uint8_t)tr[kh][r];
            }
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                v16i acc = mfma_i8(kt[db * 2 + 0], dc[0], v16i{});
                acc = mfma_i8(kt[db * 2 + 1], dc[1], acc);
                if (dump_here) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<int>(a.dump, dumpoff::ACC1)[(32 * qs + l32) * 64 + 32 * db + 8 * (r / 4) + 4 * h + (r % 4)] =
                            acc[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dq[qs][db][r] = __builtin_fmaf((float)acc[r], wq, dq[qs][db][r]);
            }
        }
    };

    // the K^T block of each step is shared by the workgroup's four waves:
    // each wave stages one quarter (loaded with its dS codes, through
    // registers so no LDS DMA forces a full wait) into a double-buffered LDS
    // tile
    __shared__ v4i kts[2][256];
    DqStep ring[DQ_DEPTH];
#pragma unroll
    for (int j = 0; j < DQ_DEPTH; ++j) load(j, ring[j]);
    for (int t0 = 0; t0 < wg_end; t0 += DQ_DEPTH) {
#pragma unroll
        for (int j = 0; j < DQ_DEPTH; ++j) {
            const int t = t0 + j;
            if (t < wg_end) {
                dq_wait<7 * (DQ_DEPTH - 1)>(ring[j]);   // this slot's loads have landed
                kts[t & 1][64 * wave + lane] = ring[j].kq;
                lds_barrier();   // LDS only: the prefetch stays in flight
                if (t < t_end) step(t, ring[j], kts[t & 1]);
                load(t + DQ_DEPTH, ring[j]);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the ring's last, unused loads
    if (!live) return;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) dq_epilogue(a, dq[qs], bh, qblk * BLK + 32 * qs + l32, h, rowbase);
}

// ------------------------------------------------------------------ MXFP8
// The same two kernels with OCP E4M3 codes and E8M0 exponents per 32x32 block
// on the scaled FP8 MFMA (block scales applied inside the instruction, so
// dK, dV and dQ accumulate in the MFMA accumulators with no per-tile
// multiply).  A 32x32 block of P or dS (32 queries of one half of the query
// block x the 32 keys of one wave) lies within one wave, so the block maxima
// need no exchange between waves, and the key-block kernel synchronizes once
// per query block (double-buffered operand tiles).  The dS codes handed to
// the dQ kernel carry four exponent bytes per tile (byte 2 * key half + query
// half) in the slot of the INT8 block scale.

struct DkdvMxSmem {
    v4i q_r[2][256];     // Q row-operand codes (A operand of Q K^T)
    v4i q_t[2][256];     // Q transposed codes (B operand of dS^T Q)
    v4i do_t[2][256];    // dO transposed codes (B operand of P^T dO)
    v8h do16[2][512];    // dO in FP16, swizzled rows (A operand of dO V^T)
    float lse2[2][128];  // [0, 64): log2-domain LSE, [64, 128): -Delta
    uint32_t qs[2][4];   // [0]: Q block exponents, [1]: dO block exponents
};

// Codes of a 32x32 block held as 16 registers x 64 lanes (E4M3(x / 2^e)),
// packed four registers to a dword in register order.
__device__ __forceinline__ v4i fp8_block_codes(const float (&x)[16], float scale) {
    return v4i{(int)fp8_quad(x[0], x[1], x[2], x[3], scale), (int)fp8_quad(x[4], x[5], x[6], x[7], scale),
               (int)fp8_quad(x[8], x[9], x[10], x[11], scale), (int)fp8_quad(x[12], x[13], x[14], x[15], scale)};
}

// S = Q K^T (dequantized in the MFMA) and P = exp2(S log2(e)/8 + bias_j -
// lse2_i) for one 64-query x 32-key tile (lane = key, registers = queries);
// MASK only on the causal diagonal and the ragged last key block.
template <bool CAUSAL, bool MASK>
__device__ __forceinline__ void dkdv_probs_mx(const DkdvMxSmem& sm, int buf, v8i kop, uint32_t q_w, int sk_e,
                                              float brow, int i, int key, int N, int lane, int h,
                                              float (&p)[2][16]) {
    // all operands first (the LSE row is read by every lane, so no divergent
    // branch splits the reads from the MFMAs), then both query halves' MFMAs
    v8i qa[2];
    float lv[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        qa[qb] = cat8(sm.q_r[buf][(qb * 2 + 0) * 64 + lane], sm.q_r[buf][(qb * 2 + 1) * 64 + lane]);
        lv[qb] = sm.lse2[buf][32 * qb + lane % 32];
        asm volatile("" : "+v"(lv[qb]));
    }
    v16f sx[2], corr[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) sx[qb] = mfma_fp8(qa[qb], kop, v16f{}, ebyte(q_w, 2 * qb + h), sk_e);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
        corr[qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(h == 0 ? -lv[qb] : 1.0f, brow, v16f{}, 0, 0, 0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[qb][r], SCORE_SCALE_LOG2, corr[qb][r]));
            if (MASK) {
                asm volatile("" : "+v"(pv));   // a select, not a branch around each exp
                const int qq = i * BLK + 32 * qb + 8 * (r / 4) + 4 * h + (r % 4);
                pv = (key >= N || (CAUSAL && key > qq)) ? 0.0f : pv;
            }
            p[qb][r] = pv;
        }
    }
}

template <bool CAUSAL, bool SMOOTHQ>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv_mx(BwdArgs a) {
    __shared__ DkdvMxSmem sm;
    const int tid = threadIdx.x, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: per-wave values live in SGPRs
    int bh, g;
    map_group_bwd(a.ngroups, a.BH, true, bh, g, CAUSAL);
    const int T = a.T;
    const int kvb = 2 * g + wave / 2, kh = wave % 2;
    const bool live = kvb < T;
    const int key = kvb * BLK + 32 * kh + l32;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const size_t rowbase = bh * np;

    v8i kop = v8i{};
    v8h vh[4];
    float kbias = 0.0f;
    int sk_e = E8M0_ONE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vh[ks] = v8h{};
    if (live) {
        const v4i* src = (const v4i*)(a.k_r + (bt + kvb) * 4096);
        kop = cat8(src[(kh * 2 + 0) * 64 + lane], src[(kh * 2 + 1) * 64 + lane]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vh[ks] = *(const v8h*)(a.v16 + (rowbase + key) * HD + 16 * ks + 8 * h);
        if (SMOOTHQ) kbias = a.bias[rowbase + key];
        sk_e = ebyte(((const uint32_t*)a.sk)[bt + kvb], 2 * kh + h);   // column = key, 32-channel block h
    }
    const float brow = h == 0 ? 1.0f : kbias;
    const int e_one = opaque(E8M0_ONE);
    const v8i ones = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                         0x38383838};

    const int i0 = CAUSAL ? min(2 * g, T - 1) : 0;
    const v4i* qrg = (const v4i*)(a.q_r + bt * 4096);
    const v4i* qtg = (const v4i*)(a.q_t + bt * 4096);
    const v4i* dtg = (const v4i*)(a.do_t + bt * 4096);
    auto fetch = [&](int i, int b) {
        dma16_to_lds(qrg + (size_t)i * 256 + tid, &sm.q_r[b][64 * wave]);
        dma16_to_lds(qtg + (size_t)i * 256 + tid, &sm.q_t[b][64 * wave]);
        dma16_to_lds(dtg + (size_t)i * 256 + tid, &sm.do_t[b][64 * wave]);
        const v4i* hs = (const v4i*)(a.do16 + (rowbase + (size_t)i * BLK) * HD);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = 256 * j + tid, row = s / 8;
            dma16_to_lds(hs + row * 8 + ((s % 8) ^ ((row >> 1) & 7)), (v4i*)sm.do16[b] + 256 * j + 64 * wave);
        }
        if (wave == 0 && lane < 32)
            dma16_to_lds((lane < 16 ? a.lse2 : a.delta) + rowbase + (size_t)i * BLK + 4 * (lane % 16), &sm.lse2[b][0]);
        if (wave == 1 && lane < 2) dma4_to_lds((lane == 0 ? a.sq : a.sdo) + bt + i, &sm.qs[b][0]);
    };

    v16f dk[2] = {v16f{}, v16f{}}, dv[2] = {v16f{}, v16f{}};   // [db]: lane = channel, regs = keys
    v16f csum = v16f{};   // Q-smoothing: every column holds sum over queries of dS^ for key (row)

    v4i dc_prev[2] = {v4i{}, v4i{}};
    uint32_t e_prev = 0;
    size_t tix_prev = 0;
    bool have_prev = false;
    auto store_prev = [&]() {
        v4i* dst = (v4i*)(a.ds_codes + tix_prev * 4096) + kh * 128 + lane;
        __builtin_nontemporal_store(dc_prev[0], dst);
        __builtin_nontemporal_store(dc_prev[1], dst + 64);
        if (lane == 0) ((uint16_t*)(a.ds_scale + tix_prev))[kh] = (uint16_t)e_prev;   // bytes 2 kh, 2 kh + 1
    };

    fetch(i0, 0);
    const bool ragged_keys = (kvb == T - 1) && (a.N & (BLK - 1)) != 0;
    for (int i = i0; i < T; ++i) {
        const int buf = (i - i0) & 1;
        // query block i has landed in buf, and every wave is done with the
        // other buffer (query block i - 1), which the next fetch overwrites
        wait_vmem();
        lds_barrier();
        if (i + 1 < T) fetch(i + 1, buf ^ 1);
        if (have_prev) store_prev();
        have_prev = false;
        if (!live || (CAUSAL && i < kvb)) continue;
        const bool masked = (CAUSAL && i == kvb) || ragged_keys;
        const uint32_t q_w = sm.qs[buf][0], do_w = sm.qs[buf][1];
        float p[2][16];   // [qb]: lane = key, registers = queries
        if (masked) dkdv_probs_mx<CAUSAL, true>(sm, buf, kop, q_w, sk_e, brow, i, key, a.N, lane, h, p);
        else dkdv_probs_mx<CAUSAL, false>(sm, buf, kop, q_w, sk_e, brow, i, key, a.N, lane, h, p);
        // P codes per 32x32 block (query half qb x this wave's keys)
        int eP[2];
        v4i pc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            uint32_t pm = 0;
#pragma unroll
            for (int r = 0; r < 16; r += 2) pm = umax(pm, umax(__float_as_uint(p[qb][r]), __float_as_uint(p[qb][r + 1])));
            eP[qb] = mx_exponent(wave_max64(__uint_as_float(pm)));
            pc[qb] = fp8_block_codes(p[qb], pow2f(eP[qb]));
        }
        // dV += P^T dO: A = P codes (row = key, 32-query block h), B = dO^T
        {
            const v8i pa = cat8(pc[0], pc[1]);
            const int pe = (h ? eP[1] : eP[0]) + 127;
#pragma unroll
            for (int db = 0; db < 2; ++db)
                dv[db] = mfma_fp8(pa, cat8(sm.do_t[buf][(db * 2 + 0) * 64 + lane], sm.do_t[buf][(db * 2 + 1) * 64 + lane]),
                                  dv[db], pe, ebyte(do_w, 2 * h + db));
        }
        // dS = P * (dO V^T - Delta) (FP16 MFMA, -Delta as the accumulator input)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = 32 * qb + l32;
            v16f nd;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 d4 = *(const float4*)&sm.lse2[buf][64 + 32 * qb + 8 * r4 + 4 * h];
                nd[4 * r4 + 0] = d4.x;
                nd[4 * r4 + 1] = d4.y;
                nd[4 * r4 + 2] = d4.z;
                nd[4 * r4 + 3] = d4.w;
            }
            v16f dpd = mfma_f16(sm.do16[buf][swz(row, 0 + h)], vh[0], nd);
            dpd = mfma_f16(sm.do16[buf][swz(row, 2 + h)], vh[1], dpd);
            dpd = mfma_f16(sm.do16[buf][swz(row, 4 + h)], vh[2], dpd);
            dpd = mfma_f16(sm.do16[buf][swz(row, 6 + h)], vh[3], dpd);
#pragma unroll
            for (int r = 0; r < 16; ++r) p[qb][r] = p[qb][r] * dpd[r];
        }
        int eS[2];
        v4i dc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) m = max_abs2f(m, p[qb][r], p[qb][r + 1]);
            eS[qb] = mx_exponent(wave_max64(m));
            dc[qb] = fp8_block_codes(p[qb], pow2f(eS[qb]));
        }
        // dK += dS^T Q (and the dS column sums for the Q-smoothing term)
        {
            const v8i da = cat8(dc[0], dc[1]);
            const int de = (h ? eS[1] : eS[0]) + 127;
#pragma unroll
            for (int db = 0; db < 2; ++db)
                dk[db] = mfma_fp8(da, cat8(sm.q_t[buf][(db * 2 + 0) * 64 + lane], sm.q_t[buf][(db * 2 + 1) * 64 + lane]),
                                  dk[db], de, ebyte(q_w, 2 * h + db));
            if (SMOOTHQ) csum = mfma_fp8(da, ones, csum, de, e_one);
        }
        dc_prev[0] = dc[0];
        dc_prev[1] = dc[1];
        e_prev = (uint32_t)(eS[0] + 127) | ((uint32_t)(eS[1] + 127) << 8);
        tix_prev = (size_t)bh * a.ntiles + ds_tile_index(CAUSAL, i, kvb, T);
        have_prev = true;
    }
    if (have_prev) store_prev();

    if (!live) return;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const float muq = SMOOTHQ ? a.mu_q[(size_t)bh * HD + 32 * db + l32] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dk[db][r] = (SMOOTHQ ? __builtin_fmaf(csum[r], muq, dk[db][r]) : dk[db][r]) * 0.125f;
    }
    if (a.rk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = kvb * BLK + 32 * kh + 8 * (r / 4) + 4 * h + (r % 4);
            const bool ok = kk < a.N;
            const float rr = ok ? a.rk[rowbase + kk] : 0.0f;
            const uint16_t* krow = a.k_in + ((size_t)bh * a.N + (ok ? kk : 0)) * HD;
            const float kn0 = ok ? qk_normed(krow[l32], rr) : 0.0f;
            const float kn1 = ok ? qk_normed(krow[32 + l32], rr) : 0.0f;
            const float mean = half_sum32(__builtin_fmaf(dk[1][r], kn1, dk[0][r] * kn0)) * (1.0f / HD);
            dk[0][r] = rr * __builtin_fmaf(-kn0, mean, dk[0][r]);
            dk[1][r] = rr * __builtin_fmaf(-kn1, mean, dk[1][r]);
        }
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int d = 32 * db + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = kvb * BLK + 32 * kh + 8 * (r / 4) + 4 * h + (r % 4);
            if (kk < a.N) {
                a.dk[((size_t)bh * a.N + kk) * HD + d] = (uint16_t)f32_to_bf16_rne(dk[db][r]);
                a.dv[((size_t)bh * a.N + kk) * HD + d] = (uint16_t)f32_to_bf16_rne(dv[db][r]);
            }
        }
    }
}

// dQ from the stored E4M3 dS codes: each 32-key half of a tile is transposed
// on the MFMA as its product with an E4M3 identity (the codes in the first 32
// k positions, zeros in the other 32; every output is one exact product),
// re-coded (exact: the values are E4M3 values), and contracted with the K^T
// codes, the block exponents applied inside the instruction.
template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void k_bwd_dq_mx(BwdArgs a) {
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, h = lane / 32,
              l32 = lane % 32;
    const int T = a.T;
    int bh, g;
    map_group_bwd((T + DQ_BLOCKS_PER_WG - 1) / DQ_BLOCKS_PER_WG, a.BH, false, bh, g, CAUSAL);
    const int qblk_wg_last = DQ_BLOCKS_PER_WG * g + DQ_BLOCKS_PER_WG - 1;
    const int qblk = min(DQ_BLOCKS_PER_WG * g + wave, T - 1);
    const bool live = DQ_BLOCKS_PER_WG * g + wave < T;
    const int t_end = !live ? 0 : CAUSAL ? qblk + 1 : T;
    const int wg_end = CAUSAL ? min(qblk_wg_last, T - 1) + 1 : T;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const size_t rowbase = bh * np;
    const size_t tile0 = (size_t)bh * a.ntiles + ds_tile_index(CAUSAL, qblk, 0, T);
    const v4i* dsg = (const v4i*)(a.ds_codes + tile0 * 4096) + lane;
    const float* dss = a.ds_scale + tile0;            // exponent words, loaded as their bit patterns
    const v4i* ktg_wave = (const v4i*)(a.k_t + bt * 4096) + 64 * wave + lane;
    const float* skg = a.sk + bt;

    // E4M3 identity (B operand): column n = l32 has 1.0 at k position n,
    // which lies in half (n % 8) / 4, byte 4 (n / 8) + n % 4
    v8i eye = v8i{};
    if (h == (l32 % 8) / 4) eye[l32 / 8] = E4M3_ONE << (8 * (l32 % 4));
    const int e_one = opaque(E8M0_ONE);

    auto load = [&](int t, DqStep& s) {   // seven untracked loads per slot, as in the INT8 kernel
        const int td = min(t, max(t_end - 1, 0));
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) s.ds[qs][kh] = gload_nt(dsg + (size_t)td * 256 + (kh * 2 + qs) * 64);
        s.kq = gload(ktg_wave + (size_t)min(t, wg_end - 1) * 256);
        s.sds = gload1(dss + td);
        s.sk = gload1(skg + td);
    };
    v16f dq[2][2] = {{v16f{}, v16f{}}, {v16f{}, v16f{}}};
    auto step = [&](const DqStep& s, const v4i* kts) {
        v8i kt[2];
#pragma unroll
        for (int db = 0; db < 2; ++db) kt[db] = cat8(kts[(db * 2 + 0) * 64 + lane], kts[(db * 2 + 1) * 64 + lane]);
        const uint32_t ds_w = __float_as_uint(s.sds), sk_w = __float_as_uint(s.sk);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            v4i dc[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const v16f tr = mfma_fp8(cat8(s.ds[qs][kh], v4i{}), eye, v16f{}, e_one, e_one);
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = tr[r];
                dc[kh] = fp8_block_codes(x, 1.0f);
            }
            const v8i db8 = cat8(dc[0], dc[1]);
            const int de = ebyte(ds_w, 2 * h + qs);   // key half h, query half qs
#pragma unroll
            for (int db = 0; db < 2; ++db) dq[qs][db] = mfma_fp8(kt[db], db8, dq[qs][db], ebyte(sk_w, 2 * h + db), de);
        }
    };

    __shared__ v4i kts[2][256];
    DqStep ring[DQ_DEPTH];
#pragma unroll
    for (int j = 0; j < DQ_DEPTH; ++j) load(j, ring[j]);
    for (int t0 = 0; t0 < wg_end; t0 += DQ_DEPTH) {
#pragma unroll
        for (int j = 0; j < DQ_DEPTH; ++j) {
            const int t = t0 + j;
            if (t < wg_end) {
                dq_wait<7 * (DQ_DEPTH - 1)>(ring[j]);
                kts[t & 1][64 * wave + lane] = ring[j].kq;
                lds_barrier();
                if (t < t_end) step(ring[j], kts[t & 1]);
                load(t + DQ_DEPTH, ring[j]);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!live) return;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) dq_epilogue(a, dq[qs], bh, qblk * BLK + 32 * qs + l32, h, rowbase);
}

// Instantiation by (causal, Q-smoothing, all-INT8 dO V^T, tile dump).
#define SAGEBWD_LAUNCH_BWD(KERNEL)                                                                   \
    dim3 grid(a.ngroups * BH), block(64 * BWD_WAVES);                                                \
    switch ((causal ? 8 : 0) | (smooth_q ? 4 : 0) | (int8_dp ? 2 : 0) | (dump ? 1 : 0)) {            \
        case 0: hipLaunchKernelGGL((KERNEL<false, false, false, false>), grid, block, 0, st, a); break; \
        case 1: hipLaunchKernelGGL((KERNEL<false, false, false, true>), grid, block, 0, st, a); break;  \
        case 2: hipLaunchKernelGGL((KERNEL<false, false, true, false>), grid, block, 0, st, a); break;  \
        case 3: hipLaunchKernelGGL((KERNEL<false, false, true, true>), grid, block, 0, st, a); break;   \
        case 4: hipLaunchKernelGGL((KERNEL<false, true, false, false>), grid, block, 0, st, a); break;  \
        case 5: hipLaunchKernelGGL((KERNEL<false, true, false, true>), grid, block, 0, st, a); break;   \
        case 6: hipLaunchKernelGGL((KERNEL<false, true, true, false>), grid, block, 0, st, a); break;   \
        case 7: hipLaunchKernelGGL((KERNEL<false, true, true, true>), grid, block, 0, st, a); break;    \
        case 8: hipLaunchKernelGGL((KERNEL<true, false, false, false>), grid, block, 0, st, a); break;  \
        case 9: hipLaunchKernelGGL((KERNEL<true, false, false, true>), grid, block, 0, st, a); break;   \
        case 10: hipLaunchKernelGGL((KERNEL<true, false, true, false>), grid, block, 0, st, a); break;  \
        case 11: hipLaunchKernelGGL((KERNEL<true, false, true, true>), grid, block, 0, st, a); break;   \
        case 12: hipLaunchKernelGGL((KERNEL<true, true, false, false>), grid, block, 0, st, a); break;  \
        case 13: hipLaunchKernelGGL((KERNEL<true, true, false, true>), grid, block, 0, st, a); break;   \
        case 14: hipLaunchKernelGGL((KERNEL<true, true, true, false>), grid, block, 0, st, a); break;   \
        default: hipLaunchKernelGGL((KERNEL<true, true, true, true>), grid, block, 0, st, a); break;    \
    }                                                                                                \
    return 0;

int launch_bwd_dkdv(const BwdArgs& a, int BH, bool causal, bool smooth_q, bool int8_dp, bool mx, hipStream_t st,
                    bool dump) {
    if (mx) {
        dim3 grid(a.ngroups * BH), block(64 * BWD_WAVES);
        if (causal) {
            if (smooth_q) hipLaunchKernelGGL((k_bwd_dkdv_mx<true, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_bwd_dkdv_mx<true, false>), grid, block, 0, st, a);
        } else {
            if (smooth_q) hipLaunchKernelGGL((k_bwd_dkdv_mx<false, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_bwd_dkdv_mx<false, false>), grid, block, 0, st, a);
        }
        return 0;
    }
    SAGEBWD_LAUNCH_BWD(k_bwd_dkdv)
}

#undef SAGEBWD_LAUNCH_BWD

int launch_bwd_dq(const BwdArgs& a, int BH, bool causal, bool mx, hipStream_t st, bool dump) {
    dim3 grid(((a.T + DQ_BLOCKS_PER_WG - 1) / DQ_BLOCKS_PER_WG) * BH), block(64 * BWD_WAVES);
    if (mx) {
        if (causal) hipLaunchKernelGGL((k_bwd_dq_mx<true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dq_mx<false>), grid, block, 0, st, a);
        return 0;
    }
    if (causal) {
        if (dump) hipLaunchKernelGGL((k_bwd_dq<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dq<true, false>), grid, block, 0, st, a);
    } else {
        if (dump) hipLaunchKernelGGL((k_bwd_dq<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_dq<false, false>), grid, block, 0, st, a);
    }
    return 0;
}

}  // namespace sagebwd
