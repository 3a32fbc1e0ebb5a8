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
// Two kernels, no atomics, bitwise repeatable, nothing of size N^2 kept
// between them:
//   k_bwd_dkdv  a workgroup of 4 waves owns two 64-key blocks (each wave 32
//               keys) and walks the query blocks.  It computes S (lane = key),
//               so P and dS codes leave the accumulator as the A operand of
//               P^T dO and dS^T Q (contraction over queries).
//   k_bwd_dq    a workgroup of 4 waves owns two 64-query blocks (each wave 32
//               queries) and walks the key blocks.  It recomputes S, P,
//               dP - Delta and dS in the forward's layout (lane = query), so
//               the dS codes leave the accumulator as the B operand of
//               dQ^T = K^T dS^T (contraction over keys); its dS values and
//               codes are bitwise the key-block kernel's.
// A 64x64 quantization tile of P or dS is held by a pair of waves, which
// exchange their partial maxima through LDS, so each kernel synchronizes its
// workgroup once per step.  The streamed operand tiles go global -> LDS by DMA
// into three buffers, each fetched a whole step before it is read; FP16 rows
// are stored with their 16-byte chunks XOR-swizzled by row so column reads do
// not collide on LDS banks.
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
// DPP row broadcasts that leave the maximum in lane 63 (wave_max64_v returns
// that register, for a store from lane 63; wave_max64 reads it once).
__device__ __forceinline__ uint32_t wave_max64_v(float f) {
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
    return v;
}
__device__ __forceinline__ float wave_max64(float f) {
    return __uint_as_float(__builtin_amdgcn_readlane(wave_max64_v(f), 63));
}
// Two such maxima with their reduction steps interleaved (the two
// dependency chains fill each other's DPP wait states).
__device__ __forceinline__ void wave_max64x2(float f0, float f1, float& m0, float& m1) {
    uint32_t v = __float_as_uint(f0), w = __float_as_uint(f1);
    v = umax(v, dppu<0xB1>(v));
    w = umax(w, dppu<0xB1>(w));
    v = umax(v, dppu<0x4E>(v));
    w = umax(w, dppu<0x4E>(w));
    v = umax(v, dppu<0x141>(v));
    w = umax(w, dppu<0x141>(w));
    v = umax(v, dppu<0x140>(v));
    w = umax(w, dppu<0x140>(w));
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    w = umax(w, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x142, 0xA, 0xF, false));
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    w = umax(w, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x143, 0xC, 0xF, false));
    m0 = __uint_as_float(__builtin_amdgcn_readlane(v, 63));
    m1 = __uint_as_float(__builtin_amdgcn_readlane(w, 63));
}

// Four signed codes rne(x * inv) packed into one dword.
__device__ __forceinline__ int pack_codes(float x0, float x1, float x2, float x3, float inv) {
    return (int)pack4(code_bits(x0, inv), code_bits(x1, inv), code_bits(x2, inv), code_bits(x3, inv));
}

// Codes of a 32x32 block held as 16 registers x 64 lanes (E4M3(x / 2^e)),
// packed four registers to a dword in register order.
__device__ __forceinline__ v4i fp8_block_codes(const float (&x)[16], float scale) {
    return v4i{(int)fp8_quad(x[0], x[1], x[2], x[3], scale), (int)fp8_quad(x[4], x[5], x[6], x[7], scale),
               (int)fp8_quad(x[8], x[9], x[10], x[11], scale), (int)fp8_quad(x[12], x[13], x[14], x[15], scale)};
}

// FP16 rows of 8 chunks of 16 bytes in LDS: chunk c of row r sits at slot
// c ^ ((r / 2) % 8), so any 16 consecutive rows read at one chunk cover all
// 64 banks (with c ^ (r % 8), rows r and r + 8 would collide).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

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

constexpr int DKDV_BUFS = 3;

struct DkdvSmem {
    v4i q_r[DKDV_BUFS][256];     // Q row-operand codes (A operand of Q K^T)
    v4i q_t[DKDV_BUFS][256];     // Q transposed codes (B operand of dS^T Q)
    v4i do_t[DKDV_BUFS][256];    // dO transposed codes (B operand of P^T dO)
    v8h do16[DKDV_BUFS][512];    // dO in FP16, [64 rows][8 chunks], swizzled (A operand of dO V^T)
    float lse2[DKDV_BUFS][128];  // [0, 64): log2-domain LSE, [64, 128): -Delta of the query block
    float qs[DKDV_BUFS][4];      // [0]: Q block scale, [1]: dO block scale
    alignas(16) float red[DKDV_BUFS][2][4];   // partial tile maxima [key block][P, |dS| of wave 0, P, |dS| of wave 1]
};

// P for one 64-query x 32-key half tile in the S layout (lane = key,
// registers = queries): P = exp2(sc A + (bias_j - lse2_i)), log2 domain.  The
// outer difference bias_j - lse2_i is one subtraction per score (this lane's
// key bias minus the query's lse2, read from LDS while the score MFMAs run;
// as an FP32 rank-2 MFMA it sat in the score's dependency chain and was
// slower), then one FMA before the exp.  MASK only on the causal diagonal tile
// and the ragged last key block, so the common path carries no per-element
// selects (a masked P is a select after its exp, not a branch around it).
// dP - Delta (the same layout) is formed here too: it does not depend on P, so
// its MFMAs are scheduled one by one between groups of the score arithmetic
// instead of stalling the wave later.
template <bool CAUSAL, bool MASK, bool INT8DP>
__device__ __forceinline__ void dkdv_probs(const DkdvSmem& sm, int buf, const v4i (&kop)[2], float sc, float kbias,
                                           int i, int key, int N, int lane, int h, float (&p)[2][16],
                                           v16f (&dpd)[2], const v8h (&vh)[4], const v4i (&vop)[2], float sV,
                                           uint8_t* dp = nullptr) {
    // the score operands first, then both query halves' MFMAs
    v4i qa[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        qa[qb][0] = sm.q_r[buf][(qb * 2 + 0) * 64 + lane];
        qa[qb][1] = sm.q_r[buf][(qb * 2 + 1) * 64 + lane];
    }
    v16i s[2];
    v16f corr[2];
    s[0] = mfma_i8(qa[0][0], kop[0], v16i{});
    s[1] = mfma_i8(qa[1][0], kop[0], v16i{});
    s[0] = mfma_i8(qa[0][1], kop[1], s[0]);
    s[1] = mfma_i8(qa[1][1], kop[1], s[1]);
    // bias_j - lse2_i for queries 32 qb + 8 (r/4) + 4 h + r%4
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float4 l4 = *(const float4*)&sm.lse2[buf][32 * qb + 8 * r4 + 4 * h];
            corr[qb][4 * r4 + 0] = kbias - l4.x;
            corr[qb][4 * r4 + 1] = kbias - l4.y;
            corr[qb][4 * r4 + 2] = kbias - l4.z;
            corr[qb][4 * r4 + 3] = kbias - l4.w;
        }
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

    const int i0 = CAUSAL ? min(2 * g, T - 1) : 0;
    // query block i -> LDS buffer b by DMA; LDS slot s of the FP16 dO tile
    // holds global chunk (s / 8, (s % 8) ^ (s / 16 % 8)), the swizzled layout
    // (the all-INT8 dO V^T stages the dO row-operand codes there instead)
    const v4i* qrg = (const v4i*)(a.q_r + bt * 4096);
    const v4i* qtg = (const v4i*)(a.q_t + bt * 4096);
    const v4i* dtg = (const v4i*)(a.do_t + bt * 4096);
    // the head's code blocks and FP16 dO rows as buffer resources: per-lane
    // offsets fixed, the block's offset wave-uniform
    const uint32_t cb = (uint32_t)T * 4096u;
    const rsrc_t r_qr = raw_rsrc(qrg, cb), r_qt = raw_rsrc(qtg, cb), r_dt = raw_rsrc(dtg, cb);
    const rsrc_t r_do = INT8DP ? raw_rsrc(a.do_r + bt * 4096, cb) : raw_rsrc(a.do16 + rowbase * HD, 2u * cb);
    const uint32_t off16 = 16u * (uint32_t)tid;
    uint32_t offh[2];   // byte offset of this lane's chunk of a swizzled FP16 dO block, j = 0, 1
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t s = 256u * j + (uint32_t)tid, row = s / 8;
        offh[j] = 16u * (row * 8 + ((s % 8) ^ ((row >> 1) & 7)));
    }
    auto fetch = [&](int i, int b) {
        bdma16_to_lds(r_qr, off16, (uint32_t)i * 4096u, &sm.q_r[b][64 * wave]);
        bdma16_to_lds(r_qt, off16, (uint32_t)i * 4096u, &sm.q_t[b][64 * wave]);
        bdma16_to_lds(r_dt, off16, (uint32_t)i * 4096u, &sm.do_t[b][64 * wave]);
        if (INT8DP) {
            bdma16_to_lds(r_do, off16, (uint32_t)i * 4096u, (v4i*)sm.do16[b] + 64 * wave);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bdma16_to_lds(r_do, offh[j], (uint32_t)i * 8192u, (v4i*)sm.do16[b] + 256 * j + 64 * wave);
        }
        // wave-uniform branches first, so the other waves skip them on the scalar unit
        if (wave == 0) {
            if (lane < 32)
                dma16_to_lds((lane < 16 ? a.lse2 : a.delta) + rowbase + (size_t)i * BLK + 4 * (lane % 16),
                             &sm.lse2[b][0]);
        } else if (wave == 1) {
            if (lane < 2) dma4_to_lds((lane == 0 ? a.sq : a.sdo) + bt + i, &sm.qs[b][0]);
        }
    };

    v16f dk[2] = {v16f{}, v16f{}}, dv[2] = {v16f{}, v16f{}};   // [db]: lane = channel, regs = keys
    float gsum = 0.0f;                                          // sum_i s_dS colsum(dS codes), this half

    fetch(i0, 0);
    if (i0 + 1 < T) fetch(i0 + 1, 1);
    wait_vmem();
    lds_barrier();
    const bool ragged_keys = (kvb == T - 1) && (a.N & (BLK - 1)) != 0;
    // One barrier per step.  Before it: the scores, P, dP - Delta and dS of
    // the step and both partial tile maxima (P and |dS|), written to LDS in
    // the slots of the step's buffer (lane 63 holds the wave's maximum; the
    // slots are rewritten three steps later, when every wave has read them).
    // After it: both block scales (the pair's four maxima in one 16-byte
    // read), the P and dS codes, and the dV and dK products.  Query block i
    // sits in LDS buffer (i - i0) % 3; the
    // DMA of block i + 2 is issued right after step i's barrier (its buffer
    // was last read in step i - 1, which every wave has finished by then) and
    // waited for before step i + 1's barrier, a whole step later.  The loop
    // runs three steps per iteration so that each LDS buffer is a
    // compile-time constant (every LDS address a base register plus an
    // immediate).
    auto step = [&](int i, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const bool active = live && (!CAUSAL || i >= kvb);
        const bool masked = (CAUSAL && i == kvb) || ragged_keys;
        float p[2][16], ds[2][16];           // [qb]: lane = key, regs = queries
        const float sQ = sm.qs[buf][0];
        const float sc = tile_scale(sQ, sK);
        uint8_t* dp = (DUMP && bh == a.dump_bh && kvb == a.dump_t && i == a.dump_i) ? a.dump : nullptr;
        if (active) {
            v16f dpe[2];
            if (masked)
                dkdv_probs<CAUSAL, true, INT8DP>(sm, buf, kop, sc, kbias, i, key, a.N, lane, h, p, dpe, vh, vop, sV,
                                                 DUMP ? dp : nullptr);
            else
                dkdv_probs<CAUSAL, false, INT8DP>(sm, buf, kop, sc, kbias, i, key, a.N, lane, h, p, dpe, vh, vop, sV,
                                                  DUMP ? dp : nullptr);
            if (DUMP && dp) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<float>(dp, dumpoff::F1)[(32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] = p[qb][r];
            }
            // one v_max3_f32 per two values (P >= 0, so the wave reduction
            // may compare bit patterns)
            float pm0 = 0.0f, pm1 = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                pm0 = max3f(pm0, p[0][r], p[0][r + 1]);
                pm1 = max3f(pm1, p[1][r], p[1][r + 1]);
            }
            const float pml = __builtin_fmaxf(pm0, pm1);
            // dS = P * (dP - Delta)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) ds[qb][r] = p[qb][r] * dpe[qb][r];
            float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                m0 = max_abs2f(m0, ds[0][r], ds[0][r + 1]);
                m1 = max_abs2f(m1, ds[1][r], ds[1][r + 1]);
            }
            // both wave reductions, then one 8-byte store from lane 63
            const uint32_t pm = wave_max64_v(pml);
            const uint32_t dsm = wave_max64_v(max3f(m0, m1, m1));
            if (lane == 63) *(v2i*)&sm.red[buf][wave / 2][2 * kh] = v2i{(int)pm, (int)dsm};
            if (DUMP && dp) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<float>(dp, dumpoff::F2)[(32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] = ds[qb][r];
            }
        }
        // this wave's DMA of block i + 1 has landed; after the barrier every
        // wave's has, every partial maximum of this step is visible, and every
        // wave is done with step i - 1's buffer
        wait_vmem();
        lds_barrier();
        if (i + 2 < T) fetch(i + 2, (buf + 2) % DKDV_BUFS);
        if (active) {
            // the B operands of this step's dV and dK products, read from LDS
            // before the code arithmetic so that it covers their latency
            v4i dob[4], qtb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dob[j] = sm.do_t[buf][j * 64 + lane];
                qtb[j] = sm.q_t[buf][j * 64 + lane];
            }
            __builtin_amdgcn_sched_barrier(0);
            // both partial maxima are >= 0: the larger is the larger bit pattern
            float sP, invP, sdS, invdS;
            const v4i rm = *(const v4i*)&sm.red[buf][wave / 2][0];
            block_scale(__uint_as_float(umax((uint32_t)rm[0], (uint32_t)rm[2])), sP, invP);
            block_scale(__uint_as_float(umax((uint32_t)rm[1], (uint32_t)rm[3])), sdS, invdS);
            // P codes, then the dV products; the dS codes are formed while
            // they run, then the dK products, under which dV is updated
            v4i pc[2], dc[2];
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
                pc[qs] = v4i{pack_codes(p[qs][0], p[qs][1], p[qs][2], p[qs][3], invP),
                             pack_codes(p[qs][4], p[qs][5], p[qs][6], p[qs][7], invP),
                             pack_codes(p[qs][8], p[qs][9], p[qs][10], p[qs][11], invP),
                             pack_codes(p[qs][12], p[qs][13], p[qs][14], p[qs][15], invP)};
            if (DUMP && dp) {
                if (lane == 0 && kh == 0) {
                    dump_at<float>(dp, dumpoff::SC)[0] = sP;
                    dump_at<float>(dp, dumpoff::SC)[1] = sdS;
                }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = (32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64);
                        dp[dumpoff::C1 + o] = (uint8_t)code_bits(p[qb][r], invP);
                        dp[dumpoff::C2 + o] = (uint8_t)code_bits(ds[qb][r], invdS);
                    }
            }
            // dV += s_P s_dO (P codes^T dO codes), dK += s_dS s_Q (dS codes^T Q codes)
            const float wv = sP * sm.qs[buf][1];
            const float wk = sdS * sQ;
            v16i av[2], ak[2];
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                av[db] = mfma_i8(pc[0], dob[db * 2 + 0], v16i{});
                av[db] = mfma_i8(pc[1], dob[db * 2 + 1], av[db]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
                dc[qs] = v4i{pack_codes(ds[qs][0], ds[qs][1], ds[qs][2], ds[qs][3], invdS),
                             pack_codes(ds[qs][4], ds[qs][5], ds[qs][6], ds[qs][7], invdS),
                             pack_codes(ds[qs][8], ds[qs][9], ds[qs][10], ds[qs][11], invdS),
                             pack_codes(ds[qs][12], ds[qs][13], ds[qs][14], ds[qs][15], invdS)};
            if (SMOOTHQ) {
                int cs = 0;
#pragma unroll
                for (int qs = 0; qs < 2; ++qs)
#pragma unroll
                    for (int d4 = 0; d4 < 4; ++d4) cs = __builtin_amdgcn_sdot4(dc[qs][d4], 0x01010101, cs, false);
                gsum = __builtin_fmaf((float)cs, sdS, gsum);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                ak[db] = mfma_i8(dc[0], qtb[db * 2 + 0], v16i{});
                ak[db] = mfma_i8(dc[1], qtb[db * 2 + 1], ak[db]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (DUMP && dp) {
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = (32 * kh + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + 32 * db + l32;
                        dump_at<int>(dp, dumpoff::ACC1)[o] = av[db][r];
                        dump_at<int>(dp, dumpoff::ACC2)[o] = ak[db][r];
                    }
            }
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) dv[db][r] = __builtin_fmaf((float)av[db][r], wv, dv[db][r]);
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) dk[db][r] = __builtin_fmaf((float)ak[db][r], wk, dk[db][r]);
        }
    };
    int i = i0;
    for (; i + 2 < T; i += 3) {
        step(i, IntC<0>{});
        step(i + 1, IntC<1>{});
        step(i + 2, IntC<2>{});
    }
    if (i < T) step(i, IntC<0>{});
    if (i + 1 < T) step(i + 1, IntC<1>{});

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

// dQ recomputes each tile's scores, P, dP - Delta and dS in the forward's
// layout, S^T = K Q^T (lane = query, registers = keys), so that the dS codes
// leave the accumulator as the B operand of dQ^T = K^T dS^T (contraction
// over keys) with no transposition, and nothing of size N^2 is kept between
// the two backward kernels.  Every product is formed from the key-block
// kernel's operands in the same k order (the score correction is the same
// rounded sum of bias_j and -lse2_i, the FP16 dO V^T MFMAs take the same
// channel chunks in the same sequence from the same -Delta input, and the
// FMAs are written out), so its P, dS, tile maxima, scales and codes are
// bitwise the key-block kernel's; the tile replay test checks this.
//
// Work split as in the forward: a workgroup of 4 waves owns 128 query rows
// (two query blocks), each wave 32 of them, and walks the key blocks; a
// 64x64 quantization tile of dS is held by the pair of waves of one query
// block, which exchange their partial maxima through LDS.  Each key block's
// K codes (both layouts), FP16 V rows, key bias and block scale go global ->
// LDS by DMA into one of three buffers: the DMA for step t + 2 is issued
// right after step t's barrier (the buffer it overwrites was last read in
// step t - 1, which every wave has finished by then), so each step waits at
// its one barrier for a DMA issued a whole step earlier.

constexpr int DQ_BUFS = 3;

struct DqSmem {
    v4i k[DQ_BUFS][256];     // K row-operand codes (A operand of K Q^T)
    v4i kt[DQ_BUFS][256];    // K transposed codes (A operand of K^T dS^T)
    v8h v16[DQ_BUFS][512];   // V in FP16, [64 rows][8 chunks], swizzled (A operand of V dO^T);
                             // all-INT8 dO V^T: V row-operand codes in its first 4 KB
    float bias[DQ_BUFS][64]; // Q-smoothing key bias (log2 domain; 0 without Q-smoothing)
    float sk[DQ_BUFS][4];    // [0]: K block scale (MXFP8: its exponent word), [1]: V block scale (all-INT8)
    alignas(8) float red[DQ_BUFS][2][2];   // partial |dS| maxima [query block][its two waves] (INT8)
};

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

// The persistent operands of one wave's 32 queries.
struct DqQuery {
    v4i qop[2];       // Q row-operand codes (B operand of K Q^T)
    v8h dob[4];       // dO in FP16, channels 16 ks + 8 h .. + 7 (B operand of V dO^T)
    v4i dor[2];       // all-INT8 dO V^T: dO row-operand codes (B operand of V dO^T)
    float nlse;       // -lse2 of this lane's query (log2 domain)
    float brow;       // non-causal MXFP8: B operand of the rank-2 score correction, -lse2 (h = 0) or 1 (h = 1)
    float bnd;        // B operand of the rank-1 product that puts -Delta in every row: -Delta (h = 0) or 0
    float sdo;        // dO block scale (all-INT8 dO V^T)
    uint32_t qw;      // Q block scale (MXFP8: the exponent bytes of this half, channel halves 0, 1)
};

// One key-block step of one wave up to the dS values: scores, P, dP - Delta
// and dS = P (dP - Delta) for 32 queries x 64 keys (lane = query, registers
// = keys 32 kb + 8 (r/4) + 4 h + r%4), one 32-key half after the other.
// MASK only for the causal diagonal tile and the ragged last key block.
template <bool CAUSAL, bool MASK, bool MX, bool INT8DP>
__device__ __forceinline__ void dq_scores(const DqSmem& sm, int buf, const DqQuery& qd, int t, int q, int N, int lane,
                                          int h, float (&ds)[2][16], int (&sdump)[2][16], bool dump) {
    const int l32 = lane % 32;
    const uint32_t kw = __float_as_uint(sm.sk[buf][0]);
    const float sc = MX ? SCORE_SCALE_LOG2 : tile_scale(__uint_as_float(qd.qw), sm.sk[buf][0]);
    const float wdp = INT8DP ? qd.sdo * sm.sk[buf][1] : 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        v16i s;
        v16f sx;
        if (MX) {
            const v8i ka = cat8(sm.k[buf][(kb * 2 + 0) * 64 + lane], sm.k[buf][(kb * 2 + 1) * 64 + lane]);
            sx = mfma_fp8(ka, cat8(qd.qop[0], qd.qop[1]), v16f{}, ebyte(kw, 2 * kb + h), ebyte(qd.qw, h));
        } else {
            s = mfma_i8(sm.k[buf][(kb * 2 + 0) * 64 + lane], qd.qop[0], v16i{});
            s = mfma_i8(sm.k[buf][(kb * 2 + 1) * 64 + lane], qd.qop[1], s);
        }
        // bias_j - lse2_i: one addition per score (the same rounded sum as the
        // key-block kernels form); in the non-causal MXFP8 form, whose
        // registers that would spill, [1 | bias] [-lse2 | 1]^T on the FP32
        // MFMA instead (32x32x2: lane l carries A[l%32][l/32] and
        // B[l/32][l%32]).  -Delta_i in every row as [1 | 0] [-Delta | 0]^T on
        // the same MFMA.
        v16f corr;
        if (MX && !CAUSAL) {
            corr = __builtin_amdgcn_mfma_f32_32x32x2f32(h == 0 ? 1.0f : sm.bias[buf][32 * kb + l32], qd.brow, v16f{},
                                                        0, 0, 0);
        } else {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 b4 = *(const float4*)&sm.bias[buf][32 * kb + 8 * r4 + 4 * h];
                corr[4 * r4 + 0] = b4.x + qd.nlse;
                corr[4 * r4 + 1] = b4.y + qd.nlse;
                corr[4 * r4 + 2] = b4.z + qd.nlse;
                corr[4 * r4 + 3] = b4.w + qd.nlse;
            }
        }
        const v16f nd = __builtin_amdgcn_mfma_f32_32x32x2f32(h == 0 ? 1.0f : 0.0f, qd.bnd, v16f{}, 0, 0, 0);
        // dP^T - Delta: the key-block kernel's products with the operands
        // swapped, the same channels in the same k steps from the same -Delta
        v16f dpd;
        if (INT8DP) {
            const v4i* vr = (const v4i*)sm.v16[buf];
            v16i ai = mfma_i8(vr[(kb * 2 + 0) * 64 + lane], qd.dor[0], v16i{});
            ai = mfma_i8(vr[(kb * 2 + 1) * 64 + lane], qd.dor[1], ai);
#pragma unroll
            for (int r = 0; r < 16; ++r) dpd[r] = __builtin_fmaf((float)ai[r], wdp, nd[r]);
        } else {
            const int row = 32 * kb + l32;
            dpd = mfma_f16(sm.v16[buf][swz(row, 0 + h)], qd.dob[0], nd);
            dpd = mfma_f16(sm.v16[buf][swz(row, 2 + h)], qd.dob[1], dpd);
            dpd = mfma_f16(sm.v16[buf][swz(row, 4 + h)], qd.dob[2], dpd);
            dpd = mfma_f16(sm.v16[buf][swz(row, 6 + h)], qd.dob[3], dpd);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (dump) sdump[kb][r] = MX ? __float_as_int(sx[r]) : s[r];
            const float sv = MX ? sx[r] : (float)s[r];
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, sc, corr[r]));
            if (MASK) {
                asm volatile("" : "+v"(pv));   // a select, not a branch around each exp
                const int key = t * BLK + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                pv = (key >= N || (CAUSAL && key > q)) ? 0.0f : pv;
            }
            ds[kb][r] = pv * dpd[r];
        }
        // the second half's MFMAs wait until the first half is done, so the
        // two halves' accumulators are never live at once
        if (kb == 0) __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool CAUSAL, bool MX, bool INT8DP, bool DUMP>
__global__ __launch_bounds__(256, 3) void k_bwd_dq(BwdArgs a) {
    __shared__ DqSmem sm;
    const int tid = threadIdx.x, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: per-wave values live in SGPRs
    int bh, g;
    map_group_bwd(a.ngroups, a.BH, false, bh, g, CAUSAL);
    const int T = a.T;
    const int qblk = 2 * g + wave / 2, qhalf = wave % 2;
    const bool live = qblk < T;
    const int t_last_wg = CAUSAL ? min(2 * g + 1, T - 1) : T - 1;   // steps of the workgroup
    const int t_last = !live ? -1 : CAUSAL ? qblk : T - 1;          // steps this wave computes
    const bool ragged = (a.N & (BLK - 1)) != 0;
    const size_t bt = (size_t)bh * T;
    const size_t np = (size_t)T * BLK;
    const size_t rowbase = bh * np;
    const int q = qblk * BLK + 32 * qhalf + l32;                    // this lane's query (padded index)

    DqQuery qd;
    qd.qop[0] = qd.qop[1] = qd.dor[0] = qd.dor[1] = v4i{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qd.dob[ks] = v8h{};
    float ndl = 0.0f, lse2 = 0.0f;
    qd.qw = 0;
    qd.sdo = 0.0f;
    if (live) {
        const v4i* src = (const v4i*)(a.q_r + (bt + qblk) * 4096);
        qd.qop[0] = src[(qhalf * 2 + 0) * 64 + lane];
        qd.qop[1] = src[(qhalf * 2 + 1) * 64 + lane];
        if (INT8DP) {
            const v4i* dsrc = (const v4i*)(a.do_r + (bt + qblk) * 4096);
            qd.dor[0] = dsrc[(qhalf * 2 + 0) * 64 + lane];
            qd.dor[1] = dsrc[(qhalf * 2 + 1) * 64 + lane];
            qd.sdo = a.sdo[bt + qblk];
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qd.dob[ks] = *(const v8h*)(a.do16 + (rowbase + q) * HD + 16 * ks + 8 * h);
        }
        ndl = a.delta[rowbase + q];
        lse2 = a.lse2[rowbase + q];
        const uint32_t w = ((const uint32_t*)a.sq)[bt + qblk];
        qd.qw = MX ? (uint32_t)ebyte(w, 2 * qhalf + 0) | ((uint32_t)ebyte(w, 2 * qhalf + 1) << 8) : w;
    }
    qd.nlse = -lse2;
    qd.brow = h == 0 ? -lse2 : 1.0f;
    qd.bnd = h == 0 ? ndl : 0.0f;

    const v4i* kg = (const v4i*)(a.k_r + bt * 4096);
    const v4i* ktg = (const v4i*)(a.k_t + bt * 4096);
    // the head's code blocks and FP16 V rows as buffer resources: per-lane
    // offsets fixed, the block's offset wave-uniform
    const uint32_t cb = (uint32_t)T * 4096u;
    const rsrc_t r_k = raw_rsrc(kg, cb), r_kt = raw_rsrc(ktg, cb);
    const rsrc_t r_v = INT8DP ? raw_rsrc(a.v_r + bt * 4096, cb) : raw_rsrc(a.v16 + rowbase * HD, 2u * cb);
    const uint32_t off16 = 16u * (uint32_t)tid;
    // LDS slot s of the FP16 V tile holds global chunk (s / 8, (s % 8) ^ (s / 16 % 8)), the swizzled layout
    uint32_t offh[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t s = 256u * j + (uint32_t)tid, row = s / 8;
        offh[j] = 16u * (row * 8 + ((s % 8) ^ ((row >> 1) & 7)));
    }
    auto fetch = [&](int t, int b) {
        bdma16_to_lds(r_k, off16, (uint32_t)t * 4096u, &sm.k[b][64 * wave]);
        bdma16_to_lds(r_kt, off16, (uint32_t)t * 4096u, &sm.kt[b][64 * wave]);
        if (INT8DP) {
            bdma16_to_lds(r_v, off16, (uint32_t)t * 4096u, (v4i*)sm.v16[b] + 64 * wave);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bdma16_to_lds(r_v, offh[j], (uint32_t)t * 8192u, (v4i*)sm.v16[b] + 256 * j + 64 * wave);
        }
        if (wave == 2 && lane < 16) dma16_to_lds(a.bias + rowbase + (size_t)t * BLK + 4 * lane, &sm.bias[b][0]);
        if (wave == 3 && lane < (INT8DP ? 2 : 1)) dma4_to_lds((lane == 0 ? a.sk : a.sv) + bt + t, &sm.sk[b][0]);
    };

    v16f dq[2] = {v16f{}, v16f{}};   // [db]: lane = query, registers = channels 32 db + 8 (r/4) + 4 h + r%4
    uint8_t* dp_sel = (DUMP && bh == a.dump_bh && qblk == a.dump_i) ? a.dump : nullptr;
    const int qloc = 32 * qhalf + l32;

    // bufc: IntC<b> when the step's LDS buffer b = t % 3 is known at compile
    // time (the main loop runs three steps per iteration, so every LDS address
    // is a base register plus an immediate), IntC<-1> otherwise
    auto step = [&](int t, auto maybe_masked, auto bufc) {
        const int buf = decltype(bufc)::value >= 0 ? decltype(bufc)::value : t % DQ_BUFS;
        const bool active = t <= t_last;
        float ds[2][16];
        int sd[2][16];
        uint8_t* dp = (DUMP && dp_sel && t == a.dump_t) ? dp_sel : nullptr;
        if (active) {
            if (decltype(maybe_masked)::value && ((CAUSAL && t == qblk) || (ragged && t == T - 1)))
                dq_scores<CAUSAL, true, MX, INT8DP>(sm, buf, qd, t, q, a.N, lane, h, ds, sd, DUMP && dp);
            else
                dq_scores<CAUSAL, false, MX, INT8DP>(sm, buf, qd, t, q, a.N, lane, h, ds, sd, DUMP && dp);
            if (DUMP && dp) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
                        dump_at<int>(dp, dumpoff::A)[qloc * 64 + kk] = sd[kb][r];
                        dump_at<float>(dp, dumpoff::F2)[qloc * 64 + kk] = ds[kb][r];
                    }
            }
            if (!MX) {
                float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    m0 = max_abs2f(m0, ds[0][r], ds[0][r + 1]);
                    m1 = max_abs2f(m1, ds[1][r], ds[1][r + 1]);
                }
                const uint32_t dsm = wave_max64_v(__builtin_fmaxf(m0, m1));
                if (lane == 63) sm.red[buf][wave / 2][qhalf] = __uint_as_float(dsm);
            }
        }
        // this wave's DMA of step t + 1 (issued a step ago) has landed; after
        // the barrier every wave's has, and every partial maximum is visible
        wait_vmem();
        lds_barrier();
        if (t + 2 <= t_last_wg) fetch(t + 2, (t + 2) % DQ_BUFS);
        if (!active) return;
        const uint32_t kw = __float_as_uint(sm.sk[buf][0]);
        if (MX) {
            // 32x32 blocks (this wave's queries x key half kb) lie within the wave
            int eS[2];
            v4i dc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float m = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) m = max_abs2f(m, ds[kb][r], ds[kb][r + 1]);
                eS[kb] = mx_exponent(wave_max64(m));
                dc[kb] = fp8_block_codes(ds[kb], pow2f(eS[kb]));
                if (DUMP && dp) {
                    // codes u8[q][k] at C1, exponents at [2 key half + query half] after the four P ones
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dp[dumpoff::C1 + qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] =
                            (uint8_t)((uint32_t)dc[kb][r / 4] >> (8 * (r % 4)));
                    if (lane == 0) dump_at<int>(dp, dumpoff::SC + 16)[2 * kb + qhalf] = eS[kb];
                }
            }
            // dQ^T += K^T dS^T: B = the codes (k block h = key half h, scale
            // of this lane's query for key half h)
            const v8i db8 = cat8(dc[0], dc[1]);
            const int de = (h ? eS[1] : eS[0]) + 127;
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const v8i ka = cat8(sm.kt[buf][(db * 2 + 0) * 64 + lane], sm.kt[buf][(db * 2 + 1) * 64 + lane]);
                dq[db] = mfma_fp8(ka, db8, dq[db], ebyte(kw, 2 * h + db), de);
            }
        } else {
            float sdS, invdS;
            // both partial maxima are >= 0: the larger is the larger bit pattern
            const v2i rm = *(const v2i*)&sm.red[buf][wave / 2][0];
            block_scale(__uint_as_float(umax((uint32_t)rm[0], (uint32_t)rm[1])), sdS, invdS);
            v4i dc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                dc[kb] = v4i{pack_codes(ds[kb][0], ds[kb][1], ds[kb][2], ds[kb][3], invdS),
                             pack_codes(ds[kb][4], ds[kb][5], ds[kb][6], ds[kb][7], invdS),
                             pack_codes(ds[kb][8], ds[kb][9], ds[kb][10], ds[kb][11], invdS),
                             pack_codes(ds[kb][12], ds[kb][13], ds[kb][14], ds[kb][15], invdS)};
            if (DUMP && dp) {
                if (lane == 0 && qhalf == 0) dump_at<float>(dp, dumpoff::SC)[0] = sdS;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dp[dumpoff::C1 + qloc * 64 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4)] =
                            (uint8_t)code_bits(ds[kb][r], invdS);
            }
            const float wq = sdS * __uint_as_float(kw);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                v16i acc = mfma_i8(sm.kt[buf][(db * 2 + 0) * 64 + lane], dc[0], v16i{});
                acc = mfma_i8(sm.kt[buf][(db * 2 + 1) * 64 + lane], dc[1], acc);
                if (DUMP && dp) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dump_at<int>(dp, dumpoff::ACC1)[qloc * 64 + 32 * db + 8 * (r / 4) + 4 * h + (r % 4)] = acc[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dq[db][r] = __builtin_fmaf((float)acc[r], wq, dq[db][r]);
            }
        }
    };

    fetch(0, 0);
    if (t_last_wg >= 1) fetch(1, 1);
    wait_vmem();
    lds_barrier();
    // Only the last two steps can hold a masked tile (the causal diagonal and
    // the ragged last key block come last), so they run in a loop of their
    // own and the main loop carries one form of the step.
    const int t_tail = t_last_wg > 1 ? t_last_wg - 1 : 0;
    int t = 0;
    for (; t + 2 < t_tail; t += 3) {
        step(t, Flag<false>{}, IntC<0>{});
        step(t + 1, Flag<false>{}, IntC<1>{});
        step(t + 2, Flag<false>{}, IntC<2>{});
    }
    for (; t < t_tail; ++t) step(t, Flag<false>{}, IntC<-1>{});
    for (; t <= t_last_wg; ++t) step(t, Flag<true>{}, IntC<-1>{});
    if (!live) return;
    dq_epilogue(a, dq, bh, q, h, rowbase);
}

// ------------------------------------------------------------------ MXFP8
// The same two kernels with OCP E4M3 codes and E8M0 exponents per 32x32 block
// on the scaled FP8 MFMA (block scales applied inside the instruction, so
// dK, dV and dQ accumulate in the MFMA accumulators with no per-tile
// multiply).  A 32x32 block of P or dS (32 queries of one half of the query
// block x the 32 keys of one wave) lies within one wave, so the block maxima
// need no exchange between waves, and the key-block kernel synchronizes once
// per query block (double-buffered operand tiles).  The dQ kernel is the
// INT8 one's recomputing kernel instantiated for E4M3 codes: its 32x32 dS
// blocks (32 queries of a wave x one 32-key half) also lie within one wave.

struct DkdvMxSmem {
    v4i q_r[2][256];     // Q row-operand codes (A operand of Q K^T)
    v4i q_t[2][256];     // Q transposed codes (B operand of dS^T Q)
    v4i do_t[2][256];    // dO transposed codes (B operand of P^T dO)
    v8h do16[2][512];    // dO in FP16, swizzled rows (A operand of dO V^T)
    float lse2[2][128];  // [0, 64): log2-domain LSE, [64, 128): -Delta
    uint32_t qs[2][4];   // [0]: Q block exponents, [1]: dO block exponents
};

// S = Q K^T (dequantized in the MFMA) and P = exp2(S log2(e)/8 + bias_j -
// lse2_i) for one 64-query x 32-key tile (lane = key, registers = queries),
// the correction bias_j - lse2_i one subtraction per score as in the INT8
// kernel; dP - Delta (FP16 MFMA, -Delta as the accumulator input) is formed
// here too, its MFMAs placed one by one between groups of the exps.  MASK
// only on the causal diagonal and the ragged last key block.
template <bool CAUSAL, bool MASK>
__device__ __forceinline__ void dkdv_probs_mx(const DkdvMxSmem& sm, int buf, v8i kop, uint32_t q_w, int sk_e,
                                              float kbias, int i, int key, int N, int lane, int h,
                                              float (&p)[2][16], v16f (&dpe)[2], const v8h (&vh)[4],
                                              uint8_t* dp = nullptr) {
    v8i qa[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
        qa[qb] = cat8(sm.q_r[buf][(qb * 2 + 0) * 64 + lane], sm.q_r[buf][(qb * 2 + 1) * 64 + lane]);
    v16f sx[2], corr[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) sx[qb] = mfma_fp8(qa[qb], kop, v16f{}, ebyte(q_w, 2 * qb + h), sk_e);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float4 l4 = *(const float4*)&sm.lse2[buf][32 * qb + 8 * r4 + 4 * h];
            corr[qb][4 * r4 + 0] = kbias - l4.x;
            corr[qb][4 * r4 + 1] = kbias - l4.y;
            corr[qb][4 * r4 + 2] = kbias - l4.z;
            corr[qb][4 * r4 + 3] = kbias - l4.w;
        }
    __builtin_amdgcn_sched_barrier(0);
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
        v16f d = mfma_f16(sm.do16[buf][swz(row, 0 + h)], vh[0], nd);
        d = mfma_f16(sm.do16[buf][swz(row, 2 + h)], vh[1], d);
        d = mfma_f16(sm.do16[buf][swz(row, 4 + h)], vh[2], d);
        dpe[qb] = mfma_f16(sm.do16[buf][swz(row, 6 + h)], vh[3], d);
    }
    if (dp) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dump_at<float>(dp, dumpoff::A)[(32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64)] = sx[qb][r];
    }
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
    // the score MFMAs first, then each dP MFMA between groups of exps
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    }
}

// MX tile dump: the code bytes of register r of query half qb (dword r / 4,
// byte r % 4) and the exponents of the 32 x 32 blocks at [2 key half + query half].
__device__ __forceinline__ void dump_mx_block(uint8_t* dp, int off_f, int off_c, int off_e, const float (&x)[16],
                                              v4i codes, int e, int qb, int kh, int h, int lane, int key) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int o = (32 * qb + 8 * (r / 4) + 4 * h + (r % 4)) * 64 + (key % 64);
        dump_at<float>(dp, off_f)[o] = x[r];
        dp[off_c + o] = (uint8_t)((uint32_t)codes[r / 4] >> (8 * (r % 4)));
    }
    if (lane == 0) dump_at<int>(dp, off_e)[2 * kh + qb] = e;
}

template <bool CAUSAL, bool SMOOTHQ, bool DUMP>
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
        // wave-uniform branches first, so the other waves skip them on the scalar unit
        if (wave == 0) {
            if (lane < 32)
                dma16_to_lds((lane < 16 ? a.lse2 : a.delta) + rowbase + (size_t)i * BLK + 4 * (lane % 16),
                             &sm.lse2[b][0]);
        } else if (wave == 1) {
            if (lane < 2) dma4_to_lds((lane == 0 ? a.sq : a.sdo) + bt + i, &sm.qs[b][0]);
        }
    };

    v16f dk[2] = {v16f{}, v16f{}}, dv[2] = {v16f{}, v16f{}};   // [db]: lane = channel, regs = keys
    v16f csum = v16f{};   // Q-smoothing: every column holds sum over queries of dS^ for key (row)

    fetch(i0, 0);
    const bool ragged_keys = (kvb == T - 1) && (a.N & (BLK - 1)) != 0;
    for (int i = i0; i < T; ++i) {
        const int buf = (i - i0) & 1;
        // query block i has landed in buf, and every wave is done with the
        // other buffer (query block i - 1), which the next fetch overwrites
        wait_vmem();
        lds_barrier();
        if (i + 1 < T) fetch(i + 1, buf ^ 1);
        if (!live || (CAUSAL && i < kvb)) continue;
        const bool masked = (CAUSAL && i == kvb) || ragged_keys;
        const uint32_t q_w = sm.qs[buf][0], do_w = sm.qs[buf][1];
        float p[2][16];   // [qb]: lane = key, registers = queries
        uint8_t* dp = (DUMP && bh == a.dump_bh && kvb == a.dump_t && i == a.dump_i) ? a.dump : nullptr;
        v16f dpe[2];
        if (masked) dkdv_probs_mx<CAUSAL, true>(sm, buf, kop, q_w, sk_e, kbias, i, key, a.N, lane, h, p, dpe, vh, DUMP ? dp : nullptr);
        else dkdv_probs_mx<CAUSAL, false>(sm, buf, kop, q_w, sk_e, kbias, i, key, a.N, lane, h, p, dpe, vh, DUMP ? dp : nullptr);
        // dS = P * (dP - Delta), then the four 32x32 block maxima (P and |dS| of
        // both query halves) reduced together, so the dS chain does not wait
        // for the P codes and the dV products
        float ds[2][16];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) ds[qb][r] = p[qb][r] * dpe[qb][r];
        float pmx[2], smx[2];
        {
            float pm[2] = {0.0f, 0.0f}, m[2] = {0.0f, 0.0f};
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    pm[qb] = max3f(pm[qb], p[qb][r], p[qb][r + 1]);
                    m[qb] = max_abs2f(m[qb], ds[qb][r], ds[qb][r + 1]);
                }
            wave_max64x2(pm[0], pm[1], pmx[0], pmx[1]);
            wave_max64x2(m[0], m[1], smx[0], smx[1]);
        }
        // P codes per 32x32 block (query half qb x this wave's keys)
        int eP[2];
        v4i pc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            eP[qb] = mx_exponent(pmx[qb]);
            pc[qb] = fp8_block_codes(p[qb], pow2f(eP[qb]));
            if (DUMP && dp) dump_mx_block(dp, dumpoff::F1, dumpoff::C1, dumpoff::SC, p[qb], pc[qb], eP[qb], qb, kh, h, lane, key);
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
        int eS[2];
        v4i dc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            eS[qb] = mx_exponent(smx[qb]);
            dc[qb] = fp8_block_codes(ds[qb], pow2f(eS[qb]));
            if (DUMP && dp)
                dump_mx_block(dp, dumpoff::F2, dumpoff::C2, dumpoff::SC + 16, ds[qb], dc[qb], eS[qb], qb, kh, h, lane, key);
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
    }

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
        switch ((causal ? 4 : 0) | (smooth_q ? 2 : 0) | (dump ? 1 : 0)) {
            case 0: hipLaunchKernelGGL((k_bwd_dkdv_mx<false, false, false>), grid, block, 0, st, a); break;
            case 1: hipLaunchKernelGGL((k_bwd_dkdv_mx<false, false, true>), grid, block, 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_bwd_dkdv_mx<false, true, false>), grid, block, 0, st, a); break;
            case 3: hipLaunchKernelGGL((k_bwd_dkdv_mx<false, true, true>), grid, block, 0, st, a); break;
            case 4: hipLaunchKernelGGL((k_bwd_dkdv_mx<true, false, false>), grid, block, 0, st, a); break;
            case 5: hipLaunchKernelGGL((k_bwd_dkdv_mx<true, false, true>), grid, block, 0, st, a); break;
            case 6: hipLaunchKernelGGL((k_bwd_dkdv_mx<true, true, false>), grid, block, 0, st, a); break;
            default: hipLaunchKernelGGL((k_bwd_dkdv_mx<true, true, true>), grid, block, 0, st, a); break;
        }
        return 0;
    }
    SAGEBWD_LAUNCH_BWD(k_bwd_dkdv)
}

#undef SAGEBWD_LAUNCH_BWD

int launch_bwd_dq(const BwdArgs& a, int BH, bool causal, bool int8_dp, bool mx, hipStream_t st, bool dump) {
    dim3 grid(a.ngroups * BH), block(64 * BWD_WAVES);
    if (mx) {
        switch ((causal ? 2 : 0) | (dump ? 1 : 0)) {
            case 0: hipLaunchKernelGGL((k_bwd_dq<false, true, false, false>), grid, block, 0, st, a); break;
            case 1: hipLaunchKernelGGL((k_bwd_dq<false, true, false, true>), grid, block, 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_bwd_dq<true, true, false, false>), grid, block, 0, st, a); break;
            default: hipLaunchKernelGGL((k_bwd_dq<true, true, false, true>), grid, block, 0, st, a); break;
        }
        return 0;
    }
    switch ((causal ? 4 : 0) | (int8_dp ? 2 : 0) | (dump ? 1 : 0)) {
        case 0: hipLaunchKernelGGL((k_bwd_dq<false, false, false, false>), grid, block, 0, st, a); break;
        case 1: hipLaunchKernelGGL((k_bwd_dq<false, false, false, true>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_bwd_dq<false, false, true, false>), grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_bwd_dq<false, false, true, true>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_bwd_dq<true, false, false, false>), grid, block, 0, st, a); break;
        case 5: hipLaunchKernelGGL((k_bwd_dq<true, false, false, true>), grid, block, 0, st, a); break;
        case 6: hipLaunchKernelGGL((k_bwd_dq<true, false, true, false>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((k_bwd_dq<true, false, true, true>), grid, block, 0, st, a); break;
    }
    return 0;
}

}  // namespace sagebwd
