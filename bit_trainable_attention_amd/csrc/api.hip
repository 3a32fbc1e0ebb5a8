// C ABI of the library: argument validation, workspace layout and the launch
// sequence of the forward and backward passes.  Declarations and the full
// contract are in include/sagebwd.h.
#include "sagebwd.h"

#include <algorithm>
#include <mutex>

#include "attn.h"
#include "prep.h"

namespace {

using namespace sagebwd;

enum Region {
    R_MU_Q = 0, R_MU_K, R_Q_R, R_K_R, R_V_T, R_Q_T, R_K_T, R_DO_T,
    R_S_Q, R_S_K, R_S_V, R_S_DO, R_CORR, R_BIAS, R_DELTA, R_LSE2, R_DO16, R_V16,
    R_DO_R, R_V_R, R_RQ, R_RK, R_SUMS, R_COUNT
};

struct Layout {
    size_t off[R_COUNT];
    size_t bytes[R_COUNT];
    size_t total;
};

constexpr int32_t MAX_N = 1 << 18;
constexpr int64_t MAX_BH = 65535;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Which regions a pass uses: the forward needs Q/K row codes and V
// transposed codes; the backward needs Q/K in both layouts and its own
// per-row data; the inspection call prepares everything.
enum Pass { PASS_FWD, PASS_BWD };

Layout make_layout(const sagebwd_params& p, Pass pass) {
    Layout L{};
    const size_t BH = (size_t)p.B * p.H;
    const size_t T = ((size_t)p.N + BLK - 1) / BLK;
    const size_t Np = T * BLK;
    const size_t nchunk = ((size_t)p.N + SUM_CHUNK - 1) / SUM_CHUNK;
    const bool bwd = pass == PASS_BWD;
    size_t sz[R_COUNT] = {};
    sz[R_MU_Q] = BH * HD * 4;
    sz[R_MU_K] = BH * HD * 4;
    sz[R_Q_R] = BH * T * 4096;
    sz[R_K_R] = BH * T * 4096;
    sz[R_V_T] = BH * T * 4096;
    sz[R_Q_T] = BH * T * 4096;     // the forward writes these too, for a backward that reuses them
    sz[R_K_T] = BH * T * 4096;
    sz[R_DO_T] = bwd ? BH * T * 4096 : 0;
    sz[R_S_Q] = BH * T * 4;
    sz[R_S_K] = BH * T * 4;
    sz[R_S_V] = BH * T * 4;
    sz[R_S_DO] = bwd ? BH * T * 4 : 0;
    sz[R_CORR] = BH * Np * 4;
    sz[R_BIAS] = BH * Np * 4;
    sz[R_DELTA] = bwd ? BH * Np * 4 : 0;
    sz[R_LSE2] = bwd ? BH * Np * 4 : 0;
    sz[R_DO16] = bwd ? BH * Np * HD * 2 : 0;
    sz[R_V16] = bwd ? BH * Np * HD * 2 : 0;
    const bool i8dp = bwd && p.int8_dp;            // row-operand dO and V codes for INT8 dO V^T
    sz[R_DO_R] = i8dp ? BH * T * 4096 : 0;
    sz[R_V_R] = i8dp ? BH * T * 4096 : 0;
    sz[R_RQ] = p.qk_norm ? BH * Np * 4 : 0;         // QK-norm factors of Q and K tokens
    sz[R_RK] = p.qk_norm ? BH * Np * 4 : 0;
    sz[R_SUMS] = BH * 2 * nchunk * HD * 8;
    size_t o = 0;
    for (int r = 0; r < R_COUNT; ++r) {
        L.off[r] = o;
        L.bytes[r] = sz[r];
        o += align256(sz[r]);
    }
    L.total = o;
    return L;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int check_params(const sagebwd_params* p) {
    if (!p) return SAGEBWD_ERR_INVALID_ARG;
    if (p->B < 1 || p->H < 1 || p->N < 1) return SAGEBWD_ERR_INVALID_ARG;
    if ((p->causal != 0 && p->causal != 1) || (p->smooth_q != 0 && p->smooth_q != 1) ||
        (p->smooth_k != 0 && p->smooth_k != 1) || (p->int8_dp != 0 && p->int8_dp != 1) ||
        (p->qk_norm != 0 && p->qk_norm != 1) || (p->mxfp8 != 0 && p->mxfp8 != 1) || (p->fp4 != 0 && p->fp4 != 1))
        return SAGEBWD_ERR_INVALID_ARG;
    if (p->D != HD) return SAGEBWD_ERR_UNSUPPORTED;
    if (p->mxfp8 && p->int8_dp) return SAGEBWD_ERR_UNSUPPORTED;   // the INT8 ablation has no MXFP8 form
    if (p->fp4 && (p->mxfp8 || p->int8_dp)) return SAGEBWD_ERR_UNSUPPORTED;
    if (p->N > MAX_N || (int64_t)p->B * p->H > MAX_BH) return SAGEBWD_ERR_UNSUPPORTED;
    return SAGEBWD_OK;
}

int check_tensor(const void* ptr) {
    if (!ptr) return SAGEBWD_ERR_INVALID_ARG;
    if (!aligned(ptr, 16)) return SAGEBWD_ERR_INVALID_ARG;
    return SAGEBWD_OK;
}

int check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
    if (!ws || !aligned(ws, 256)) return SAGEBWD_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return SAGEBWD_ERR_WORKSPACE;
    return SAGEBWD_OK;
}

template <class T>
T* region(void* ws, const Layout& L, int r) {
    return L.bytes[r] ? (T*)((char*)ws + L.off[r]) : nullptr;
}

int hip_status() { return hipGetLastError() == hipSuccess ? SAGEBWD_OK : SAGEBWD_ERR_HIP; }

// The workspace of sagebwd_fwd_noalloc: one static device array, which each
// GPU holds at its own address.  Host code never uses the array's name as a
// device pointer: the address of each device's copy is looked up once, with
// that device current, and kept.
static __device__ __align__(256) unsigned char scratch[SAGEBWD_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;

// Address of this device's copy of the scratch array, or null on failure.
void* scratch_ptr(int device) {
    static std::mutex mu;
    static void* ptrs[SCRATCH_MAX_DEVICES] = {};
    if (device < 0 || device >= SCRATCH_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[device]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptrs[device] = ptr;
    }
    return ptrs[device];
}

int operand_format(const sagebwd_params& p) { return p.fp4 ? FMT_FP4 : p.mxfp8 ? FMT_MXFP8 : FMT_INT8; }

// Means + quantization of Q, K, V into the regions of this layout.
void run_prepare_qkv(const sagebwd_params& p, const Layout& L, const void* Q, const void* K, const void* V,
                     void* ws, bool want_row, bool want_vt, bool want_qkt, hipStream_t st) {
    const int BH = p.B * p.H;
    const int T = (p.N + BLK - 1) / BLK;
    float* rq = region<float>(ws, L, R_RQ);     // null without QK-norm
    float* rk = region<float>(ws, L, R_RK);
    if (rq) launch_rownorm((const uint16_t*)Q, (const uint16_t*)K, rq, rk, p.N, T, BH, st);
    MeansArgs m{};
    m.q = (const uint16_t*)Q;
    m.k = (const uint16_t*)K;
    m.rq = rq;
    m.rk = rk;
    m.sums = region<double>(ws, L, R_SUMS);
    m.mu_q = region<float>(ws, L, R_MU_Q);
    m.mu_k = region<float>(ws, L, R_MU_K);
    m.N = p.N;
    m.BH = BH;
    m.smooth_q = p.smooth_q;
    m.smooth_k = p.smooth_k;
    launch_means(m, st);

    QuantArgs a{};
    a.q = (const uint16_t*)Q;
    a.k = (const uint16_t*)K;
    a.v = (const uint16_t*)V;
    a.rq = rq;
    a.rk = rk;
    a.mu_q = m.mu_q;
    a.mu_k = m.mu_k;
    a.q_r = want_row ? region<int8_t>(ws, L, R_Q_R) : nullptr;
    a.k_r = want_row ? region<int8_t>(ws, L, R_K_R) : nullptr;
    a.q_t = want_qkt ? region<int8_t>(ws, L, R_Q_T) : nullptr;
    a.k_t = want_qkt ? region<int8_t>(ws, L, R_K_T) : nullptr;
    a.v_t = want_vt ? region<int8_t>(ws, L, R_V_T) : nullptr;
    a.sq = region<float>(ws, L, R_S_Q);
    a.sk = region<float>(ws, L, R_S_K);
    a.sv = region<float>(ws, L, R_S_V);
    a.corr = region<float>(ws, L, R_CORR);
    a.bias = region<float>(ws, L, R_BIAS);
    a.N = p.N;
    a.T = T;
    a.smooth_q = p.smooth_q;
    a.smooth_k = p.smooth_k;
    // V's block scales are only needed by the forward and the inspection call
    launch_quantize(a, BH, want_vt ? 3 : 2, operand_format(p), st);
}

// Where the backward reads the quantized Q and K (means, codes in both
// layouts, scales, LSE correction, Q-smoothing bias): its own workspace after
// re-quantizing, or the workspace of the forward that produced them.
struct QkSource {
    void* ws;
    Layout L;
};

void run_bwd_pre(const sagebwd_params& p, const Layout& L, const QkSource& qk, const void* V, const void* O,
                 const float* LSE, const void* dO, void* ws, hipStream_t st) {
    BwdPreArgs b{};
    b.dout = (const uint16_t*)dO;
    b.o = (const uint16_t*)O;
    b.v = (const uint16_t*)V;
    b.lse = LSE;
    b.corr = region<float>(qk.ws, qk.L, R_CORR);
    b.delta = region<float>(ws, L, R_DELTA);
    b.lse2 = region<float>(ws, L, R_LSE2);
    b.do_t = region<int8_t>(ws, L, R_DO_T);
    b.sdo = region<float>(ws, L, R_S_DO);
    b.do16 = region<_Float16>(ws, L, R_DO16);
    b.v16 = region<_Float16>(ws, L, R_V16);
    b.do_r = region<int8_t>(ws, L, R_DO_R);       // null unless int8_dp
    b.v_r = region<int8_t>(ws, L, R_V_R);
    b.sv = b.v_r ? region<float>(ws, L, R_S_V) : nullptr;
    b.N = p.N;
    b.T = (p.N + BLK - 1) / BLK;
    launch_bwd_pre(b, p.B * p.H, p.mxfp8 != 0, st);
}

FwdArgs fwd_args(const sagebwd_params& p, const Layout& L, void* ws, void* O, float* LSE) {
    FwdArgs a{};
    a.q_r = region<int8_t>(ws, L, R_Q_R);
    a.k_r = region<int8_t>(ws, L, R_K_R);
    a.v_t = region<int8_t>(ws, L, R_V_T);
    a.sq = region<float>(ws, L, R_S_Q);
    a.sk = region<float>(ws, L, R_S_K);
    a.sv = region<float>(ws, L, R_S_V);
    a.corr = region<float>(ws, L, R_CORR);
    a.bias = region<float>(ws, L, R_BIAS);
    a.o = (uint16_t*)O;
    a.lse = LSE;
    a.N = p.N;
    a.T = (p.N + BLK - 1) / BLK;
    a.ngroups = (a.T + 1) / 2;
    a.BH = p.B * p.H;
    a.dump = nullptr;
    a.dump_bh = a.dump_i = a.dump_t = -1;
    return a;
}

BwdArgs bwd_args(const sagebwd_params& p, const Layout& L, const QkSource& qk, void* ws, const void* Q,
                 const void* K, void* dQ, void* dK, void* dV) {
    BwdArgs a{};
    a.q_in = (const uint16_t*)Q;
    a.k_in = (const uint16_t*)K;
    a.q_r = region<int8_t>(qk.ws, qk.L, R_Q_R);
    a.k_r = region<int8_t>(qk.ws, qk.L, R_K_R);
    a.q_t = region<int8_t>(qk.ws, qk.L, R_Q_T);
    a.k_t = region<int8_t>(qk.ws, qk.L, R_K_T);
    a.do_t = region<int8_t>(ws, L, R_DO_T);
    a.do_r = region<int8_t>(ws, L, R_DO_R);
    a.v_r = region<int8_t>(ws, L, R_V_R);
    a.sv = a.v_r ? region<float>(ws, L, R_S_V) : nullptr;   // written by the backward's own preparation
    a.sq = region<float>(qk.ws, qk.L, R_S_Q);
    a.sk = region<float>(qk.ws, qk.L, R_S_K);
    a.sdo = region<float>(ws, L, R_S_DO);
    a.bias = region<float>(qk.ws, qk.L, R_BIAS);
    a.delta = region<float>(ws, L, R_DELTA);
    a.lse2 = region<float>(ws, L, R_LSE2);
    a.do16 = region<_Float16>(ws, L, R_DO16);
    a.v16 = region<_Float16>(ws, L, R_V16);
    a.mu_q = region<float>(qk.ws, qk.L, R_MU_Q);
    a.rq = region<float>(qk.ws, qk.L, R_RQ);
    a.rk = region<float>(qk.ws, qk.L, R_RK);
    a.dq = (uint16_t*)dQ;
    a.dk = (uint16_t*)dK;
    a.dv = (uint16_t*)dV;
    a.N = p.N;
    a.T = (p.N + BLK - 1) / BLK;
    a.ngroups = (a.T + 1) / 2;
    a.BH = p.B * p.H;
    a.dump = nullptr;
    a.dump_bh = a.dump_i = a.dump_t = -1;
    return a;
}

// The two attention kernels of the backward.  which: 1 the dK/dV kernel, 2
// the dQ kernel, 3 both; kernel_dump selects which of them (1: dK/dV, 2: dQ)
// runs its debug instantiation.  The two are independent: each recomputes
// the scores, P and dS it needs.
void run_bwd_attn(const sagebwd_params& p, const BwdArgs& a, int which, int kernel_dump, hipStream_t st) {
    const int BH = p.B * p.H;
    if (which & 1) launch_bwd_dkdv(a, BH, p.causal, p.smooth_q, p.int8_dp, p.mxfp8, st, kernel_dump == 1);
    if (which & 2) launch_bwd_dq(a, BH, p.causal, p.int8_dp, p.mxfp8, st, kernel_dump == 2);
}

}  // namespace

extern "C" {

size_t sagebwd_fwd_workspace_size(const sagebwd_params* p) {
    if (check_params(p) != SAGEBWD_OK) return 0;
    return make_layout(*p, PASS_FWD).total;
}

size_t sagebwd_bwd_workspace_size(const sagebwd_params* p) {
    if (check_params(p) != SAGEBWD_OK) return 0;
    return make_layout(*p, PASS_BWD).total;
}

const char* sagebwd_status_string(int status) {
    switch (status) {
        case SAGEBWD_OK: return "ok";
        case SAGEBWD_ERR_INVALID_ARG: return "invalid argument";
        case SAGEBWD_ERR_UNSUPPORTED: return "unsupported shape";
        case SAGEBWD_ERR_WORKSPACE: return "workspace too small";
        case SAGEBWD_ERR_HIP: return "HIP launch error";
        case SAGEBWD_ERR_SCRATCH: return "workspace exceeds the built-in scratch buffer";
        default: return "unknown status";
    }
}

int sagebwd_fwd_stage(const sagebwd_params* p, int stage, const void* Q, const void* K, const void* V, void* O,
                      float* LSE, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (stage != SAGEBWD_STAGE_FWD_PREPARE && stage != SAGEBWD_STAGE_FWD_ATTN) return SAGEBWD_ERR_INVALID_ARG;
    for (const void* t : {Q, K, V, (const void*)O}) {
        if ((rc = check_tensor(t))) return rc;
    }
    if (!LSE || !aligned(LSE, 4)) return SAGEBWD_ERR_INVALID_ARG;
    const Layout L = make_layout(*p, PASS_FWD);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (stage == SAGEBWD_STAGE_FWD_PREPARE) {
        run_prepare_qkv(*p, L, Q, K, V, ws, true, true, !p->fp4, st);
        return hip_status();
    }
    const FwdArgs a = fwd_args(*p, L, ws, O, LSE);
    launch_fwd(a, p->B * p->H, p->causal, p->smooth_q, operand_format(*p), st);
    return hip_status();
}

int sagebwd_fwd(const sagebwd_params* p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                void* ws, size_t ws_bytes, void* stream) {
    int rc = sagebwd_fwd_stage(p, SAGEBWD_STAGE_FWD_PREPARE, Q, K, V, O, LSE, ws, ws_bytes, stream);
    if (rc) return rc;
    return sagebwd_fwd_stage(p, SAGEBWD_STAGE_FWD_ATTN, Q, K, V, O, LSE, ws, ws_bytes, stream);
}

int sagebwd_fwd_noalloc(const sagebwd_params* p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                        void* stream) {
    int rc = check_params(p);
    if (rc) return rc;
    for (const void* t : {Q, K, V, (const void*)O}) {
        if ((rc = check_tensor(t))) return rc;
    }
    if (!LSE || !aligned(LSE, 4)) return SAGEBWD_ERR_INVALID_ARG;
    const size_t need = make_layout(*p, PASS_FWD).total;
    if (need > SAGEBWD_NOALLOC_SCRATCH_BYTES) return SAGEBWD_ERR_SCRATCH;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) return SAGEBWD_ERR_HIP;
    void* ws = scratch_ptr(device);
    if (!ws) return SAGEBWD_ERR_HIP;
    return sagebwd_fwd(p, Q, K, V, O, LSE, ws, SAGEBWD_NOALLOC_SCRATCH_BYTES, stream);
}

int sagebwd_bwd_stage(const sagebwd_params* p, int stage, const void* Q, const void* K, const void* V,
                      const void* O, const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                      const void* fwd_ws, size_t fwd_ws_bytes, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (stage != SAGEBWD_STAGE_BWD_PREPARE && stage != SAGEBWD_STAGE_BWD_DKDV && stage != SAGEBWD_STAGE_BWD_DQ &&
        stage != SAGEBWD_STAGE_BWD_ATTN)
        return SAGEBWD_ERR_INVALID_ARG;
    if (p->fp4) return SAGEBWD_ERR_UNSUPPORTED;   // the FP4 mode is an inference forward
    for (const void* t : {Q, K, V, O, dO, (const void*)dQ, (const void*)dK, (const void*)dV}) {
        if ((rc = check_tensor(t))) return rc;
    }
    if (!LSE || !aligned(LSE, 4)) return SAGEBWD_ERR_INVALID_ARG;
    const Layout L = make_layout(*p, PASS_BWD);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    QkSource qk{ws, L};
    if (fwd_ws) {
        qk.L = make_layout(*p, PASS_FWD);
        if ((rc = check_ws(qk.L, fwd_ws, fwd_ws_bytes))) return rc;
        const uintptr_t f0 = (uintptr_t)fwd_ws, f1 = f0 + qk.L.total, w0 = (uintptr_t)ws, w1 = w0 + L.total;
        if (f0 < w1 && w0 < f1) return SAGEBWD_ERR_INVALID_ARG;   // the two workspaces overlap
        qk.ws = const_cast<void*>(fwd_ws);   // read only
    }
    hipStream_t st = (hipStream_t)stream;
    if (stage == SAGEBWD_STAGE_BWD_PREPARE) {
        if (!fwd_ws) run_prepare_qkv(*p, L, Q, K, V, ws, true, false, true, st);
        run_bwd_pre(*p, L, qk, V, O, LSE, dO, ws, st);
        return hip_status();
    }
    const BwdArgs a = bwd_args(*p, L, qk, ws, Q, K, dQ, dK, dV);
    run_bwd_attn(*p, a, stage == SAGEBWD_STAGE_BWD_ATTN ? 3 : stage == SAGEBWD_STAGE_BWD_DKDV ? 1 : 2, 0, st);
    return hip_status();
}

// The whole backward: preparation, then the dK/dV kernel and the dQ kernel.
static int bwd_pass(const sagebwd_params* p, const void* Q, const void* K, const void* V, const void* O,
             const float* LSE, const void* dO, void* dQ, void* dK, void* dV, const void* fwd_ws,
             size_t fwd_ws_bytes, void* ws, size_t ws_bytes, hipStream_t st) {
    int rc = sagebwd_bwd_stage(p, SAGEBWD_STAGE_BWD_PREPARE, Q, K, V, O, LSE, dO, dQ, dK, dV, fwd_ws, fwd_ws_bytes,
                               ws, ws_bytes, st);
    if (rc) return rc;
    return sagebwd_bwd_stage(p, SAGEBWD_STAGE_BWD_ATTN, Q, K, V, O, LSE, dO, dQ, dK, dV, fwd_ws, fwd_ws_bytes, ws,
                             ws_bytes, st);
}

int sagebwd_bwd(const sagebwd_params* p, const void* Q, const void* K, const void* V, const void* O,
                const float* LSE, const void* dO, void* dQ, void* dK, void* dV, const void* fwd_ws,
                size_t fwd_ws_bytes, void* ws, size_t ws_bytes, void* stream) {
    return bwd_pass(p, Q, K, V, O, LSE, dO, dQ, dK, dV, fwd_ws, fwd_ws_bytes, ws, ws_bytes, (hipStream_t)stream);
}

int sagebwd_debug_tile(const sagebwd_params* p, int kernel, int bh, int qblock, int kblock, const void* Q,
                       const void* K, const void* V, void* O, float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                       void* dump, size_t dump_bytes, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(p);
    if (rc) return rc;
    const int T = (p->N + BLK - 1) / BLK;
    if (kernel < 0 || kernel > 2 || bh < 0 || bh >= p->B * p->H || qblock < 0 || qblock >= T || kblock < 0 ||
        kblock >= T || (p->causal && kblock > qblock))
        return SAGEBWD_ERR_INVALID_ARG;
    if (!dump || dump_bytes < (size_t)dumpoff::BYTES) return SAGEBWD_ERR_INVALID_ARG;
    if (p->fp4 && kernel != 0) return SAGEBWD_ERR_UNSUPPORTED;   // FP4: forward only
    if (kernel == 0) {
        if ((rc = sagebwd_fwd_stage(p, SAGEBWD_STAGE_FWD_PREPARE, Q, K, V, O, LSE, ws, ws_bytes, stream))) return rc;
        const Layout L = make_layout(*p, PASS_FWD);
        FwdArgs a = fwd_args(*p, L, ws, O, LSE);
        a.dump = (uint8_t*)dump;
        a.dump_bh = bh;
        a.dump_i = qblock;
        a.dump_t = kblock;
        launch_fwd(a, p->B * p->H, p->causal, p->smooth_q, operand_format(*p), (hipStream_t)stream, true);
        return hip_status();
    }
    if ((rc = sagebwd_bwd_stage(p, SAGEBWD_STAGE_BWD_PREPARE, Q, K, V, O, LSE, dO, dQ, dK, dV, nullptr, 0, ws,
                                ws_bytes, stream)))
        return rc;
    const Layout L = make_layout(*p, PASS_BWD);
    BwdArgs a = bwd_args(*p, L, QkSource{ws, L}, ws, Q, K, dQ, dK, dV);
    a.dump = (uint8_t*)dump;
    a.dump_bh = bh;
    a.dump_i = qblock;
    a.dump_t = kblock;
    // kernel 1: the dK/dV kernel; kernel 2: both (the dQ kernel dumps)
    run_bwd_attn(*p, a, kernel == 1 ? 1 : 3, kernel, (hipStream_t)stream);
    return hip_status();
}

int sagebwd_prepare(const sagebwd_params* p, const void* Q, const void* K, const void* V, const void* O,
                    const float* LSE, const void* dO, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(p);
    if (rc) return rc;
    for (const void* t : {Q, K, V}) {
        if ((rc = check_tensor(t))) return rc;
    }
    const bool with_bwd = dO != nullptr;
    if (with_bwd && p->fp4) return SAGEBWD_ERR_UNSUPPORTED;
    if (with_bwd) {
        if ((rc = check_tensor(O)) || (rc = check_tensor(dO))) return rc;
        if (!LSE || !aligned(LSE, 4)) return SAGEBWD_ERR_INVALID_ARG;
    } else if (O || LSE) {
        return SAGEBWD_ERR_INVALID_ARG;
    }
    const Layout L = make_layout(*p, PASS_BWD);
    if ((rc = check_ws(L, ws, ws_bytes))) return rc;
    hipStream_t st = (hipStream_t)stream;
    run_prepare_qkv(*p, L, Q, K, V, ws, true, true, !p->fp4, st);
    if (with_bwd) run_bwd_pre(*p, L, QkSource{ws, L}, V, O, LSE, dO, ws, st);
    return hip_status();
}

int sagebwd_ws_region(const sagebwd_params* p, int region_id, size_t* offset, size_t* bytes) {
    int rc = check_params(p);
    if (rc) return rc;
    if (region_id < 0 || region_id >= R_SUMS || !offset || !bytes) return SAGEBWD_ERR_INVALID_ARG;
    const Layout L = make_layout(*p, PASS_BWD);
    *offset = L.off[region_id];
    *bytes = L.bytes[region_id];
    return SAGEBWD_OK;
}

}  // extern "C"
