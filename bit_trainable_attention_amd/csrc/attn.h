// Argument blocks and launchers of the attention kernels.
#pragma once
#include "common.h"

namespace sagebwd {

// Tile dump of the debug instantiations (row-major [row][col] blocks):
//   A     i32 [64][64]  score accumulator Q_code K_code^T       [query][key]
//   F1    f32 [64][64]  fwd: 127 P^ before rounding; dkdv: P
//   C1    u8  [64][64]  fwd: P~ codes; dkdv: P codes; dq: dS codes
//   ACC1  i32 [64][64]  fwd: P~ V_code [query][ch]; dkdv: P^T dO [key][ch];
//                       dq: dS K [query][ch]
//   F2    f32 [64][64]  dkdv, dq: dS
//   C2    u8  [64][64]  dkdv: dS codes
//   ACC2  i32 [64][64]  dkdv: dS^T Q [key][ch]
//   SC    f32 [4]       dkdv: s_P, s_dS; dq: s_dS
namespace dumpoff {
constexpr int A = 0, F1 = 16384, C1 = 32768, ACC1 = 36864, F2 = 53248, C2 = 69632, ACC2 = 73728, SC = 90112,
              BYTES = 90368;
}

// Compile-time flag passed to the loop-step lambdas of the attention kernels.
template <bool B>
struct Flag {
    static constexpr bool value = B;
};
template <int V>
struct IntC {
    static constexpr int value = V;
};

struct FwdArgs {
    const int8_t *q_r, *k_r, *v_t;     // code blocks [BH][T][4096]
    const float *sq, *sk, *sv;         // [BH][T] (MX: 4 exponent bytes per block)
    const float *corr, *bias;          // [BH][Np]
    uint16_t* o;                       // bf16 [BH][N][64]
    float* lse;                        // [BH][N]
    int N, T, ngroups, BH;             // ngroups = ceil(T / 2): 128 query rows per workgroup
    uint8_t* dump;                     // tile dump (debug instantiation only)
    int dump_bh, dump_i, dump_t;       // which (head, query block, key block) to dump
};

struct BwdArgs {
    const int8_t *q_r, *k_r, *q_t, *k_t, *do_t;
    const int8_t *do_r, *v_r;          // row-operand dO and V codes (INT8 dO V^T only)
    const float *sq, *sk, *sdo, *sv;   // [BH][T] (sv: INT8 dO V^T only)
    const float *bias, *delta, *lse2;  // [BH][Np]
    const _Float16 *do16, *v16;        // [BH][Np][64]
    const float* mu_q;                 // [BH][64]
    const uint16_t *q_in, *k_in;       // bf16 Q, K as passed in [BH][N][64] (QK-norm gradient)
    const float *rq, *rk;              // QK-norm factors [BH][Np], or null (no QK-norm)
    uint16_t *dq, *dk, *dv;            // bf16 [BH][N][64]
    int N, T, ngroups, BH;             // ngroups = ceil(T / 2): two 64-row blocks per workgroup
    uint8_t* dump;                     // tile dump (debug instantiation only)
    int dump_bh, dump_i, dump_t;       // which (head, query block, key block) to dump
};

// fmt: FMT_INT8, FMT_MXFP8 or FMT_FP4 (each with a tile-dump instantiation)
int launch_fwd(const FwdArgs& a, int BH, bool causal, bool smooth_q, int fmt, hipStream_t st, bool dump = false);
// int8_dp: the all-INT8 ablation, dO V^T from INT8 codes instead of FP16;
// mx: MXFP8 codes and block exponents (neither int8_dp nor a tile dump)
int launch_bwd_dkdv(const BwdArgs& a, int BH, bool causal, bool smooth_q, bool int8_dp, bool mx, hipStream_t st,
                    bool dump = false);
// int8_dp, mx: as launch_bwd_dkdv (the dQ kernel recomputes dS the same way)
int launch_bwd_dq(const BwdArgs& a, int BH, bool causal, bool int8_dp, bool mx, hipStream_t st, bool dump = false);

template <class T>
__device__ __forceinline__ T* dump_at(uint8_t* d, int off) { return (T*)(d + off); }

__device__ __forceinline__ float tile_scale(float sq, float sk) { return (sq * sk) * SCORE_SCALE_LOG2; }

}  // namespace sagebwd
