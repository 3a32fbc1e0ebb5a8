// Argument blocks and launchers of the preparation kernels.
#pragma once
#include "common.h"

namespace sagebwd {

constexpr int SUM_CHUNK = 256;   // tokens per partial column sum

struct MeansArgs {
    const uint16_t* q;
    const uint16_t* k;
    const float *rq, *rk;              // QK-norm factors [BH][Np], or null
    double* sums;      // [BH][2][nchunk][64]
    float* mu_q;       // [BH][64]
    float* mu_k;
    int N, BH, smooth_q, smooth_k;
};

struct QuantArgs {
    const uint16_t *q, *k, *v;         // bf16 [BH][N][64]
    const float *rq, *rk;              // QK-norm factors [BH][Np], or null
    const float *mu_q, *mu_k;          // [BH][64]
    int8_t *q_r, *k_r;                 // row operand layout (nullable)
    int8_t *q_t, *k_t, *v_t;           // transposed operand layout (nullable)
    float *sq, *sk, *sv;               // [BH][T] (MX: 4 exponent bytes per block)
    float* corr;                       // [BH][Np]
    float* bias;                       // [BH][Np]
    int N, T, smooth_q, smooth_k;
};

struct BwdPreArgs {
    const uint16_t *dout, *o, *v;      // bf16 [BH][N][64]
    const float* lse;                  // [BH][N]
    const float* corr;                 // [BH][Np]
    float *delta, *lse2;               // [BH][Np]: -rowsum(dO*O), log2-domain LSE
    int8_t* do_t;                      // transposed operand layout
    float* sdo;                        // [BH][T] (MX: 4 exponent bytes per block)
    int8_t *do_r, *v_r;                // row-operand dO and V codes, or null (INT8 dO V^T only)
    float* sv;                         // [BH][T] V block scales, with v_r
    _Float16 *do16, *v16;              // [BH][Np][64]
    int N, T;
};

int launch_rownorm(const uint16_t* q, const uint16_t* k, float* rq, float* rk, int N, int T, int BH, hipStream_t st);
int launch_means(const MeansArgs& m, hipStream_t st);
// fmt: FMT_INT8, FMT_MXFP8 or FMT_FP4 (Q, K row FP4 blocks and V class FP4
// blocks in q_r, k_r, v_t; q_t, k_t unused)
int launch_quantize(const QuantArgs& a, int BH, int ntensors, int fmt, hipStream_t st);
int launch_bwd_pre(const BwdPreArgs& a, int BH, bool mx, hipStream_t st);

}  // namespace sagebwd
