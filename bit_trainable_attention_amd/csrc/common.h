// Shared device helpers for the gfx950 SageBwd kernels.
//
// MFMA conventions used throughout (32x32 tiles, one wave of 64 lanes; lane
// l, half h = l/32):
//   INT8  v_mfma_i32_32x32x32_i8 : A lane l holds row l%32 and 16 k-bytes,
//                                  B lane l holds column l%32 and the same 16
//                                  k positions; D lane l, register r holds
//                                  element (row 8*(r/4) + 4*h + r%4, column l%32).
//   FP16  v_mfma_f32_32x32x16_f16: A/B lane l hold 8 halves of row/column l%32;
//                                  D as above.
// Because the k positions of A and B in one lane agree, any fixed assignment
// of the contraction index to (half, byte) works as long as both operands use
// it.  Two code layouts per 64x64 block follow from this:
//   row operand  (token is the M/N index, channel the k index),
//   transposed   (channel is the M/N index, token the k index, with the
//                 token order of a D register column: byte b of half h is
//                 token 8*(b/4) + 4*h + b%4 of the 32-token k-step),
// so the P / dS codes produced in D registers feed the next MFMA directly.
//   FP8   v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3): A/B lane l hold 32
//         k-bytes of row/column l%32, byte b at k = 32*(b/16) + 16*h + b%16,
//         so the two 16-byte chunks of the INT8 layouts (k-steps 0 and 1)
//         form one operand; each lane also passes the E8M0 scale of row/column
//         l%32 for the 32-k block h, and every product is multiplied by the
//         two scales.  D as above, in float32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sagebwd {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int BLK = 64;                    // tokens per block, tile side
constexpr int FMT_INT8 = 0, FMT_MXFP8 = 1, FMT_FP4 = 2;   // operand formats of a pass
constexpr int HD = 64;                     // head dimension
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float LOG2_127 = 6.988684686772166f;
constexpr float SCORE_SCALE_LOG2 = LOG2E * 0.125f;   // 1/sqrt(64) folded into log2 domain
// 1.5 * 2^23: adding it rounds a float in (-2^22, 2^22) to the nearest
// integer (ties to even) and leaves that integer in the low mantissa bits.
constexpr float MAGIC = 12582912.0f;
constexpr uint32_t MAGIC_BITS = 0x4B400000u;
constexpr float A_MIN = 0x1p-100f;         // smaller block absmax -> all-zero block
constexpr float R127 = 1.0f / 127.0f;      // correctly rounded float32 of 1/127

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// QK-norm of one bf16 element with its token's factor r: bf16(fp32(x r)),
// returned as float32.
__device__ __forceinline__ float qk_normed(uint32_t bits16, float r) {
    return bf16_to_f32(f32_to_bf16_rne(bf16_to_f32(bits16) * r));
}
constexpr double QK_NORM_EPS = 1e-6;

// 127/a, correctly rounded, for finite a >= 2^-100, in five VALU instructions
// instead of the twelve of the generic IEEE division: with a' = a 2^-4
// (exact) and n = 127 2^-4, q0 = n rcp(a') and one fused correction
// q = q0 + (n - a' q0) rcp(a').  The pre-scale keeps rcp(a') a normal number
// up to the largest finite a.  On gfx950 this q equals the correctly rounded
// quotient for every float32 a in [2^-121, 2^128), which was checked
// exhaustively (all 2^23 mantissas at every exponent) against the compiled
// division by sagebwd_check_block_scale.
__device__ __forceinline__ float div127(float a) {
    const float as = a * 0x1p-4f;
    const float y = __builtin_amdgcn_rcpf(as);
    const float q0 = 7.9375f * y;
    return __builtin_fmaf(__builtin_fmaf(-as, q0, 7.9375f), y, q0);
}

// a/127, correctly rounded, in three VALU instructions: q0 = a RN(1/127),
// the residual r = a - 127 q0 (exact in one FMA: it is a small multiple of
// ulp(q0), subnormal near a = 2^-100, which this build keeps), and one fused
// correction q = q0 + r RN(1/127).  Equal to the correctly rounded quotient
// for every float32 a in [2^-100, 2^128) (sagebwd_check_block_scale compares
// all of them with the IEEE division on the GPU).
__device__ __forceinline__ float quot127(float a) {
    const float q0 = a * R127;
    return __builtin_fmaf(__builtin_fmaf(-127.0f, q0, a), R127, q0);
}

// Per-block scale from an absmax: s = a/127 and inv = 127/a, both the
// correctly rounded float32 quotients; blocks with a < 2^-100 are all-zero.
__device__ __forceinline__ void block_scale(float a, float& s, float& inv) {
    if (a >= A_MIN) {
        s = quot127(a);
        inv = div127(a);
    } else {
        s = 0.0f;
        inv = 0.0f;
    }
}

// round-half-even(x * inv) of the exact product, as magic-biased float bits:
// the low byte is the two's-complement int8 code.
__device__ __forceinline__ uint32_t code_bits(float x, float inv) {
    return __float_as_uint(__builtin_fmaf(x, inv, MAGIC));
}
__device__ __forceinline__ int code_int(float x, float inv) {
    return (int)(code_bits(x, inv) - MAGIC_BITS);
}
// MXFP8 (OCP E4M3 codes, one E8M0 power-of-two scale per 32 x 32 block):
// the least e with 448 2^e >= a, clamped to [-126, 127].  a = m 2^E with m in
// [1, 2): e = E - 8, plus 1 when m > 1.75 (448 = 1.75 2^8); zero and
// subnormal a clamp to -126.
__device__ __forceinline__ int mx_exponent(float a) {
    const uint32_t u = __float_as_uint(a);
    const int e = (int)((u >> 23) & 0xFFu) - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return e < -126 ? -126 : (e > 127 ? 127 : e);
}
// FP4 (E2M1, one E8M0 scale per 32 values): the least e with 6 2^e >= a,
// clamped to [-126, 127].  a = m 2^E with m in [1, 2): e = E - 2, plus 1
// when m > 1.5 (6 = 1.5 2^2); zero and subnormal a clamp to -126.
__device__ __forceinline__ int fp4_exponent(float a) {
    const uint32_t u = __float_as_uint(a);
    const int e = (int)((u >> 23) & 0xFFu) - 129 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    return e < -126 ? -126 : (e > 127 ? 127 : e);
}
// Two E2M1 codes rne(x / scale), rne(y / scale) (scale a power of two) into
// byte SEL of old (x in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float x, float y, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x, y, scale, SEL);
}
// Eight E2M1 codes of x[0..7] / scale in one dword (value i in nibble i).
__device__ __forceinline__ uint32_t fp4_oct(const float* x, float scale) {
    uint32_t w = fp4_pair<0>(__float_as_uint(x[0]), x[0], x[1], scale);   // every nibble is overwritten
    w = fp4_pair<1>(w, x[2], x[3], scale);
    w = fp4_pair<2>(w, x[4], x[5], scale);
    return fp4_pair<3>(w, x[6], x[7], scale);
}
// 2^e as a float32 (e in [-126, 127]).
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
// Two E4M3 codes rne(x / scale), rne(y / scale) (scale a power of two) in the
// low (hi = false) or high 16 bits of old.
typedef short v2s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8_pair(uint32_t old, float x, float y, float scale, bool hi) {
    v2s o = __builtin_bit_cast(v2s, old);
    o = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, x, y, scale, true)
           : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, x, y, scale, false);
    return __builtin_bit_cast(uint32_t, o);
}
// Four E4M3 codes of x0..x3 / scale packed in one dword (byte 0 from x0).
__device__ __forceinline__ uint32_t fp8_quad(float x0, float x1, float x2, float x3, float scale) {
    // the two pairs overwrite the low and then the high half, so the starting
    // value is never read: x0's own bits let its register serve when x0 is
    // dead here (a literal 0 costs a move every time)
    return fp8_pair(fp8_pair(__float_as_uint(x0), x0, x1, scale, false), x2, x3, scale, true);
}

// Value of E4M3 code byte j of w (j a constant after unrolling).
__device__ __forceinline__ float fp8_value(uint32_t w, int j) {
    switch (j) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
    }
}

// rne(v) for v already scaled (0 <= v < 2^22), as magic-biased bits.
__device__ __forceinline__ uint32_t round_bits(float v) {
    return __float_as_uint(v + MAGIC);
}

// Pack the low bytes of four words into one dword (byte 0 from a).
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);   // [a0, b0, 0, 0]
    uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000c0cu);   // [0, 0, c0, d0]
    return lo | hi;
}

__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f16(v8h a, v8h b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// E4M3 x E4M3 with E8M0 scales sa (this lane's row of A) and sb (column of B),
// each a biased exponent in bits 0..7.
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ v8i cat8(v4i x, v4i y) { return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]}; }
// Byte i of a word of four block exponents.
__device__ __forceinline__ int ebyte(uint32_t w, int i) { return (int)((w >> (8 * i)) & 0xFFu); }
// A value the compiler cannot fold: a literal scale operand would be encoded
// as an inline float constant rather than as the integer exponent.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}
constexpr int E8M0_ONE = 127;              // biased exponent of 2^0
constexpr int E4M3_ONE = 0x38;             // E4M3 code of 1.0
// E2M1 x E2M1 on the scaled MFMA: each half of the wave holds the 32 values
// of its own 32-k block (16 bytes, value i in nibble i), sa/sb as mfma_fp8.
__device__ __forceinline__ v16f mfma_fp4(v4i a, v4i b, v16f c, int sa, int sb) {
    const v8i a8 = cat8(a, v4i{}), b8 = cat8(b, v4i{});
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}
constexpr uint32_t E2M1_ONES = 0x22222222u;   // eight E2M1 codes of 1.0
constexpr int FP4_EXP_OFF = 2048;             // exponent bytes after the codes of an FP4 block


// max(a, b, c) and max(a, |b|, |c|), written so the compiler sees them (it
// forms v_max3_f32 itself and inserts the wait states an MFMA or
// transcendental result needs before a VALU instruction reads it).  The
// operands are arithmetic results, never signaling NaNs, so no quieting is
// needed; the compiler knows this of the results it can see.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}
__device__ __forceinline__ float max_abs2f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, __builtin_fabsf(b)), __builtin_fabsf(c));
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

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
// The same through a raw buffer resource: the address is the resource's base
// plus a per-lane byte offset (a VGPR) plus a wave-uniform byte offset (an
// SGPR), so a stream walked block by block costs no vector-ALU address
// arithmetic per copy; reads beyond the resource's size return zeros.
// The resource's last word sets a 32-bit data format (untyped loads need a
// nonzero one); its size is in bytes (stride 0).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bdma16_to_lds(rsrc_t r, uint32_t lane_off, uint32_t wave_off, void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, lane_off,
                                             wave_off, 0, 0);
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

// Byte offsets of element (token r, channel c) inside a 64x64 code block.
__host__ __device__ constexpr int row_operand_offset(int r, int c) {
    return (((r / 32) * 2 + c / 32) * 64 + 32 * ((c % 32) / 16) + r % 32) * 16 + c % 16;
}
__host__ __device__ constexpr int transposed_operand_offset(int r, int c) {
    return (((c / 32) * 2 + r / 32) * 64 + 32 * ((r % 8) / 4) + c % 32) * 16 + 4 * ((r % 32) / 8) + r % 4;
}

}  // namespace sagebwd
