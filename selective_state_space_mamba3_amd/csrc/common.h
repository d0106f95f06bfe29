// Device helpers shared by the gfx950 kernels of the Mamba-3 forward path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// v_mfma_f32_16x16x4_f32, one 16x16 block, fp32 in / fp32 accumulate.
// Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; register r of the
// result in lane l is D[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Split fp32 products on v_mfma_f32_16x16x32_bf16.  Lane l supplies
// A[l % 16][k] and B[k][l % 16] for eight k-slots (the same slot -> k map
// for both operands, so any assignment of the contraction index to slots is
// valid); the result layout matches mfma16.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma_bf16(uintx4 a, uintx4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
// Six-term form: each fp32 operand as head + middle + tail bf16 pieces, each
// the round-to-nearest bf16 of what the earlier ones leave (x = h + m + t + e,
// |e| <= 2^-24 |x|), and the products h h, h m, m h, h t, t h, m m
// accumulated in fp32, smallest first; the dropped m t, t m and t t are
// below 2^-24, so a product is exact to about 2^-23, fp32 level.
__device__ __forceinline__ floatx4 mfma_bf16x6(uintx4 ah, uintx4 am, uintx4 at, uintx4 bh, uintx4 bm, uintx4 bt,
                                                floatx4 c) {
  c = mfma_bf16(am, bm, c);
  c = mfma_bf16(ah, bt, c);
  c = mfma_bf16(at, bh, c);
  c = mfma_bf16(ah, bm, c);
  c = mfma_bf16(am, bh, c);
  return mfma_bf16(ah, bh, c);
}
// Split two fp32 values into three bf16 pieces each (first value in the low
// 16 bits of each word).
__device__ __forceinline__ void split2_bf16x3(float x0, float x1, unsigned& h, unsigned& m, unsigned& t) {
  h = __builtin_bit_cast(unsigned, __builtin_convertvector((floatx2){x0, x1}, bf16x2));
  const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
  m = __builtin_bit_cast(unsigned, __builtin_convertvector((floatx2){r0, r1}, bf16x2));
  const float s0 = r0 - __uint_as_float(m << 16), s1 = r1 - __uint_as_float(m & 0xffff0000u);
  t = __builtin_bit_cast(unsigned, __builtin_convertvector((floatx2){s0, s1}, bf16x2));
}
__device__ __forceinline__ void split8_bf16x3(const float* v, uintx4& h, uintx4& m, uintx4& t) {
  unsigned a[4], b[4], c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2_bf16x3(v[2 * i], v[2 * i + 1], a[i], b[i], c[i]);
  h = uintx4{a[0], a[1], a[2], a[3]};
  m = uintx4{b[0], b[1], b[2], b[3]};
  t = uintx4{c[0], c[1], c[2], c[3]};
}
// Exchange a word with the neighbouring lane (lanes 2i and 2i + 1; DPP quad_perm 1,0,3,2).
__device__ __forceinline__ unsigned swap_pair_u(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
}

// exp(x) through the hardware exp2 (v_exp_f32): relative error about
// |x| * 2^-23 from the log2(e) scaling, used where the result multiplies
// terms that are themselves negligible once |x| is large.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// sigmoid(u) with the hardware exp2 and reciprocal (a few ulp); saturates
// cleanly: exp2 of a large argument is +inf and its reciprocal zero.
__device__ __forceinline__ float sigmoid_fast(float u) {
  return __builtin_amdgcn_rcpf(1.f + exp_fast(-u));
}

// u * sigmoid(u) with the hardware exp2 and reciprocal (about 2 ulp).
__device__ __forceinline__ float silu_fast(float u) { return u * sigmoid_fast(u); }

// Cross-lane helpers on DPP (register-to-register lane shifts; no LDS).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
// Inclusive prefix sum within each 32-lane half of the wave: shifts by
// 1, 2, 4, 8 inside 16-lane rows, then lane 15 of rows 0 / 2 into rows 1 / 3.
__device__ __forceinline__ float scan32_f(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  v += dpp_f<0x142, 0xa>(v);
  return v;
}
// Inclusive prefix sum over the whole wave (adds lane 31 into rows 2 and 3).
__device__ __forceinline__ float scan64_f(float v) {
  v = scan32_f(v);
  v += dpp_f<0x143, 0xc>(v);
  return v;
}
// Value of lane i + 1 (zero in lane 63).
__device__ __forceinline__ float next_lane_f(float v) { return dpp_f<0x130>(v); }
__device__ __forceinline__ float read_lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float sigmoidf_acc(float u) {
  // 1 / (1 + e^-u) without overflow for large |u|.
  if (u >= 0.f) return 1.f / (1.f + expf(-u));
  const float e = expf(u);
  return e / (1.f + e);
}

__device__ __forceinline__ float siluf_acc(float u) { return u * sigmoidf_acc(u); }

__device__ __forceinline__ float softplusf_acc(float u) {
  // max(u, 0) + log1p(e^-|u|): exact for large |u|, no overflow.
  return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
}

// sin and cos of the reduced argument r (|r| <= pi/4) in quadrant q: Taylor
// polynomials whose truncation error (below 1e-12) is far under float32
// rounding, then the quadrant's swap and signs.
__device__ __forceinline__ void sincos_poly(float r, int q, float* s_out, float* c_out) {
  const float r2 = r * r;
  // sin r = r - r^3/3! + r^5/5! - ... ; cos r = 1 - r^2/2! + r^4/4! - ...
  float sp = fmaf(r2, -1.f / 39916800.f, 1.f / 362880.f);
  sp = fmaf(r2, sp, -1.f / 5040.f);
  sp = fmaf(r2, sp, 1.f / 120.f);
  sp = fmaf(r2, sp, -1.f / 6.f);
  const float sn = fmaf(r * r2, sp, r);
  float cp = fmaf(r2, 1.f / 479001600.f, -1.f / 3628800.f);
  cp = fmaf(r2, cp, 1.f / 40320.f);
  cp = fmaf(r2, cp, -1.f / 720.f);
  cp = fmaf(r2, cp, 1.f / 24.f);
  cp = fmaf(r2, cp, -0.5f);
  const float cs = fmaf(r2, cp, 1.f);
  switch (q & 3) {
    case 0: *s_out = sn; *c_out = cs; break;
    case 1: *s_out = cs; *c_out = -sn; break;
    case 2: *s_out = -sn; *c_out = -cs; break;
    default: *s_out = -cs; *c_out = sn; break;
  }
}

// sin and cos of x, accurate to a few ulp.  The argument is reduced by pi/2
// (k = rint(x 2/pi), r = x - k pi/2) with pi/2 split into three float32
// pieces applied by fused multiply-adds (Cody-Waite), or in float64 for
// |x| >= 8192; then sincos_poly.  The pieces of pi/2 come from Machin's
// formula evaluated to 60 digits.
__device__ __forceinline__ void sincos_acc(float x, float* s_out, float* c_out) {
  float r;
  int q;
  if (fabsf(x) < 8192.f) {
    const float k = rintf(x * 0x1.45f306p-1f);
    r = fmaf(-k, 0x1.921fb6p+0f, x);
    r = fmaf(-k, -0x1.777a5cp-25f, r);
    r = fmaf(-k, -0x1.ee59dap-50f, r);
    q = (int)k;
  } else {
    const double xd = (double)x;
    const double kd = rint(xd * 0x1.45f306dc9c883p-1);
    double rd = fma(-kd, 0x1.921fb54442d18p+0, xd);
    rd = fma(-kd, 0x1.1a62633145c07p-54, rd);
    r = (float)rd;
    q = (int)(kd - 4.0 * floor(kd * 0.25));  // k mod 4 without integer overflow
  }
  sincos_poly(r, q, s_out, c_out);
}

// sin and cos of x from the hardware sine and cosine (v_sin_f32 / v_cos_f32,
// arguments in revolutions) after the same three-part fused reduction by
// 2 pi (the pi/2 pieces times four), for |x| < 8192; sincos_acc beyond.
// Measured on gfx950 over 4M arguments in |x| < 8192: at most 3.9e-7 from
// the float64 sine and cosine (sincos_acc: 7e-8).
__device__ __forceinline__ void sincos_hw(float x, float* s_out, float* c_out) {
  if (fabsf(x) < 8192.f) {
    const float k = rintf(x * 0x1.45f306p-3f);
    float r = fmaf(-k, 0x1.921fb6p+2f, x);
    r = fmaf(-k, -0x1.777a5cp-23f, r);
    r = fmaf(-k, -0x1.ee59dap-48f, r);
    const float rev = r * 0x1.45f306p-3f;
    *s_out = __builtin_amdgcn_sinf(rev);
    *c_out = __builtin_amdgcn_cosf(rev);
  } else {
    sincos_acc(x, s_out, c_out);
  }
}

// The same for an argument held in float64, reduced in float64 whatever its
// size.  The decode steps form theta = angle_state + dt angle exactly in
// float64 from its float32 parts, so that an accumulated angle of large
// magnitude (|theta| of 1e4 has a float32 spacing of 1e-3) loses nothing to
// a float32 rounding of the sum before its sine is taken.
__device__ __forceinline__ void sincos_acc_d(double x, float* s_out, float* c_out) {
  const double kd = rint(x * 0x1.45f306dc9c883p-1);
  double rd = fma(-kd, 0x1.921fb54442d18p+0, x);
  rd = fma(-kd, 0x1.1a62633145c07p-54, rd);
  sincos_poly((float)rd, (int)(kd - 4.0 * floor(kd * 0.25)), s_out, c_out);
}

// fp16 matrix products of split fp32 operands (v_mfma_f32_16x16x32_f16; the
// operand layout is that of mfma_bf16).  A value v, first scaled by a power
// of two so that the block's largest magnitude lies in [2^14, 2^15), is
// held as a head h = fp16(v) and a tail l = fp16(v - h) (the remainder v - h
// is exact in fp32 before its one rounding to fp16); v - h - l is
// below 2^-22 |v| for normal heads, and h h' + h l' + l h' leaves out
// l l' < 2^-22 |v v'|: about 2^-21 relative per product, at the level of an
// fp32 dot product's own rounding.
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mfma_f16(uintx4 a, uintx4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c, 0,
                                                0, 0);
}
// Split two fp32 values x0 s, x1 s (s a power of two) into fp16 head and
// tail words (x0 in the low half of each word), the scaling folded into
// v_fma_mix{lo,hi}_f16, which round a fused x s + c to fp16 in one half of
// the word and keep the other half: the heads fp16(x s) and the tails
// fp16(x s - h).  The compiler's hazard tracking does not see inside an asm
// statement, and an MFMA that reads a VGPR needs two wait states after a VALU
// instruction writes it, so the block ends with them (s_nop 1) before either
// word can reach an MFMA operand.
__device__ __forceinline__ void split2_f16s(float x0, float x1, float s, unsigned& h, unsigned& l) {
  unsigned hw, lw;
  asm("v_fma_mixlo_f16 %0, %2, %4, 0\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0\n\t"
      "v_fma_mixlo_f16 %1, %2, %4, -%0 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %3, %4, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(hw), "=&v"(lw)
      : "v"(x0), "v"(x1), "v"(s));
  h = hw;
  l = lw;
}
// Exponent e such that 2^e m lies in [2^14, 2^15) for m > 0 (0 for m = 0 or
// non-finite m), at most 120 (so that 2^e is a finite float; for finite m
// the frexp exponent is at most 128, so e >= -113 without a lower clamp).
__device__ __forceinline__ int f16_scale_exp(float m) {
  const int e = min(15 - __builtin_amdgcn_frexp_expf(m), 120);
  return (m > 0.f && m <= 3.0e38f) ? e : 0;
}
// max(|a|, |b|, m) for m >= 0 (one v_max3_f32 with absolute-value
// modifiers; a NaN operand may be dropped, the NaN itself still reaches the
// products it belongs to).
__device__ __forceinline__ float max3_abs(float a, float b, float m) {
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)), m);
}
// Maximum of non-negative v over lanes l, l ^ 16, l ^ 32, l ^ 48 (v_permlane16/32_swap).
__device__ __forceinline__ float max_xor16_32(float v) {
  const unsigned u = __float_as_uint(v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned w = max(s16[0], s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(max(s32[0], s32[1]));
}
// Maximum of non-negative v over the 64 lanes of a wave (in every lane).
__device__ __forceinline__ float wave_max_nn(float v) {
  unsigned u = __float_as_uint(v);
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xf, 0xf, false));  // quad_perm 2,3,0,1
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xf, 0xf, false));  // row_ror 4
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xf, 0xf, false));  // row_ror 8
  return max_xor16_32(__uint_as_float(u));
}

// Workgroup barrier for hand-offs through LDS only.  It waits for this wave's
// LDS operations (lgkmcnt) and then meets the other waves, but unlike
// __syncthreads() it does not wait for outstanding global loads (vmcnt), so
// prefetches issued before it stay in flight.  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ floatx4 lds_read4(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}

// Raw buffer access (buffer_load / buffer_store with a scalar resource and a
// 32-bit per-lane byte offset).  The resource covers [base, base + bytes):
// loads past the end return zero and stores past the end are dropped, which
// masks partial chunks without branches.  0x00020000 is the gfx9-family
// third descriptor word for 32-bit raw data.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// The size must be wave-uniform; readfirstlane tells the compiler so, which
// keeps the descriptor in scalar registers.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
__device__ __forceinline__ floatx4 buf_load4(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ float buf_load1(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t byte_off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4, v), r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store1(rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, byte_off, 0, 0);
}

// Map a hardware workgroup id to a logical work unit so that consecutive
// logical units land on the same XCD: the dispatcher hands workgroup i to
// XCD i % 8, so logical units are dealt out in eight contiguous runs.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n) {
  const uint32_t per = n / 8u, rem = n % 8u;
  const uint32_t xcd = i % 8u, j = i / 8u;
  return xcd < rem ? xcd * (per + 1u) + j : rem * (per + 1u) + (xcd - rem) * per + j;
}

}  // namespace m3
