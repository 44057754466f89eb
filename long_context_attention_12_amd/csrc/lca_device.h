// lca_device.h — device helpers shared by the gfx950 kernels: storage-format
// conversions (bf16, e4m3fn, e2m1/E8M0), MFMA operand types, wave reductions
// and the RoPE angle. Every conversion here is written from the format's
// definition and rounds to nearest even exactly as the format specifies.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---- bfloat16 --------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even on the 16 dropped bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// Two floats to two bf16 (round to nearest even) in one gfx950 instruction
// (v_cvt_pk_bf16_f32); lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// ---- OCP FP8 E4M3FN (bias 7, max 448, subnormal step 2^-9) -------------------
__device__ __forceinline__ uint8_t f32_to_e4m3fn(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                         // below 2^-6: multiples of 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));   // 8 -> 0x08 (2^-6)
  } else {
    int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
    uint32_t q = static_cast<uint32_t>(__builtin_rintf(ldexpf(a, 3 - e)));  // [8, 16]
    if (q == 16u) { q = 8u; ++e; }
    int ef = e + 7;
    if (ef > 15 || (ef == 15 && q - 8u > 6u)) { ef = 15; q = 14u; }
    code = (static_cast<uint32_t>(ef) << 3) | (q - 8u);
  }
  return static_cast<uint8_t>(sign | code);
}
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
  uint32_t ef = (c >> 3) & 0xfu, mt = c & 7u;
  float mag = ef == 0 ? static_cast<float>(mt) * 0.001953125f
                      : ldexpf(static_cast<float>(8u + mt), static_cast<int>(ef) - 10);
  return (c & 0x80u) ? -mag : mag;
}

// ---- OCP MX E2M1 element and E8M0 scale ---------------------------------------
// Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; halfway cases go to the even code.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  float a = fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}
// floor(log2(amax)) - 2, clamped to the E8M0 range; amax > 0 and finite.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int e;
  (void)frexpf(amax, &e);                       // amax in [2^(e-1), 2^e)
  int E = (e - 1) - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// ---- direct HBM -> LDS copies ---------------------------------------------------
// One 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes at `gptr` land at
// LDS byte address lds_addr + 16 * l. Issued as inline asm so that the
// compiler does not track it: every wait on these copies in the ring loop is
// explicit (wait_vmcnt); a loop that uses it issues no other vector-memory
// access it would have to wait for. The instruction has no register results.
__device__ __forceinline__ void lds_copy16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
               : "memory", "m0");
}

// Same, 4 bytes per lane: lane l's dword at `gptr` lands at lds_addr + 4 * l.
__device__ __forceinline__ void lds_copy4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p)));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N (6-bit field split over [3:0] and [15:14]); expcnt
  // and lgkmcnt at their maxima, i.e. not waited on
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait for every LDS (and scalar-memory) operation of this wave: lgkmcnt = 0,
// vmcnt and expcnt left at their maximum (no wait).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// ---- wave reductions (64 lanes) -----------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- RoPE ----------------------------------------------------------------------
// Pair i of the R rotated channels turns at frequency theta_i = base^(-2i/R),
// i.e. the i-th power of the ratio r = base^(-2/R). The host takes r once per
// call (rope_ratio); a kernel raises it to the i-th power by squaring, eight
// fp64 steps for i < 256, in place of an fp64 power per lane (the power sat on
// the critical path of the kernels that build angle tables). The product with
// the position and the reduction to [-pi, pi] stay in double, so positions
// near 2^20 keep full float32 accuracy; sin and cos of the reduced angle are
// taken in float32.
inline double rope_ratio(float base, int R) {
  return R > 0 && base > 0.f ? pow(static_cast<double>(base), -2.0 / static_cast<double>(R)) : 1.0;
}

__device__ __forceinline__ double rope_freq(double r, int i) {
  double f = 1.0, p = r;
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    if ((i >> bit) & 1) f *= p;
    p *= p;
  }
  return f;
}

__device__ __forceinline__ void rope_sincos(double pos, int i, double r, float* s, float* c) {
  double ang = pos * rope_freq(r, i);
  const double two_pi = 6.283185307179586476925286766559;
  ang = ang - two_pi * rint(ang / two_pi);
  const float a = static_cast<float>(ang);
  *s = sinf(a);
  *c = cosf(a);
}

// Entries visible at position p (p >= 0, m >= 1): (p + 1) / m. Positions below
// 2^32 take a 32-bit unsigned division (a 64-bit one costs several times the
// instructions, and kernels evaluate this in their prologues).
__host__ __device__ __forceinline__ int64_t n_visible(int64_t p, int m) {
  const uint64_t q = static_cast<uint64_t>(p) + 1u;
  if (q <= 0xffffffffull) return static_cast<int64_t>(static_cast<uint32_t>(q) / static_cast<uint32_t>(m));
  return static_cast<int64_t>(q / static_cast<uint64_t>(m));
}

}  // namespace lca
