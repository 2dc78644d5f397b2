// Device helpers shared by the libsdv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sdv.h"

#define SDV_DEV __device__ __forceinline__

namespace sdv {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// SplitMix64 counter hash (Steele, Lea, Flood 2014), nested over
// (seed, request, position, draw); written from the published definition.
SDV_DEV uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
SDV_DEV uint64_t sm(uint64_t x) { return mix64(x + 0x9E3779B97F4A7C15ull); }

// 24-bit uniform in [0, 1 - 2^-24], exact in fp32 and fp64.
SDV_DEV double uniform24(uint64_t seed, uint64_t r, uint64_t pos, uint64_t draw) {
  uint64_t h = sm(sm(sm(sm(seed) ^ r) ^ pos) ^ draw);
  return (double)(uint32_t)(h >> 40) * 0x1p-24;
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A 32-bit word holds two bf16 values, element 0 in the low half.
SDV_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
SDV_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
SDV_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round fp32 to bf16, nearest-even; NaN stays NaN (quietened).
SDV_DEV uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

// Raw hardware exp2 (v_exp_f32): exact for -inf -> 0, NaN -> NaN.
SDV_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Wave64 reductions.
SDV_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
SDV_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SDV_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SDV_DEV int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
// Inclusive prefix sum over the wave (fp64).
SDV_DEV double wave_incl_scan_d(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// 16-byte streaming (non-temporal) load / store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
SDV_DEV uint4 ld_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
SDV_DEV void st_nt(void* p, uint4 v) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, (u32x4*)p);
}

SDV_DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// Row statistics across the library's boundary: (m, Z) with m = max(row)/T
// and Z = sum exp(row/T - m).  Inside the kernels a row is held as (ref, Zi):
// ref = fp32(max * c) with c = log2(e)/T, Zi = sum 2^(x*c - ref).  Z is taken
// relative to the reported (rounded) m, so that reading a reported pair back
// gives the frame it came from, to within the fp32 rounding of Z.
constexpr double kLog2eD = 1.4426950408889634074;

SDV_DEV float2 stats_report(float M, float ref, double Zi, float inv_t) {
  const float m = M * inv_t;
  if (M == -__builtin_huge_valf()) return make_float2(m, 0.0f);  // all -inf: (-inf, 0)
  return make_float2(m, (float)(Zi * exp2((double)ref - (double)m * kLog2eD)));
}

// A reported pair in the kernels' frame; returns SD_ST_NONFINITE for NaN,
// m = +inf or Z outside (0, inf), SD_ST_ZERO_Z for m = -inf, else 0.
SDV_DEV int stats_read(float2 mz, float* ref, double* Zi) {
  *ref = 0.0f;
  *Zi = 0.0;
  const float m = mz.x, Z = mz.y;
  if (isnan(m) || isnan(Z) || m == __builtin_huge_valf()) return SD_ST_NONFINITE;
  if (m == -__builtin_huge_valf()) return SD_ST_ZERO_Z;
  if (!(Z > 0.0f) || Z == __builtin_huge_valf()) return SD_ST_NONFINITE;
  const double e = (double)m * kLog2eD;
  *ref = (float)e;
  *Zi = (double)Z * exp2(e - (double)*ref);
  return 0;
}

}  // namespace sdv

// Host-side helpers.
static inline size_t sdv_align256(size_t x) { return (x + 255) & ~(size_t)255; }
