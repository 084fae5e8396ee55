// Device/host helpers shared by the libsas kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SAS_BLK 64
#define SAS_DEV __device__ __forceinline__

namespace sas {

// ------------------------------------------------------------- element types
// bf16 values travel as raw 16-bit patterns in global memory.
SAS_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even float -> bf16 (inputs are finite).
SAS_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

struct ElemF32 {
  using T = float;
  static SAS_DEV float ld(const T* p) { return *p; }
  static SAS_DEV void st(T* p, float v) { *p = v; }
};

struct ElemBF16 {
  using T = uint16_t;
  static SAS_DEV float ld(const T* p) { return bf16_to_f32(*p); }
  static SAS_DEV void st(T* p, float v) { *p = f32_to_bf16(v); }
};

// 2^x on the transcendental unit without the denormal range fix-up of exp2f
// (softmax weights below 2^-126 flush to zero, which is harmless).
SAS_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------- wave64 reductions
SAS_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
SAS_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
SAS_DEV int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Number of set bits of a 64-bit lane mask below the calling lane.
SAS_DEV int mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

SAS_DEV int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

constexpr float kLog2e = 1.4426950408889634f;
// Smallest log-gate the external gate uses: its kernels keep the log-gate as
// an exponent offset of the tile's weights and divide their sum by g again,
// so g is held at e^-60 or more to keep the weights clear of underflow.
constexpr float kMinExtLogGate = -60.f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace sas
