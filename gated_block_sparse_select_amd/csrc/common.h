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

// A 16-byte load with the non-temporal hint, for data a kernel reads once:
// keeping such a stream out of the caches measured faster for the decode K/V
// tiles (96 vs 109 us per batch-64 call on one box) and the pooling pass
// (52 vs 57 us).  Tiles that other workgroups read again stay on the
// ordinary path (the same hint on the attention kernels' tile loads cost
// up to 10%).
SAS_DEV uint4 load_stream(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 2^x on the transcendental unit without the denormal range fix-up of exp2f
// (softmax weights below 2^-126 flush to zero, which is harmless).
SAS_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------- block geometry
// Block i of batch entry b holds the token rows [w + lo, w + hi) inside the
// 64-row window [w, w + 64) that the kernels load.  Without a table
// (geo == nullptr) block i is rows [64 i, 64 i + 64).  With a table (first
// token, length per block, packed documents) the window starts at the
// block's first token, or at n - 64 for a short last block near the end of
// the tensors; entries are clamped so that the window stays inside [0, n)
// whatever the table holds (n >= 64).
struct BlockGeo {
  int w, lo, hi;
};
SAS_DEV BlockGeo block_geo(const int32_t* __restrict__ geo, int b, int nb, int n, int i) {
  if (geo == nullptr) return BlockGeo{i * SAS_BLK, 0, SAS_BLK};
  const int2 e = reinterpret_cast<const int2*>(geo)[size_t(b) * nb + i];
  const int len = min(max(e.y, 0), SAS_BLK);
  const int st = min(max(e.x, 0), n - len);
  const int w = min(st, n - SAS_BLK);
  return BlockGeo{w, st - w, st - w + len};
}

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
