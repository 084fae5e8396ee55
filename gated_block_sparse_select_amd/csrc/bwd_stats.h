// Row statistics of the backward's dZ-tile path (gfx950): for one (batch,
// query head, q-block) unit, stats[unit] = [-lse/tau for the window's 64 rows |
// -D for them], D = rowsum(dO o O) (the chain rule through the softmax of the
// SAS review page, paper.oopus.info, §2.3 and §2.6); (-inf, 0) on window
// rows outside the block, so every weight there is 0.  256 threads per unit,
// 16 lanes per row at d = 128 (8 at d = 64); o and dO are read once, with
// non-temporal 16-byte loads.
#pragma once

#include "common.h"

namespace sas {

template <int D>
SAS_DEV void bwd_stats_unit(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
                            const float* __restrict__ lse, float* __restrict__ stats, int Hq, int n,
                            float tau, const int32_t* __restrict__ geo, int nqb, int unit,
                            int tid) {
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;   // rows per pass
  const int bh = unit / nqb, i = unit % nqb;
  const BlockGeo gi = block_geo(geo, bh / Hq, nqb, n, i);
  const int c = tid % CPR;
  float* st = stats + size_t(unit) * 128;
  const size_t row0 = size_t(bh) * n + gi.w;
  float acc[64 / RPP];
#pragma unroll
  for (int p = 0; p < 64 / RPP; ++p) {
    const size_t off = (row0 + p * RPP + tid / CPR) * D + c * 8;
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, load_stream(reinterpret_cast<const uint4*>(o + off)));
    const bf16x8_t g = __builtin_bit_cast(bf16x8_t, load_stream(reinterpret_cast<const uint4*>(dO + off)));
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x = __builtin_fmaf(float(a[e]), float(g[e]), x);
    acc[p] = x;
  }
#pragma unroll
  for (int p = 0; p < 64 / RPP; ++p) {
#pragma unroll
    for (int w = CPR / 2; w > 0; w >>= 1) acc[p] += __shfl_xor(acc[p], w);
    const int r = p * RPP + tid / CPR;
    if (c == 0) {
      const bool ok = r >= gi.lo && r < gi.hi;
      st[r] = ok ? -lse[row0 + r] / tau : -INFINITY;
      st[64 + r] = ok ? -acc[p] : 0.f;
    }
  }
}

}  // namespace sas
