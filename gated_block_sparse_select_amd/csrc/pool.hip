// Mean-pooled block scores: the stand-in selector of the 32K training workload
// (a score per history block computed from q and K_{B_m}, SAS review page,
// paper.oopus.info, §2.2 selector equation).
//
//   pass 1 (HBM-bound, one pass over q and k): qbar[b,kv,i,:] = mean of the
//     rows (64, or the block's own rows of a block table) x G heads of
//     q-block i; kbar[b,kv,m,:] = mean of key block m; 0 for an empty block.
//   pass 2 (small): s[b,kv,i,m] = qbar_i . kbar_m / sqrt(d) for all (i, m).
#include "common.h"
#include "launch.h"

namespace sas {

template <class E>
SAS_DEV void load8(const typename E::T* p, float* o);

template <>
SAS_DEV void load8<ElemBF16>(const uint16_t* p, float* o) {
  const uint4 u = load_stream(reinterpret_cast<const uint4*>(p));
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = __uint_as_float(w[e] << 16);
    o[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

template <>
SAS_DEV void load8<ElemF32>(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// grid: B*Hkv*nb workgroups of 256 threads.  Thread t owns 8 columns
// (cg = t % (D/8)) and a strided set of rows (rg = t / (D/8)).
template <class E, int D>
__global__ void __launch_bounds__(256) pool_means_kernel(const typename E::T* __restrict__ q,
                                                         const typename E::T* __restrict__ k,
                                                         float* __restrict__ qbar,
                                                         float* __restrict__ kbar, int Hq,
                                                         int Hkv, int n,
                                                         const int32_t* __restrict__ geo, int nb) {
  constexpr int CG = D / 8;        // column groups of 8
  constexpr int RG = 256 / CG;     // row groups
  const int G = Hq / Hkv;
  const int blk = blockIdx.x % nb;
  const int bk = blockIdx.x / nb;  // b*Hkv + kv
  const int b = bk / Hkv, kv = bk % Hkv;
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  const BlockGeo bg = block_geo(geo, b, nb, n, blk);
  const int r0 = bg.w + bg.lo, nr = bg.hi - bg.lo;   // the block's own rows

  float aq[8] = {0, 0, 0, 0, 0, 0, 0, 0}, ak[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < G; ++g) {
    const typename E::T* base =
        q + ((size_t(b) * Hq + kv * G + g) * n + size_t(r0)) * D + cg * 8;
    for (int r = rg; r < nr; r += RG) {
      float x[8];
      load8<E>(base + size_t(r) * D, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) aq[e] += x[e];
    }
  }
  {
    const typename E::T* base = k + ((size_t(b) * Hkv + kv) * n + size_t(r0)) * D + cg * 8;
    for (int r = rg; r < nr; r += RG) {
      float x[8];
      load8<E>(base + size_t(r) * D, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) ak[e] += x[e];
    }
  }
  __shared__ float red[2][RG][D];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rg][cg * 8 + e] = aq[e];
    red[1][rg][cg * 8 + e] = ak[e];
  }
  __syncthreads();
  if (threadIdx.x < 2 * D) {
    const int which = threadIdx.x / D, c = threadIdx.x % D;
    float acc = 0.f;
    for (int r = 0; r < RG; ++r) acc += red[which][r][c];
    const size_t o = (size_t(bk) * nb + blk) * D + c;
    const float rows = float(nr > 0 ? nr : 1);   // an empty block keeps the zero sum
    if (which == 0) qbar[o] = acc * (1.0f / (rows * float(G)));
    else kbar[o] = acc * (1.0f / rows);
  }
}

// grid: (B*Hkv) * ceil(nb/16) workgroups of 256 threads; 16 q-rows per group.
template <int D>
__global__ void __launch_bounds__(256) pool_dot_kernel(const float* __restrict__ qbar,
                                                       const float* __restrict__ kbar,
                                                       float* __restrict__ s, int nb,
                                                       float inv_sqrt_d) {
  constexpr int R = 16;
  const int tiles = (nb + R - 1) / R;
  const int bk = blockIdx.x / tiles;
  const int i0 = (blockIdx.x % tiles) * R;
  __shared__ float qs[R][D];
  for (int e = threadIdx.x; e < R * D; e += 256) {
    const int r = e / D, c = e % D;
    qs[r][c] = (i0 + r < nb) ? qbar[(size_t(bk) * nb + i0 + r) * D + c] : 0.f;
  }
  __syncthreads();
  for (int m = threadIdx.x; m < nb; m += 256) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    const float* kr = kbar + (size_t(bk) * nb + m) * D;
    for (int c = 0; c < D; c += 4) {
      const float4 kk = *reinterpret_cast<const float4*>(kr + c);
#pragma unroll
      for (int r = 0; r < R; ++r)
        acc[r] += qs[r][c] * kk.x + qs[r][c + 1] * kk.y + qs[r][c + 2] * kk.z + qs[r][c + 3] * kk.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (i0 + r < nb) s[(size_t(bk) * nb + i0 + r) * nb + m] = acc[r] * inv_sqrt_d;
  }
}

hipError_t launch_pool(int dtype, const void* q, const void* k, float* s, float* ws, int B,
                       int Hq, int Hkv, int n, int d, const int32_t* geo, int nb, hipStream_t st) {
  float* qbar = ws;
  float* kbar = ws + size_t(B) * Hkv * nb * d;
  {
    ProfScope ps("sas_pool_means_kernel", st);
    dim3 grid(B * Hkv * nb);
    if (dtype == 1) {
      if (d == 128)
        hipLaunchKernelGGL((pool_means_kernel<ElemBF16, 128>), grid, dim3(256), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, qbar, kbar, Hq, Hkv, n, geo, nb);
      else
        hipLaunchKernelGGL((pool_means_kernel<ElemBF16, 64>), grid, dim3(256), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, qbar, kbar, Hq, Hkv, n, geo, nb);
    } else {
      if (d == 128)
        hipLaunchKernelGGL((pool_means_kernel<ElemF32, 128>), grid, dim3(256), 0, st,
                           (const float*)q, (const float*)k, qbar, kbar, Hq, Hkv, n, geo, nb);
      else
        hipLaunchKernelGGL((pool_means_kernel<ElemF32, 64>), grid, dim3(256), 0, st,
                           (const float*)q, (const float*)k, qbar, kbar, Hq, Hkv, n, geo, nb);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_pool_dot_kernel", st);
    dim3 grid(B * Hkv * ((nb + 15) / 16));
    const float isd = 1.0f / sqrtf(float(d));
    if (d == 128)
      hipLaunchKernelGGL(pool_dot_kernel<128>, grid, dim3(256), 0, st, qbar, kbar, s, nb, isd);
    else
      hipLaunchKernelGGL(pool_dot_kernel<64>, grid, dim3(256), 0, st, qbar, kbar, s, nb, isd);
  }
  return hipGetLastError();
}

}  // namespace sas
