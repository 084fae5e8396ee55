// SIMT (vector ALU, float32 arithmetic) forward and backward of SAS gated
// block-sparse attention: the path for float32 tensors (the small float32
// workload, where fp32 MFMA would not meet a 1e-5 tolerance any better and
// the work is launch-bound).
//
//   o = softmax(tau q K_S^T + log g_S) V_S        (SAS review page §2.3)
//   log g_m = s_m - LSE(s over history), g_0 = 1  (§2.4)
//   gate gradient of a kept block = sum of its logit gradients (§2.6)
//
// One thread per (query head, query row); K/V tiles of the kept blocks are
// staged through LDS as float32.  The external gate (sas.h) is computed as
// written: unbiased logits, values of kept block m scaled by g = exp(log g).
// Block tables (packed documents, block_geo): a block is a 64-row window
// whose rows [lo, hi) are its own tokens; key j of the current block is
// visible from row t iff lo <= j <= t, and only a block's own rows and keys
// are stored.
#include "common.h"
#include "launch.h"
#include "sas.h"

namespace sas {

// ---------------------------------------------------------------- forward
// grid: B*Hkv*nqb; block: G*64 threads (thread = head g, row r).
template <class E, int D>
__global__ void __launch_bounds__(1024) fwd_simt_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ k,
    const typename E::T* __restrict__ v, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const float* __restrict__ lg, typename E::T* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int n, int topk, float tau, int gate,
    const int32_t* __restrict__ geo, int nqb) {
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const int i = blockIdx.x % nqb;
  const int bk = blockIdx.x / nqb;
  const int b = bk / Hkv, kv = bk % Hkv;
  const BlockGeo gi = block_geo(geo, b, nqb, n, i);
  if (gi.hi == gi.lo) return;   // a padding block holds no token (uniform exit)
  const int G = Hq / Hkv;
  const int g = threadIdx.x / SAS_BLK, r = threadIdx.x % SAS_BLK;
  const int h = kv * G + g;
  const size_t qrow = (size_t(b) * Hq + h) * n + size_t(gi.w) + r;

  __shared__ float Ks[SAS_BLK][D + 1];
  __shared__ float Vs[SAS_BLK][D + 1];

  float qr[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = E::ld(q + qrow * D + c) * tau;
    acc[c] = 0.f;
  }
  float mrun = -INFINITY, lrun = 0.f;
  const int c_sel = cnt[bk * size_t(nqb) + i];
  const size_t kvbase = (size_t(b) * Hkv + kv) * n;
  for (int t = 0; t <= c_sel; ++t) {
    const int blk = (t < c_sel) ? idx[(bk * size_t(nqb) + i) * topk + t] : i;
    const float lgt = (t < c_sel) ? lg[(bk * size_t(nqb) + i) * topk + t] : 0.f;
    const float bias = ext ? 0.f : lgt;       // logit bias
    const float w = ext ? expf(lgt) : 1.f;    // value weight
    const int w0 = (t < c_sel) ? block_geo(geo, b, nqb, n, blk).w : gi.w;
    __syncthreads();
    for (int e = threadIdx.x; e < SAS_BLK * D; e += blockDim.x) {
      const int rr = e / D, cc = e % D;
      const size_t gx = (kvbase + size_t(w0) + rr) * D + cc;
      Ks[rr][cc] = E::ld(k + gx);
      Vs[rr][cc] = E::ld(v + gx);
    }
    __syncthreads();
    // causal on the current block, over its own keys
    const int jmin = (t < c_sel) ? 0 : gi.lo;
    const int jmax = (t < c_sel) ? SAS_BLK : r + 1;
    for (int j = jmin; j < jmax; ++j) {
      float z = bias;
#pragma unroll
      for (int c = 0; c < D; ++c) z += qr[c] * Ks[j][c];
      if (z > mrun) {
        const float corr = expf(mrun - z);
        lrun *= corr;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] *= corr;
        mrun = z;
      }
      const float p = expf(z - mrun);
      lrun += p;
      const float pw = p * w;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] += pw * Vs[j][c];
    }
  }
  if (r < gi.lo || r >= gi.hi) return;   // a window row of another block
  const float inv = 1.f / lrun;
#pragma unroll
  for (int c = 0; c < D; ++c) E::st(o + qrow * D + c, acc[c] * inv);
  lse[qrow] = mrun + logf(lrun);
}

// ---------------------------------------------------------------- backward
// D[row] = sum_c dO[row,c] * o[row,c]; one thread per row.
template <class E, int D>
__global__ void __launch_bounds__(256) bwd_rowdot_kernel(const typename E::T* __restrict__ o,
                                                         const typename E::T* __restrict__ dO,
                                                         float* __restrict__ Dv, size_t rows) {
  const size_t r = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= rows) return;
  float a = 0.f;
  for (int c = 0; c < D; ++c) a += E::ld(o + r * D + c) * E::ld(dO + r * D + c);
  Dv[r] = a;
}

// dQ, the per-slot gate gradient and the gate Jacobian row of ds.
// grid: B*Hkv*nqb; block G*64 (thread = head g, row r).
template <class E, int D>
__global__ void __launch_bounds__(1024) bwd_dq_simt_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ k,
    const typename E::T* __restrict__ v, const typename E::T* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const float* __restrict__ lg, const float* __restrict__ s,
    const float* __restrict__ s_lse, typename E::T* __restrict__ dq, float* __restrict__ ds,
    int Hq, int Hkv, int n, int topk, float tau, int gate, const int32_t* __restrict__ geo,
    int nqb) {
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const int i = blockIdx.x % nqb;
  const int bk = blockIdx.x / nqb;
  const int b = bk / Hkv, kv = bk % Hkv;
  const BlockGeo gi = block_geo(geo, b, nqb, n, i);
  const int G = Hq / Hkv;
  const int g = threadIdx.x / SAS_BLK, r = threadIdx.x % SAS_BLK;
  const int h = kv * G + g;
  const size_t qrow = (size_t(b) * Hq + h) * n + size_t(gi.w) + r;
  const bool row_ok = r >= gi.lo && r < gi.hi;
  const size_t rowsel = bk * size_t(nqb) + i;

  __shared__ float Ks[SAS_BLK][D + 1];
  __shared__ float Vs[SAS_BLK][D + 1];
  __shared__ float wsum[16];
  __shared__ float dlg_s[2048];  // topk <= blocks per sequence <= 2048
  __shared__ int slot_of[2048];

  float qr[D], dor[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = E::ld(q + qrow * D + c);
    dor[c] = E::ld(dO + qrow * D + c);
    acc[c] = 0.f;
  }
  const float L = lse[qrow], Drow = Dv[qrow];
  // an empty padding block keeps nothing (cnt 0) and still writes its ds row
  const int c_sel = gi.hi > gi.lo ? cnt[rowsel] : 0;
  const size_t kvbase = (size_t(b) * Hkv + kv) * n;
  const int nwaves = blockDim.x / 64;
  for (int t = 0; t <= c_sel && gi.hi > gi.lo; ++t) {
    const int blk = (t < c_sel) ? idx[rowsel * topk + t] : i;
    const float lgt = (t < c_sel) ? lg[rowsel * topk + t] : 0.f;
    const float bias = ext ? 0.f : lgt;
    const float w = ext ? expf(lgt) : 1.f;
    const int w0 = (t < c_sel) ? block_geo(geo, b, nqb, n, blk).w : gi.w;
    __syncthreads();
    for (int e = threadIdx.x; e < SAS_BLK * D; e += blockDim.x) {
      const int rr = e / D, cc = e % D;
      const size_t gx = (kvbase + size_t(w0) + rr) * D + cc;
      Ks[rr][cc] = E::ld(k + gx);
      Vs[rr][cc] = E::ld(v + gx);
    }
    __syncthreads();
    // rows outside the block contribute nothing; the current block's own keys
    const int jmin = (t < c_sel) ? 0 : gi.lo;
    const int jmax = !row_ok ? 0 : (t < c_sel) ? SAS_BLK : r + 1;
    float tsum = 0.f;
    for (int j = jmin; j < jmax; ++j) {
      float z = bias, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        z += tau * qr[c] * Ks[j][c];
        dp += dor[c] * Vs[j][c];
      }
      const float p = expf(z - L);
      dp *= w;
      const float dz = p * (dp - Drow);
      tsum += ext ? p * dp : dz;   // gate gradient: d/dlog g
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] += dz * Ks[j][c];
    }
    if (t < c_sel) {
      tsum = wave_sum(tsum);
      if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = tsum;
      __syncthreads();
      if (threadIdx.x == 0) {
        float a = 0.f;
        for (int w = 0; w < nwaves; ++w) a += wsum[w];
        dlg_s[t] = a;
      }
    }
  }
  if (row_ok) {
#pragma unroll
    for (int c = 0; c < D; ++c) E::st(dq + qrow * D + c, acc[c] * tau);
  }

  // gate Jacobian: ds[i,m] = [m kept] dlg - pi_m * sum(dlg), pi = softmax(s[i,:i])
  for (int m = threadIdx.x; m < nqb; m += blockDim.x) slot_of[m] = -1;
  __syncthreads();
  for (int t = threadIdx.x; t < c_sel; t += blockDim.x) slot_of[idx[rowsel * topk + t]] = t;
  __syncthreads();
  float tot = 0.f;
  for (int t = 0; t < c_sel; ++t) tot += dlg_s[t];
  const float sl = s_lse[rowsel];
  const float* srow = s + rowsel * nqb;
  float* dsrow = ds + rowsel * nqb;
  const int hist = sl > -INFINITY ? i : 0;   // a row without candidates has no gate
  for (int m = threadIdx.x; m < nqb; m += blockDim.x) {
    float val = 0.f;
    if (m < hist) {
      const int sl_m = slot_of[m];
      if (gate == SAS_GATE_SIGMOID)   // d log sigmoid(s) / ds = sigmoid(-s), no coupling
        val = sl_m >= 0 ? dlg_s[sl_m] / (1.f + expf(srow[m])) : 0.f;
      else
        val = (sl_m >= 0 ? dlg_s[sl_m] : 0.f) - expf(srow[m] - sl) * tot;
    }
    dsrow[m] = val;
  }
}

// dK, dV of key block m.  grid: B*Hkv*nkb; block 64 (thread = key row j).
template <class E, int D>
__global__ void __launch_bounds__(64) bwd_dkdv_simt_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ k,
    const typename E::T* __restrict__ v, const typename E::T* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dv, const float* __restrict__ lg,
    const int32_t* __restrict__ rev_off, const int32_t* __restrict__ rev_list,
    typename E::T* __restrict__ dk, typename E::T* __restrict__ dv, int Hq, int Hkv, int n,
    int topk, float tau, int gate, const int32_t* __restrict__ geo, int nb) {
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const int m = blockIdx.x % nb;
  const int bk = blockIdx.x / nb;
  const int b = bk / Hkv, kv = bk % Hkv;
  const BlockGeo gm = block_geo(geo, b, nb, n, m);
  if (gm.hi == gm.lo) return;   // a padding block holds no token (uniform exit)
  const int G = Hq / Hkv;
  const int j = threadIdx.x;
  const size_t krow = (size_t(b) * Hkv + kv) * n + size_t(gm.w) + j;

  __shared__ float Qs[SAS_BLK][D + 1];
  __shared__ float Os[SAS_BLK][D + 1];
  __shared__ float Ls[SAS_BLK], Ds[SAS_BLK];

  float kr[D], vr[D], ak[D], av[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    kr[c] = E::ld(k + krow * D + c);
    vr[c] = E::ld(v + krow * D + c);
    ak[c] = 0.f;
    av[c] = 0.f;
  }
  const int32_t* off = rev_off + size_t(bk) * (nb + 1);
  const int32_t* lst = rev_list + size_t(bk) * nb * (topk + 1);
  for (int e = off[m]; e < off[m + 1]; ++e) {
    const int32_t ent = lst[e];
    const int i = ent & 0xFFFF;
    const int slot = (ent >> 16) & 0xFFFF;
    const bool own = slot == 0xFFFF;
    const float lgt = own ? 0.f : lg[(bk * size_t(nb) + i) * topk + slot];
    const float bias = ext ? 0.f : lgt;
    const float w = ext ? expf(lgt) : 1.f;
    const BlockGeo gq = block_geo(geo, b, nb, n, i);
    for (int g = 0; g < G; ++g) {
      const size_t row0 = (size_t(b) * Hq + kv * G + g) * n + size_t(gq.w);
      __syncthreads();
      for (int x = threadIdx.x; x < SAS_BLK * D; x += 64) {
        const int rr = x / D, cc = x % D;
        Qs[rr][cc] = E::ld(q + (row0 + rr) * D + cc);
        Os[rr][cc] = E::ld(dO + (row0 + rr) * D + cc);
      }
      Ls[threadIdx.x] = lse[row0 + threadIdx.x];
      Ds[threadIdx.x] = Dv[row0 + threadIdx.x];
      __syncthreads();
      // the q-block's own rows; on the own block, rows at or after key j
      for (int t = own ? max(j, gq.lo) : gq.lo; t < gq.hi; ++t) {
        float z = bias, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          z += tau * Qs[t][c] * kr[c];
          dp += Os[t][c] * vr[c];
        }
        const float p = expf(z - Ls[t]);
        const float dz = p * (w * dp - Ds[t]);
        const float pw = p * w;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          av[c] += pw * Os[t][c];
          ak[c] += dz * Qs[t][c];
        }
      }
    }
  }
  if (j < gm.lo || j >= gm.hi) return;   // a window row of another block
#pragma unroll
  for (int c = 0; c < D; ++c) {
    E::st(dk + krow * D + c, ak[c] * tau);
    E::st(dv + krow * D + c, av[c]);
  }
}

template <class E, int D>
static hipError_t fwd_go(const void* q, const void* k, const void* v, const int32_t* idx,
                         const int32_t* cnt, const float* lg, void* o, float* lse, int B, int Hq,
                         int Hkv, int n, int topk, float tau, int gate, const int32_t* geo, int nqb,
                         hipStream_t st) {
  using T = typename E::T;
  ProfScope ps("sas_fwd_simt_kernel", st);
  hipLaunchKernelGGL((fwd_simt_kernel<E, D>), dim3(B * Hkv * nqb), dim3((Hq / Hkv) * SAS_BLK), 0,
                     st, (const T*)q, (const T*)k, (const T*)v, idx, cnt, lg, (T*)o, lse, Hq, Hkv,
                     n, topk, tau, gate, geo, nqb);
  return hipGetLastError();
}

hipError_t launch_fwd_simt(int dtype, const void* q, const void* k, const void* v,
                           const int32_t* idx, const int32_t* cnt, const float* lg, void* o,
                           float* lse, int B, int Hq, int Hkv, int n, int d, int topk, float tau,
                           int gate, const int32_t* geo, int nqb, hipStream_t st) {
  if (dtype == 0) {
    if (d == 64) return fwd_go<ElemF32, 64>(q, k, v, idx, cnt, lg, o, lse, B, Hq, Hkv, n, topk, tau, gate, geo, nqb, st);
    return fwd_go<ElemF32, 128>(q, k, v, idx, cnt, lg, o, lse, B, Hq, Hkv, n, topk, tau, gate, geo, nqb, st);
  }
  if (d == 64) return fwd_go<ElemBF16, 64>(q, k, v, idx, cnt, lg, o, lse, B, Hq, Hkv, n, topk, tau, gate, geo, nqb, st);
  return fwd_go<ElemBF16, 128>(q, k, v, idx, cnt, lg, o, lse, B, Hq, Hkv, n, topk, tau, gate, geo, nqb, st);
}

template <class E, int D>
static hipError_t bwd_go(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, const int32_t* idx, const int32_t* cnt,
                         const float* lg, const float* s, const float* s_lse, void* dq, void* dk,
                         void* dv, float* ds, float* Dws, const int32_t* rev_off,
                         const int32_t* rev_list, int B, int Hq, int Hkv, int n, int topk,
                         float tau, int gate, const int32_t* geo, int nb, hipStream_t st) {
  using T = typename E::T;
  const size_t rows = size_t(B) * Hq * n;
  {
    ProfScope ps("sas_bwd_rowdot_kernel", st);
    hipLaunchKernelGGL((bwd_rowdot_kernel<E, D>), dim3((rows + 255) / 256), dim3(256), 0, st,
                       (const T*)o, (const T*)dO, Dws, rows);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_dq_simt_kernel", st);
    hipLaunchKernelGGL((bwd_dq_simt_kernel<E, D>), dim3(B * Hkv * nb), dim3((Hq / Hkv) * SAS_BLK),
                       0, st, (const T*)q, (const T*)k, (const T*)v, (const T*)dO, lse, Dws, idx,
                       cnt, lg, s, s_lse, (T*)dq, ds, Hq, Hkv, n, topk, tau, gate, geo, nb);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_dkdv_simt_kernel", st);
    hipLaunchKernelGGL((bwd_dkdv_simt_kernel<E, D>), dim3(B * Hkv * nb), dim3(SAS_BLK), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)dO, lse, Dws, lg, rev_off,
                       rev_list, (T*)dk, (T*)dv, Hq, Hkv, n, topk, tau, gate, geo, nb);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_simt(int dtype, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse, const int32_t* idx,
                           const int32_t* cnt, const float* lg, const float* s,
                           const float* s_lse, void* dq, void* dk, void* dv, float* ds, float* Dws,
                           const int32_t* rev_off, const int32_t* rev_list, int B, int Hq,
                           int Hkv, int n, int d, int topk, float tau, int gate,
                           const int32_t* geo, int nb, hipStream_t st) {
#define SAS_BWD_ARGS q, k, v, o, dO, lse, idx, cnt, lg, s, s_lse, dq, dk, dv, ds, Dws, rev_off, \
                     rev_list, B, Hq, Hkv, n, topk, tau, gate, geo, nb, st
  if (dtype == 0) {
    if (d == 64) return bwd_go<ElemF32, 64>(SAS_BWD_ARGS);
    return bwd_go<ElemF32, 128>(SAS_BWD_ARGS);
  }
  if (d == 64) return bwd_go<ElemBF16, 64>(SAS_BWD_ARGS);
  return bwd_go<ElemBF16, 128>(SAS_BWD_ARGS);
#undef SAS_BWD_ARGS
}

}  // namespace sas
