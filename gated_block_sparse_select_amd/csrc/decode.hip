// Single-token decode over a contiguous KV cache.
//
// The query of batch entry b is token T = seq_len-1; its current block i = T/64
// holds the tokens [64 i, seq_len).  Each kv-group selects Top-K history blocks
// from its score row and adds their log-gates (SAS review page, paper.oopus.info,
// §2.2, §2.4); the current block is unbiased (§2.4, g_0 = 1).
//
// The step is HBM-bound (one pass over the kept K/V tiles), so it runs on the
// vector units with perfectly coalesced 16-byte loads: a 64-token tile of one
// kv-head is one contiguous 64*d element chunk of the cache.
//   1. select (select.hip, decode rows) -> idx / log-gate in the workspace;
//   2. split kernel: grid (b, kv, split); each workgroup streams a contiguous
//      range of the (cnt+1) tiles for all G query heads of the group and
//      writes an unnormalised partial (acc, running max, running sum);
//   3. combine kernel: merges the splits per query head.
#include "common.h"
#include "launch.h"

namespace sas {

template <class E>
struct Vec16;  // one 16-byte chunk of elements, unpacked to float
template <>
struct Vec16<ElemBF16> {
  static constexpr int N = 8;
  static SAS_DEV void unpack(const uint4& u, float* o) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = __uint_as_float(w[e] << 16);
      o[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
};
template <>
struct Vec16<ElemF32> {
  static constexpr int N = 4;
  static SAS_DEV void unpack(const uint4& u, float* o) {
    o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
    o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
  }
};

// grid: B*Hkv*nsplit workgroups of 256 threads.
// Thread t owns element group dg = t % CPR (EPC elements) of keys
// kg + (256/CPR)*u, u < KPT, in every tile.
template <class E, int D, int GMAX>
__global__ void __launch_bounds__(256) decode_split_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ kc,
    const typename E::T* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ lg, float* __restrict__ part_acc, float* __restrict__ part_ml,
    int Hq, int Hkv, int cap, int topk, int nsplit, float tau2) {
  constexpr int EPC = Vec16<E>::N;        // elements per 16-byte chunk
  constexpr int CPR = D / EPC;            // chunks per key row
  constexpr int KG = 256 / CPR;           // key groups per workgroup
  constexpr int KPT = SAS_BLK / KG;       // keys per thread per tile
  const int split = blockIdx.x % nsplit;
  const int bk = blockIdx.x / nsplit;
  const int b = bk / Hkv, kv = bk % Hkv;
  const int G = Hq / Hkv;
  const int t = threadIdx.x;
  const int dg = t % CPR, kg = t / CPR;
  const int wave = t >> 6;

  int L = seq_lens[b];
  L = L < 1 ? 1 : (L > cap ? cap : L);
  const int icur = (L - 1) / SAS_BLK;
  const int c_sel = cnt[bk];
  const int ntiles = c_sel + 1;
  const int per = (ntiles + nsplit - 1) / nsplit;
  const int t0 = split * per, t1 = min(ntiles, t0 + per);

  // query values of this thread's element group for all heads, pre-scaled by
  // tau*log2(e) so scores are in the exp2 domain
  float qv[GMAX][EPC];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      const typename E::T* qp = q + (size_t(b) * Hq + kv * G + g) * D + dg * EPC;
      float tmp[EPC];
      Vec16<E>::unpack(*reinterpret_cast<const uint4*>(qp), tmp);
#pragma unroll
      for (int e = 0; e < EPC; ++e) qv[g][e] = tmp[e] * tau2;
    }
  }
  float acc[GMAX][EPC];
  float mrun[GMAX], lpart[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    mrun[g] = -INFINITY;
    lpart[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
  }
  __shared__ float red[4][GMAX];

  const size_t cache0 = (size_t(b) * Hkv + kv) * size_t(cap) * D;
  for (int tile = t0; tile < t1; ++tile) {
    const int blk = tile < c_sel ? idx[size_t(bk) * topk + tile] : icur;
    const float bias2 = tile < c_sel ? lg[size_t(bk) * topk + tile] * kLog2e : 0.f;
    const int nvalid = tile < c_sel ? SAS_BLK : L - icur * SAS_BLK;
    const typename E::T* kt = kc + cache0 + size_t(blk) * SAS_BLK * D;
    const typename E::T* vt = vc + cache0 + size_t(blk) * SAS_BLK * D;
    uint4 kr[KPT], vr[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = u * 256 + t;  // chunk index inside the contiguous tile
      kr[u] = reinterpret_cast<const uint4*>(kt)[c];
      vr[u] = reinterpret_cast<const uint4*>(vt)[c];
    }
    float sc[KPT][GMAX];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      float kx[EPC];
      Vec16<E>::unpack(kr[u], kx);
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) a += qv[g][e] * kx[e];
        sc[u][g] = a;
      }
    }
    // sum over the CPR lanes holding one key row
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1)
#pragma unroll
      for (int u = 0; u < KPT; ++u)
#pragma unroll
        for (int g = 0; g < GMAX; ++g) sc[u][g] += __shfl_xor(sc[u][g], o);
    float tmax[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int key = kg + KG * u;
        sc[u][g] = key < nvalid ? sc[u][g] + bias2 : -INFINITY;
        mx = fmaxf(mx, sc[u][g]);
      }
      for (int o = CPR; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      tmax[g] = mx;
    }
    __syncthreads();
    if ((t & 63) == 0)
#pragma unroll
      for (int g = 0; g < GMAX; ++g) red[wave][g] = tmax[g];
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) continue;
      const float mt = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
      const float mnew = fmaxf(mrun[g], mt);
      const float corr = exp2f(mrun[g] - mnew);
      mrun[g] = mnew;
      lpart[g] *= corr;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[g][e] *= corr;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const float p = exp2f(sc[u][g] - mnew);
        lpart[g] += p;
        float vx[EPC];
        Vec16<E>::unpack(vr[u], vx);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] += p * vx[e];
      }
    }
  }
  // reduce acc / lpart over the KG key groups that share an element group
  __shared__ float racc[GMAX][D];
  __shared__ float rl[GMAX];
  for (int x = t; x < GMAX * D; x += 256) racc[x / D][x % D] = 0.f;
  if (t < GMAX) rl[t] = 0.f;
  __syncthreads();
  for (int k2 = 0; k2 < KG; ++k2) {
    if (kg == k2) {
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g >= G) continue;
#pragma unroll
        for (int e = 0; e < EPC; ++e) racc[g][dg * EPC + e] += acc[g][e];
        if (dg == 0) rl[g] += lpart[g];
      }
    }
    __syncthreads();
  }
  for (int x = t; x < G * D; x += 256) {
    const int g = x / D, c = x % D;
    part_acc[((size_t(b) * Hq + kv * G + g) * nsplit + split) * D + c] = racc[g][c];
  }
  if (t == 0) {
    // thread 0 holds the workgroup-wide running max of every head
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) continue;
      const size_t pi = ((size_t(b) * Hq + kv * G + g) * nsplit + split) * 2;
      part_ml[pi] = (t0 < t1) ? mrun[g] : -INFINITY;
      part_ml[pi + 1] = rl[g];
    }
  }
}

// grid: B*Hq workgroups of D threads.
template <class E, int D>
__global__ void __launch_bounds__(128) decode_combine_kernel(const float* __restrict__ part_acc,
                                                             const float* __restrict__ part_ml,
                                                             typename E::T* __restrict__ o,
                                                             int nsplit) {
  const size_t bh = blockIdx.x;
  const int c = threadIdx.x;
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, part_ml[(bh * nsplit + sp) * 2]);
  float l = 0.f, a = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float m = part_ml[(bh * nsplit + sp) * 2];
    if (m == -INFINITY) continue;
    const float w = exp2f(m - M);
    l += w * part_ml[(bh * nsplit + sp) * 2 + 1];
    a += w * part_acc[(bh * nsplit + sp) * D + c];
  }
  E::st(o + bh * D + c, a / l);
}

int decode_nsplit(int B, int Hkv, int topk) {
  const int pairs = B * Hkv;
  int ns = (2048 + pairs - 1) / pairs;
  if (ns > topk + 1) ns = topk + 1;
  if (ns < 1) ns = 1;
  return ns;
}

template <class E, int D, int GMAX>
static void split_go(const void* q, const void* kc, const void* vc, const int32_t* sl,
                     const int32_t* idx, const int32_t* cnt, const float* lg, float* pa,
                     float* pm, int B, int Hq, int Hkv, int cap, int topk, int ns, float tau2,
                     hipStream_t st) {
  using T = typename E::T;
  hipLaunchKernelGGL((decode_split_kernel<E, D, GMAX>), dim3(B * Hkv * ns), dim3(256), 0, st,
                     (const T*)q, (const T*)kc, (const T*)vc, sl, idx, cnt, lg, pa, pm, Hq, Hkv,
                     cap, topk, ns, tau2);
}

template <class E, int D>
static void split_g(int G, const void* q, const void* kc, const void* vc, const int32_t* sl,
                    const int32_t* idx, const int32_t* cnt, const float* lg, float* pa, float* pm,
                    int B, int Hq, int Hkv, int cap, int topk, int ns, float tau2,
                    hipStream_t st) {
  if (G <= 1) split_go<E, D, 1>(q, kc, vc, sl, idx, cnt, lg, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, st);
  else if (G <= 2) split_go<E, D, 2>(q, kc, vc, sl, idx, cnt, lg, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, st);
  else if (G <= 4) split_go<E, D, 4>(q, kc, vc, sl, idx, cnt, lg, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, st);
  else if (G <= 8) split_go<E, D, 8>(q, kc, vc, sl, idx, cnt, lg, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, st);
  else split_go<E, D, 16>(q, kc, vc, sl, idx, cnt, lg, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, st);
}

hipError_t launch_decode(int dtype, const void* q, const void* kc, const void* vc,
                         const int32_t* seq_lens, const int32_t* idx, const int32_t* cnt,
                         const float* lg, float* part_acc, float* part_ml, void* o, int B, int Hq,
                         int Hkv, int cap, int d, int topk, int nsplit, float tau,
                         hipStream_t st) {
  const int G = Hq / Hkv;
  const float tau2 = tau * kLog2e;
  {
    ProfScope ps("sas_decode_split_kernel", st);
    if (dtype == 1) {
      if (d == 128) split_g<ElemBF16, 128>(G, q, kc, vc, seq_lens, idx, cnt, lg, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, st);
      else split_g<ElemBF16, 64>(G, q, kc, vc, seq_lens, idx, cnt, lg, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, st);
    } else {
      if (d == 128) split_g<ElemF32, 128>(G, q, kc, vc, seq_lens, idx, cnt, lg, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, st);
      else split_g<ElemF32, 64>(G, q, kc, vc, seq_lens, idx, cnt, lg, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, st);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_decode_combine_kernel", st);
    if (dtype == 1) {
      if (d == 128) hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 128>), dim3(B * Hq), dim3(128), 0, st, part_acc, part_ml, (uint16_t*)o, nsplit);
      else hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 64>), dim3(B * Hq), dim3(64), 0, st, part_acc, part_ml, (uint16_t*)o, nsplit);
    } else {
      if (d == 128) hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 128>), dim3(B * Hq), dim3(128), 0, st, part_acc, part_ml, (float*)o, nsplit);
      else hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 64>), dim3(B * Hq), dim3(64), 0, st, part_acc, part_ml, (float*)o, nsplit);
    }
  }
  return hipGetLastError();
}

}  // namespace sas
