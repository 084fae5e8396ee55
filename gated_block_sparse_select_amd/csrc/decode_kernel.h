#pragma once

// Single-token decode kernels, for a contiguous KV cache (decode.hip) and for
// a paged pool of one-block pages (decode_paged.hip).
//
// The query of batch entry b is token T = seq_len-1; its current block i = T/64
// holds the tokens [64 i, seq_len).  Each kv-group selects Top-K history blocks
// from its score row and adds their log-gates (SAS review page, paper.oopus.info,
// §2.2, §2.4); the current block is unbiased (§2.4, g_0 = 1).
//
// The step is HBM-bound (one pass over the kept K/V tiles), so it runs on the
// vector units with perfectly coalesced 16-byte loads: a 64-token tile of one
// kv-head is one contiguous 64*d element chunk of the cache (or of one page).
// One kernel does the whole step for a (b, kv-group, split): wave 0 (or, for
// rows over 2048 blocks, the whole workgroup) selects the row's blocks into
// LDS, then the workgroup streams its share of the kept tiles plus the
// current block with two tiles of loads in flight.  When one
// workgroup covers a whole row (enough rows to fill the GPU) it writes o
// directly; otherwise it writes an unnormalised partial (output, max, sum)
// and a combine kernel merges the splits.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"
#include "sas.h"
#include "select_row.h"

namespace sas {

template <class E>
struct Vec16;  // one 16-byte chunk of elements
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
  // acc + dot(q, k) over the 8 elements, accumulated in float32
  static SAS_DEV float dot(const uint4& q, const uint4& k, float acc) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w}, kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, qw[e]),
                                            __builtin_bit_cast(bf2, kw[e]), acc, false);
    return acc;
  }
};
template <>
struct Vec16<ElemF32> {
  static constexpr int N = 4;
  static SAS_DEV void unpack(const uint4& u, float* o) {
    o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
    o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
  }
  static SAS_DEV float dot(const uint4& q, const uint4& k, float acc) {
    acc = __builtin_fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    return __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  }
};

// Sum over aligned groups of W lanes (W = 8, 16 or 32) with DPP lane
// permutations: swap neighbours, swap pairs, mirror within 8, mirror within
// 16 (then one swap across the two rows of 16 for W = 32).
template <int CTRL>
SAS_DEV float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int W>
SAS_DEV float group_sum(float x) {
  static_assert(W == 8 || W == 16 || W == 32, "group width");
  x = dpp_add<0xB1>(x);     // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);     // quad_perm [2,3,0,1]
  x = dpp_add<0x141>(x);    // row_half_mirror
  if (W >= 16) x = dpp_add<0x140>(x);   // row_mirror
  if (W == 32) x += __shfl_xor(x, 16);
  return x;
}

// grid: B*Hkv*nsplit workgroups of 256 threads.
// Thread t owns chunk dg = t % CPR (EPC elements) of keys kg + KG*u, u < KPT,
// of every tile, kg = t / CPR: a group of CPR lanes reads one key row (256 B
// at d = 128 bf16) and the tile is one contiguous stretch of the cache.  Each
// key group keeps its own online softmax (running max, sum, output chunk) for
// all G heads, so tiles need no workgroup barrier.  NB register buffers
// rotate (the tile loop is unrolled by NB) so that the loads of the next
// NB-1 tiles are in flight while one is computed.  The KG groups are merged once,
// through LDS, at the end.
//
// SW = 1: wave 0 selects (rows of up to 64*CPL candidates); SW = 4: the whole
// workgroup selects (up to 256*CPL).  PAGED: K/V come from a pool of one-block
// pages [num_pages, Hkv, 64, d]; block m of sequence b lives in page
// page_table[b, m] (clamped into [0, num_pages)); otherwise from the
// contiguous cache [B, Hkv, cap, d].
template <class E, int D, int GMAX, int CPL, int SW, bool PAGED>
__global__ void __launch_bounds__(256) decode_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ kc,
    const typename E::T* __restrict__ vc, const int32_t* __restrict__ page_table, int num_pages,
    const int32_t* __restrict__ seq_lens, const float* __restrict__ s,
    int32_t* __restrict__ idx_out, typename E::T* __restrict__ o, float* __restrict__ part_acc,
    float* __restrict__ part_ml, int Hq, int Hkv, int cap, int topk, int nsplit, float tau2,
    int gate) {
  static_assert(SW == 1 || SW == 4, "select by one wave or by the workgroup's four");
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
  const int wave = t >> 6, lane = t & 63;

  const int nkb = cap / SAS_BLK;
  int L = seq_lens[b];
  L = L < 1 ? 1 : (L > cap ? cap : L);
  const int icur = (L - 1) / SAS_BLK;
  // block m of this sequence -> page holding it (paged pool) or m itself
  auto where = [&](int m) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int p = page_table[size_t(b) * nkb + m];
      return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
    } else {
      return m;
    }
  };

  // this thread's chunk of every head's query (scores are scaled by
  // tau*log2(e) afterwards, so they are in the exp2 domain)
  uint4 qv[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
    qv[g] = g < G ? *reinterpret_cast<const uint4*>(q + (size_t(b) * Hq + kv * G + g) * D + dg * EPC)
                  : make_uint4(0u, 0u, 0u, 0u);

  // selection of this row: kept blocks and base-2 log-gates in LDS
  __shared__ int32_t sblk[SAS_MAX_BLOCKS];
  __shared__ float sgate[SAS_MAX_BLOCKS];
  __shared__ int scnt;
  int32_t* orow = (idx_out != nullptr && split == 0) ? idx_out + size_t(bk) * topk : nullptr;
  // the external gate keeps its log-gate as the tile's exponent offset
  // (clamped at -60, so no weight underflows) and divides the tile's weight
  // sum by g again: o = sum g P v / sum P
  const bool ext = gate == SAS_GATE_EXTERNAL;
  auto emit = [&](int pos, int m, float g) __attribute__((always_inline)) {
    sblk[pos] = where(m);
    sgate[pos] = (ext ? fmaxf(g, kMinExtLogGate) : g) * kLog2e;
    if (orow) orow[pos] = m;
  };
  const float* srow = s + size_t(bk) * nkb;
  if constexpr (SW == 1) {
    if (wave == 0) {
      float lse;
      const int keff = select_row<CPL>(srow, icur, topk, gate, lane, lse, emit);
      if (orow)
        for (int p = keff + lane; p < topk; p += 64) orow[p] = -1;
      if (lane == 0) scnt = keff;
    }
  } else {
    __shared__ float sel_red[6 * SW];
    float lse;
    const int keff = select_row_wg<CPL, SW>(srow, icur, topk, gate, wave, lane, lse,
                                            (__attribute__((address_space(3))) float*)sel_red, emit);
    if (orow)
      for (int p = keff + t; p < topk; p += 256) orow[p] = -1;
    if (t == 0) scnt = keff;
  }
  __syncthreads();
  const int c_sel = scnt;
  const int ntiles = c_sel + 1;
  const int per = (ntiles + nsplit - 1) / nsplit;
  const int t0 = split * per, t1 = min(ntiles, t0 + per);

  float acc[GMAX][EPC];
  float mrun[GMAX], lrun[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    mrun[g] = -INFINITY;
    lrun[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
  }

  const size_t cache0 = (size_t(b) * Hkv + kv) * size_t(cap) * D;
  const int cur = where(icur);
  // register buffers: NB-1 tiles of loads stay in flight while one is computed
  constexpr int NB = 3;
  uint4 kb[NB][KPT], vb[NB][KPT];
  auto load = [&]<int B>(int tile) __attribute__((always_inline)) {
    const int blk = tile < c_sel ? sblk[tile] : cur;
    const size_t base = PAGED ? (size_t(blk) * Hkv + kv) * SAS_BLK * D : cache0 + size_t(blk) * SAS_BLK * D;
    const uint4* kt = reinterpret_cast<const uint4*>(kc + base);
    const uint4* vt = reinterpret_cast<const uint4*>(vc + base);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      kb[B][u] = kt[u * 256 + t];
      vb[B][u] = vt[u * 256 + t];
    }
  };
  // Lazy running max (exp2 domain): raised only when a tile's max exceeds it
  // by more than kSlack somewhere in the wave, so most tiles skip the rescale;
  // weights stay below 2^kSlack and the final acc / l is exact whatever max
  // was used.
  constexpr float kSlack = 8.f;
  constexpr bool kBF16 = std::is_same<E, ElemBF16>::value;
  auto compute = [&]<int B>(int tile) __attribute__((always_inline)) {
    const float bias2 = tile < c_sel ? sgate[tile] : 0.f;
    const float wsum_scale = ext ? fast_exp2(-bias2) : 1.f;   // 1/g for the external gate
    const int nvalid = tile < c_sel ? SAS_BLK : L - icur * SAS_BLK;
    float sc[KPT][GMAX];
#pragma unroll
    for (int u = 0; u < KPT; ++u)
#pragma unroll
      for (int g = 0; g < GMAX; ++g)
        sc[u][g] = g < G ? group_sum<CPR>(Vec16<E>::dot(qv[g], kb[B][u], 0.f)) : 0.f;
    // bf16: V of key pairs (2x, 2x+1) regrouped once per tile, shared by all
    // heads: word w of vp[x][h] holds elements 2w+h of the two keys, so
    // acc += p0 v0 + p1 v1 is one v_dot2_f32_bf16 per element.
    uint32_t vp[KPT / 2][2][4];
    if constexpr (kBF16) {
#pragma unroll
      for (int x = 0; x < KPT / 2; ++x) {
        const uint4 a = vb[B][2 * x], c = vb[B][2 * x + 1];
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vp[x][0][w] = __builtin_amdgcn_perm(cw[w], aw[w], 0x05040100u);
          vp[x][1][w] = __builtin_amdgcn_perm(cw[w], aw[w], 0x07060302u);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) continue;
      float mt = -INFINITY;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        sc[u][g] = kg + KG * u < nvalid ? __builtin_fmaf(sc[u][g], tau2, bias2) : -INFINITY;
        mt = fmaxf(mt, sc[u][g]);
      }
      if (mt == -INFINITY) continue;   // no valid key of this group in the tile
      if (__any(mt > mrun[g] + kSlack)) {
        const float mnew = fmaxf(mrun[g], mt);
        const float corr = fast_exp2(mrun[g] - mnew);
        mrun[g] = mnew;
        lrun[g] *= corr;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] *= corr;
      }
      float ts = 0.f;   // this tile's weight sum
      if constexpr (kBF16) {
        typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
        const bf2 ones = __builtin_bit_cast(bf2, 0x3F803F80u);
#pragma unroll
        for (int x = 0; x < KPT / 2; ++x) {
          // the weights actually used (bf16) also form the normaliser
          const bf2 pp = {(__bf16)fast_exp2(sc[2 * x][g] - mrun[g]),
                          (__bf16)fast_exp2(sc[2 * x + 1][g] - mrun[g])};
          ts = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ts, false);
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              acc[g][2 * w + h] = __builtin_amdgcn_fdot2_f32_bf16(
                  pp, __builtin_bit_cast(bf2, vp[x][h][w]), acc[g][2 * w + h], false);
        }
      } else {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
          const float p = fast_exp2(sc[u][g] - mrun[g]);
          ts += p;
          float vx[EPC];
          Vec16<E>::unpack(vb[B][u], vx);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[g][e] = __builtin_fmaf(p, vx[e], acc[g][e]);
        }
      }
      lrun[g] = __builtin_fmaf(ts, wsum_scale, lrun[g]);
    }
  };
  [&]<int... X>(std::integer_sequence<int, X...>) __attribute__((always_inline)) {
    ((t0 + X < t1 ? load.template operator()<X>(t0 + X) : void()), ...);
  }(std::make_integer_sequence<int, NB>{});
  int tile = t0;
  for (; tile + NB <= t1; tile += NB)
    [&]<int... X>(std::integer_sequence<int, X...>) __attribute__((always_inline)) {
      ((compute.template operator()<X>(tile + X),
        (tile + X + NB < t1 ? load.template operator()<X>(tile + X + NB) : void())),
       ...);
    }(std::make_integer_sequence<int, NB>{});
  [&]<int... X>(std::integer_sequence<int, X...>) __attribute__((always_inline)) {
    ((tile + X < t1 ? compute.template operator()<X>(tile + X) : void()), ...);
  }(std::make_integer_sequence<int, NB - 1>{});

  // merge the KG key groups: M = max of the group maxima, each group's sum
  // and output chunk scaled by 2^(m_k - M)
  __shared__ float sm[KG][GMAX], sl[KG][GMAX];
  __shared__ float sacc[KG][GMAX][D];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) continue;
#pragma unroll
    for (int e = 0; e < EPC; ++e) sacc[kg][g][dg * EPC + e] = acc[g][e];
    if (dg == 0) {
      sm[kg][g] = mrun[g];
      sl[kg][g] = lrun[g];
    }
  }
  __syncthreads();
  for (int x = t; x < G * D; x += 256) {
    const int g = x / D, c = x % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KG; ++k) M = fmaxf(M, sm[k][g]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        if (sm[k][g] == -INFINITY) continue;
        const float w = fast_exp2(sm[k][g] - M);
        a = __builtin_fmaf(w, sacc[k][g][c], a);
        l = __builtin_fmaf(w, sl[k][g], l);
      }
    }
    const size_t bh = size_t(b) * Hq + kv * G + g;
    if (nsplit == 1) {
      E::st(o + bh * D + c, a / l);   // the current block always has a valid key
    } else {
      const size_t pb = bh * nsplit + split;
      part_acc[pb * D + c] = a;
      if (c == 0) {
        part_ml[pb * 2] = M;
        part_ml[pb * 2 + 1] = l;
      }
    }
  }
}

// grid: B*Hq workgroups of D threads.
template <class E, int D>
__global__ void __launch_bounds__(128) decode_combine_kernel(const float* __restrict__ part_acc,
                                                             const float* __restrict__ part_ml,
                                                             typename E::T* __restrict__ o,
                                                             int nsplit) {
  // the splits' (max, sum) pairs go to LDS with parallel loads, so the merge
  // below issues its partial-output loads back to back instead of one
  // dependent load per split (decode_nsplit never exceeds 512)
  __shared__ float sm[512], sl[512];
  const size_t bh = blockIdx.x;
  const int c = threadIdx.x;
  for (int sp = c; sp < nsplit; sp += D) {
    sm[sp] = part_ml[(bh * nsplit + sp) * 2];
    sl[sp] = part_ml[(bh * nsplit + sp) * 2 + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, sm[sp]);
  float l = 0.f, a = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < nsplit; ++sp) {
    const float m = sm[sp];
    const float x = part_acc[(bh * nsplit + sp) * D + c];
    if (m != -INFINITY) {   // a split without keys contributes nothing
      const float w = fast_exp2(m - M);
      l += w * sl[sp];
      a += w * x;
    }
  }
  E::st(o + bh * D + c, a / l);
}


// ---- launch: dtype -> d -> select mode -> heads per group
template <class E, int D, int GMAX, int CPL, int SW, bool PAGED>
static void dec_go(const void* q, const void* kc, const void* vc, const int32_t* pt, int np,
                   const int32_t* sl, const float* s, int32_t* idx_out, void* o, float* pa,
                   float* pm, int B, int Hq, int Hkv, int cap, int topk, int ns, float tau2,
                   int gate, hipStream_t st) {
  using T = typename E::T;
  hipLaunchKernelGGL((decode_kernel<E, D, GMAX, CPL, SW, PAGED>), dim3(B * Hkv * ns), dim3(256), 0, st,
                     (const T*)q, (const T*)kc, (const T*)vc, pt, np, sl, s, idx_out, (T*)o, pa, pm,
                     Hq, Hkv, cap, topk, ns, tau2, gate);
}

template <class E, int D, int CPL, int SW, bool PAGED>
static void dec_g(int G, const void* q, const void* kc, const void* vc, const int32_t* pt, int np,
                  const int32_t* sl, const float* s, int32_t* idx_out, void* o, float* pa,
                  float* pm, int B, int Hq, int Hkv, int cap, int topk, int ns, float tau2,
                  int gate, hipStream_t st) {
  if (G <= 4) dec_go<E, D, 4, CPL, SW, PAGED>(q, kc, vc, pt, np, sl, s, idx_out, o, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, gate, st);
  else if (G <= 8) dec_go<E, D, 8, CPL, SW, PAGED>(q, kc, vc, pt, np, sl, s, idx_out, o, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, gate, st);
  else dec_go<E, D, 16, CPL, SW, PAGED>(q, kc, vc, pt, np, sl, s, idx_out, o, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, gate, st);
}

template <class E, int D, bool PAGED>
static void dec_c(int G, const void* q, const void* kc, const void* vc, const int32_t* pt, int np,
                  const int32_t* sl, const float* s, int32_t* idx_out, void* o, float* pa,
                  float* pm, int B, int Hq, int Hkv, int cap, int topk, int ns, float tau2,
                  int gate, hipStream_t st) {
  // history rows hold up to cap/64 - 1 candidate blocks
  const int nkb = cap / SAS_BLK;
  if (nkb <= 8 * 64)
    dec_g<E, D, 8, 1, PAGED>(G, q, kc, vc, pt, np, sl, s, idx_out, o, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, gate, st);
  else if (!PAGED || nkb <= 32 * 64)
    dec_g<E, D, 32, 1, PAGED>(G, q, kc, vc, pt, np, sl, s, idx_out, o, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, gate, st);
  else if constexpr (PAGED)
    dec_g<E, D, 32, 4, PAGED>(G, q, kc, vc, pt, np, sl, s, idx_out, o, pa, pm, B, Hq, Hkv, cap, topk, ns, tau2, gate, st);
}

// The decode step (and, when rows are split, the combine kernel) for either
// cache layout; kernel names for the profiling hooks differ per layout.
template <bool PAGED>
hipError_t launch_decode_any(int dtype, const void* q, const void* kc, const void* vc,
                             const int32_t* page_table, int num_pages, const int32_t* seq_lens,
                             const float* s, int32_t* idx_out, float* part_acc, float* part_ml,
                             void* o, int B, int Hq, int Hkv, int cap, int d, int topk, int nsplit,
                             float tau, int gate, hipStream_t st) {
  const int G = Hq / Hkv;
  const float tau2 = tau * kLog2e;
  {
    ProfScope ps(PAGED ? "sas_decode_paged_kernel" : "sas_decode_kernel", st);
    if (dtype == 1) {
      if (d == 128) dec_c<ElemBF16, 128, PAGED>(G, q, kc, vc, page_table, num_pages, seq_lens, s, idx_out, o, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, gate, st);
      else dec_c<ElemBF16, 64, PAGED>(G, q, kc, vc, page_table, num_pages, seq_lens, s, idx_out, o, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, gate, st);
    } else {
      if (d == 128) dec_c<ElemF32, 128, PAGED>(G, q, kc, vc, page_table, num_pages, seq_lens, s, idx_out, o, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, gate, st);
      else dec_c<ElemF32, 64, PAGED>(G, q, kc, vc, page_table, num_pages, seq_lens, s, idx_out, o, part_acc, part_ml, B, Hq, Hkv, cap, topk, nsplit, tau2, gate, st);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
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
