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
// When one workgroup covers a whole row (enough rows to fill the GPU), one
// kernel does the whole step: wave 0 (or, for rows over 2048 blocks, the
// whole workgroup) selects the row's blocks into LDS, then the workgroup
// streams the kept tiles plus the current block with two tiles of loads in
// flight and writes o.  Otherwise (small batches, long contexts) a select
// kernel selects each row once, into the workspace, and the row's tiles are
// split over several workgroups; each writes an unnormalised partial
// (output, max, sum), and a combine kernel merges them.  (Merging inside the
// split kernel, by the last workgroup of a row to finish, was measured
// slower: the device-scope fences and the row's serialised atomics cost more
// than the extra launch.)
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

// x plus x of the lane that the DPP control CTRL selects (a permutation
// within each row of 16 lanes, so no source lane is out of bounds; bound_ctrl
// set lets the compiler fold the move into the add for every control)
template <int CTRL>
SAS_DEV float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Floor of the running maxima (exp2 domain) in place of -inf, so that
// exp2(m - mrun) and the rescale exp2(mrun - mnew) never see -inf - -inf: a
// weight against it is exp2(-inf) = 0 for invalid keys, and the first valid
// key (any finite score is far above it) rescales everything before it by 0.
constexpr float kMaxFloor = -1.0e30f;

// Sums of N values over aligned groups of W lanes (W = 8, 16 or 32) with DPP
// lane permutations: swap neighbours, swap pairs, mirror within 8, rotate by
// 8 within 16 (then one swap across the two rows of 16 for W = 32).  Each level
// runs over all N values before the next, so the N reduction chains
// interleave (no dependent DPP back to back).
template <int W, int N>
SAS_DEV void group_sum_all(float* x) {
  static_assert(W == 8 || W == 16 || W == 32, "group width");
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0xB1>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x4E>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x141>(x[i]);
  if constexpr (W >= 16) {   // rotate by 8 within the row: the other half
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = dpp_add<0x128>(x[i]);
  }
  if constexpr (W == 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 16);
  }
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
// SW = 4: the four waves select rows of up to 256*CPL candidates
// (select_row_hier for topk <= 64, select_row_wg otherwise).  PAGED: K/V come from a pool of one-block
// pages [num_pages, Hkv, 64, d]; block m of sequence b lives in page
// page_table[b, m] (clamped into [0, num_pages)); otherwise from the
// contiguous cache [B, Hkv, cap, d].
//
// PRESEL (split rows): the row's selection comes from the workspace (written
// by decode_select_kernel: kept blocks / pages and base-2 log-gates, the
// current block after them, and the count), and split s streams the tiles s,
// s + nsplit, ... of it, so it can fetch its first tile's block at once.
template <class E, int D, int GMAX, int CPL, int SW, bool PAGED, bool PRESEL>
__global__ void __launch_bounds__(256) decode_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ kc,
    const typename E::T* __restrict__ vc, const int32_t* __restrict__ page_table, int num_pages,
    const int32_t* __restrict__ seq_lens, const float* __restrict__ s,
    int32_t* __restrict__ idx_out, typename E::T* __restrict__ o, DecodeScratch ws, int Hq,
    int Hkv, int cap, int topk, int nsplit, float tau2, int gate) {
  static_assert(SW == 4, "the workgroup's four waves select");
  constexpr int EPC = Vec16<E>::N;        // elements per 16-byte chunk
  constexpr int CPR = D / EPC;            // chunks per key row
  constexpr int KG = 256 / CPR;           // key groups per workgroup
  constexpr int KPT = SAS_BLK / KG;       // keys per thread per tile
  // register buffers: NB-1 tiles of loads stay in flight while one is
  // computed.  With the non-temporal K/V loads two measured fastest (94.4 vs
  // 95.8 us for three and 104 for four at batch 64), and two leave the
  // eight-head groups without spills.
  constexpr int NB = 2;
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
  // the external gate keeps its log-gate as the tile's exponent offset
  // (clamped at -60, so no weight underflows) and divides the tile's weight
  // sum by g again: o = sum g P v / sum P
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const size_t e0 = size_t(bk) * (topk + 1);   // this row's workspace selection
  // tiles p = t0 + r*ts, r < nloc, of the row's kept blocks followed by the
  // current block (position c_sel)
  int c_sel, t0, ts, nloc;
  if constexpr (PRESEL) {
    // the select kernel wrote the kept blocks (pages), their gates and the
    // current block at position c_sel; split s takes tiles s, s + nsplit, ...
    c_sel = ws.sel_cnt[bk];
    t0 = split;
    ts = nsplit;
    nloc = split <= c_sel ? (c_sel - split) / nsplit + 1 : 0;
  } else {
    int32_t* orow = idx_out != nullptr ? idx_out + size_t(bk) * topk : nullptr;
    auto emit = [&](int pos, int m, int tg, float g) __attribute__((always_inline)) {
      sblk[pos] = PAGED ? tg : m;
      sgate[pos] = (ext ? fmaxf(g, kMinExtLogGate) : g) * kLog2e;
      if (orow) orow[pos] = m;
    };
    auto tag_of = [&](int m) __attribute__((always_inline)) { return where(m); };
    const float* srow = s + size_t(bk) * nkb;
    __shared__ float sel_red[6 * SW];
    float lse;
    if (topk <= 64) {
      __shared__ float cval[SW * 64];
      __shared__ int cidx[SW * 64], ctag[SW * 64];
      __shared__ uint32_t thr[SW + 4];
      // four waves merge in one level: no second-level segments
      const int keff = select_row_hier<CPL, SW>(
          srow, nkb, icur, topk, gate, wave, lane, lse,
          (__attribute__((address_space(3))) float*)sel_red,
          (__attribute__((address_space(3))) float*)cval,
          (__attribute__((address_space(3))) int*)cidx,
          (__attribute__((address_space(3))) int*)ctag,
          (__attribute__((address_space(3))) uint32_t*)thr,
          (__attribute__((address_space(3))) float*)cval,
          (__attribute__((address_space(3))) int*)cidx,
          (__attribute__((address_space(3))) int*)ctag, tag_of, emit);
      if (wave == 0) {
        if (orow)
          for (int p = keff + lane; p < topk; p += 64) orow[p] = -1;
        if (lane == 0) scnt = keff;
      }
    } else {
      const int keff = select_row_wg<CPL, SW>(srow, nkb, icur, topk, gate, wave, lane, lse,
                                              (__attribute__((address_space(3))) float*)sel_red,
                                              tag_of, emit);
      if (orow)
        for (int p = keff + t; p < topk; p += 64 * SW) orow[p] = -1;
      if (t == 0) scnt = keff;
    }
    __syncthreads();
    c_sel = scnt;
    t0 = 0;
    ts = 1;
    nloc = c_sel + 1;
  }

  float acc[GMAX][EPC];
  float mrun[GMAX], lrun[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    mrun[g] = kMaxFloor;
    lrun[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
  }

  const size_t cache0 = (size_t(b) * Hkv + kv) * size_t(cap) * D;
  const int cur = PRESEL ? 0 : where(icur);
  // tile p: its block (page) and base-2 log-gate; the current block (p ==
  // c_sel) is unbiased
  auto blk_of = [&](int p) __attribute__((always_inline)) {
    if constexpr (PRESEL) return ws.sel_blk[e0 + p];
    else return p < c_sel ? sblk[p] : cur;
  };
  auto bias_of = [&](int p) __attribute__((always_inline)) {
    if constexpr (PRESEL) return ws.sel_gate[e0 + p];
    else return p < c_sel ? sgate[p] : 0.f;
  };
  uint4 kb[NB][KPT], vb[NB][KPT];
  auto load = [&]<int B>(int r) __attribute__((always_inline)) {
    const int blk = blk_of(t0 + r * ts);
    const size_t base = PAGED ? (size_t(blk) * Hkv + kv) * SAS_BLK * D : cache0 + size_t(blk) * SAS_BLK * D;
    const uint4* kt = reinterpret_cast<const uint4*>(kc + base);
    const uint4* vt = reinterpret_cast<const uint4*>(vc + base);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      kb[B][u] = load_stream(kt + u * 256 + t);
      vb[B][u] = load_stream(vt + u * 256 + t);
    }
  };
  // Lazy running max (exp2 domain): raised only when a tile's max exceeds it
  // by more than kSlack somewhere in the wave, so most tiles skip the rescale;
  // weights stay below 2^kSlack and the final acc / l is exact whatever max
  // was used.
  constexpr float kSlack = 8.f;
  constexpr bool kBF16 = std::is_same<E, ElemBF16>::value;
  auto compute = [&]<int B>(int r) __attribute__((always_inline)) {
    const int tile = t0 + r * ts;
    const float bias2 = bias_of(tile);
    const float wsum_scale = ext ? fast_exp2(-bias2) : 1.f;   // 1/g for the external gate
    const int nvalid = tile < c_sel ? SAS_BLK : L - icur * SAS_BLK;
    // every head slot g < GMAX is computed (those >= G have a zero query, and
    // their results are never stored), so the loop has no per-head branch.
    // Up to four heads reduce all their sums together; wider groups reduce
    // head by head (KPT chains at a time), which bounds the live values.
    float sc[GMAX][KPT];
    if constexpr (GMAX <= 4) {
#pragma unroll
      for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int u = 0; u < KPT; ++u) sc[g][u] = Vec16<E>::dot(qv[g], kb[B][u], 0.f);
      group_sum_all<CPR, KPT * GMAX>(&sc[0][0]);
    } else {
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) sc[g][u] = Vec16<E>::dot(qv[g], kb[B][u], 0.f);
        group_sum_all<CPR, KPT>(&sc[g][0]);
      }
    }
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
      // a group without a valid key in the tile has mt = -inf: it adds
      // weights exp2(-inf - mrun) = 0 and never raises mrun
      float mt = -INFINITY;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        sc[g][u] = kg + KG * u < nvalid ? __builtin_fmaf(sc[g][u], tau2, bias2) : -INFINITY;
        mt = fmaxf(mt, sc[g][u]);
      }
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
          const bf2 pp = {(__bf16)fast_exp2(sc[g][2 * x] - mrun[g]),
                          (__bf16)fast_exp2(sc[g][2 * x + 1] - mrun[g])};
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
          const float p = fast_exp2(sc[g][u] - mrun[g]);
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
    ((X < nloc ? load.template operator()<X>(X) : void()), ...);
  }(std::make_integer_sequence<int, NB>{});
  int r = 0;
  for (; r + NB <= nloc; r += NB)
    [&]<int... X>(std::integer_sequence<int, X...>) __attribute__((always_inline)) {
      ((compute.template operator()<X>(r + X),
        (r + X + NB < nloc ? load.template operator()<X>(r + X + NB) : void())),
       ...);
    }(std::make_integer_sequence<int, NB>{});
  [&]<int... X>(std::integer_sequence<int, X...>) __attribute__((always_inline)) {
    ((r + X < nloc ? compute.template operator()<X>(r + X) : void()), ...);
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
    float M = kMaxFloor;
#pragma unroll
    for (int k = 0; k < KG; ++k) M = fmaxf(M, sm[k][g]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      // a group that saw no valid key (mrun still kMaxFloor, acc = l = 0)
      // weighs 0 here unless no group saw one (a split without keys), when
      // every term is 0 anyway
      const float w = fast_exp2(sm[k][g] - M);
      a = __builtin_fmaf(w, sacc[k][g][c], a);
      l = __builtin_fmaf(w, sl[k][g], l);
    }
    const size_t bh = size_t(b) * Hq + kv * G + g;
    if constexpr (!PRESEL) {
      E::st(o + bh * D + c, a / l);   // the current block always has a valid key
    } else {
      const size_t pb = bh * nsplit + split;
      ws.part_acc[pb * D + c] = a;
      if (c == 0) {
        ws.part_ml[pb * 2] = M;
        ws.part_ml[pb * 2 + 1] = l;
      }
    }
  }
}

// The selection of split rows, once per (b, kv-group): NW waves select the
// row (select_row for NW = 1, select_row_wg otherwise) into the workspace -
// kept blocks (pages when PAGED), base-2 log-gates, count - and write
// idx_out.
template <int CPL, int NW, bool PAGED>
__global__ void __launch_bounds__(64 * NW) decode_select_kernel(
    const int32_t* __restrict__ page_table, int num_pages, const int32_t* __restrict__ seq_lens,
    const float* __restrict__ s, int32_t* __restrict__ idx_out, DecodeScratch ws, int Hkv,
    int cap, int topk, int gate) {
  const int bk = blockIdx.x;
  const int b = bk / Hkv;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int nkb = cap / SAS_BLK;
  auto where = [&](int m) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int p = page_table[size_t(b) * nkb + m];
      return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
    } else {
      return m;
    }
  };
  int L = seq_lens[b];
  L = L < 1 ? 1 : (L > cap ? cap : L);
  const int icur = (L - 1) / SAS_BLK;
  const int cur = where(icur);   // issued now, used at the end
  const bool ext = gate == SAS_GATE_EXTERNAL;
  int32_t* orow = idx_out != nullptr ? idx_out + size_t(bk) * topk : nullptr;
  const size_t e0 = size_t(bk) * (topk + 1);
  auto emit = [&](int pos, int m, int tg, float g) __attribute__((always_inline)) {
    ws.sel_blk[e0 + pos] = PAGED ? tg : m;
    ws.sel_gate[e0 + pos] = (ext ? fmaxf(g, kMinExtLogGate) : g) * kLog2e;
    if (orow) orow[pos] = m;
  };
  auto tag_of = [&](int m) __attribute__((always_inline)) { return where(m); };
  const float* srow = s + size_t(bk) * nkb;
  float lse;
  // the number kept, known to wave 0 (and to every wave after select_row_wg)
  int keff;
  if constexpr (NW == 1) {
    keff = select_row<CPL>(srow, nkb, icur, topk, gate, lane, lse, tag_of, emit);
  } else {
    __shared__ float sel_red[6 * NW];
    if (topk <= 64) {
      __shared__ float cval[NW * 64], mval[4 * 64];
      __shared__ int cidx[NW * 64], ctag[NW * 64], midx[4 * 64], mtag[4 * 64];
      __shared__ uint32_t thr[NW + 4];
      keff = select_row_hier<CPL, NW>(srow, nkb, icur, topk, gate, wave, lane, lse,
                                      (__attribute__((address_space(3))) float*)sel_red,
                                      (__attribute__((address_space(3))) float*)cval,
                                      (__attribute__((address_space(3))) int*)cidx,
                                      (__attribute__((address_space(3))) int*)ctag,
                                      (__attribute__((address_space(3))) uint32_t*)thr,
                                      (__attribute__((address_space(3))) float*)mval,
                                      (__attribute__((address_space(3))) int*)midx,
                                      (__attribute__((address_space(3))) int*)mtag, tag_of, emit);
    } else {
      keff = select_row_wg<CPL, NW>(srow, nkb, icur, topk, gate, wave, lane, lse,
                                    (__attribute__((address_space(3))) float*)sel_red, tag_of,
                                    emit);
    }
  }
  if (wave != 0) return;
  // the current block follows the kept ones, unbiased
  if (lane == 0) {
    ws.sel_blk[e0 + keff] = cur;
    ws.sel_gate[e0 + keff] = 0.f;
    ws.sel_cnt[bk] = keff;
  }
  if (orow)
    for (int p = keff + lane; p < topk; p += 64) orow[p] = -1;
}

// grid: B*Hq workgroups of 256 threads: merges the nsplit partials of one
// (b, head): M = max of the splits' maxima, o = sum 2^(m - M) acc / sum
// 2^(m - M) l.  Thread t takes column t % D of the splits t / D + (256/D) k;
// the first KM of them are loaded together with the (max, sum) pairs, so a
// call waits on one round of loads (more splits than that take further
// rounds).  The column sums of the 256/D thread groups are added in group
// order, so the result is deterministic.
template <class E, int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(const float* __restrict__ part_acc,
                                                             const float* __restrict__ part_ml,
                                                             typename E::T* __restrict__ o,
                                                             int nsplit) {
  constexpr int NG = 256 / D, KM = 16;
  __shared__ float sm[512], sl[512];   // decode_nsplit never exceeds 512
  __shared__ float ra[NG][D], rl[NG][D];
  const size_t bh = blockIdx.x;
  const int t = threadIdx.x, c = t % D, grp = t / D;
  const float* pa = part_acc + bh * nsplit * D + c;
  float x[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int sp = grp + NG * k;
    x[k] = sp < nsplit ? pa[size_t(sp) * D] : 0.f;
  }
  for (int sp = t; sp < nsplit; sp += 256) {
    sm[sp] = part_ml[(bh * nsplit + sp) * 2];
    sl[sp] = part_ml[(bh * nsplit + sp) * 2 + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, sm[sp]);
  float a = 0.f, l = 0.f;
  auto add = [&](int sp, float xv) __attribute__((always_inline)) {
    const float m = sm[sp];
    if (m != -INFINITY) {   // a split without keys contributes nothing
      const float w = fast_exp2(m - M);
      l = __builtin_fmaf(w, sl[sp], l);
      a = __builtin_fmaf(w, xv, a);
    }
  };
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (grp + NG * k < nsplit) add(grp + NG * k, x[k]);
  for (int sp = grp + NG * KM; sp < nsplit; sp += NG) add(sp, pa[size_t(sp) * D]);
  ra[grp][c] = a;
  rl[grp][c] = l;
  __syncthreads();
  if (grp != 0) return;
#pragma unroll
  for (int g = 1; g < NG; ++g) {
    a += ra[g][c];
    l += rl[g][c];
  }
  E::st(o + bh * D + c, a / l);   // the current block always has a valid key
}

// ---- launch: dtype -> d -> select mode -> heads per group
template <class E, int D, int GMAX, int CPL, int SW, bool PAGED, bool PRESEL>
static void dec_go(const void* q, const void* kc, const void* vc, const int32_t* pt, int np,
                   const int32_t* sl, const float* s, int32_t* idx_out, void* o,
                   const DecodeScratch& ws, int B, int Hq, int Hkv, int cap, int topk, int ns,
                   float tau2, int gate, hipStream_t st) {
  using T = typename E::T;
  hipLaunchKernelGGL((decode_kernel<E, D, GMAX, CPL, SW, PAGED, PRESEL>), dim3(B * Hkv * ns),
                     dim3(256), 0, st, (const T*)q, (const T*)kc, (const T*)vc, pt, np, sl, s,
                     idx_out, (T*)o, ws, Hq, Hkv, cap, topk, ns, tau2, gate);
}

template <class E, int D, int CPL, int SW, bool PAGED, bool PRESEL>
static void dec_g(int G, const void* q, const void* kc, const void* vc, const int32_t* pt, int np,
                  const int32_t* sl, const float* s, int32_t* idx_out, void* o,
                  const DecodeScratch& ws, int B, int Hq, int Hkv, int cap, int topk, int ns,
                  float tau2, int gate, hipStream_t st) {
#define SAS_DEC_ARGS q, kc, vc, pt, np, sl, s, idx_out, o, ws, B, Hq, Hkv, cap, topk, ns, tau2, gate, st
  if (G <= 4) dec_go<E, D, 4, CPL, SW, PAGED, PRESEL>(SAS_DEC_ARGS);
  else if (G <= 8) dec_go<E, D, 8, CPL, SW, PAGED, PRESEL>(SAS_DEC_ARGS);
  else dec_go<E, D, 16, CPL, SW, PAGED, PRESEL>(SAS_DEC_ARGS);
#undef SAS_DEC_ARGS
}

template <class E, int D, bool PAGED>
static void dec_c(int G, const void* q, const void* kc, const void* vc, const int32_t* pt, int np,
                  const int32_t* sl, const float* s, int32_t* idx_out, void* o,
                  const DecodeScratch& ws, int B, int Hq, int Hkv, int cap, int topk, int ns,
                  float tau2, int gate, hipStream_t st) {
#define SAS_DEC_ARGS G, q, kc, vc, pt, np, sl, s, idx_out, o, ws, B, Hq, Hkv, cap, topk, ns, tau2, gate, st
  if (ns > 1) {   // rows selected beforehand (decode_select_kernel), tiles split
    dec_g<E, D, 1, 4, PAGED, true>(SAS_DEC_ARGS);
    return;
  }
  // history rows hold up to cap/64 - 1 candidate blocks; the workgroup's four
  // waves select (select_row_hier for topk <= 64, select_row_wg otherwise)
  const int nkb = cap / SAS_BLK;
  if (nkb <= 2 * 256)
    dec_g<E, D, 2, 4, PAGED, false>(SAS_DEC_ARGS);
  else if (!PAGED || nkb <= 8 * 256)
    dec_g<E, D, 8, 4, PAGED, false>(SAS_DEC_ARGS);
  else if constexpr (PAGED)
    dec_g<E, D, 32, 4, PAGED, false>(SAS_DEC_ARGS);
#undef SAS_DEC_ARGS
}

template <bool PAGED>
static void dec_select(const int32_t* pt, int np, const int32_t* sl, const float* s,
                       int32_t* idx_out, const DecodeScratch& ws, int B, int Hkv, int cap, int topk,
                       int gate, hipStream_t st) {
#define SAS_SEL_ARGS pt, np, sl, s, idx_out, ws, Hkv, cap, topk, gate
  // one wave for rows of up to 512 blocks, 16 waves (1..8 candidates per lane)
  // beyond: a lone row is pure latency, so more waves shorten the search
  const int nkb = cap / SAS_BLK;
  if (nkb <= 8 * 64)
    hipLaunchKernelGGL((decode_select_kernel<8, 1, PAGED>), dim3(B * Hkv), dim3(64), 0, st, SAS_SEL_ARGS);
  else if (nkb <= 1024)
    hipLaunchKernelGGL((decode_select_kernel<1, 16, PAGED>), dim3(B * Hkv), dim3(1024), 0, st, SAS_SEL_ARGS);
  else if (nkb <= 2048)
    hipLaunchKernelGGL((decode_select_kernel<2, 16, PAGED>), dim3(B * Hkv), dim3(1024), 0, st, SAS_SEL_ARGS);
  else if (nkb <= 4096)
    hipLaunchKernelGGL((decode_select_kernel<4, 16, PAGED>), dim3(B * Hkv), dim3(1024), 0, st, SAS_SEL_ARGS);
  else
    hipLaunchKernelGGL((decode_select_kernel<8, 16, PAGED>), dim3(B * Hkv), dim3(1024), 0, st, SAS_SEL_ARGS);
#undef SAS_SEL_ARGS
}

// The decode step for either cache layout: one fused kernel when one
// workgroup covers a row (nsplit == 1); otherwise the select kernel, the
// split kernel and the combine kernel.  Kernel names for the
// profiling hooks differ per layout.
template <bool PAGED>
hipError_t launch_decode_any(int dtype, const void* q, const void* kc, const void* vc,
                             const int32_t* page_table, int num_pages, const int32_t* seq_lens,
                             const float* s, int32_t* idx_out, const DecodeScratch& ws, void* o,
                             int B, int Hq, int Hkv, int cap, int d, int topk, int nsplit,
                             float tau, int gate, hipStream_t st) {
  const int G = Hq / Hkv;
  const float tau2 = tau * kLog2e;
  if (nsplit > 1) {
    ProfScope ps(PAGED ? "sas_decode_paged_select_kernel" : "sas_decode_select_kernel", st);
    dec_select<PAGED>(page_table, num_pages, seq_lens, s, idx_out, ws, B, Hkv, cap, topk, gate, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps(PAGED ? "sas_decode_paged_kernel" : "sas_decode_kernel", st);
#define SAS_DEC_ARGS G, q, kc, vc, page_table, num_pages, seq_lens, s, idx_out, o, ws, B, Hq, Hkv, cap, topk, nsplit, tau2, gate, st
    if (dtype == 1) {
      if (d == 128) dec_c<ElemBF16, 128, PAGED>(SAS_DEC_ARGS);
      else dec_c<ElemBF16, 64, PAGED>(SAS_DEC_ARGS);
    } else {
      if (d == 128) dec_c<ElemF32, 128, PAGED>(SAS_DEC_ARGS);
      else dec_c<ElemF32, 64, PAGED>(SAS_DEC_ARGS);
    }
#undef SAS_DEC_ARGS
  }
  e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  {
    ProfScope ps("sas_decode_combine_kernel", st);
    if (dtype == 1) {
      if (d == 128) hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 128>), dim3(B * Hq), dim3(256), 0, st, ws.part_acc, ws.part_ml, (uint16_t*)o, nsplit);
      else hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 64>), dim3(B * Hq), dim3(256), 0, st, ws.part_acc, ws.part_ml, (uint16_t*)o, nsplit);
    } else {
      if (d == 128) hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 128>), dim3(B * Hq), dim3(256), 0, st, ws.part_acc, ws.part_ml, (float*)o, nsplit);
      else hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 64>), dim3(B * Hq), dim3(256), 0, st, ws.part_acc, ws.part_ml, (float*)o, nsplit);
    }
  }
  return hipGetLastError();
}

}  // namespace sas
