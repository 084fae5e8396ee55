// LSE-normalised Top-K block selection of one score row by one wave64 (SAS
// review page, paper.oopus.info: §2.2 keeps the Top-K history blocks by
// selector score, §2.4 sets log g_m = s_m - LSE(s over all history blocks)).
//
// Candidates m < i sit in registers, CPL per lane with m = j*64 + lane, so
// scanning j ascending and lanes ascending visits m in ascending order.  Each
// candidate gets a 32-bit order-preserving key of its float value (-0.0
// canonicalised to +0.0); a 32-step bitwise search with wave population
// counts (ballots, so the counting stays in scalar registers) finds the K-th
// largest key T exactly; all keys > T are kept, and keys == T are kept lowest
// index first until K blocks are chosen.  The kept blocks are emitted in
// ascending order.  Every comparison is on the exact float bits, so the
// result is bit-identical to a sort by (score desc, index asc).  A score of
// -inf marks a block that is not a candidate (in a packed batch, a block of
// an earlier document): it is left out of the LSE and never kept, so a row
// keeps min(K, finite scores) blocks and a row without one gets LSE -inf.
#pragma once

#include <utility>

#include "common.h"
#include "sas.h"

namespace sas {

SAS_DEV uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Log-gate of a kept block with score x in a row with candidate LSE lse, for
// each gate kind (sas.h): x - lse (softmax; also the external gate's log g),
// log sigmoid(x) (sigmoid), 0 (hard).
SAS_DEV float log_gate_of(int gate, float x, float lse) {
  if (gate == SAS_GATE_SIGMOID) return fminf(x, 0.f) - log1pf(expf(-fabsf(x)));
  if (gate == SAS_GATE_HARD) return 0.f;
  return x - lse;
}

// order_key(-inf): below the key of every finite score, which is at least
// order_key(-FLT_MAX) = kNoKey + 1.  A key <= kNoKey is not a candidate.
constexpr uint32_t kNoKey = 0x007FFFFFu;

// Sum over the wave of a per-lane count c <= CPL, from the population counts
// of its bits (one ballot per bit).
template <int CPL>
SAS_DEV int wave_count_small(uint32_t c) {
  constexpr int NBITS = CPL < 2 ? 1 : CPL < 4 ? 2 : CPL < 8 ? 3 : CPL < 16 ? 4 : CPL < 32 ? 5 : 6;
  int n = 0;
#pragma unroll
  for (int b = 0; b < NBITS; ++b) n += __popcll(__ballot((c >> b) & 1u)) << b;
  return n;
}

// Threshold of a wave's keys for topk: keys > T are kept, then keys == T
// lowest position first until need_eq are kept.  With search, T is the
// largest th such that at least topk keys are >= th (a 32-step bitwise
// search), or kNoKey when fewer than topk candidates exist (then every
// candidate is kept).  Without search (the caller knows every candidate is
// kept) T = kNoKey; topk == 0 keeps nothing (T = ~0, no key exceeds it).
//
// Each step counts the keys >= th | bit over the wave.  VCNT = false: one
// ballot and scalar population count per key slot - fewest instructions, best
// when several waves share a SIMD and hide each other's waits.  VCNT = true:
// each lane counts its own keys in a vector register and the wave sums those
// counts with a ballot per bit (wave_count_small) - far fewer scalar reads of
// vector-written masks, each of which stalls a lone wave, so it is the faster
// form for a wave that runs alone.
//
// lo, hi (optional): bounds of the result known to the caller - at least
// topk keys are >= lo (so lo <= T) and no key exceeds hi.  The search builds
// T from its top bit down, one bit per step, and every value in [lo, hi]
// shares the bits above the highest bit where lo and hi differ, so the
// search starts with those bits set and tests only the bits below: the same
// T in fewer steps.  lo = 0 (the default) is no bound.
template <int CPL, bool VCNT = false>
SAS_DEV void wave_threshold(const uint32_t (&key)[CPL], int topk, bool search, uint32_t& T,
                            int& need_eq, uint32_t lo = 0u, uint32_t hi = ~0u) {
  T = topk > 0 ? kNoKey : ~0u;
  need_eq = 0;
  if (!search || topk <= 0) return;
  uint32_t th = 0u;   // largest th with at least topk keys >= th
  int top = 31;
  if (lo != 0u && lo <= hi) {
    const uint32_t diff = lo ^ hi;
    top = diff == 0u ? -1 : 31 - __builtin_clz(diff);
    th = top < 0 ? lo : lo & ~((2u << top) - 1u);   // 2u << 31 wraps to 0: th = 0
  }
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t c = th | (1u << bit);
    int n_ge = 0;
    if constexpr (VCNT) {
      uint32_t cl = 0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) cl += key[j] >= c ? 1u : 0u;
      n_ge = wave_count_small<CPL>(cl);
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) n_ge += __popcll(__ballot(key[j] >= c));
    }
    if (n_ge >= topk) th = c;
  }
  if (th > kNoKey) {
    T = th;
    int n_gt = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) n_gt += __popcll(__ballot(key[j] > T));
    need_eq = topk - n_gt;
  }
}

// Keeps the keys wave_threshold chose: keep(j, pos) runs on the lane holding
// the pos-th kept key, positions ascending in (j, lane) order.  Returns the
// number kept (wave-uniform).
template <int CPL, class Keep>
SAS_DEV int wave_keep(const uint32_t (&key)[CPL], uint32_t T, int need_eq, Keep&& keep) {
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const bool eq = key[j] == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = key[j] > T || (eq && eq_seen + mask_rank(eqm) < need_eq);
    eq_seen += __popcll(eqm);
    const uint64_t tm = __ballot(take);
    if (take) keep(j, base + mask_rank(tm));
    base += __popcll(tm);
  }
  return base;
}

// No per-candidate tag: emit receives 0.
struct NoTag {
  SAS_DEV int operator()(int) const { return 0; }
};

// Selects min(topk, candidates) of the blocks m < i of srow.  Scores are
// loaded for m < nk (nk >= i, a bound known at launch, so these loads need not
// wait for i) and masked to m < i.  tag(m) is loaded alongside (for instance
// the page of block m) and handed to emit, so that emitting waits on no
// further memory access.  emit(pos, m, tag, log_gate) is called by the lane
// holding the pos-th kept block (pos ascending with m), with the log-gate of
// the gate kind.  Returns the number kept (wave-uniform); lse receives the
// LSE over the candidates, -inf if there is none.
//
// Non-candidates (m >= i or a score of -inf) carry key kNoKey or below, under
// every candidate's key, so the search ends with T <= kNoKey exactly when
// fewer than topk candidates exist, and then every key > kNoKey is kept.  The
// number kept is the running output position, so no separate candidate count
// is needed.
template <int CPL, class Tag, class Emit>
SAS_DEV int select_row(const float* __restrict__ srow, int nk, int i, int topk, int gate, int lane,
                       float& lse, Tag&& tag_of, Emit&& emit) {
  float val[CPL];
  uint32_t key[CPL];
  int tag[CPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = j * 64 + lane;
    const float x = m < nk ? srow[m] : -INFINITY;
    tag[j] = m < nk ? tag_of(m) : 0;
    val[j] = m < i ? x : -INFINITY;
    key[j] = order_key(val[j]);
    mx = fmaxf(mx, val[j]);
  }
  mx = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) se += expf(val[j] - mx);   // -inf terms add 0
  se = wave_sum(se);
  lse = mx > -INFINITY ? mx + logf(se) : -INFINITY;

  // topk >= i keeps every candidate without a search
  uint32_t T;
  int need_eq;
  wave_threshold(key, topk, topk < i, T, need_eq);
  return wave_keep(key, T, need_eq, [&](int j, int pos) __attribute__((always_inline)) {
    emit(pos, j * 64 + lane, tag[j], log_gate_of(gate, val[j], lse));
  });
}

// The same selection by a workgroup of NW waves, for topk <= 64 and rows of up
// to NW*64*CPL candidates (long decode contexts), with no barrier inside the
// searches.  Wave w holds the contiguous candidates [w*64*CPL, (w+1)*64*CPL),
// m = w*64*CPL + j*64 + lane, and first keeps the top min(topk, its
// candidates) of its own share (by score descending, then index ascending)
// into its segment of LDS (SEG = 32 slots when topk <= 32, else 64).  The
// segments are then merged the same way: by wave 0 alone for NW = 4; for
// NW >= 8 in two levels, four waves each keeping the top of NW/4 segments,
// then wave 0 the top of their four.  This is exact: a block among the top
// topk of a set in that strict order is among the top topk of any subset
// holding it, so every kept block survives each level; and segments read in
// slot order list their blocks in ascending m, so ties at the threshold
// still go lowest index first.  Each merge search starts from bounds: the
// largest threshold of the segments it merges (at least topk keys reach it)
// and the row's largest key.
//
// The LSE is over every candidate: the maximum, then the exp sum (per wave,
// summed in wave order, so the result is deterministic), through red (2*NW
// words).  cval, cidx and ctag hold NW*64 entries, thr NW + 4 words, and
// mval, midx, mtag 4*64 entries (the second level's inputs).  Every thread of
// the workgroup must call it (it contains __syncthreads); emit(pos, m, tag,
// log_gate) is called by wave 0's lanes only, and the return value (the
// number kept) and lse are valid in wave 0 only.
template <int CPL, int NW, class Tag, class Emit>
SAS_DEV int select_row_hier(const float* __restrict__ srow, int nk, int i, int topk, int gate,
                            int wave, int lane, float& lse,
                            __attribute__((address_space(3))) float* red,
                            __attribute__((address_space(3))) float* cval,
                            __attribute__((address_space(3))) int* cidx,
                            __attribute__((address_space(3))) int* ctag,
                            __attribute__((address_space(3))) uint32_t* thr,
                            __attribute__((address_space(3))) float* mval,
                            __attribute__((address_space(3))) int* midx,
                            __attribute__((address_space(3))) int* mtag, Tag&& tag_of,
                            Emit&& emit) {
  static_assert(NW == 4 || NW == 8 || NW == 16, "four, eight or sixteen waves");
  const int m0 = wave * 64 * CPL;
  const int seg = topk <= 32 ? 32 : 64;
  // a threshold that bounds a merge from below: only a real candidate key
  // (a wave with fewer than topk candidates keeps them all and bounds nothing)
  auto bound = [](uint32_t T) { return T > kNoKey && T != ~0u ? T : 0u; };
  float val[CPL];
  uint32_t key[CPL];
  int tag[CPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = m0 + j * 64 + lane;
    const float x = m < nk ? srow[m] : -INFINITY;
    tag[j] = m < nk ? tag_of(m) : 0;
    val[j] = m < i ? x : -INFINITY;
    key[j] = order_key(val[j]);
    mx = fmaxf(mx, val[j]);
  }
  // this wave's share: positions [m0, min(i, m0 + 64*CPL)); a share of at
  // most topk positions keeps every candidate without a search
  const int share = min(max(i - m0, 0), 64 * CPL);
  {
    uint32_t T;
    int need_eq;
    wave_threshold<CPL, (NW <= 4)>(key, topk, topk < share, T, need_eq);
    const int s0 = wave * seg;
    const int kept = wave_keep(key, T, need_eq, [&](int j, int pos) __attribute__((always_inline)) {
      cval[s0 + pos] = val[j];
      cidx[s0 + pos] = m0 + j * 64 + lane;
      ctag[s0 + pos] = tag[j];
    });
    if (lane >= kept && lane < seg) cval[s0 + lane] = -INFINITY;
    if (lane == 0) thr[wave] = bound(T);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float gmx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) gmx = fmaxf(gmx, red[w]);
  const uint32_t hi = order_key(gmx);   // no candidate's key exceeds it
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) se += expf(val[j] - gmx);   // -inf terms add 0
  se = wave_sum(se);
  if (lane == 0) red[NW + wave] = se;

  // merge of the segments [s_first, s_first + nseg) held in (v, x, g) (R rows
  // of 64 slots): the threshold of their top topk; keep(r, pos) on the lane
  // holding each kept slot, positions ascending
  auto merge = [&]<int R>(const __attribute__((address_space(3))) float* v, int row0, int s_first,
                          int nseg, auto&& keep) __attribute__((always_inline)) {
    float v2[R];
    uint32_t k2[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      v2[r] = v[(row0 + r) * 64 + lane];
      k2[r] = order_key(v2[r]);
    }
    uint32_t lo = 0u;
    for (int s = 0; s < nseg; ++s) lo = max(lo, thr[s_first + s]);
    uint32_t T;
    int need_eq;
    wave_threshold<R, true>(k2, topk, topk < i, T, need_eq, lo, hi);
    const int kept = wave_keep(k2, T, need_eq, [&](int r, int pos) __attribute__((always_inline)) {
      keep(row0 + r, pos, v2[r]);
    });
    return std::make_pair(kept, T);
  };

  if constexpr (NW >= 8) {
    // first level: wave q < 4 merges segments [q*NW/4, (q+1)*NW/4)
    constexpr int G1 = NW / 4;
    if (wave < 4) {
      auto lvl1 = [&]<int R>() __attribute__((always_inline)) {
        const auto kt = merge.template operator()<R>(
            cval, wave * R, wave * G1, G1, [&](int row, int pos, float vv) __attribute__((always_inline)) {
              mval[wave * seg + pos] = vv;
              midx[wave * seg + pos] = cidx[row * 64 + lane];
              mtag[wave * seg + pos] = ctag[row * 64 + lane];
            });
        if (lane >= kt.first && lane < seg) mval[wave * seg + lane] = -INFINITY;
        if (lane == 0) thr[NW + wave] = bound(kt.second);
      };
      if (seg == 32) lvl1.template operator()<G1 / 2>();
      else lvl1.template operator()<G1>();
    }
  }
  __syncthreads();
  if (wave != 0) return 0;
  float gse = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) gse += red[NW + w];
  lse = gmx > -INFINITY ? gmx + logf(gse) : -INFINITY;
  // last level: wave 0 over four segments (of the first level for NW >= 8,
  // of phase A for NW = 4)
  constexpr bool TWO = NW >= 8;
  const __attribute__((address_space(3))) float* v = TWO ? mval : cval;
  const __attribute__((address_space(3))) int* x = TWO ? midx : cidx;
  const __attribute__((address_space(3))) int* g = TWO ? mtag : ctag;
  auto last = [&]<int R>() __attribute__((always_inline)) {
    return merge.template operator()<R>(
               v, 0, TWO ? NW : 0, 4, [&](int row, int pos, float vv) __attribute__((always_inline)) {
                 emit(pos, x[row * 64 + lane], g[row * 64 + lane], log_gate_of(gate, vv, lse));
               })
        .first;
  };
  return seg == 32 ? last.template operator()<2>() : last.template operator()<4>();
}

// The same selection by a workgroup of NW waves, for any topk and rows of up
// to NW*64*CPL candidates (long decode contexts).  Wave w holds the contiguous
// candidates [w*64*CPL, (w+1)*64*CPL), m = w*64*CPL + j*64 + lane, so waves in
// order, then j, then lanes visit m ascending.  The maximum, the exp sum
// (summed in wave order, so the result is deterministic) and every count of
// the threshold search are combined across waves through red, an LDS array of
// at least 6*NW words; each of the 32 search rounds costs one barrier (its
// counts alternate between two slots, so a slot is rewritten only after every
// wave has read it).  Ties at the threshold and output positions follow from
// the per-wave counts of the waves before.  Every thread of the workgroup must
// call it (it contains __syncthreads).
template <int CPL, int NW, class Tag, class Emit>
SAS_DEV int select_row_wg(const float* __restrict__ srow, int nk, int i, int topk, int gate,
                          int wave, int lane, float& lse,
                          __attribute__((address_space(3))) float* red, Tag&& tag_of,
                          Emit&& emit) {
  __attribute__((address_space(3))) int* ired =
      reinterpret_cast<__attribute__((address_space(3))) int*>(red);
  const int m0 = wave * 64 * CPL;
  float val[CPL];
  uint32_t key[CPL];
  int tag[CPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = m0 + j * 64 + lane;
    const float x = m < nk ? srow[m] : -INFINITY;
    tag[j] = m < nk ? tag_of(m) : 0;
    val[j] = m < i ? x : -INFINITY;
    key[j] = order_key(val[j]);
    mx = fmaxf(mx, val[j]);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float gmx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) gmx = fmaxf(gmx, red[w]);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) se += expf(val[j] - gmx);   // -inf terms add 0
  se = wave_sum(se);
  if (lane == 0) red[NW + wave] = se;
  __syncthreads();
  float gse = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) gse += red[NW + w];
  lse = gmx > -INFINITY ? gmx + logf(gse) : -INFINITY;

  uint32_t T = topk > 0 ? kNoKey : ~0u;
  const bool search = topk > 0 && topk < i;   // uniform over the workgroup
  uint32_t th = 0u;   // largest th with at least topk keys >= th
  if (search) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = th | (1u << bit);
      int n = 0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) n += __popcll(__ballot(key[j] >= c));
      const int slot = 2 * NW + (bit & 1) * NW;
      if (lane == 0) ired[slot + wave] = n;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += ired[slot + w];
      if (tot >= topk) th = c;
    }
  }
  // ties are kept only when the search found a candidate threshold (at least
  // topk candidates); per-wave counts above and at it (the waves before this
  // one decide its tie budget and its first output position)
  const bool ties = search && th > kNoKey;
  if (ties) T = th;
  int gt = 0, eqn = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    gt += __popcll(__ballot(key[j] > T));
    eqn += __popcll(__ballot(ties && key[j] == T));
  }
  if (lane == 0) {
    ired[4 * NW + wave] = gt;
    ired[5 * NW + wave] = eqn;
  }
  __syncthreads();
  int n_gt = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n_gt += ired[4 * NW + w];
  const int need_eq = ties ? topk - n_gt : 0;
  int base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w >= wave) break;
    const int e_w = ired[5 * NW + w];
    base += ired[4 * NW + w] + min(e_w, max(0, need_eq - eq_before));
    eq_before += e_w;
  }

  int eq_seen = eq_before;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = m0 + j * 64 + lane;
    const bool eq = ties && key[j] == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = key[j] > T || (eq && eq_seen + mask_rank(eqm) < need_eq);
    eq_seen += __popcll(eqm);
    const uint64_t tm = __ballot(take);
    if (take) emit(base + mask_rank(tm), m, tag[j], log_gate_of(gate, val[j], lse));
    base += __popcll(tm);
  }
  return n_gt + need_eq;
}

// candidates per lane for history rows of up to nkb blocks
inline int select_cpl(int nkb) {
  const int need = (nkb + 63) / 64;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 16 ? 16 : 32;
}

}  // namespace sas
