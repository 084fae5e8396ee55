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

#include "common.h"

namespace sas {

SAS_DEV uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selects min(topk, candidates) of the blocks m < i of srow.  emit(pos, m,
// log_gate) is called by the lane holding the pos-th kept block (pos
// ascending with m).  Returns the number kept (wave-uniform); lse receives
// the LSE over the candidates, -inf if there is none.
template <int CPL, class Emit>
SAS_DEV int select_row(const float* __restrict__ srow, int i, int topk, int lane, float& lse,
                       Emit&& emit) {
  float val[CPL];
  uint32_t key[CPL];
  float mx = -INFINITY;
  int nc = 0;   // candidates: m < i with a finite score
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = j * 64 + lane;
    val[j] = m < i ? srow[m] : -INFINITY;
    const bool ok = val[j] > -INFINITY;
    key[j] = ok ? order_key(val[j]) : 0u;  // 0 is below every candidate's key
    nc += __popcll(__ballot(ok));
    mx = fmaxf(mx, val[j]);
  }
  mx = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    if (key[j] != 0u) se += expf(val[j] - mx);
  se = wave_sum(se);
  lse = nc > 0 ? mx + logf(se) : -INFINITY;

  const int keff = topk < nc ? topk : nc;
  uint32_t T = 0u;  // every candidate is kept when keff == nc
  int need_eq = 0;
  if (keff < nc && keff > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      int n_ge = 0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) n_ge += __popcll(__ballot(key[j] >= c));
      if (n_ge >= keff) T = c;
    }
    int n_gt = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) n_gt += __popcll(__ballot(key[j] > T));
    need_eq = keff - n_gt;
  }

  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = j * 64 + lane;
    bool take;
    if (keff == 0) {
      take = false;
    } else if (keff == nc) {
      take = key[j] != 0u;
    } else {
      const bool eq = key[j] == T;
      const uint64_t eqm = __ballot(eq);
      take = key[j] > T || (eq && eq_seen + mask_rank(eqm) < need_eq);
      eq_seen += __popcll(eqm);
    }
    const uint64_t tm = __ballot(take);
    if (take) emit(base + mask_rank(tm), m, val[j] - lse);
    base += __popcll(tm);
  }
  return keff;
}

// The same selection by a workgroup of NW waves, for rows of up to
// NW*64*CPL candidates (long decode contexts).  Wave w holds the contiguous
// candidates [w*64*CPL, (w+1)*64*CPL), m = w*64*CPL + j*64 + lane, so waves in
// order, then j, then lanes visit m ascending.  The maximum, the exp sum
// (summed in wave order, so the result is deterministic) and every count of
// the threshold search are combined across waves through red, an LDS array of
// at least 7*NW words; each of the 32 search rounds costs one barrier (its
// counts alternate between two slots, so a slot is rewritten only after every
// wave has read it).  Ties at the threshold and output positions follow from
// the per-wave counts of the waves before.  Every thread of the workgroup must
// call it (it contains __syncthreads).
template <int CPL, int NW, class Emit>
SAS_DEV int select_row_wg(const float* __restrict__ srow, int i, int topk, int wave, int lane,
                          float& lse, __attribute__((address_space(3))) float* red, Emit&& emit) {
  __attribute__((address_space(3))) int* ired =
      reinterpret_cast<__attribute__((address_space(3))) int*>(red);
  const int m0 = wave * 64 * CPL;
  float val[CPL];
  uint32_t key[CPL];
  float mx = -INFINITY;
  int ncw = 0;   // this wave's candidates (m < i, finite score)
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = m0 + j * 64 + lane;
    val[j] = m < i ? srow[m] : -INFINITY;
    const bool ok = val[j] > -INFINITY;
    key[j] = ok ? order_key(val[j]) : 0u;
    ncw += __popcll(__ballot(ok));
    mx = fmaxf(mx, val[j]);
  }
  mx = wave_max(mx);
  if (lane == 0) {
    red[wave] = mx;
    ired[6 * NW + wave] = ncw;
  }
  __syncthreads();
  float gmx = -INFINITY;
  int nc = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    gmx = fmaxf(gmx, red[w]);
    nc += ired[6 * NW + w];
  }
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    if (key[j] != 0u) se += expf(val[j] - gmx);
  se = wave_sum(se);
  if (lane == 0) red[NW + wave] = se;
  __syncthreads();
  float gse = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) gse += red[NW + w];
  lse = nc > 0 ? gmx + logf(gse) : -INFINITY;

  const int keff = topk < nc ? topk : nc;
  uint32_t T = 0u;
  int need_eq = 0;
  const bool search = keff < nc && keff > 0;   // uniform over the workgroup
  if (search) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      int n = 0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) n += __popcll(__ballot(key[j] >= c));
      const int slot = 2 * NW + (bit & 1) * NW;
      if (lane == 0) ired[slot + wave] = n;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += ired[slot + w];
      if (tot >= keff) T = c;
    }
  }
  // per-wave counts above and at the threshold (waves before this one decide
  // its tie budget and its first output position)
  int gt = 0, eqn = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    gt += __popcll(__ballot(key[j] > T));
    eqn += __popcll(__ballot(search && key[j] == T));
  }
  if (lane == 0) {
    ired[4 * NW + wave] = gt;
    ired[5 * NW + wave] = eqn;
  }
  __syncthreads();
  int n_gt = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n_gt += ired[4 * NW + w];
  if (search) need_eq = keff - n_gt;
  int base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w >= wave) break;
    const int e_w = ired[5 * NW + w];
    if (keff == nc) {
      base += ired[6 * NW + w];
    } else if (search) {
      base += ired[4 * NW + w] + min(e_w, max(0, need_eq - eq_before));
    }
    eq_before += e_w;
  }

  int eq_seen = eq_before;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = m0 + j * 64 + lane;
    bool take;
    if (keff == 0) {
      take = false;
    } else if (keff == nc) {
      take = key[j] != 0u;
    } else {
      const bool eq = key[j] == T;
      const uint64_t eqm = __ballot(eq);
      take = key[j] > T || (eq && eq_seen + mask_rank(eqm) < need_eq);
      eq_seen += __popcll(eqm);
    }
    const uint64_t tm = __ballot(take);
    if (take) emit(base + mask_rank(tm), m, val[j] - lse);
    base += __popcll(tm);
  }
  return keff;
}

// candidates per lane for history rows of up to nkb blocks
inline int select_cpl(int nkb) {
  const int need = (nkb + 63) / 64;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 16 ? 16 : 32;
}

}  // namespace sas
