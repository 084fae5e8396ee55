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
// result is bit-identical to a sort by (score desc, index asc).
#pragma once

#include "common.h"

namespace sas {

SAS_DEV uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selects min(topk, i) of the blocks m < i of srow.  emit(pos, m, log_gate)
// is called by the lane holding the pos-th kept block (pos ascending with m).
// Returns the number kept (wave-uniform); lse receives LSE(srow[0..i)), -inf
// for i == 0.
template <int CPL, class Emit>
SAS_DEV int select_row(const float* __restrict__ srow, int i, int topk, int lane, float& lse,
                       Emit&& emit) {
  float val[CPL];
  uint32_t key[CPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = j * 64 + lane;
    const bool ok = m < i;
    val[j] = ok ? srow[m] : -INFINITY;
    key[j] = ok ? order_key(val[j]) : 0u;  // 0 is below every finite key
    mx = fmaxf(mx, val[j]);
  }
  mx = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    if (j * 64 + lane < i) se += expf(val[j] - mx);
  se = wave_sum(se);
  lse = (i > 0) ? mx + logf(se) : -INFINITY;

  const int keff = topk < i ? topk : i;
  uint32_t T = 0u;  // keep every valid key when keff == i
  int need_eq = 0;
  if (keff < i && keff > 0) {
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
    } else if (keff == i) {
      take = m < i;
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
