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

// Selects min(topk, candidates) of the blocks m < i of srow.  emit(pos, m,
// log_gate) is called by the lane holding the pos-th kept block (pos
// ascending with m), with the log-gate of the gate kind.  Returns the number kept (wave-uniform); lse receives
// the LSE over the candidates, -inf if there is none.
//
// Non-candidates (m >= i or a score of -inf) carry key kNoKey, below every
// candidate's key, so the search ends with T <= kNoKey exactly when fewer
// than topk candidates exist, and then every key > kNoKey is kept.  The number kept is the
// running output position, so no separate candidate count is needed.
template <int CPL, class Emit>
SAS_DEV int select_row(const float* __restrict__ srow, int i, int topk, int gate, int lane,
                       float& lse, Emit&& emit) {
  float val[CPL];
  uint32_t key[CPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = j * 64 + lane;
    val[j] = m < i ? srow[m] : -INFINITY;
    key[j] = order_key(val[j]);
    mx = fmaxf(mx, val[j]);
  }
  mx = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) se += expf(val[j] - mx);   // -inf terms add 0
  se = wave_sum(se);
  lse = mx > -INFINITY ? mx + logf(se) : -INFINITY;

  // keep keys > T, then keys == T lowest index first until need_eq are kept;
  // topk == 0 keeps nothing (no key exceeds ~0), topk >= i every candidate
  uint32_t T = topk > 0 ? kNoKey : ~0u;
  int need_eq = 0;
  if (topk > 0 && topk < i) {
    uint32_t th = 0u;   // largest th with at least topk keys >= th
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = th | (1u << bit);
      int n_ge = 0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) n_ge += __popcll(__ballot(key[j] >= c));
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

  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = j * 64 + lane;
    const bool eq = key[j] == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = key[j] > T || (eq && eq_seen + mask_rank(eqm) < need_eq);
    eq_seen += __popcll(eqm);
    const uint64_t tm = __ballot(take);
    if (take) emit(base + mask_rank(tm), m, log_gate_of(gate, val[j], lse));
    base += __popcll(tm);
  }
  return base;
}

// The same selection by a workgroup of NW waves, for rows of up to
// NW*64*CPL candidates (long decode contexts).  Wave w holds the contiguous
// candidates [w*64*CPL, (w+1)*64*CPL), m = w*64*CPL + j*64 + lane, so waves in
// order, then j, then lanes visit m ascending.  The maximum, the exp sum
// (summed in wave order, so the result is deterministic) and every count of
// the threshold search are combined across waves through red, an LDS array of
// at least 6*NW words; each of the 32 search rounds costs one barrier (its
// counts alternate between two slots, so a slot is rewritten only after every
// wave has read it).  Ties at the threshold and output positions follow from
// the per-wave counts of the waves before.  Every thread of the workgroup must
// call it (it contains __syncthreads).
template <int CPL, int NW, class Emit>
SAS_DEV int select_row_wg(const float* __restrict__ srow, int i, int topk, int gate, int wave,
                          int lane, float& lse, __attribute__((address_space(3))) float* red,
                          Emit&& emit) {
  __attribute__((address_space(3))) int* ired =
      reinterpret_cast<__attribute__((address_space(3))) int*>(red);
  const int m0 = wave * 64 * CPL;
  float val[CPL];
  uint32_t key[CPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int m = m0 + j * 64 + lane;
    val[j] = m < i ? srow[m] : -INFINITY;
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
    if (take) emit(base + mask_rank(tm), m, log_gate_of(gate, val[j], lse));
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
