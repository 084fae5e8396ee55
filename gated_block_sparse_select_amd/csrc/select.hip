// LSE-normalised Top-K block selection (SAS review page, paper.oopus.info:
// §2.2 keeps the Top-K history blocks by selector score, §2.4 sets
// log g_m = s_m - LSE(s over all history blocks)).
//
// One wave64 per score row.  Candidates m < i sit in registers, CPL per lane
// with m = j*64 + lane, so scanning j ascending and lanes ascending visits m in
// ascending order.  Each candidate gets a 32-bit order-preserving key of its
// float value (-0.0 canonicalised to +0.0); a 32-step bitwise search with wave
// population counts (ballots, so the counting stays in scalar registers)
// finds the K-th largest key T exactly; all keys > T are
// kept, and keys == T are kept lowest index first until K blocks are chosen.
// The kept blocks are then compacted in ascending order with ballots.  Every
// comparison is on the exact float bits, so the result is bit-identical to a
// sort by (score desc, index asc).
#include "common.h"
#include "launch.h"

namespace sas {

SAS_DEV uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CPL>
__global__ void __launch_bounds__(64) select_kernel(const float* __restrict__ s,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ cnt,
                                                     float* __restrict__ lg,
                                                     float* __restrict__ slse, int rows,
                                                     int nqb, int nkb, int topk,
                                                     const int32_t* __restrict__ seq_lens,
                                                     int hkv, int cap) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  int i;
  if (seq_lens) {
    int L = seq_lens[row / hkv];
    L = L < 1 ? 1 : (L > cap ? cap : L);
    i = (L - 1) / SAS_BLK;
  } else {
    i = row % nqb;
  }
  const float* srow = s + size_t(row) * nkb;

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
  const float lse = (i > 0) ? mx + logf(se) : -INFINITY;

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

  int32_t* irow = idx ? idx + size_t(row) * topk : nullptr;
  float* grow = lg ? lg + size_t(row) * topk : nullptr;
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
    if (take) {
      const int pos = base + mask_rank(tm);
      irow[pos] = m;
      grow[pos] = val[j] - lse;
    }
    base += __popcll(tm);
  }
  for (int p = keff + lane; p < topk; p += 64) {
    irow[p] = -1;
    grow[p] = -INFINITY;
  }
  if (lane == 0) {
    cnt[row] = keff;
    slse[row] = lse;
  }
}

template <int CPL>
static void go(const float* s, int32_t* idx, int32_t* cnt, float* lg, float* slse, int rows,
               int nqb, int nkb, int topk, const int32_t* sl, int hkv, int cap, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel<CPL>, dim3(rows), dim3(64), 0, st, s, idx, cnt, lg, slse, rows,
                     nqb, nkb, topk, sl, hkv, cap);
}

hipError_t launch_select(const float* s, int32_t* idx, int32_t* cnt, float* lg, float* slse,
                         int rows, int nqb, int nkb, int topk, const int32_t* seq_lens, int hkv,
                         int cap, hipStream_t st) {
  ProfScope ps("sas_select_kernel", st);
  // candidates per lane: history length is at most nkb (training) / nkb (decode)
  const int need = (nkb + 63) / 64;
  if (need <= 1) go<1>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, st);
  else if (need <= 2) go<2>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, st);
  else if (need <= 4) go<4>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, st);
  else if (need <= 8) go<8>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, st);
  else if (need <= 16) go<16>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, st);
  else go<32>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, st);
  return hipGetLastError();
}

}  // namespace sas
