// bf16 matrix-core forward of SAS gated block-sparse attention (gfx950).
//
//   o = softmax(tau q K_S^T + log g_S) V_S     (SAS review page, paper.oopus.info,
//                                               §2.3 equation; §2.6 fused kernel)
// over the kept history blocks (bias = log-gate) and the causally masked current
// block (bias 0, g_0 = 1 per §2.4).
//
// Workgroup = one (batch, kv-head, 64-query block) and up to 4 query heads of
// that group (GQA: the heads share the K/V tiles in LDS).  Two waves per head,
// 32 query rows each, so every SIMD holds two waves and one wave's softmax
// (VALU) runs while the other's matrix-core work proceeds.
//   S^T = K Q^T   (A = K tile rows from LDS, B = Q rows held in registers),
//   so each lane owns one query row: row max / sum need a single lane swap;
//   O^T += V^T P^T (A = V tile read transposed from LDS, B = P from registers).
// K/V tiles are double-buffered in LDS; the next tile's global loads are in
// flight while the current one is computed.  Softmax runs in the exp2 domain.
// Workgroups are issued largest q-block first (most tiles first).
//
// Block tables (packed documents of any length): each block is a 64-row
// window of the token axis of which rows [lo, hi) are the block's own
// tokens (block_geo).  Kept history blocks are whole blocks; on the current
// block, key j is visible from row t iff lo <= j <= t; rows outside [lo, hi)
// are computed but not stored.
//
// EXT (the external gate, g scales the values after an unbiased softmax):
// the kernel is the same with the log-gate kept as the tile's exponent
// offset, so the weights P g reach the PV product unchanged, and the tile's
// weight sum is multiplied by 1/g before it joins the normaliser, which then
// sums the unbiased weights: O / l = sum g P v / sum P.
#include <type_traits>
#include <utility>

#include "launch.h"
#include "mfma_common.h"
#include "sas.h"

namespace sas {

template <int D, int GC, bool EXT>
__global__ void __launch_bounds__(128 * GC) fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const float* __restrict__ lg, uint16_t* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int n, int topk, float tau2, int BH, int h_off,
    int hchunks, const int32_t* __restrict__ geo, int nqb) {
  // A one-head workgroup has only two waves: with two stages (64 KB of LDS at
  // d = 128 instead of 96 KB) two of them fit on a CU, so all four SIMDs work.
  constexpr int NS = GC == 1 ? 2 : kFwdStages;
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;           // bytes of one 64 x D tile
  constexpr int JT = TB / 1024;           // 1 KB DMA slices per tile
  constexpr int JW = 2 * JT / (2 * GC);   // slices per wave per stage (K and V)
  static_assert((2 * JT) % (2 * GC) == 0 && JT % JW == 0, "slices must split evenly over the waves");
  constexpr int TK = 100, TV = 101;       // LDS buffer tags: K tiles, V tiles

  const int G = Hq / Hkv;
  int bid = blockIdx.x;
  const int hc = bid % hchunks;
  bid /= hchunks;
  const int bk = bid % BH;
  const int i = nqb - 1 - bid / BH;
  const int b = bk / Hkv, kv = bk % Hkv;
  const BlockGeo gi = block_geo(geo, b, nqb, n, i);
  if (gi.hi == gi.lo) return;   // a padding block holds no token (uniform exit)
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int h = kv * G + h_off + hc * GC + (wave >> 1);
  const int rt = wave & 1;
  const bool row_ok = rt * 32 + lr >= gi.lo && rt * 32 + lr < gi.hi;
  const size_t rowsel = size_t(bk) * nqb + i;
  const int c_sel = cnt[rowsel];
  const int ntiles = c_sel + 1;
  const int32_t* irow = idx + rowsel * topk;
  const float* grow = lg + rowsel * topk;

  const size_t qrow = (size_t(b) * Hq + h) * n + size_t(gi.w) + rt * 32 + lr;
  bf16x8 qop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qop[c] = *reinterpret_cast<const bf16x8*>(q + qrow * D + c * 16 + hh * 8);

  const size_t kv0 = (size_t(b) * Hkv + kv) * size_t(n);
  // tile t -> ring stage BUF: K and V of block idx[t] (or the current block)
  // the first half of the waves move K slices, the others V slices (JW
  // divides JT, so no wave straddles the two)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bool k_side = wv * JW < JT;
  const int slice0 = (wv * JW) % JT;
  uint32_t pat[4];
  dma_lane_pattern<D>(lane, slice0, pat);
  auto issue = [&]<int BUF>(int t) __attribute__((always_inline)) {
    const int w0 = t < c_sel ? (geo ? block_geo(geo, b, nqb, n, irow[t]).w : irow[t] * SAS_BLK)
                             : gi.w;
    const uint16_t* src = (k_side ? k : v) + (kv0 + size_t(w0)) * D;
    dma_slices<JW>(src, k_side ? stage_buf<TK, BUF, TB>() : stage_buf<TV, BUF, TB>(), slice0, pat);
  };
  issue.template operator()<0>(0);
  if constexpr (NS > 2) {
    if (1 < ntiles) issue.template operator()<1>(1);
  }

  uint32_t ko[D / 16], vo[D / 32][2];
  {
    int koff[D / 16], voff[D / 32][2];
    row_offsets<D>(lane, koff);
    tr_offsets<D>(lane, voff);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) ko[c] = lane_off(koff[c]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) vo[dt][w] = lane_off(voff[dt][w]);
  }

  // Running row max in the exp2 domain.  It is raised only when a tile's max
  // exceeds it by more than kRescaleSlack (wave-uniform decision), so most
  // tiles skip the O rescale; weights stay below 2^kRescaleSlack, and the
  // final O / l is exact whatever max was used.
  constexpr float kRescaleSlack = 8.0f;
  float mrow = -INFINITY, lrow = 0.f;
  f32x16 O[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) O[dt][j] = 0.f;

  // one tile from ring stage ST; CUR: the causal current block
  auto tile = [&]<int ST, bool CUR>(int t) __attribute__((always_inline)) {
    lds_cchar* Kt = stage_buf<TK, ST, TB>();
    lds_cchar* Vt = stage_buf<TV, ST, TB>();
    const float bias2 = CUR ? 0.f : (EXT ? fmaxf(grow[t], kMinExtLogGate) : grow[t]) * kLog2e;

    f32x16 S[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) S[kt][j] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        S[kt] = mfma32(ld16(Kt + kt * 32 * ROWB, ko[c]), qop[c], S[kt]);
    }
    // K-chunk reads run 4 products ahead of the products that use them
#pragma unroll
    for (int x = 0; x < 4; ++x) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int x = 0; x < D / 8 - 4; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (CUR) {  // causal mask of the current block: key j visible iff lo <= j <= row
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kt * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (key > rt * 32 + lr || key < gi.lo) S[kt][j] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, S[kt][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * tau2 + bias2;   // tau2 > 0: max commutes with the affine map
    if (__any(mt > mrow + kRescaleSlack)) {
      const float mnew = fmaxf(mrow, mt);
      const float alpha = fast_exp2(mrow - mnew);
      mrow = mnew;
      lrow *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) O[dt][j] *= alpha;
    }
    const float c0 = bias2 - mrow;
    bf16x8 P[4];
    float ts = 0.f;   // EXT: this tile's weight sum
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int jc = 0; jc < 2; ++jc) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(S[kt][8 * jc + e], tau2, c0));
        P[kt * 2 + jc] = pack_bf16x8(p);
        // normalise by the weights actually used
        if constexpr (EXT) ts = sum_bf16x8(P[kt * 2 + jc], ts);
        else lrow = sum_bf16x8(P[kt * 2 + jc], lrow);
      }
    if constexpr (EXT) lrow = __builtin_fmaf(ts, fast_exp2(-bias2), lrow);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        O[dt] = mfma32(ldtr_pair(Vt + ch * 16 * ROWB, vo[dt][0], vo[dt][1]), P[ch], O[dt]);
    // transposed V reads run 4 products ahead
#pragma unroll
    for (int x = 0; x < 8; ++x) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int x = 0; x < D / 8 - 4; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // kept tile t in stage ST: its DMA landed (and the stage it refills is free)
  // after the wait + barrier; then the tile NS-1 ahead is put in flight
  auto kept = [&]<int ST>(int t) __attribute__((always_inline)) {
    vm_wait_barrier<JW * (NS - 2)>();
    if (t + NS - 1 < ntiles) issue.template operator()<(ST + NS - 1) % NS>(t + NS - 1);
    tile.template operator()<ST, false>(t);
  };

  int t = 0;
#pragma nounroll
  for (; t + NS <= c_sel; t += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      (kept.template operator()<S>(t + S), ...);
    }(std::make_integer_sequence<int, NS>{});
  // t % NS == 0 here; finish the kept tiles, then the current block
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((t + S < c_sel ? kept.template operator()<S>(t + S) : void()), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
  vm_wait_barrier<0>();
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((c_sel % NS == S ? tile.template operator()<S, true>(c_sel) : void()), ...);
  }(std::make_integer_sequence<int, NS>{});

  lrow += __shfl_xor(lrow, 32);
  if (!row_ok) return;   // a window row of another block (no barrier follows)
  const float inv = 1.f / lrow;
  uint16_t* orow = o + qrow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(O[dt][4 * jg + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * jg + 4 * hh) = r;
    }
  if (hh == 0) lse[qrow] = (mrow + log2f(lrow)) * kLn2;
}

bool mfma_supported(int d, int G) { return (d == 64 || d == 128) && G >= 1 && G <= 16; }

template <int D, int GC>
static void fwd_launch(int nblocks, const void* q, const void* k, const void* v,
                       const int32_t* idx, const int32_t* cnt, const float* lg, void* o, float* lse,
                       int Hq, int Hkv, int n, int topk, float tau2, int BH, int h_off,
                       int hchunks, bool ext, const int32_t* geo, int nqb, hipStream_t st) {
  if (ext)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, GC, true>), dim3(nblocks), dim3(128 * GC), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, cnt, lg,
                       (uint16_t*)o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, geo, nqb);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<D, GC, false>), dim3(nblocks), dim3(128 * GC), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, cnt, lg,
                       (uint16_t*)o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, geo, nqb);
}

template <int D>
static void fwd_dispatch(int gc, int nblocks, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* cnt, const float* lg, void* o,
                         float* lse, int Hq, int Hkv, int n, int topk, float tau2, int BH,
                         int h_off, int hchunks, bool ext, const int32_t* geo, int nqb,
                         hipStream_t st) {
  switch (gc) {
    case 1: fwd_launch<D, 1>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, ext, geo, nqb, st); break;
    case 2: fwd_launch<D, 2>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, ext, geo, nqb, st); break;
    default: fwd_launch<D, 4>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, ext, geo, nqb, st); break;
  }
}

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* cnt, const float* lg, void* o, float* lse, int B,
                           int Hq, int Hkv, int n, int d, int topk, float tau, int gate,
                           const int32_t* geo, int nqb, hipStream_t st) {
  ProfScope ps("sas_fwd_mfma_kernel", st);
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const int G = Hq / Hkv;
  const int BH = B * Hkv;
  const float tau2 = tau * kLog2e;
  // heads in chunks of 4, then 2, then 1 (each launch covers hchunks chunks)
  for (const HeadChunks& hc : head_chunks(G)) {
    if (d == 128) fwd_dispatch<128>(hc.gc, BH * nqb * hc.count, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, hc.h_off, hc.count, ext, geo, nqb, st);
    else fwd_dispatch<64>(hc.gc, BH * nqb * hc.count, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, hc.h_off, hc.count, ext, geo, nqb, st);
  }
  return hipGetLastError();
}

}  // namespace sas
