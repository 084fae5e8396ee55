// bf16 matrix-core backward of SAS gated block-sparse attention (gfx950).
//
// With P = softmax(Z), Z = tau q K^T + bias (log-gate on kept blocks, 0 with
// the causal mask on the current block), O = P V and upstream dO:
//   D = rowsum(dO o O),  dP = dO V^T,  dZ = P o (dP - D),
//   dQ = tau dZ K,  dK = tau sum_h dZ^T Q_h,  dV = sum_h P^T dO_h,
//   dlg[i, m] = sum over the group's heads, rows of q-block i and keys of
//               block m of dZ  (the block gate gradient of the SAS review
//               page, paper.oopus.info, §2.6),
//   ds[i, m] = [m kept] dlg[i, m] - pi_i[m] sum_{kept m'} dlg[i, m'],
//               pi_i = softmax of s[i, :] over the row's candidates (m < i,
//               finite score)  (chain rule through §2.4); with the sigmoid
//               gate, ds[i, m] = [m kept] dlg[i, m] sigmoid(-s[i, m]).
//
// Three kernels:
//  * dq kernel, q-block outer (same workgroup shape and tile pipeline as the
//    forward): recomputes S^T and dP^T per kept tile, accumulates dQ^T =
//    K^T dZ^T, writes D for the key-outer kernel and the per-tile dZ sums
//    (per head chunk) for the gate Jacobian.
//  * ds kernel: sums the head-chunk partials in a fixed order and applies the
//    gate Jacobian to one score row per workgroup.
//  * dk/dv kernel, key-block outer: one workgroup per (batch, kv-head, key
//    block) walks the reverse list of q-blocks that read the block (its own
//    current block first) for every head of the group, with dK and dV held in
//    registers - no atomics, so the result is deterministic.
// The split recomputes S and dP in both passes (7 tile products instead of 5)
// in exchange for no atomics and no per-pair partial buffers.
//
// Block tables (packed documents of any length, block_geo): a block is a
// 64-row window whose rows [lo, hi) are its own tokens.  The dq kernel
// zeroes dZ on the other rows of a q-block's window and gives them the
// statistics (-inf, 0), so the key-outer kernel's weights there are 0; only
// a block's own rows (dq) and keys (dk, dv) are stored.
//
// EXT, the external gate (g scales block m's values after an unbiased
// softmax): with P_b = g P, the weight the forward's PV product used,
//   dV = sum_h P_b^T dO_h,  dZ = P (g dP - D) = P_b (dP - D/g),
//   dlg[i, m] = sum over block m of P g dP = sum of P_b dP,
// so the kernels keep the log-gate as the tile's exponent offset and only
// replace D by D/g (and, in the dq kernel, sum P_b dP for the gate).
#include <type_traits>
#include <utility>

#include "launch.h"
#include "mfma_common.h"
#include "sas.h"

namespace sas {

// ------------------------------------------------------------------ dq kernel
template <int D, int GC, bool EXT>
__global__ void __launch_bounds__(128 * GC) bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ lg, uint16_t* __restrict__ dq, float* __restrict__ stats,
    float* __restrict__ dlgp, int Hq, int Hkv, int n, int topk, float tau, float tau2, int BH,
    int h_off, int hchunks, int nch, int chunk0, const int32_t* __restrict__ geo, int nqb) {
  constexpr int NS = kDqStages;
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;
  constexpr int JT = TB / 1024;
  constexpr int JW = 2 * JT / (2 * GC);
  static_assert((2 * JT) % (2 * GC) == 0 && JT % JW == 0, "slices must split evenly over the waves");
  constexpr int TK = 200, TV = 201;       // LDS buffer tags: K tiles, V tiles
  __shared__ float part[2][8];            // per-wave dZ sums of the last two tiles

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
  const int chunk = chunk0 + hc;
  const size_t rowsel = size_t(bk) * nqb + i;
  const int c_sel = cnt[rowsel];
  const int ntiles = c_sel + 1;
  const int32_t* irow = idx + rowsel * topk;
  const float* grow = lg + rowsel * topk;

  const size_t qrow = (size_t(b) * Hq + h) * n + size_t(gi.w) + rt * 32 + lr;
  bf16x8 qop[D / 16], dop[D / 16];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const size_t off = qrow * D + c * 16 + hh * 8;
    qop[c] = *reinterpret_cast<const bf16x8*>(q + off);
    dop[c] = *reinterpret_cast<const bf16x8*>(dO + off);
    const bf16x8 oo = *reinterpret_cast<const bf16x8*>(o + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart += float(dop[c][e]) * float(oo[e]);
  }
  // rows of the window outside the block: o and lse there belong to other
  // blocks (or to no block), so their D and lse are replaced by 0
  const float Drow = row_ok ? dpart + __shfl_xor(dpart, 32) : 0.f;
  const float lse_r = row_ok ? lse[qrow] : 0.f;
  const float lse2 = lse_r * kLog2e;
  if (hh == 0) {
    // per-row statistics of this (head, q-block) for the key-block-outer pass:
    // [-lse / tau for the 64 rows | -D for the 64 rows]; (-inf, 0) outside the
    // block, so the weights there are 0
    float* st = stats + ((size_t(b) * Hq + h) * nqb + i) * 128;
    st[rt * 32 + lr] = row_ok ? -lse_r / tau : -INFINITY;
    st[64 + rt * 32 + lr] = -Drow;
  }

  const size_t kv0 = (size_t(b) * Hkv + kv) * size_t(n);
  // the first half of the waves move K slices, the others V slices
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

  uint32_t ko[D / 16], to[D / 32][2];
  {
    int koff[D / 16], toff[D / 32][2];
    row_offsets<D>(lane, koff);
    tr_offsets<D>(lane, toff);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) ko[c] = lane_off(koff[c]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) to[dt][w] = lane_off(toff[dt][w]);
  }

  f32x16 dQ[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) dQ[dt][j] = 0.f;

  // one tile from ring stage ST; CUR = the causal current block
  auto tile = [&]<int ST, bool CUR>(int t) __attribute__((always_inline)) {
    lds_cchar* Kt = stage_buf<TK, ST, TB>();
    lds_cchar* Vt = stage_buf<TV, ST, TB>();
    const float bias2 = CUR ? 0.f : (EXT ? fmaxf(grow[t], kMinExtLogGate) : grow[t]) * kLog2e;
    const float zoff = bias2 - lse2;
    const float Dg = EXT ? Drow * fast_exp2(-bias2) : 0.f;   // EXT: D / g
    float zs = 0.f;
    bf16x8 dZp[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {   // one 32-key half at a time
      f32x16 S, P2;
      // dP starts at -D (this lane's row), so the products give dP - D;
      // EXT keeps dP itself (its gate gradient needs it)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        S[j] = 0.f;
        P2[j] = EXT ? 0.f : -Drow;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        S = mfma32(ld16(Kt + kt * 32 * ROWB, ko[c]), qop[c], S);
        P2 = mfma32(ld16(Vt + kt * 32 * ROWB, ko[c]), dop[c], P2);
      }
#pragma unroll
      for (int jc = 0; jc < 2; ++jc) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 8 * jc + e;
          float p = fast_exp2(__builtin_fmaf(S[j], tau2, zoff));
          const int key = kt * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (CUR && (key > rt * 32 + lr || key < gi.lo)) p = 0.f;
          if constexpr (EXT) {
            x[e] = row_ok ? p * (P2[j] - Dg) : 0.f;
            if (!CUR && row_ok) zs = __builtin_fmaf(p, P2[j], zs);
          } else {
            x[e] = row_ok ? p * P2[j] : 0.f;
          }
        }
        dZp[kt * 2 + jc] = pack_bf16x8(x);
        // the block-gate gradient of the dZ used
        if constexpr (!EXT) zs = sum_bf16x8(dZp[kt * 2 + jc], zs);
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        dQ[dt] = mfma32(ldtr_pair(Kt + ch * 16 * ROWB, to[dt][0], to[dt][1]), dZp[ch], dQ[dt]);
    if (!CUR) {
      zs = wave_sum(zs);
      if (lane == 0) part[t & 1][wave] = zs;
    }
  };
  auto publish = [&](int t) __attribute__((always_inline)) {   // gate gradient of tile t
    if (tid == 0) {
      float a = 0.f;
      for (int w = 0; w < 2 * GC; ++w) a += part[t & 1][w];
      dlgp[(rowsel * nch + chunk) * topk + t] = a;
    }
  };
  // kept tile t in stage ST: wait for it (and for the stage it refills to be
  // free), publish the gate gradient of tile t-1, refill, compute
  auto kept = [&]<int ST>(int t) __attribute__((always_inline)) {
    vm_wait_barrier<JW * (NS - 2)>();
    if (t > 0) publish(t - 1);
    if (t + NS - 1 < ntiles) issue.template operator()<(ST + NS - 1) % NS>(t + NS - 1);
    tile.template operator()<ST, false>(t);
  };
  int t = 0;
#pragma nounroll
  for (; t + NS <= c_sel; t += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      (kept.template operator()<S>(t + S), ...);
    }(std::make_integer_sequence<int, NS>{});
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((t + S < c_sel ? kept.template operator()<S>(t + S) : void()), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
  vm_wait_barrier<0>();
  if (c_sel > 0) publish(c_sel - 1);
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((c_sel % NS == S ? tile.template operator()<S, true>(c_sel) : void()), ...);
  }(std::make_integer_sequence<int, NS>{});

  if (!row_ok) return;   // a window row of another block (no barrier follows)
  uint16_t* drow = dq + qrow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(dQ[dt][4 * jg + e] * tau);
      *reinterpret_cast<bf16x4*>(drow + dt * 32 + 8 * jg + 4 * hh) = r;
    }
}

// ------------------------------------------------------------------ ds kernel
// grid: one workgroup (256 threads) per score row (b, kv, i).
__global__ void __launch_bounds__(256) bwd_ds_kernel(const float* __restrict__ dlgp,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ cnt,
                                                     const float* __restrict__ s,
                                                     const float* __restrict__ s_lse,
                                                     float* __restrict__ ds, int nqb, int topk,
                                                     int nch, int gate) {
  __shared__ float dl[2048];      // topk <= 2048
  __shared__ int slot_of[2048];   // blocks per sequence <= 2048
  __shared__ float tot_s;
  const size_t row = blockIdx.x;
  const int i = int(row % nqb);
  const int c = cnt[row];
  for (int sl = threadIdx.x; sl < c; sl += 256) {
    float a = 0.f;
    for (int ch = 0; ch < nch; ++ch) a += dlgp[(row * nch + ch) * topk + sl];
    dl[sl] = a;
  }
  for (int m = threadIdx.x; m < nqb; m += 256) slot_of[m] = -1;
  __syncthreads();
  for (int sl = threadIdx.x; sl < c; sl += 256) slot_of[idx[row * topk + sl]] = sl;
  if (threadIdx.x == 0) {
    float a = 0.f;
    for (int sl = 0; sl < c; ++sl) a += dl[sl];
    tot_s = a;
  }
  __syncthreads();
  const float tot = tot_s;
  const float sl_ = s_lse[row];
  const int hist = sl_ > -INFINITY ? i : 0;   // a row without candidates has no gate
  for (int m = threadIdx.x; m < nqb; m += 256) {
    float val = 0.f;
    if (m < hist) {
      const int sm = slot_of[m];
      if (gate == SAS_GATE_SIGMOID)   // d log sigmoid(s) / ds = sigmoid(-s), no coupling
        val = sm >= 0 ? dl[sm] / (1.f + expf(s[row * nqb + m])) : 0.f;
      else
        val = (sm >= 0 ? dl[sm] : 0.f) - expf(s[row * nqb + m] - sl_) * tot;
    }
    ds[row * nqb + m] = val;
  }
}

// ------------------------------------------------------------------ dk/dv kernel
// grid: nkb*B*Hkv workgroups of 4 waves; wave = (key half kh, row half rh).
// The (q-block, head) steps of the reverse list stream through a ring of
// kKvStages stages, each holding the Q and dO tiles of one (q-block, head) and
// its row statistics [-lse/tau | -D]; the K and V rows of the wave's key half
// stay in registers.  The statistics are the start values of the two
// accumulators, so S = Q K^T - lse/tau (tau2*S + bias2 is the base-2 log of
// P) and dP = dO V^T - D come out of the matrix cores ready for the
// elementwise step.
//
// Each step runs in four phases fenced with sched_barrier: S and dP (LDS
// reads two 16-column chunks ahead of the products that use them), P and dZ
// of rows 0..15 of the wave's 32, the dV/dK products of those rows overlapped
// with P and dZ of rows 16..31, then the dV/dK products of rows 16..31.  The
// list entries (q-block and base-2 log-gate) are staged in LDS first, so the
// loop issues no scalar memory loads (those return out of order and would
// force every LDS wait to drain all outstanding LDS reads).
//
// DZ (the dZ-tile path): each step's bf16 dZ operands are also stored, one
// 8 KB tile per (q-block, kept slot or own block, head), for the dq kernel;
// the own block's step then also masks the window's keys before the block's
// first token, so that the stored tile is exactly the one dq needs.
template <int D, bool EXT, bool DZ>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ stats, const float* __restrict__ lg,
    const int32_t* __restrict__ rev_off, const int32_t* __restrict__ rev_list,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, uint16_t* __restrict__ dz, int Hq,
    int Hkv, int n, int topk, float tau, float tau2, const int32_t* __restrict__ geo, int nkb,
    int pph) {
  static_assert(!(EXT && DZ), "the external gate's dq needs dP itself: no dZ store path");
  constexpr int NS = kKvStages;
  static_assert(NS == 4, "stage arithmetic below assumes a 4-stage ring");
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;
  constexpr int CPR = D / 8;
  constexpr int JT = TB / 1024;
  constexpr int JW = 2 * JT / 4;        // Q + dO slices per wave per step
  constexpr int PER = JW + 1;           // plus the row statistics
  constexpr int TQ = 300, TO = 301, TS = 302, TL = 303;   // LDS buffer tags

  const int G = Hq / Hkv;
  // Grid in phases of pph (batch, kv-head) pairs (pph divides B*Hkv; the
  // host picks the largest whose Q/dO fit the last-level cache, so a phase's
  // re-read tiles stay there); inside a phase, key-block-major: consecutive
  // workgroups take the same key block of consecutive pairs.  Workgroups are
  // dealt round-robin to the XCDs, so an XCD serves the key blocks m, m+1,
  // ... of one or two pairs at a time; their reverse lists walk similar
  // q-block ranges in ascending order, so a Q/dO tile one of them loads is
  // often still in that XCD's L2 when the next needs it.  Each phase starts
  // the longest lists (small m) first.
  const int ph = blockIdx.x / (nkb * pph), pr = blockIdx.x % (nkb * pph);
  const int m = pr / pph;
  const int bk = ph * pph + pr % pph;
  const int b = bk / Hkv, kv = bk % Hkv;
  const BlockGeo gm = block_geo(geo, b, nkb, n, m);
  if (gm.hi == gm.lo) return;   // a padding block holds no token (uniform exit)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int kh = wave & 1, rh = wave >> 1;

  const size_t kvrow0 = (size_t(b) * Hkv + kv) * n + size_t(gm.w);
  const size_t krow = kvrow0 + kh * 32 + lr;
  bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    kop[c] = *reinterpret_cast<const bf16x8*>(k + krow * D + c * 16 + hh * 8);
    vop[c] = *reinterpret_cast<const bf16x8*>(v + krow * D + c * 16 + hh * 8);
  }

  f32x16 dK[D / 32], dV[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      dK[dt][j] = 0.f;
      dV[dt][j] = 0.f;
    }

  // list entries of this key block -> LDS: q-block | (first row of its
  // window << 11) and base-2 log-gate (0 for the own block, entry 0); the
  // window row is below 2^17 and the q-block below 2^11
  __shared__ int2 meta[SAS_MAX_BLOCKS];
  // DZ: the dZ slot of each entry (its place in the q-block's kept list,
  // topk for the own block)
  typedef __attribute__((address_space(3))) int16_t lds_i16;
  lds_i16* mslot = reinterpret_cast<lds_i16*>(stage_buf<TL, 0, DZ ? 2 * SAS_MAX_BLOCKS : 4>());
  const int32_t* lst = rev_list + size_t(bk) * nkb * (topk + 1);
  const int32_t e0 = rev_off[size_t(bk) * (nkb + 1) + m];
  const int32_t e1 = rev_off[size_t(bk) * (nkb + 1) + m + 1];
  for (int e = tid; e < e1 - e0; e += 256) {
    const int32_t ent = lst[e0 + e];
    const int iq = ent & 0xFFFF, slot = (ent >> 16) & 0xFFFF;
    const float l = slot == 0xFFFF ? 0.f : lg[(size_t(bk) * nkb + iq) * topk + slot];
    const float b2 = (EXT ? fmaxf(l, kMinExtLogGate) : l) * kLog2e;
    const int wq = geo ? block_geo(geo, b, nkb, n, iq).w : iq * SAS_BLK;
    meta[e] = make_int2(iq | (wq << 11), __float_as_int(b2));
    if constexpr (DZ) mslot[e] = int16_t(slot == 0xFFFF ? topk : slot);
  }
  __syncthreads();
  const int nsteps = (e1 - e0) * G;
  const int nmain = nsteps - G;

  // DMA cursor: the next step to issue, as (list entry, head).  The first
  // half of the waves move Q slices, the others dO slices; every wave moves
  // the 256 B of row statistics of its row half (lane l: word l%32 of the
  // -lse/tau rows for l < 32, of the -D rows for l >= 32).
  int ie = 0, ih = 0;
  const bool q_side = wave * JW < JT;
  const int slice0 = (wave * JW) % JT;
  const size_t hstride = size_t(n) * D * 2;
  const char* src_base = reinterpret_cast<const char*>(q_side ? q : dO) +
                         (size_t(b) * Hq + kv * G) * hstride;
  const float* st_base = stats + (size_t(b) * Hq + kv * G) * size_t(nkb) * 128 + rh * 32;
  const uint32_t st_lane = uint32_t(((lane >> 5) * 64 + (lane & 31)) * 4);
  uint32_t pat[4];
  dma_lane_pattern<D>(lane, slice0, pat);
  auto issue = [&]<int BUF>() __attribute__((always_inline)) {
    const int ent = __builtin_amdgcn_readfirstlane(meta[ie].x);
    const int iq = ent & 2047;
    const char* tile = src_base + size_t(ih) * hstride + size_t(ent >> 11) * ROWB;
    dma_slices<JW>(tile, q_side ? stage_buf<TQ, BUF, TB>() : stage_buf<TO, BUF, TB>(), slice0, pat);
    __builtin_amdgcn_global_load_lds(
        (glb_void*)(uniform_ptr(st_base + (size_t(ih) * nkb + iq) * 128) + opaque(st_lane)),
        (lds_void*)(stage_buf<TS, BUF, 1024>() + wave * 256), 4, 0, 0);
    if (++ih == G) {
      ih = 0;
      ++ie;
    }
  };
  // wait until the loads of all but the `ahead` most recently issued steps
  // have landed, then barrier
  auto wait_ahead = [&](int ahead) __attribute__((always_inline)) {
    if (ahead >= 2) vm_wait_barrier<2 * PER>();
    else if (ahead == 1) vm_wait_barrier<PER>();
    else vm_wait_barrier<0>();
  };

  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((S < nsteps ? issue.template operator()<S>() : void()), ...);
  }(std::make_integer_sequence<int, NS - 1>{});

  uint32_t qo[D / 16], to[D / 32][2];
  {
    int roff[D / 16], toff[D / 32][2];
    row_offsets<D>(lane, roff);
    tr_offsets<D>(lane, toff);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qo[c] = lane_off(rh * 32 * ROWB + roff[c]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) to[dt][w] = lane_off(rh * 32 * ROWB + toff[dt][w]);
  }
  // statistics of rows rh*32 + 8*jg + 4*hh + 0..3 (16 B per group jg) in this
  // wave's 256 B copy
  const uint32_t so = lane_off(wave * 256 + 4 * hh * 4);
  typedef __attribute__((ext_vector_type(4))) float f32x4;
  typedef const __attribute__((address_space(3))) f32x4 lds_f32x4;

  // P and dZ = P o (dP - D) of row chunk jc as bf16 operands (register
  // j = 8*jc + e holds row rh*32 + 8*(j/4) + 4*hh + j%4 of this lane's key);
  // own-block steps mask the keys above each query row.
  auto elementwise = [&]<int JC>(const f32x16& S, const f32x16& P2, float bias2, bool own,
                                 bf16x8& Pp, bf16x8& Zp) __attribute__((always_inline)) {
    float pv[8], zv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * JC + e;
      float p = fast_exp2(__builtin_fmaf(S[j], tau2, bias2));
      // DZ: also the window's keys before the block (their dZ is stored for dq)
      if (own && (kh * 32 + lr > rh * 32 + 8 * (j >> 2) + 4 * hh + (j & 3) ||
                  (DZ && kh * 32 + lr < gm.lo)))
        p = 0.f;
      pv[e] = p;
      zv[e] = p * P2[j];
    }
    Pp = pack_bf16x8(pv);
    Zp = pack_bf16x8(zv);
  };

  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  // S = Q K^T - lse/tau and dP = dO V^T - D (EXT: - D/g) of the step in
  // stage ST: the statistics seed the accumulators, then the products over
  // the d chunks (row chunks read two ahead).
  auto sdp = [&]<int ST>(float bias2, f32x16& S, f32x16& P2) __attribute__((always_inline)) {
    lds_cchar* Qt = stage_buf<TQ, ST, TB>();
    lds_cchar* Ot = stage_buf<TO, ST, TB>();
    lds_cchar* St = stage_buf<TS, ST, 1024>();
    const float ig = EXT ? fast_exp2(-bias2) : 1.f;
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const f32x4 l4 = *reinterpret_cast<lds_f32x4*>(St + so + jg * 32);
      const f32x4 d4 = *reinterpret_cast<lds_f32x4*>(St + so + 128 + jg * 32);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S[4 * jg + r] = l4[r];
        P2[4 * jg + r] = EXT ? d4[r] * ig : d4[r];
      }
    }
    bf16x8 qa[NC], oa[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qa[c] = ld16(Qt, qo[c]);
      oa[c] = ld16(Ot, qo[c]);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      S = mfma32(qa[c], kop[c], S);
      P2 = mfma32(oa[c], vop[c], P2);
    }
  };
  // transposed Q / dO operands (rows 0..15 and 16..31 of the wave) of the
  // step in stage ST
  auto tr_ops = [&]<int ST>(bf16x8 (&tO)[2][NT], bf16x8 (&tQ)[2][NT]) __attribute__((always_inline)) {
    lds_cchar* Qt = stage_buf<TQ, ST, TB>();
    lds_cchar* Ot = stage_buf<TO, ST, TB>();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        tO[h][dt] = ldtr_pair(Ot + h * 16 * ROWB, to[dt][0], to[dt][1]);
        tQ[h][dt] = ldtr_pair(Qt + h * 16 * ROWB, to[dt][0], to[dt][1]);
      }
  };
  // dV += P^T dO, dK += dZ^T Q over the wave's 32 rows
  auto dvdk = [&](const bf16x8 (&Pp)[2], const bf16x8 (&Zp)[2], const bf16x8 (&tO)[2][NT],
                  const bf16x8 (&tQ)[2][NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        dV[dt] = mfma32(Pp[h], tO[h][dt], dV[dt]);
        dK[dt] = mfma32(Zp[h], tQ[h][dt], dK[dt]);
      }
  };

  // Software pipeline over the steps: iteration s forms P and dZ of step s
  // (vector work on the S / dP accumulated in iteration s - 1) while the
  // matrix cores compute S and dP of step s + 1, then runs the dV/dK
  // products of step s.  The vector work of one step thus overlaps the
  // products of the next instead of waiting for its own.
  //
  // Ring: step s lives in stage s % NS.  Iteration s reads stage s (the
  // transposed operands) and stage s + 1 (statistics and rows); after its
  // barrier, stage s - 1 is free and is refilled with step s + NS - 1.
  // DZ: the dZ tile of (q-block iq, kept slot, head) is the 8 KB at
  //   dz + ((((b*Hkv + kv)*nqb + iq)*(topk + 1) + slot)*G + head) * 8192 B,
  // in this kernel's register order: wave (kh, rh) stores Zp[h] as the 1 KB
  // slice (kh*2 + rh)*2 + h, 16 B per lane in lane order (one contiguous
  // store per slice).  Lane l's 16 B hold key kh*32 + l%32 and rows
  // rh*32 + 16h + 4(l/32) + {0..3} (first 8 B) and + 8 + {0..3} (last 8 B).
  auto ztile = [&](int e, int head) __attribute__((always_inline)) {
    const int iq = __builtin_amdgcn_readfirstlane(meta[e].x) & 2047;
    const int slot = __builtin_amdgcn_readfirstlane(int(mslot[e]));
    return reinterpret_cast<uint16_t*>(const_cast<char*>(uniform_ptr(
        dz + ((((size_t(bk) * nkb + iq) * (topk + 1) + slot) * G + head) << 12))));
  };
  const uint32_t zlane = lane_off((kh * 2 + rh) * 2048 + lane * 16);   // bytes
  // Buffer stores: the tile's base lives in a scalar descriptor (8 KB of
  // records, so no store can leave the tile) and each lane adds one 32-bit
  // offset; the non-temporal policy keeps the stream (8 KB per workgroup and
  // step), read back only by the dq kernel, from displacing the re-read Q/dO
  // tiles.  (A
  // flat store would also count in lgkmcnt and make every LDS wait of the
  // loop wait for it.)
  auto store_dz = [&](uint16_t* zt, const bf16x8 (&Zp)[2]) __attribute__((always_inline)) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(zt, 0, 8192, 0x00020000);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Zp[h]), rs, int(zlane),
                                             h * 1024, 2 /* nt */);
  };
  f32x16 S, P2;
  float bias = 0.f;
  uint16_t* zt = nullptr;   // DZ: dZ tile of step s
  int ce = 0, chd = 0;   // list entry / head of step s + 1 (the next one to start)
  auto advance = [&]() __attribute__((always_inline)) {
    if (++chd == G) {
      chd = 0;
      ++ce;
    }
  };
  // prologue (steps 0 .. NS-2 were issued above): S and dP of step 0, an
  // own-block step (no gate)
  wait_ahead(min(NS - 2, nsteps - 1));
  sdp.template operator()<0>(0.f, S, P2);
  if constexpr (DZ) zt = ztile(0, 0);
  advance();

  // iteration s in stage ST; CHECKED: the ring's end may fall inside
  auto iter = [&]<int ST, bool CHECKED>(int s) __attribute__((always_inline)) {
    constexpr int ST1 = (ST + 1) % NS;
    const bool own = CHECKED && s < G;
    bf16x8 tO[2][NT], tQ[2][NT], Pp[2], Zp[2];
    if (!CHECKED || s + 1 < nsteps) {
      // step s + 1 landed (at most one later step still in flight); every
      // wave is done with stage s - 1
      // (DZ: the two dZ stores of step s - 1 follow step s + 2's DMA, and
      // vmcnt counts loads and stores in issue order; the CHECKED waits are
      // stricter, so they stay correct)
      if (CHECKED) wait_ahead(min(NS - 3, nsteps - 2 - s));
      else vm_wait_barrier<(NS - 3) * PER + (DZ ? 2 : 0)>();
      if (!CHECKED || s + NS - 1 < nsteps) issue.template operator()<(ST + NS - 1) % NS>();
      // base-2 log-gate of step s + 1 (0 for the own block, list entry 0)
      const float bias_n = __int_as_float(meta[ce].y);
      const float bias_s = bias;
      uint16_t* zt_n = DZ ? ztile(ce, chd) : nullptr;
      f32x16 Sn, P2n;
      tr_ops.template operator()<ST>(tO, tQ);
      sdp.template operator()<ST1>(bias_n, Sn, P2n);
      elementwise.template operator()<0>(S, P2, bias_s, own, Pp[0], Zp[0]);
      elementwise.template operator()<1>(S, P2, bias_s, own, Pp[1], Zp[1]);
      // issue order: the matrix products of step s + 1 with the vector work
      // of step s between them
#pragma unroll
      for (int i = 0; i < 2 * NC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      if constexpr (DZ) store_dz(zt, Zp);
      dvdk(Pp, Zp, tO, tQ);
      S = Sn;
      P2 = P2n;
      bias = bias_n;
      zt = zt_n;
      advance();
    } else {
      // last step: nothing further to start
      tr_ops.template operator()<ST>(tO, tQ);
      elementwise.template operator()<0>(S, P2, bias, own, Pp[0], Zp[0]);
      elementwise.template operator()<1>(S, P2, bias, own, Pp[1], Zp[1]);
      if constexpr (DZ) store_dz(zt, Zp);
      dvdk(Pp, Zp, tO, tQ);
    }
  };
  int s = 0;
#pragma nounroll
  for (; s < G; s += NS)
    [&]<int... S_>(std::integer_sequence<int, S_...>) __attribute__((always_inline)) {
      ((s + S_ < nsteps ? iter.template operator()<S_, true>(s + S_) : void()), ...);
    }(std::make_integer_sequence<int, NS>{});
#pragma nounroll
  for (; s + 2 * NS - 1 < nsteps; s += NS)
    [&]<int... S_>(std::integer_sequence<int, S_...>) __attribute__((always_inline)) {
      (iter.template operator()<S_, false>(s + S_), ...);
    }(std::make_integer_sequence<int, NS>{});
#pragma nounroll
  for (; s < nsteps; s += NS)
    [&]<int... S_>(std::integer_sequence<int, S_...>) __attribute__((always_inline)) {
      ((s + S_ < nsteps ? iter.template operator()<S_, true>(s + S_) : void()), ...);
    }(std::make_integer_sequence<int, NS>{});
  __syncthreads();

  // Reduce the two row halves through LDS (float32 [32 keys][D] per key half,
  // in the stage-0 Q / dO buffers), then write coalesced bf16 rows: first dV,
  // then dK (scaled by tau).
  __attribute__((address_space(3))) float* red[2] = {
      reinterpret_cast<__attribute__((address_space(3))) float*>(stage_buf<TQ, 0, TB>()),
      reinterpret_cast<__attribute__((address_space(3))) float*>(stage_buf<TO, 0, TB>())};
  static_assert(32 * D * 4 <= TB, "reduction buffer");
  const size_t out0 = kvrow0 * D;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const f32x16* acc = pass == 0 ? dV : dK;
    __attribute__((address_space(3))) float* rk = red[kh];
    if (rh == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          rk[(8 * (j >> 2) + 4 * hh + (j & 3)) * D + dt * 32 + lr] = acc[dt][j];
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          rk[(8 * (j >> 2) + 4 * hh + (j & 3)) * D + dt * 32 + lr] += acc[dt][j];
    }
    __syncthreads();
    uint16_t* dst = (pass == 0 ? dv : dk) + out0;
    const float sc = pass == 0 ? 1.f : tau;
    for (int c = tid; c < 64 * CPR; c += 256) {
      const int key = c / CPR;
      if (key < gm.lo || key >= gm.hi) continue;   // a window row of another block
      const __attribute__((address_space(3))) float* src = red[key >> 5] + (key & 31) * D + (c % CPR) * 8;
      bf16x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (__bf16)(src[e] * sc);
      *reinterpret_cast<bf16x8*>(dst + c * 8) = r;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ dZ path
// When the workspace holds a dZ tile for every (head, q-block, kept or own
// block), the key-block-outer kernel stores the dZ it forms (bf16, the values
// its dK product uses) and dq becomes one product per tile,
//   dQ_i = tau sum over the tiles of q-block i of dZ_tile K_tile,
// so dq does not form S and dP again: the backward executes five tile
// products (S and dP recomputed once, in the key-outer pass, then dV, dK and
// dQ; review page §2.6) instead of seven.  The row statistics the key-outer
// pass seeds its accumulators with come from a small pass over o and dO
// (bwd_stats.h), launched with the reverse lists (revidx.hip).

// grid: (batch, kv-head, q-block i, head chunk) as the dq kernel; 2*GC waves,
// wave w = query head w/2 of the chunk and half w%2 of the d columns, all 64
// rows of the window (two waves per SIMD, so one wave's LDS reads overlap the
// other's products).  Per tile (kept blocks in list order, then the own
// block) a ring stage holds the K tile (shared by the chunk's heads) and each
// head's dZ tile; dQ^T += K^T dZ^T with both operands read transposed from
// LDS.  The dZ tile arrives in the key-outer kernel's register order (8-byte
// pieces of one key and four consecutive rows); each lane of a
// DS_READ_B64_TR_B16 names the piece its 4 x 4 transpose needs, so the
// operand comes out as 8 keys of one row.  On the way into LDS, 16-byte chunk
// c of every 1 KB slice moves to c ^ ((c >> 5) << 3), so that the 64 pieces of
// one read fall in distinct 8-byte bank slots two lanes at a time.  The sum
// of each kept tile's dZ over the chunk's heads is the block-gate gradient
// partial the ds kernel reads (review page §2.6).
constexpr int kDqzStages = 3;
template <int D, int GC>
__global__ void __launch_bounds__(128 * GC) bwd_dqz_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ dz,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, uint16_t* __restrict__ dq,
    float* __restrict__ dlgp, int Hq, int Hkv, int n, int topk, int K, float tau, int BH,
    int h_off, int hchunks, int nch, int chunk0, const int32_t* __restrict__ geo, int nqb) {
  constexpr int NS = kDqzStages;
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;
  constexpr int JT = TB / 1024;
  constexpr int JWK = JT / (2 * GC);      // K slices per wave
  constexpr int ZB = 64 * 64 * 2;         // bytes of a dZ tile
  constexpr int JWZ = ZB / 1024 / 2;      // dZ slices per wave (half its head's tile)
  constexpr int PER = JWK + JWZ;          // DMA instructions per wave per tile
  constexpr int DT = D / 64;              // 32-column d tiles per wave
  static_assert(JT % (2 * GC) == 0, "K slices must split evenly over the waves");
  constexpr int TK = 400, TZ = 401;       // LDS buffer tags
  __shared__ float part[2][GC];           // per-head dZ sums of the last two tiles

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int hw = wave >> 1, dh = wave & 1;   // head of the chunk, d half
  const int hg = h_off + hc * GC + hw;       // head within the group
  const int h = kv * G + hg;
  const int chunk = chunk0 + hc;
  const size_t rowsel = size_t(bk) * nqb + i;
  const int c_sel = cnt[rowsel];
  const int ntiles = c_sel + 1;
  const int32_t* irow = idx + rowsel * K;
  const uint16_t* zrow = dz + ((rowsel * size_t(topk + 1) * G + hg) << 12);
  const size_t zstride = size_t(G) << 12;   // between the slots of one head

  const size_t kv0 = (size_t(b) * Hkv + kv) * size_t(n);
  const int slice0 = wave * JWK;
  uint32_t patk[4];
  dma_lane_pattern<D>(lane, slice0, patk);
  const uint32_t patz = uint32_t(lane ^ ((lane >> 5) << 3)) * 16;
  auto issue = [&]<int BUF>(int t) __attribute__((always_inline)) {
    const int w0 = t < c_sel ? (geo ? block_geo(geo, b, nqb, n, irow[t]).w : irow[t] * SAS_BLK)
                             : gi.w;
    dma_slices<JWK>(k + (kv0 + size_t(w0)) * D, stage_buf<TK, BUF, TB>(), slice0, patk);
    const char* zg = reinterpret_cast<const char*>(zrow + size_t(t < c_sel ? t : topk) * zstride) +
                     dh * JWZ * 1024;
    lds_char* zl = stage_buf<TZ, BUF, GC * ZB>() + hw * ZB + dh * JWZ * 1024;
#pragma unroll
    for (int u = 0; u < JWZ; ++u)   // read once: the non-temporal policy (aux 2)
      __builtin_amdgcn_global_load_lds((glb_void*)(uniform_ptr(zg + u * 1024) + opaque(patz)),
                                       (lds_void*)(zl + u * 1024), 16, 0, 2);
  };
  issue.template operator()<0>(0);
  if (1 < ntiles) issue.template operator()<1>(1);

  // Transposed dZ reads.  Lane j of a 16-lane group names the piece of key
  // 16c + 4(grp >> 1) + (j >> 2) + 8w and rows 32hf + 16(grp & 1) + 4(j & 3)
  // + 0..3 (grp = lane / 16), which the key-outer kernel's wave (c >> 1, hf)
  // stored in slice half grp & 1, lane (key % 32) + 32 (j & 1), bytes
  // 8 ((j >> 1) & 1); then lane i of the group receives row 32hf +
  // 16(grp & 1) + i, keys 16c + 4(grp >> 1) + 8w + 0..3, as tr_operand
  // orders them.  zo[w] is the byte offset for c = hf = 0; chunk c adds
  // (c >> 1) * 4096 + (c & 1) * 256, row half hf adds 2048.
  uint32_t to[DT][2], zo[2];
  {
    int toff[D / 32][2];
    tr_offsets<D>(lane, toff);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) to[dt][w] = lane_off(toff[dh * DT + dt][w]);
    const int grp = lane >> 4, j = lane & 15, zh = j & 1;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int chunk = 4 * (grp >> 1) + (j >> 2) + 8 * (w ^ zh) + 32 * zh;   // swizzled
      zo[w] = lane_off(hw * ZB + (grp & 1) * 1024 + chunk * 16 + 8 * ((j >> 1) & 1));
    }
  }

  f32x16 dQ[2][DT];   // [row half][32 columns of this wave's d half]: C[m = d][n = row]
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) dQ[hf][dt][jj] = 0.f;

  auto tile = [&]<int ST, bool CUR>(int t) __attribute__((always_inline)) {
    lds_cchar* Kt = stage_buf<TK, ST, TB>();
    lds_cchar* Zt = stage_buf<TZ, ST, GC * ZB>();
    bf16x8 zb[2][4];   // dZ^T operands: 8 keys of key chunk c for one row of half hf
    bf16x8 ka[DT][4];  // K^T operands: 8 keys of key chunk c for one d column
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        zb[hf][c] = ldtr_pair(Zt + hf * 2048 + (c >> 1) * 4096 + (c & 1) * 256, zo[0], zo[1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ka[dt][c] = ldtr_pair(Kt + c * 16 * ROWB, to[dt][0], to[dt][1]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dQ[0][dt] = mfma32(ka[dt][c], zb[0][c], dQ[0][dt]);
        dQ[1][dt] = mfma32(ka[dt][c], zb[1][c], dQ[1][dt]);
      }
    if (!CUR && dh == 0) {
      float zs = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) zs = sum_bf16x8(zb[hf][c], zs);
      zs = wave_sum(zs);
      if (lane == 0) part[t & 1][hw] = zs;
    }
  };
  auto publish = [&](int t) __attribute__((always_inline)) {   // gate gradient of tile t
    if (tid == 0) {
      float a = 0.f;
      for (int w = 0; w < GC; ++w) a += part[t & 1][w];
      dlgp[(rowsel * nch + chunk) * K + t] = a;
    }
  };
  auto kept = [&]<int ST>(int t) __attribute__((always_inline)) {
    vm_wait_barrier<PER * (NS - 2)>();
    if (t > 0) publish(t - 1);
    if (t + NS - 1 < ntiles) issue.template operator()<(ST + NS - 1) % NS>(t + NS - 1);
    tile.template operator()<ST, false>(t);
  };
  int t = 0;
#pragma nounroll
  for (; t + NS <= c_sel; t += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      (kept.template operator()<S>(t + S), ...);
    }(std::make_integer_sequence<int, NS>{});
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((t + S < c_sel ? kept.template operator()<S>(t + S) : void()), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
  vm_wait_barrier<0>();
  if (c_sel > 0) publish(c_sel - 1);
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((c_sel % NS == S ? tile.template operator()<S, true>(c_sel) : void()), ...);
  }(std::make_integer_sequence<int, NS>{});

#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r = hf * 32 + lr;
    if (r < gi.lo || r >= gi.hi) continue;   // a window row of another block
    uint16_t* drow = dq + ((size_t(b) * Hq + h) * n + gi.w + r) * D + dh * (D / 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(dQ[hf][dt][4 * jg + e] * tau);
        *reinterpret_cast<bf16x4*>(drow + dt * 32 + 8 * jg + 4 * hh) = v4;
      }
  }
}

// ------------------------------------------------------------------ host side
template <int D, int GC>
static void dq_launch(int nblocks, const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* lse, const int32_t* idx, const int32_t* cnt,
                      const float* lg, void* dq, float* stats, float* dlgp, int Hq, int Hkv, int n,
                      int topk, float tau, float tau2, int BH, int h_off, int hchunks, int nch,
                      int chunk0, bool ext, const int32_t* geo, int nqb, hipStream_t st) {
#define SAS_DQ_KARGS (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o, \
    (const uint16_t*)dO, lse, idx, cnt, lg, (uint16_t*)dq, stats, dlgp, Hq, Hkv, n, topk, tau,   \
    tau2, BH, h_off, hchunks, nch, chunk0, geo, nqb
  if (ext)
    hipLaunchKernelGGL((bwd_dq_kernel<D, GC, true>), dim3(nblocks), dim3(128 * GC), 0, st,
                       SAS_DQ_KARGS);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, GC, false>), dim3(nblocks), dim3(128 * GC), 0, st,
                       SAS_DQ_KARGS);
#undef SAS_DQ_KARGS
}

template <int D>
static void dq_dispatch(int gc, int nblocks, const void* q, const void* k, const void* v,
                        const void* o, const void* dO, const float* lse, const int32_t* idx,
                        const int32_t* cnt, const float* lg, void* dq, float* stats, float* dlgp,
                        int Hq, int Hkv, int n, int topk, float tau, float tau2, int BH, int h_off,
                        int hchunks, int nch, int chunk0, bool ext, const int32_t* geo, int nqb,
                        hipStream_t st) {
#define SAS_DQ_ARGS nblocks, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, \
                    topk, tau, tau2, BH, h_off, hchunks, nch, chunk0, ext, geo, nqb, st
  switch (gc) {
    case 1: dq_launch<D, 1>(SAS_DQ_ARGS); break;
    case 2: dq_launch<D, 2>(SAS_DQ_ARGS); break;
    default: dq_launch<D, 4>(SAS_DQ_ARGS); break;
  }
#undef SAS_DQ_ARGS
}

static int n_head_chunks(int G) {
  int nch = 0;
  for (const HeadChunks& hc : head_chunks(G)) nch += hc.count;
  return nch;
}

size_t bwd_mfma_extra_ws(int B, int Hq, int Hkv, int nb, int topk) {
  const int nch = n_head_chunks(Hq / Hkv);
  return sizeof(float) * size_t(B) * Hkv * nb * nch * size_t(topk > 0 ? topk : 1);
}

template <int D>
static void dqz_dispatch(int gc, int nblocks, const void* k, const void* dz, const int32_t* idx,
                         const int32_t* cnt, void* dq, float* dlgp, int Hq, int Hkv, int n,
                         int topk, int K, float tau, int BH, int h_off, int hchunks, int nch,
                         int chunk0, const int32_t* geo, int nqb, hipStream_t st) {
#define SAS_DQZ_KARGS (const uint16_t*)k, (const uint16_t*)dz, idx, cnt, (uint16_t*)dq, dlgp, Hq, \
    Hkv, n, topk, K, tau, BH, h_off, hchunks, nch, chunk0, geo, nqb
  switch (gc) {
    case 1:
      hipLaunchKernelGGL((bwd_dqz_kernel<D, 1>), dim3(nblocks), dim3(128), 0, st, SAS_DQZ_KARGS);
      break;
    case 2:
      hipLaunchKernelGGL((bwd_dqz_kernel<D, 2>), dim3(nblocks), dim3(256), 0, st, SAS_DQZ_KARGS);
      break;
    default:
      hipLaunchKernelGGL((bwd_dqz_kernel<D, 4>), dim3(nblocks), dim3(512), 0, st, SAS_DQZ_KARGS);
      break;
  }
#undef SAS_DQZ_KARGS
}

size_t bwd_dz_bytes(int B, int Hq, int nb, int topk) {
  return size_t(B) * Hq * size_t(nb) * (size_t(topk) + 1) * 64 * 64 * 2;
}

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, const int32_t* idx,
                           const int32_t* cnt, const float* lg, const float* s,
                           const float* s_lse, void* dq, void* dk, void* dv, float* ds,
                           float* stats, const int32_t* rev_off, const int32_t* rev_list,
                           float* dlgp, void* dz, int B, int Hq, int Hkv, int n, int d, int topk,
                           float tau, int gate, const int32_t* geo, int nqb, hipStream_t st) {
  const int G = Hq / Hkv;
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const bool zpath = dz != nullptr && !ext;
  const int BH = B * Hkv;
  const float tau2 = tau * kLog2e;
  const int nch = n_head_chunks(G);
  const int K = topk > 0 ? topk : 1;
  hipError_t e = hipSuccess;
  if (!zpath) {   // (the dZ-tile path's statistics come with the reverse lists)
    ProfScope ps("sas_bwd_dq_kernel", st);
    int chunk0 = 0;
    for (const HeadChunks& hc : head_chunks(G)) {
      if (d == 128) dq_dispatch<128>(hc.gc, BH * nqb * hc.count, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, K, tau, tau2, BH, hc.h_off, hc.count, nch, chunk0, ext, geo, nqb, st);
      else dq_dispatch<64>(hc.gc, BH * nqb * hc.count, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, K, tau, tau2, BH, hc.h_off, hc.count, nch, chunk0, ext, geo, nqb, st);
      chunk0 += hc.count;
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!zpath) {
    ProfScope ps("sas_bwd_ds_kernel", st);
    hipLaunchKernelGGL(bwd_ds_kernel, dim3(BH * nqb), dim3(256), 0, st, dlgp, idx, cnt, s, s_lse,
                       ds, nqb, K, nch, gate);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("sas_bwd_dkdv_kernel", st);
    // pairs per phase: the largest divisor of B*Hkv whose Q and dO (G heads
    // each, bf16) fit 256 MiB, the size of the last-level cache; a phase
    // wider than that re-fetches its re-read tiles from HBM (measured: all
    // eight kv-heads of the 32K layer at once, 537 MB, ran the step 5-8%
    // slower than phases of two or four)
    const size_t pair_bytes = size_t(G) * size_t(n) * size_t(d) * 2 * 2;
    int pph = BH;
    while (pph > 1 && (BH % pph != 0 || size_t(pph) * pair_bytes > (size_t(256) << 20))) --pph;
#define SAS_KV_KARGS (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, \
    (const uint16_t*)dO, stats, lg, rev_off, rev_list, (uint16_t*)dk, (uint16_t*)dv, \
    (uint16_t*)dz, Hq, Hkv, n, topk, tau, tau2, geo, nqb, pph
    if (d == 128 && ext)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, true, false>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else if (d == 128 && zpath)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, false, true>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else if (d == 128)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, false, false>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else if (ext)
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, true, false>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else if (zpath)
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false, true>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false, false>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
#undef SAS_KV_KARGS
  }
  e = hipGetLastError();
  if (e != hipSuccess || !zpath) return e;
  {
    ProfScope ps("sas_bwd_dqz_kernel", st);
    int chunk0 = 0;
    for (const HeadChunks& hc : head_chunks(G)) {
      if (d == 128) dqz_dispatch<128>(hc.gc, BH * nqb * hc.count, k, dz, idx, cnt, dq, dlgp, Hq, Hkv, n, topk, K, tau, BH, hc.h_off, hc.count, nch, chunk0, geo, nqb, st);
      else dqz_dispatch<64>(hc.gc, BH * nqb * hc.count, k, dz, idx, cnt, dq, dlgp, Hq, Hkv, n, topk, K, tau, BH, hc.h_off, hc.count, nch, chunk0, geo, nqb, st);
      chunk0 += hc.count;
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_ds_kernel", st);
    hipLaunchKernelGGL(bwd_ds_kernel, dim3(BH * nqb), dim3(256), 0, st, dlgp, idx, cnt, s, s_lse,
                       ds, nqb, K, nch, gate);
  }
  return hipGetLastError();
}

}  // namespace sas
