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
    int h_off, int hchunks, int nch, int chunk0) {
  constexpr int NS = kDqStages;
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;
  constexpr int JT = TB / 1024;
  constexpr int JW = 2 * JT / (2 * GC);
  static_assert((2 * JT) % (2 * GC) == 0 && JT % JW == 0, "slices must split evenly over the waves");
  constexpr int TK = 200, TV = 201;       // LDS buffer tags: K tiles, V tiles
  __shared__ float part[2][8];            // per-wave dZ sums of the last two tiles

  const int nqb = n / SAS_BLK;
  const int G = Hq / Hkv;
  int bid = blockIdx.x;
  const int hc = bid % hchunks;
  bid /= hchunks;
  const int bk = bid % BH;
  const int i = nqb - 1 - bid / BH;
  const int b = bk / Hkv, kv = bk % Hkv;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int h = kv * G + h_off + hc * GC + (wave >> 1);
  const int rt = wave & 1;
  const int chunk = chunk0 + hc;
  const size_t rowsel = size_t(bk) * nqb + i;
  const int c_sel = cnt[rowsel];
  const int ntiles = c_sel + 1;
  const int32_t* irow = idx + rowsel * topk;
  const float* grow = lg + rowsel * topk;

  const size_t qrow = (size_t(b) * Hq + h) * n + size_t(i) * SAS_BLK + rt * 32 + lr;
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
  const float Drow = dpart + __shfl_xor(dpart, 32);
  const float lse2 = lse[qrow] * kLog2e;
  if (hh == 0) {
    // per-row statistics of this (head, q-block) for the key-block-outer pass:
    // [-lse / tau for the 64 rows | -D for the 64 rows]
    float* st = stats + ((size_t(b) * Hq + h) * nqb + i) * 128;
    st[rt * 32 + lr] = -lse[qrow] / tau;
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
    const int blk = t < c_sel ? irow[t] : i;
    const uint16_t* src = (k_side ? k : v) + (kv0 + size_t(blk) * SAS_BLK) * D;
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
          if (CUR && kt * 32 + 8 * (j >> 2) + 4 * hh + (j & 3) > rt * 32 + lr) p = 0.f;
          if constexpr (EXT) {
            x[e] = p * (P2[j] - Dg);
            if (!CUR) zs = __builtin_fmaf(p, P2[j], zs);
          } else {
            x[e] = p * P2[j];
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
template <int D, bool EXT>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ stats, const float* __restrict__ lg,
    const int32_t* __restrict__ rev_off, const int32_t* __restrict__ rev_list,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hq, int Hkv, int n, int topk,
    float tau, float tau2) {
  constexpr int NS = kKvStages;
  static_assert(NS == 4, "stage arithmetic below assumes a 4-stage ring");
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;
  constexpr int CPR = D / 8;
  constexpr int JT = TB / 1024;
  constexpr int JW = 2 * JT / 4;        // Q + dO slices per wave per step
  constexpr int PER = JW + 1;           // plus the row statistics
  constexpr int TQ = 300, TO = 301, TS = 302;   // LDS buffer tags

  const int nkb = n / SAS_BLK;
  const int G = Hq / Hkv;
  // key-block-major grid: consecutive workgroups take the same key block of
  // consecutive (batch, kv-head) pairs.  Workgroups are dealt round-robin to
  // the XCDs, so one XCD serves one kv-head's key blocks m, m+1, ... at a
  // time; their reverse lists walk similar q-block ranges in ascending order,
  // so a Q/dO tile one of them loads is often still in that XCD's L2 when the
  // next needs it.  It also starts the longest lists (small m) first.
  const int BH = gridDim.x / nkb;
  const int m = blockIdx.x / BH;
  const int bk = blockIdx.x % BH;
  const int b = bk / Hkv, kv = bk % Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int kh = wave & 1, rh = wave >> 1;

  const size_t kvrow0 = (size_t(b) * Hkv + kv) * n + size_t(m) * SAS_BLK;
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

  // list entries of this key block -> LDS: q-block and base-2 log-gate
  // (0 for the own block, entry 0)
  __shared__ int2 meta[SAS_MAX_BLOCKS];
  const int32_t* lst = rev_list + size_t(bk) * nkb * (topk + 1);
  const int32_t e0 = rev_off[size_t(bk) * (nkb + 1) + m];
  const int32_t e1 = rev_off[size_t(bk) * (nkb + 1) + m + 1];
  for (int e = tid; e < e1 - e0; e += 256) {
    const int32_t ent = lst[e0 + e];
    const int iq = ent & 0xFFFF, slot = (ent >> 16) & 0xFFFF;
    const float l = slot == 0xFFFF ? 0.f : lg[(size_t(bk) * nkb + iq) * topk + slot];
    const float b2 = (EXT ? fmaxf(l, kMinExtLogGate) : l) * kLog2e;
    meta[e] = make_int2(iq, __float_as_int(b2));
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
    const int iq = __builtin_amdgcn_readfirstlane(meta[ie].x);
    const char* tile = src_base + size_t(ih) * hstride + size_t(iq) * SAS_BLK * D * 2;
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
  // j = 8*jc + e holds row rh*32 + 8*(j/4) + 4*hh + j%4 of this lane's key)
  auto elementwise = [&]<bool OWN, int JC>(const f32x16& S, const f32x16& P2, float bias2,
                                           bf16x8& Pp, bf16x8& Zp) __attribute__((always_inline)) {
    float pv[8], zv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * JC + e;
      float p = fast_exp2(__builtin_fmaf(S[j], tau2, bias2));
      if (OWN && kh * 32 + lr > rh * 32 + 8 * (j >> 2) + 4 * hh + (j & 3)) p = 0.f;
      pv[e] = p;
      zv[e] = p * P2[j];
    }
    Pp = pack_bf16x8(pv);
    Zp = pack_bf16x8(zv);
  };

  auto step = [&]<int ST, bool OWN>(float bias2) __attribute__((always_inline)) {
    constexpr int NC = D / 16;
    constexpr int NT = D / 32;
    lds_cchar* Qt = stage_buf<TQ, ST, TB>();
    lds_cchar* Ot = stage_buf<TO, ST, TB>();
    lds_cchar* St = stage_buf<TS, ST, 1024>();
    // phase 1: S = Q K^T - lse/tau, dP = dO V^T - D (EXT: - D/g)
    f32x16 S, P2;
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
    for (int c = 0; c < 2; ++c) {
      qa[c] = ld16(Qt, qo[c]);
      oa[c] = ld16(Ot, qo[c]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 2 < NC) {
        qa[c + 2] = ld16(Qt, qo[c + 2]);
        oa[c + 2] = ld16(Ot, qo[c + 2]);
      }
      S = mfma32(qa[c], kop[c], S);
      P2 = mfma32(oa[c], vop[c], P2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase 2: transposed operands of rows 0..15, P and dZ of rows 0..15
    bf16x8 tO0[NT], tQ0[NT], tO1[NT], tQ1[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      tO0[dt] = ldtr_pair(Ot, to[dt][0], to[dt][1]);
      tQ0[dt] = ldtr_pair(Qt, to[dt][0], to[dt][1]);
    }
    bf16x8 Pp0, Zp0, Pp1, Zp1;
    elementwise.template operator()<OWN, 0>(S, P2, bias2, Pp0, Zp0);
    __builtin_amdgcn_sched_barrier(0);
    // phase 3: dV/dK of rows 0..15 with P, dZ and operands of rows 16..31
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      tO1[dt] = ldtr_pair(Ot + 16 * ROWB, to[dt][0], to[dt][1]);
      tQ1[dt] = ldtr_pair(Qt + 16 * ROWB, to[dt][0], to[dt][1]);
    }
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      dV[dt] = mfma32(Pp0, tO0[dt], dV[dt]);
      dK[dt] = mfma32(Zp0, tQ0[dt], dK[dt]);
    }
    elementwise.template operator()<OWN, 1>(S, P2, bias2, Pp1, Zp1);
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six vector ops
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 4: dV/dK of rows 16..31
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      dV[dt] = mfma32(Pp1, tO1[dt], dV[dt]);
      dK[dt] = mfma32(Zp1, tQ1[dt], dK[dt]);
    }
  };

  // step s in stage ST: wait for its DMA (and for the stage it refills to be
  // free), refill the stage NS-1 ahead, compute.  Steps 0..G-1 are the own
  // block (no gate, causal mask; rows 0..31 see none of the keys 32..63, so
  // that wave sits them out).
  int ce = 0, chd = 0;   // list entry / head of the step being computed
  auto run = [&]<int ST, bool STEADY>(int s) __attribute__((always_inline)) {
    if (STEADY) vm_wait_barrier<(NS - 2) * PER>();
    else wait_ahead(min(NS - 2, nsteps - 1 - s));
    if (STEADY || s + NS - 1 < nsteps) issue.template operator()<(ST + NS - 1) % NS>();
    const float bias2 = __int_as_float(meta[ce].y);
    if (++chd == G) {
      chd = 0;
      ++ce;
    }
    if (!STEADY && s < G) {
      if (!(kh == 1 && rh == 0)) step.template operator()<ST, true>(0.f);
    } else {
      step.template operator()<ST, false>(bias2);
    }
  };
  int s = 0;
  // own-block steps and the ring tail use the checked form
#pragma nounroll
  for (; s < G; s += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      ((s + S < nsteps ? run.template operator()<S, false>(s + S) : void()), ...);
    }(std::make_integer_sequence<int, NS>{});
#pragma nounroll
  for (; s + 2 * NS - 2 < nsteps; s += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      (run.template operator()<S, true>(s + S), ...);
    }(std::make_integer_sequence<int, NS>{});
#pragma nounroll
  for (; s < nsteps; s += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      ((s + S < nsteps ? run.template operator()<S, false>(s + S) : void()), ...);
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
      const __attribute__((address_space(3))) float* src = red[key >> 5] + (key & 31) * D + (c % CPR) * 8;
      bf16x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (__bf16)(src[e] * sc);
      *reinterpret_cast<bf16x8*>(dst + c * 8) = r;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host side
template <int D, int GC>
static void dq_launch(int nblocks, const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* lse, const int32_t* idx, const int32_t* cnt,
                      const float* lg, void* dq, float* stats, float* dlgp, int Hq, int Hkv, int n,
                      int topk, float tau, float tau2, int BH, int h_off, int hchunks, int nch,
                      int chunk0, bool ext, hipStream_t st) {
#define SAS_DQ_KARGS (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o, \
    (const uint16_t*)dO, lse, idx, cnt, lg, (uint16_t*)dq, stats, dlgp, Hq, Hkv, n, topk, tau,   \
    tau2, BH, h_off, hchunks, nch, chunk0
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
                        int hchunks, int nch, int chunk0, bool ext, hipStream_t st) {
#define SAS_DQ_ARGS nblocks, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, \
                    topk, tau, tau2, BH, h_off, hchunks, nch, chunk0, ext, st
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

size_t bwd_mfma_extra_ws(int B, int Hq, int Hkv, int n, int topk) {
  const int nch = n_head_chunks(Hq / Hkv);
  return sizeof(float) * size_t(B) * Hkv * (n / SAS_BLK) * nch * size_t(topk > 0 ? topk : 1);
}

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, const int32_t* idx,
                           const int32_t* cnt, const float* lg, const float* s,
                           const float* s_lse, void* dq, void* dk, void* dv, float* ds,
                           float* stats, const int32_t* rev_off, const int32_t* rev_list,
                           float* dlgp, int B, int Hq, int Hkv, int n, int d, int topk, float tau,
                           int gate, hipStream_t st) {
  const int G = Hq / Hkv;
  const bool ext = gate == SAS_GATE_EXTERNAL;
  const int nqb = n / SAS_BLK;
  const int BH = B * Hkv;
  const float tau2 = tau * kLog2e;
  const int nch = n_head_chunks(G);
  const int K = topk > 0 ? topk : 1;
  {
    ProfScope ps("sas_bwd_dq_kernel", st);
    int chunk0 = 0;
    for (const HeadChunks& hc : head_chunks(G)) {
      if (d == 128) dq_dispatch<128>(hc.gc, BH * nqb * hc.count, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, K, tau, tau2, BH, hc.h_off, hc.count, nch, chunk0, ext, st);
      else dq_dispatch<64>(hc.gc, BH * nqb * hc.count, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, K, tau, tau2, BH, hc.h_off, hc.count, nch, chunk0, ext, st);
      chunk0 += hc.count;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_ds_kernel", st);
    hipLaunchKernelGGL(bwd_ds_kernel, dim3(BH * nqb), dim3(256), 0, st, dlgp, idx, cnt, s, s_lse,
                       ds, nqb, K, nch, gate);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_dkdv_kernel", st);
#define SAS_KV_KARGS (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, \
    (const uint16_t*)dO, stats, lg, rev_off, rev_list, (uint16_t*)dk, (uint16_t*)dv, Hq, Hkv, n, \
    topk, tau, tau2
    if (d == 128 && ext)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else if (d == 128)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else if (ext)
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), dim3(BH * nqb), dim3(256), 0, st, SAS_KV_KARGS);
#undef SAS_KV_KARGS
  }
  return hipGetLastError();
}

}  // namespace sas
