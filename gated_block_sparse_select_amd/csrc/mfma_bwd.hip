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
//               pi_i = softmax(s[i, 0..i-1])  (chain rule through §2.4).
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
#include <type_traits>
#include <utility>

#include "launch.h"
#include "mfma_common.h"

namespace sas {

// ------------------------------------------------------------------ dq kernel
template <int D, int GC>
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
  static_assert((2 * JT) % (2 * GC) == 0, "slices must split evenly over the waves");
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
    // [lse * log2(e) for the 64 rows | D for the 64 rows]
    float* st = stats + ((size_t(b) * Hq + h) * nqb + i) * 128;
    st[rt * 32 + lr] = lse2;
    st[64 + rt * 32 + lr] = Drow;
  }

  const size_t kv0 = (size_t(b) * Hkv + kv) * size_t(n);
  auto issue = [&]<int BUF>(int t) __attribute__((always_inline)) {
    const int blk = t < c_sel ? irow[t] : i;
    const uint16_t* kb = k + (kv0 + size_t(blk) * SAS_BLK) * D;
    const uint16_t* vb = v + (kv0 + size_t(blk) * SAS_BLK) * D;
#pragma unroll
    for (int u = 0; u < JW; ++u) {
      const int j = wave * JW + u;
      if (j < JT) dma_tile_slice<D>(kb, stage_buf<TK, BUF, TB>(), j, lane);
      else dma_tile_slice<D>(vb, stage_buf<TV, BUF, TB>(), j - JT, lane);
    }
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
    const float zoff = (CUR ? 0.f : grow[t] * kLog2e) - lse2;
    float zs = 0.f;
    bf16x8 dZp[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {   // one 32-key half at a time
      f32x16 S, P2;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        S[j] = 0.f;
        P2[j] = 0.f;
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
          x[e] = p * (P2[j] - Drow);
          zs += x[e];
        }
        dZp[kt * 2 + jc] = pack_bf16x8(x);
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
                                                     int nch) {
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
  for (int m = threadIdx.x; m < nqb; m += 256) {
    float val = 0.f;
    if (m < i) {
      const int sm = slot_of[m];
      val = (sm >= 0 ? dl[sm] : 0.f) - expf(s[row * nqb + m] - sl_) * tot;
    }
    ds[row * nqb + m] = val;
  }
}

// ------------------------------------------------------------------ dk/dv kernel
// grid: B*Hkv*nkb workgroups of 4 waves; wave = (key half kh, row half rh).
// The (q-block, head) steps of the reverse list stream through a ring of
// kKvStages stages, each holding the Q and dO tiles of one (q-block, head) and
// its row statistics [lse*log2e | D]; the block's own V tile sits in LDS (its
// K rows stay in registers as the S = Q K^T operand).
template <int D>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ stats, const float* __restrict__ lg,
    const int32_t* __restrict__ rev_off, const int32_t* __restrict__ rev_list,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hq, int Hkv, int n, int topk,
    float tau, float tau2) {
  constexpr int NS = kKvStages;
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;
  constexpr int CPR = D / 8;
  constexpr int JT = TB / 1024;
  constexpr int JW = 2 * JT / 4;        // Q + dO slices per wave per step
  constexpr int PER = JW + 1;           // plus one slice of row statistics
  constexpr int TQ = 300, TO = 301, TS = 302, TVV = 303;   // LDS buffer tags

  const int nkb = n / SAS_BLK;
  const int G = Hq / Hkv;
  const int bk = blockIdx.x / nkb;
  const int m = blockIdx.x % nkb;
  const int b = bk / Hkv, kv = bk % Hkv;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int kh = wave & 1, rh = wave >> 1;

  const size_t kvrow0 = (size_t(b) * Hkv + kv) * n + size_t(m) * SAS_BLK;
  const size_t krow = kvrow0 + kh * 32 + lr;
  bf16x8 kop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    kop[c] = *reinterpret_cast<const bf16x8*>(k + krow * D + c * 16 + hh * 8);
  lds_char* Vown = stage_buf<TVV, 0, TB>();
#pragma unroll
  for (int u = 0; u < JT / 4; ++u) dma_tile_slice<D>(v + kvrow0 * D, Vown, wave * (JT / 4) + u, lane);

  f32x16 dK[D / 32], dV[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      dK[dt][j] = 0.f;
      dV[dt][j] = 0.f;
    }

  const int32_t* lst = rev_list + size_t(bk) * nkb * (topk + 1);
  const int32_t e0 = rev_off[size_t(bk) * (nkb + 1) + m];
  const int32_t e1 = rev_off[size_t(bk) * (nkb + 1) + m + 1];
  const int nsteps = (e1 - e0) * G;

  auto issue = [&]<int BUF>(int s) __attribute__((always_inline)) {
    const int32_t ent = lst[e0 + s / G];
    const int iq = ent & 0xFFFF;
    const int hq = kv * G + s % G;
    const size_t row0 = (size_t(b) * Hq + hq) * n + size_t(iq) * SAS_BLK;
#pragma unroll
    for (int u = 0; u < JW; ++u) {
      const int j = wave * JW + u;
      if (j < JT) dma_tile_slice<D>(q + row0 * D, stage_buf<TQ, BUF, TB>(), j, lane);
      else dma_tile_slice<D>(dO + row0 * D, stage_buf<TO, BUF, TB>(), j - JT, lane);
    }
    // 512 B of statistics: lanes 0..7 of each wave move 128 B
    const float* st = stats + ((size_t(b) * Hq + hq) * nkb + iq) * 128 + wave * 32;
    if (lane < 8) dma16(st + lane * 4, stage_buf<TS, BUF, 512>() + wave * 128);
  };
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((S < nsteps ? issue.template operator()<S>(S) : void()), ...);
  }(std::make_integer_sequence<int, NS - 1>{});

  uint32_t qo[D / 16], to[D / 32][2], vo[D / 16];
  {
    int roff[D / 16], toff[D / 32][2];
    row_offsets<D>(lane, roff);
    tr_offsets<D>(lane, toff);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      qo[c] = lane_off(rh * 32 * ROWB + roff[c]);
      vo[c] = lane_off(kh * 32 * ROWB + roff[c]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) to[dt][w] = lane_off(rh * 32 * ROWB + toff[dt][w]);
  }
  // row statistics of rows rh*32 + 8*jg + 4*hh + 0..3 (16 B per group)
  const uint32_t so = lane_off((rh * 32 + 4 * hh) * 4);
  const int keyw = kh * 32 + lr;  // this lane's key inside block m

  auto step = [&]<int ST>(int s) __attribute__((always_inline)) {
    lds_cchar* Qt = stage_buf<TQ, ST, TB>();
    lds_cchar* Ot = stage_buf<TO, ST, TB>();
    lds_cchar* St = stage_buf<TS, ST, 512>();
    const int32_t ent = lst[e0 + s / G];
    const int iq = ent & 0xFFFF;
    const int slot = (ent >> 16) & 0xFFFF;
    const bool own = slot == 0xFFFF;   // the block's own (causal) current block
    const float bias2 = own ? 0.f : lg[(size_t(bk) * nkb + iq) * topk + slot] * kLog2e;
    // own block: rows 0..31 see none of the keys 32..63
    if (own && kh == 1 && rh == 0) return;
    f32x16 S, P2;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      S[j] = 0.f;
      P2[j] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      S = mfma32(ld16(Qt, qo[c]), kop[c], S);
      P2 = mfma32(ld16(Ot, qo[c]), ld16(Vown, vo[c]), P2);
    }
    // S[row][key]: lane l, reg j: row = rh*32 + 8(j/4) + 4hh + j%4, key = keyw
    typedef __attribute__((ext_vector_type(4))) float f32x4;
    bf16x8 Pp[2], Zp[2];
#pragma unroll
    for (int jc = 0; jc < 2; ++jc) {
      float pv[8], zv[8];
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int jg = 2 * jc + g2;
        const f32x4 lv = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(St + so + jg * 32);
        const f32x4 dv4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(St + so + 256 + jg * 32);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int j = 4 * jg + r4;
          float p = fast_exp2(__builtin_fmaf(S[j], tau2, bias2 - lv[r4]));
          if (own && keyw > rh * 32 + 8 * jg + 4 * hh + r4) p = 0.f;
          pv[4 * g2 + r4] = p;
          zv[4 * g2 + r4] = p * (P2[j] - dv4[r4]);
        }
      }
      Pp[jc] = pack_bf16x8(pv);
      Zp[jc] = pack_bf16x8(zv);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jc = 0; jc < 2; ++jc) {
        dV[dt] = mfma32(Pp[jc], ldtr_pair(Ot + jc * 16 * ROWB, to[dt][0], to[dt][1]), dV[dt]);
        dK[dt] = mfma32(Zp[jc], ldtr_pair(Qt + jc * 16 * ROWB, to[dt][0], to[dt][1]), dK[dt]);
      }
  };
  // step s in stage ST: wait for its DMA (and for the stage it refills to be
  // free), refill the stage NS-1 ahead, compute
  auto run = [&]<int ST>(int s) __attribute__((always_inline)) {
    const int after = min(NS - 2, nsteps - 1 - s);
    if (after >= 2) vm_wait_barrier<PER * 2>();
    else if (after == 1) vm_wait_barrier<PER>();
    else vm_wait_barrier<0>();
    if (s + NS - 1 < nsteps) issue.template operator()<(ST + NS - 1) % NS>(s + NS - 1);
    step.template operator()<ST>(s);
  };
  int s = 0;
#pragma nounroll
  for (; s + NS <= nsteps; s += NS)
    [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
      (run.template operator()<S>(s + S), ...);
    }(std::make_integer_sequence<int, NS>{});
  [&]<int... S>(std::integer_sequence<int, S...>) __attribute__((always_inline)) {
    ((s + S < nsteps ? run.template operator()<S>(s + S) : void()), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
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
                      int chunk0, hipStream_t st) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, GC>), dim3(nblocks), dim3(128 * GC), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                     (const uint16_t*)dO, lse, idx, cnt, lg, (uint16_t*)dq, stats, dlgp, Hq, Hkv,
                     n, topk, tau, tau2, BH, h_off, hchunks, nch, chunk0);
}

template <int D>
static void dq_dispatch(int gc, int nblocks, const void* q, const void* k, const void* v,
                        const void* o, const void* dO, const float* lse, const int32_t* idx,
                        const int32_t* cnt, const float* lg, void* dq, float* stats, float* dlgp,
                        int Hq, int Hkv, int n, int topk, float tau, float tau2, int BH, int h_off,
                        int hchunks, int nch, int chunk0, hipStream_t st) {
#define SAS_DQ_ARGS nblocks, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, \
                    topk, tau, tau2, BH, h_off, hchunks, nch, chunk0, st
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
                           hipStream_t st) {
  const int G = Hq / Hkv;
  const int nqb = n / SAS_BLK;
  const int BH = B * Hkv;
  const float tau2 = tau * kLog2e;
  const int nch = n_head_chunks(G);
  const int K = topk > 0 ? topk : 1;
  {
    ProfScope ps("sas_bwd_dq_kernel", st);
    int chunk0 = 0;
    for (const HeadChunks& hc : head_chunks(G)) {
      if (d == 128) dq_dispatch<128>(hc.gc, BH * nqb * hc.count, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, K, tau, tau2, BH, hc.h_off, hc.count, nch, chunk0, st);
      else dq_dispatch<64>(hc.gc, BH * nqb * hc.count, q, k, v, o, dO, lse, idx, cnt, lg, dq, stats, dlgp, Hq, Hkv, n, K, tau, tau2, BH, hc.h_off, hc.count, nch, chunk0, st);
      chunk0 += hc.count;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_ds_kernel", st);
    hipLaunchKernelGGL(bwd_ds_kernel, dim3(BH * nqb), dim3(256), 0, st, dlgp, idx, cnt, s, s_lse,
                       ds, nqb, K, nch);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("sas_bwd_dkdv_kernel", st);
    if (d == 128) {
      hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(BH * nqb), dim3(256), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dO, stats, lg,
                         rev_off, rev_list, (uint16_t*)dk, (uint16_t*)dv, Hq, Hkv, n, topk, tau,
                         tau2);
    } else {
      hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(BH * nqb), dim3(256), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dO, stats, lg,
                         rev_off, rev_list, (uint16_t*)dk, (uint16_t*)dv, Hq, Hkv, n, topk, tau,
                         tau2);
    }
  }
  return hipGetLastError();
}

}  // namespace sas
