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
#include "launch.h"
#include "mfma_common.h"

namespace sas {

template <int D, int GC>
__global__ void __launch_bounds__(128 * GC) fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const float* __restrict__ lg, uint16_t* __restrict__ o,
    float* __restrict__ lse, int Hq, int Hkv, int n, int topk, float tau2, int BH, int h_off,
    int hchunks) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int ROWB = D * 2;
  constexpr int TB = 64 * ROWB;          // bytes of one 64 x D tile
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int HALF = 64 * CPR;         // chunks per tile
  constexpr int TOTAL = 2 * HALF;        // K + V chunks per stage
  constexpr int NT = 128 * GC;
  constexpr int CPT = (TOTAL + NT - 1) / NT;

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
  const size_t rowsel = size_t(bk) * nqb + i;
  const int c_sel = cnt[rowsel];
  const int ntiles = c_sel + 1;
  const int32_t* irow = idx + rowsel * topk;
  const float* grow = lg + rowsel * topk;

  const size_t qrow = (size_t(b) * Hq + h) * n + size_t(i) * SAS_BLK + rt * 32 + lr;
  bf16x8 qop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qop[c] = *reinterpret_cast<const bf16x8*>(q + qrow * D + c * 16 + hh * 8);

  const size_t kv0 = (size_t(b) * Hkv + kv) * size_t(n);
  uint4 stg[CPT];
  auto load_tile = [&](int t) {
    const int blk = t < c_sel ? irow[t] : i;
    const uint16_t* kb = k + (kv0 + size_t(blk) * SAS_BLK) * D;
    const uint16_t* vb = v + (kv0 + size_t(blk) * SAS_BLK) * D;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + NT * u;
      if (c < TOTAL) {
        const uint16_t* src = c < HALF ? kb + c * 8 : vb + (c - HALF) * 8;
        stg[u] = *reinterpret_cast<const uint4*>(src);
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* base = smem + stage * 2 * TB;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + NT * u;
      if (c < TOTAL) {
        const bool isv = c >= HALF;
        const int cc = isv ? c - HALF : c;
        const int row = cc / CPR, col = cc % CPR;
        const int off = tile_off<D>(row, col);
        *reinterpret_cast<uint4*>(base + (isv ? TB : 0) + off) = stg[u];
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  float mrow = -INFINITY, lrow = 0.f;
  f32x16 O[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) O[dt][j] = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const char* Kt = smem + stage * 2 * TB;
    const char* Vt = Kt + TB;
    const bool cur = t == c_sel;
    const float bias2 = cur ? 0.f : grow[t] * kLog2e;

    f32x16 S[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) S[kt][j] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        S[kt] = mfma32(lds_read16(Kt, tile_off<D>(kt * 32 + lr, 2 * c + hh)), qop[c], S[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float z = S[kt][j] * tau2 + bias2;
        if (cur) {
          const int key = kt * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (key > rt * 32 + lr) z = -INFINITY;
        }
        S[kt][j] = z;
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrow, mx);
    const float alpha = exp2f(mrow - mnew);
    mrow = mnew;
    lrow *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) O[dt][j] *= alpha;

    bf16x8 P[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int jc = 0; jc < 2; ++jc) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2f(S[kt][8 * jc + e] - mnew);
          lrow += p[e];
        }
        P[kt * 2 + jc] = pack_bf16x8(p);
      }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        O[dt] = mfma32(tr_operand<D>(Vt, ch * 16, dt * 32, lane), P[ch], O[dt]);

    if (t + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  lrow += __shfl_xor(lrow, 32);
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
                       int hchunks, hipStream_t st) {
  const size_t shm = size_t(4) * 64 * D * 2;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, GC>), dim3(nblocks), dim3(128 * GC), shm, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, cnt, lg,
                     (uint16_t*)o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks);
}

template <int D>
static void fwd_dispatch(int gc, int nblocks, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* cnt, const float* lg, void* o,
                         float* lse, int Hq, int Hkv, int n, int topk, float tau2, int BH,
                         int h_off, int hchunks, hipStream_t st) {
  switch (gc) {
    case 1: fwd_launch<D, 1>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, st); break;
    case 2: fwd_launch<D, 2>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, st); break;
    case 3: fwd_launch<D, 3>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, st); break;
    default: fwd_launch<D, 4>(nblocks, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, h_off, hchunks, st); break;
  }
}

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* cnt, const float* lg, void* o, float* lse, int B,
                           int Hq, int Hkv, int n, int d, int topk, float tau, hipStream_t st) {
  ProfScope ps("sas_fwd_mfma_kernel", st);
  const int G = Hq / Hkv;
  const int nqb = n / SAS_BLK;
  const int BH = B * Hkv;
  const float tau2 = tau * kLog2e;
  const int full = G / 4, rem = G % 4;
  // heads [0, 4*full) in chunks of 4, then the remaining rem heads
  if (full > 0) {
    if (d == 128) fwd_dispatch<128>(4, BH * nqb * full, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, 0, full, st);
    else fwd_dispatch<64>(4, BH * nqb * full, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, 0, full, st);
  }
  if (rem > 0) {
    if (d == 128) fwd_dispatch<128>(rem, BH * nqb, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, 4 * full, 1, st);
    else fwd_dispatch<64>(rem, BH * nqb, q, k, v, idx, cnt, lg, o, lse, Hq, Hkv, n, topk, tau2, BH, 4 * full, 1, st);
  }
  return hipGetLastError();
}

}  // namespace sas
