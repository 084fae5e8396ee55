// Reverse (per key block) lists for the key-block-outer backward pass.
//
// For each (batch, kv-head) and key block m, list every q-block whose key set
// contains m: block m itself (its own current block, always first) and then,
// in ascending order, each i > m that selected m.  Entries pack i | slot<<16,
// where slot is m's position in idx[i,:] (0xFFFF for the own block), so the
// consumer can read that pair's log-gate directly.
//
// One workgroup per (batch, kv-head).  List lengths come from LDS atomics
// (order independent) and a parallel prefix sum.  The lists are then filled
// in chunks of 64 q-blocks: a 64-bit LDS mask per key block marks the rows of
// the chunk that selected it, and each (row, slot) pair of the chunk writes
// its entry at the list cursor plus the number of earlier rows in the mask,
// so every list comes out ascending and the output is deterministic.
#include "bwd_stats.h"
#include "common.h"
#include "launch.h"

namespace sas {

constexpr int kRevMaxNb = 2048;
constexpr int kRevThreads = 1024;
constexpr int kChunkRows = 64;            // q-blocks per fill chunk (one mask bit each)

// The lists of pair bh, by one workgroup of kRevThreads threads.
SAS_DEV void revidx_pair(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                         int32_t* __restrict__ rev_off, int32_t* __restrict__ rev_list, int nb,
                         int topk, int bh) {
  __shared__ int32_t cursor[kRevMaxNb + 1];
  __shared__ unsigned long long rows[kRevMaxNb];
  __shared__ int32_t wtot[kRevThreads / 64];
  const int32_t* I = idx + size_t(bh) * nb * topk;
  const int32_t* C = cnt + size_t(bh) * nb;
  int32_t* off = rev_off + size_t(bh) * (nb + 1);
  int32_t* list = rev_list + size_t(bh) * nb * (topk + 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;

  // list lengths: the own block plus every row that kept m
  for (int m = tid; m <= nb; m += kRevThreads) cursor[m] = (m < nb) ? 1 : 0;
  __syncthreads();
  if (topk > 0) {
    for (int e = tid; e < nb * topk; e += kRevThreads) {
      const int i = e / topk, sl = e - i * topk;
      if (sl < C[i]) atomicAdd(&cursor[I[e]], 1);
    }
  }
  __syncthreads();

  // exclusive prefix sum of cursor[0..nb]: PER consecutive entries per
  // thread, an inclusive scan across each wave, then across the waves
  constexpr int PER = (kRevMaxNb + 1 + kRevThreads - 1) / kRevThreads;
  int v[PER], tot = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int j = tid * PER + p;
    v[p] = j <= nb ? cursor[j] : 0;
    tot += v[p];
  }
  int x = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kRevThreads / 64 ? wtot[lane] : 0;
    int xs = w;
#pragma unroll
    for (int o = 1; o < kRevThreads / 64; o <<= 1) {
      const int y = __shfl_up(xs, o);
      if (lane >= o) xs += y;
    }
    if (lane < kRevThreads / 64) wtot[lane] = xs - w;   // exclusive over waves
  }
  __syncthreads();
  int run = wtot[wid] + x - tot;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int j = tid * PER + p;
    if (j <= nb) cursor[j] = run;
    run += v[p];
  }
  __syncthreads();
  for (int m = tid; m <= nb; m += kRevThreads) {
    off[m] = cursor[m];
    if (m < nb) {
      list[cursor[m]] = m | int32_t(0xFFFF0000u);
      cursor[m] += 1;
    }
  }
  __syncthreads();
  if (topk == 0) return;

  for (int c0 = 0; c0 < nb; c0 += kChunkRows) {
    const int c1 = min(nb, c0 + kChunkRows);
    for (int m = tid; m < nb; m += kRevThreads) rows[m] = 0ull;
    __syncthreads();
    for (int e = c0 * topk + tid; e < c1 * topk; e += kRevThreads) {
      const int i = e / topk, sl = e - i * topk;
      if (sl < C[i]) atomicOr(&rows[I[e]], 1ull << (i - c0));
    }
    __syncthreads();
    for (int e = c0 * topk + tid; e < c1 * topk; e += kRevThreads) {
      const int i = e / topk, sl = e - i * topk;
      if (sl < C[i]) {
        const int m = I[e];
        const unsigned long long before = rows[m] & ((1ull << (i - c0)) - 1ull);
        list[cursor[m] + __popcll(before)] = i | (sl << 16);
      }
    }
    __syncthreads();
    for (int m = tid; m < nb; m += kRevThreads) cursor[m] += __popcll(rows[m]);
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kRevThreads) revidx_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt,
                                                            int32_t* __restrict__ rev_off,
                                                            int32_t* __restrict__ rev_list,
                                                            int nb, int topk) {
  revidx_pair(idx, cnt, rev_off, rev_list, nb, topk, blockIdx.x);
}

// The reverse lists together with the row statistics of the backward's
// dZ-tile path: workgroups 0 .. BH-1 build the lists (one pair each; these
// few latency-bound workgroups are dispatched first, so they run while the
// rest stream o and dO), the others compute four statistics units each
// (bwd_stats_unit, 256 threads per unit).
template <int D>
__global__ void __launch_bounds__(kRevThreads) revidx_stats_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int32_t* __restrict__ rev_off,
    int32_t* __restrict__ rev_list, int nb, int topk, int BH, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, float* __restrict__ stats,
    int Hq, int n, float tau, const int32_t* __restrict__ geo, int units) {
  if (int(blockIdx.x) < BH) {
    revidx_pair(idx, cnt, rev_off, rev_list, nb, topk, blockIdx.x);
    return;
  }
  const int unit = (int(blockIdx.x) - BH) * (kRevThreads / 256) + int(threadIdx.x) / 256;
  if (unit < units)   // uniform per 256-thread unit; no barrier follows
    bwd_stats_unit<D>(o, dO, lse, stats, Hq, n, tau, geo, nb, unit, int(threadIdx.x) % 256);
}

hipError_t launch_revidx(const int32_t* idx, const int32_t* cnt, int32_t* rev_off,
                         int32_t* rev_list, int BH, int nb, int topk, hipStream_t st) {
  ProfScope ps("sas_revidx_kernel", st);
  hipLaunchKernelGGL(revidx_kernel, dim3(BH), dim3(kRevThreads), 0, st, idx, cnt, rev_off, rev_list,
                     nb, topk);
  return hipGetLastError();
}

hipError_t launch_revidx_stats(const int32_t* idx, const int32_t* cnt, int32_t* rev_off,
                               int32_t* rev_list, int BH, int nb, int topk, const void* o,
                               const void* dO, const float* lse, float* stats, int B, int Hq, int n,
                               int d, float tau, const int32_t* geo, hipStream_t st) {
  ProfScope ps("sas_revidx_stats_kernel", st);
  const int units = B * Hq * nb;
  constexpr int per = kRevThreads / 256;
  const dim3 grid(BH + (units + per - 1) / per);
#define SAS_RS_ARGS idx, cnt, rev_off, rev_list, nb, topk, BH, (const uint16_t*)o, \
    (const uint16_t*)dO, lse, stats, Hq, n, tau, geo, units
  if (d == 128)
    hipLaunchKernelGGL((revidx_stats_kernel<128>), grid, dim3(kRevThreads), 0, st, SAS_RS_ARGS);
  else
    hipLaunchKernelGGL((revidx_stats_kernel<64>), grid, dim3(kRevThreads), 0, st, SAS_RS_ARGS);
#undef SAS_RS_ARGS
  return hipGetLastError();
}

}  // namespace sas
