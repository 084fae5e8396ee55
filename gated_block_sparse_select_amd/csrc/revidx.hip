// Reverse (per key block) lists for the key-block-outer backward pass.
//
// For each (batch, kv-head) and key block m, list every q-block whose key set
// contains m: block m itself (its own current block, always first) and then,
// in ascending order, each i > m that selected m.  Entries pack i | slot<<16,
// where slot is m's position in idx[i,:] (0xFFFF for the own block), so the
// consumer can read that pair's log-gate directly.
//
// One workgroup per (batch, kv-head).  Counts come from LDS atomics (order
// independent), offsets from a prefix sum, and the lists are filled in
// ascending i from an LDS bitmap rebuilt per chunk of 128 q-blocks, so the
// output is deterministic.
#include "common.h"
#include "launch.h"

namespace sas {

constexpr int kRevMaxNb = 2048;
constexpr int kChunk = 128;               // q-blocks per bitmap chunk
constexpr int kWords = kChunk / 32;

__global__ void __launch_bounds__(1024) revidx_kernel(const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ cnt,
                                                      int32_t* __restrict__ rev_off,
                                                      int32_t* __restrict__ rev_list, int nb,
                                                      int topk) {
  __shared__ int32_t cursor[kRevMaxNb + 1];
  __shared__ uint32_t bits[kRevMaxNb * kWords];
  const int bh = blockIdx.x;
  const int32_t* I = idx + size_t(bh) * nb * topk;
  const int32_t* C = cnt + size_t(bh) * nb;
  int32_t* off = rev_off + size_t(bh) * (nb + 1);
  int32_t* list = rev_list + size_t(bh) * nb * (topk + 1);
  const int tid = threadIdx.x;

  for (int m = tid; m <= nb; m += blockDim.x) cursor[m] = (m < nb) ? 1 : 0;
  __syncthreads();
  for (int e = tid; e < nb * topk; e += blockDim.x) {
    const int i = e / topk, sl = e % topk;
    if (sl < C[i]) atomicAdd(&cursor[I[e]], 1);
  }
  __syncthreads();
  // exclusive prefix sum over nb+1 entries (single thread: nb <= 2048)
  if (tid == 0) {
    int run = 0;
    for (int m = 0; m <= nb; ++m) {
      const int c = cursor[m];
      cursor[m] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int m = tid; m <= nb; m += blockDim.x) off[m] = cursor[m];
  for (int m = tid; m < nb; m += blockDim.x) list[cursor[m]] = m | int32_t(0xFFFF0000u);
  __syncthreads();
  for (int m = tid; m < nb; m += blockDim.x) cursor[m] += 1;

  for (int c0 = 0; c0 < nb; c0 += kChunk) {
    for (int w = tid; w < nb * kWords; w += blockDim.x) bits[w] = 0u;
    __syncthreads();
    const int c1 = min(nb, c0 + kChunk);
    for (int e = c0 * topk + tid; e < c1 * topk; e += blockDim.x) {
      const int i = e / topk, sl = e % topk;
      if (sl < C[i]) atomicOr(&bits[I[e] * kWords + (i - c0) / 32], 1u << ((i - c0) & 31));
    }
    __syncthreads();
    for (int m = tid; m < nb; m += blockDim.x) {
      int cur = cursor[m];
      for (int w = 0; w < kWords; ++w) {
        uint32_t x = bits[m * kWords + w];
        while (x) {
          const int bpos = __ffs(x) - 1;
          x &= x - 1;
          const int i = c0 + w * 32 + bpos;
          // m's slot in the ascending row idx[i, 0..cnt)
          int lo = 0, hi = C[i] - 1;
          const int32_t* row = I + size_t(i) * topk;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (row[mid] < m) lo = mid + 1; else hi = mid;
          }
          list[cur++] = i | (lo << 16);
        }
      }
      cursor[m] = cur;
    }
    __syncthreads();
  }
}

hipError_t launch_revidx(const int32_t* idx, const int32_t* cnt, int32_t* rev_off,
                         int32_t* rev_list, int BH, int nb, int topk, hipStream_t st) {
  ProfScope ps("sas_revidx_kernel", st);
  hipLaunchKernelGGL(revidx_kernel, dim3(BH), dim3(1024), 0, st, idx, cnt, rev_off, rev_list, nb,
                     topk);
  return hipGetLastError();
}

}  // namespace sas
