// Top-K block selection kernel: one wave64 per score row (training rows, or
// decode rows whose current block comes from seq_lens); the per-row logic is
// select_row.
#include "launch.h"
#include "select_row.h"

namespace sas {

template <int CPL>
__global__ void __launch_bounds__(64) select_kernel(const float* __restrict__ s,
                                                    int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ cnt,
                                                    float* __restrict__ lg,
                                                    float* __restrict__ slse, int rows,
                                                    int nqb, int nkb, int topk,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int hkv, int cap, int gate) {
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
  int32_t* irow = idx + size_t(row) * topk;
  float* grow = lg + size_t(row) * topk;
  float lse;
  const int keff = select_row<CPL>(s + size_t(row) * nkb, i, i, topk, gate, lane, lse, NoTag{},
                                   [&](int pos, int m, int, float g) {
                                     irow[pos] = m;
                                     grow[pos] = g;
                                   });
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
               int nqb, int nkb, int topk, const int32_t* sl, int hkv, int cap, int gate,
               hipStream_t st) {
  hipLaunchKernelGGL(select_kernel<CPL>, dim3(rows), dim3(64), 0, st, s, idx, cnt, lg, slse, rows,
                     nqb, nkb, topk, sl, hkv, cap, gate);
}

hipError_t launch_select(const float* s, int32_t* idx, int32_t* cnt, float* lg, float* slse,
                         int rows, int nqb, int nkb, int topk, const int32_t* seq_lens, int hkv,
                         int cap, int gate, hipStream_t st) {
  ProfScope ps("sas_select_kernel", st);
  switch (select_cpl(nkb)) {
    case 1: go<1>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, gate, st); break;
    case 2: go<2>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, gate, st); break;
    case 4: go<4>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, gate, st); break;
    case 8: go<8>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, gate, st); break;
    case 16: go<16>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, gate, st); break;
    default: go<32>(s, idx, cnt, lg, slse, rows, nqb, nkb, topk, seq_lens, hkv, cap, gate, st); break;
  }
  return hipGetLastError();
}

// Packed batches: s[b,kv,i,m] = -inf for m < first block of block i's
// document, which takes those blocks out of row i's candidates.  One 256-thread
// workgroup per score row; a row writes at most i floats.
__global__ void __launch_bounds__(256) mask_documents_kernel(const int32_t* __restrict__ doc_first,
                                                             float* __restrict__ s, int hkv,
                                                             int nb) {
  const size_t row = blockIdx.x;          // (b, kv, i)
  const int i = int(row % nb);
  const int b = int(row / (size_t(nb) * hkv));
  int f = doc_first[size_t(b) * nb + i];
  f = f < 0 ? 0 : (f > i ? i : f);
  float* srow = s + row * nb;
  for (int m = threadIdx.x; m < f; m += 256) srow[m] = -INFINITY;
}

hipError_t launch_mask_documents(const int32_t* doc_first, float* s, int B, int hkv, int nb,
                                 hipStream_t st) {
  ProfScope ps("sas_mask_documents_kernel", st);
  hipLaunchKernelGGL(mask_documents_kernel, dim3(size_t(B) * hkv * nb), dim3(256), 0, st,
                     doc_first, s, hkv, nb);
  return hipGetLastError();
}

}  // namespace sas
