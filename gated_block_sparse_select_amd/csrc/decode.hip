// Single-token decode over a contiguous KV cache [B, Hkv, cap, d]; the kernel
// template is in decode_kernel.h.
#include "decode_kernel.h"

namespace sas {

int decode_nsplit(int B, int Hkv, int topk) {
  // one workgroup per row when there are enough rows to fill the GPU (two
  // per CU); otherwise split each row's tiles over several workgroups
  const int pairs = B * Hkv;
  int ns = (512 + pairs - 1) / pairs;
  if (ns > topk + 1) ns = topk + 1;
  if (ns < 1) ns = 1;
  return ns;
}

hipError_t launch_decode(int dtype, const void* q, const void* kc, const void* vc,
                         const int32_t* seq_lens, const float* s, int32_t* idx_out,
                         const DecodeScratch& ws, void* o, int B, int Hq, int Hkv, int cap, int d,
                         int topk, int nsplit, float tau, int gate, hipStream_t st) {
  return launch_decode_any<false>(dtype, q, kc, vc, nullptr, 0, seq_lens, s, idx_out, ws, o, B,
                                  Hq, Hkv, cap, d, topk, nsplit, tau, gate, st);
}

}  // namespace sas
