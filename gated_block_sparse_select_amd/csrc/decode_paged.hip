// Single-token decode over a paged KV pool: pages of one 64-token block,
// k_pages / v_pages [num_pages, Hkv, 64, d], with a page table [B, max_blocks]
// mapping each sequence's block m to its page (the serving-side cache of the
// SAS review page, paper.oopus.info, §2.6).  Same arithmetic as the
// contiguous decode; rows longer than 2048 blocks are selected by the whole
// workgroup.  The kernel template is in decode_kernel.h.
#include "decode_kernel.h"

namespace sas {

hipError_t launch_decode_paged(int dtype, const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* page_table, int num_pages, const int32_t* seq_lens,
                               const float* s, int32_t* idx_out, const DecodeScratch& ws, void* o,
                               int B, int Hq, int Hkv, int max_blocks, int d, int topk, int nsplit,
                               float tau, int gate, hipStream_t st) {
  return launch_decode_any<true>(dtype, q, k_pages, v_pages, page_table, num_pages, seq_lens, s,
                                 idx_out, ws, o, B, Hq, Hkv, max_blocks * SAS_BLK, d, topk, nsplit,
                                 tau, gate, st);
}

}  // namespace sas
