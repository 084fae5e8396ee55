// Internal launcher declarations (host side).  Each launcher enqueues on the
// given stream and returns hipGetLastError() of its launch(es); argument
// checking happens in sas_api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sas {

// Profiling hooks used around every launch (no-ops unless enabled).
void prof_before(const char* name, hipStream_t st);
void prof_after(const char* name, hipStream_t st);

struct ProfScope {
  const char* name;
  hipStream_t st;
  ProfScope(const char* n, hipStream_t s) : name(n), st(s) { prof_before(name, st); }
  ~ProfScope() { prof_after(name, st); }
};

// ---- selection (select.hip)
// Training rows: rows = B*Hkv*nqb, q-block i = row % nqb, row stride nkb.
// Decode rows (seq_lens != nullptr): rows = B*Hkv, i = (clamp(len,1,cap)-1)/64.
hipError_t launch_mask_documents(const int32_t* doc_first, float* s, int B, int hkv, int nb,
                                 hipStream_t st);
hipError_t launch_select(const float* s, int32_t* idx, int32_t* cnt, float* log_gate,
                         float* s_lse, int rows, int nqb, int nkb, int topk,
                         const int32_t* seq_lens, int hkv, int cap, int gate, hipStream_t st);

// Block tables: geo is nullptr (block i = rows [64 i, 64 i + 64), nb = n/64)
// or a device int32 [B, nb, 2] table of (first token, length), see block_geo.

// ---- pooling (pool.hip); ws holds qbar and kbar (float32 [B*Hkv*nb*d] each)
hipError_t launch_pool(int dtype, const void* q, const void* k, float* s, float* ws, int B,
                       int Hq, int Hkv, int n, int d, const int32_t* geo, int nb, hipStream_t st);

// ---- reverse (per key block) lists (revidx.hip)
// rev_off [B*Hkv][nkb+1] (offsets into that pair's rev_list segment of
// nkb*(topk+1) entries); entries pack (i | slot<<16), slot 0xFFFF = own block.
hipError_t launch_revidx(const int32_t* idx, const int32_t* cnt, int32_t* rev_off,
                         int32_t* rev_list, int BH, int nb, int topk, hipStream_t st);
// The same lists plus, in the same launch, the bf16 backward's row statistics
// for its dZ-tile path (bwd_stats.h): stats [B*Hq*nb][128] float32.
hipError_t launch_revidx_stats(const int32_t* idx, const int32_t* cnt, int32_t* rev_off,
                               int32_t* rev_list, int BH, int nb, int topk, const void* o,
                               const void* dO, const float* lse, float* stats, int B, int Hq, int n,
                               int d, float tau, const int32_t* geo, hipStream_t st);

// ---- SIMT (float32) forward / backward (simt.hip)
hipError_t launch_fwd_simt(int dtype, const void* q, const void* k, const void* v,
                           const int32_t* idx, const int32_t* cnt, const float* lg, void* o,
                           float* lse, int B, int Hq, int Hkv, int n, int d, int topk,
                           float tau, int gate, const int32_t* geo, int nb, hipStream_t st);
hipError_t launch_bwd_simt(int dtype, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse, const int32_t* idx,
                           const int32_t* cnt, const float* lg, const float* s,
                           const float* s_lse, void* dq, void* dk, void* dv, float* ds,
                           float* Dws, const int32_t* rev_off, const int32_t* rev_list, int B,
                           int Hq, int Hkv, int n, int d, int topk, float tau, int gate,
                           const int32_t* geo, int nb, hipStream_t st);

// ---- decode (decode.hip)
// Workspace of a decode call whose rows are split over nsplit workgroups
// (unused when nsplit == 1): per (b, kv) row the selection (kept blocks or
// pages and base-2 log-gates, [B*Hkv][topk+1]; count [B*Hkv]), and per
// (b, head, split) the unnormalised partial output [.. * d] and (max, sum)
// [.. * 2].
struct DecodeScratch {
  int32_t* sel_blk;
  float* sel_gate;
  int32_t* sel_cnt;
  float* part_acc;
  float* part_ml;
};
int decode_nsplit(int B, int Hkv, int topk);
hipError_t launch_decode(int dtype, const void* q, const void* kc, const void* vc,
                         const int32_t* seq_lens, const float* s, int32_t* idx_out,
                         const DecodeScratch& ws, void* o, int B, int Hq, int Hkv, int cap, int d,
                         int topk, int nsplit, float tau, int gate, hipStream_t st);

// ---- paged decode (decode_paged.hip)
hipError_t launch_decode_paged(int dtype, const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* page_table, int num_pages, const int32_t* seq_lens,
                               const float* s, int32_t* idx_out, const DecodeScratch& ws, void* o,
                               int B, int Hq, int Hkv, int max_blocks, int d, int topk, int nsplit,
                               float tau, int gate, hipStream_t st);

}  // namespace sas
