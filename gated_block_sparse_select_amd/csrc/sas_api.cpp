// C ABI of libsas: host-side argument checks, workspace carving and dispatch
// to the gfx950 kernels.  No entry point allocates device memory or
// synchronises; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sas.h"
#include "launch.h"

namespace sas {
// bf16 tensor-core kernels (mfma_fwd.hip / mfma_bwd.hip)
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* cnt, const float* lg, void* o, float* lse, int B,
                           int Hq, int Hkv, int n, int d, int topk, float tau, int gate,
                           const int32_t* geo, int nb, hipStream_t st);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, const int32_t* idx,
                           const int32_t* cnt, const float* lg, const float* s,
                           const float* s_lse, void* dq, void* dk, void* dv, float* ds,
                           float* Dws, const int32_t* rev_off, const int32_t* rev_list,
                           float* dlgp, void* dz, int B, int Hq, int Hkv, int n, int d,
                           int topk, float tau, int gate, const int32_t* geo, int nb,
                           hipStream_t st);
size_t bwd_mfma_extra_ws(int B, int Hq, int Hkv, int nb, int topk);
size_t bwd_dz_bytes(int B, int Hq, int nb, int topk);
bool mfma_supported(int d, int G);
}  // namespace sas

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool shape_ok_common(int B, int Hq, int Hkv, int len, int d, int topk, float scale, int gate) {
  if (B < 1 || Hq < 1 || Hkv < 1) return false;
  if (gate < SAS_GATE_SOFTMAX || gate > SAS_GATE_EXTERNAL) return false;
  if (Hq % Hkv != 0) return false;
  const int G = Hq / Hkv;
  if (G > 16) return false;
  if (len < SAS_BLOCK || len % SAS_BLOCK != 0) return false;
  if (len / SAS_BLOCK > SAS_MAX_BLOCKS) return false;
  if (d != 64 && d != 128) return false;
  if (topk < 0 || topk > SAS_MAX_BLOCKS) return false;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return false;
  // element counts must fit the 32-bit grid arithmetic used for block ids
  if (int64_t(B) * Hq * (len / SAS_BLOCK) > (int64_t(1) << 30)) return false;
  return true;
}

// Blocks of a training shape: n/64 without a table, else the table's nb.
int nblocks(const sas_shape* s) { return s->blocks ? s->nb : s->n / SAS_BLOCK; }

sas_status check_shape(const sas_shape* s) {
  if (!s) return SAS_ERR_ARG;
  if (s->dtype != SAS_F32 && s->dtype != SAS_BF16) return SAS_ERR_DTYPE;
  if (s->blocks == nullptr) {
    if (s->nb != 0 && s->nb != s->n / SAS_BLOCK) return SAS_ERR_ARG;
    if (!shape_ok_common(s->B, s->Hq, s->Hkv, s->n, s->d, s->topk, s->scale, s->gate))
      return SAS_ERR_ARG;
    return SAS_OK;
  }
  // a block table: the limits of a shape with nb blocks of 64, with n free (>= 64)
  if (s->nb < 1 || s->nb > SAS_MAX_BLOCKS || s->n < SAS_BLOCK || s->n > SAS_BLOCK * SAS_MAX_BLOCKS)
    return SAS_ERR_ARG;
  if (!shape_ok_common(s->B, s->Hq, s->Hkv, s->nb * SAS_BLOCK, s->d, s->topk, s->scale, s->gate))
    return SAS_ERR_ARG;
  if (int64_t(s->B) * s->Hq * s->n > (int64_t(1) << 40)) return SAS_ERR_ARG;
  return SAS_OK;
}

sas_status check_dshape(const sas_decode_shape* s) {
  if (!s) return SAS_ERR_ARG;
  if (s->dtype != SAS_F32 && s->dtype != SAS_BF16) return SAS_ERR_DTYPE;
  if (!shape_ok_common(s->B, s->Hq, s->Hkv, s->cap, s->d, s->topk, s->scale, s->gate))
    return SAS_ERR_ARG;
  return SAS_OK;
}

sas_status check_pshape(const sas_decode_paged_shape* s) {
  if (!s) return SAS_ERR_ARG;
  if (s->dtype != SAS_F32 && s->dtype != SAS_BF16) return SAS_ERR_DTYPE;
  if (s->max_blocks < 1 || s->max_blocks > SAS_MAX_DECODE_BLOCKS || s->num_pages < 1)
    return SAS_ERR_ARG;
  // the remaining limits are those of a decode shape whose cap is one block
  if (!shape_ok_common(s->B, s->Hq, s->Hkv, SAS_BLOCK, s->d, s->topk, s->scale, s->gate))
    return SAS_ERR_ARG;
  if (int64_t(s->B) * s->Hkv * s->max_blocks > (int64_t(1) << 30)) return SAS_ERR_ARG;
  return SAS_OK;
}

// the paged decode's workspace is laid out like the contiguous decode's
sas_decode_shape as_decode_shape(const sas_decode_paged_shape* s) {
  sas_decode_shape d{};
  d.B = s->B;
  d.Hq = s->Hq;
  d.Hkv = s->Hkv;
  d.cap = SAS_BLOCK;
  d.d = s->d;
  d.topk = s->topk;
  d.scale = s->scale;
  d.dtype = s->dtype;
  d.gate = s->gate;
  return d;
}

float tau_of(float scale, int d) { return scale > 0.f ? scale : 1.0f / std::sqrt(float(d)); }

thread_local hipError_t g_last_hip = hipSuccess;

sas_status from_hip(hipError_t e) {
  if (e == hipSuccess) return SAS_OK;
  g_last_hip = e;
  return SAS_ERR_HIP;
}

// hipGetLastError() reports the last error of ANY runtime call on this thread;
// drop whatever an unrelated earlier call left there before our launches.
void clear_stale_error() { (void)hipGetLastError(); }

// ----------------------------------------------------------- bwd workspace
// The bf16 backward stores dZ (one 64 x 64 bf16 tile per head, q-block and
// kept or own block) when the workspace has room for it and the tiles take
// at most kDzMaxBytes; otherwise (and for the external gate, the float32
// path and a smaller workspace) dq recomputes S and dP instead.
constexpr size_t kDzMaxBytes = size_t(16) << 30;
struct BwdWs {
  size_t D_off, off_off, list_off, dlg_off, total, dz_off, total_dz;
};
BwdWs bwd_layout(const sas_shape* s) {
  const size_t nb = size_t(nblocks(s));
  const size_t BH = size_t(s->B) * s->Hkv;
  BwdWs w{};
  w.D_off = 0;
  // row statistics: SIMT path D [B,Hq,n]; MFMA path [-lse/tau | -D] per block's 64 window rows
  const size_t rows = std::max(size_t(s->n), nb * SAS_BLOCK);
  w.off_off = align_up(w.D_off + 2 * sizeof(float) * size_t(s->B) * s->Hq * rows);
  w.list_off = align_up(w.off_off + sizeof(int32_t) * BH * (nb + 1));
  w.dlg_off = align_up(w.list_off + sizeof(int32_t) * BH * nb * (size_t(s->topk) + 1));
  w.total = align_up(w.dlg_off + sas::bwd_mfma_extra_ws(s->B, s->Hq, s->Hkv, int(nb), s->topk));
  w.dz_off = w.total;
  w.total_dz = w.total;
  const size_t dzb = sas::bwd_dz_bytes(s->B, s->Hq, int(nb), s->topk);
  if (s->dtype == SAS_BF16 && s->gate != SAS_GATE_EXTERNAL &&
      sas::mfma_supported(s->d, s->Hq / s->Hkv) && dzb <= kDzMaxBytes)
    w.total_dz = align_up(w.dz_off + dzb);
  return w;
}

// ----------------------------------------------------------- decode workspace
// When a row's tiles are split over several workgroups: the row's selection
// (kept blocks / pages, base-2 log-gates, count) and the split workgroups'
// partial outputs with (max, sum); a small minimum otherwise.
struct DecWs {
  size_t blk_off, gate_off, cnt_off, acc_off, ml_off, total;
  int nsplit;
};
DecWs dec_layout(const sas_decode_shape* s) {
  DecWs w{};
  w.nsplit = sas::decode_nsplit(s->B, s->Hkv, s->topk);
  const bool split = w.nsplit > 1;
  const size_t rows = split ? size_t(s->B) * s->Hkv : 0;
  const size_t ent = rows * (size_t(s->topk) + 1);
  const size_t parts = split ? size_t(s->B) * s->Hq * w.nsplit : 0;
  w.blk_off = 0;
  w.gate_off = align_up(w.blk_off + sizeof(int32_t) * ent);
  w.cnt_off = align_up(w.gate_off + sizeof(float) * ent);
  w.acc_off = align_up(w.cnt_off + sizeof(int32_t) * rows);
  w.ml_off = align_up(w.acc_off + sizeof(float) * parts * s->d);
  w.total = align_up(w.ml_off + sizeof(float) * parts * 2 + 1);
  return w;
}
sas::DecodeScratch dec_scratch(const DecWs& w, void* base_v) {
  char* base = static_cast<char*>(base_v);
  return sas::DecodeScratch{reinterpret_cast<int32_t*>(base + w.blk_off),
                            reinterpret_cast<float*>(base + w.gate_off),
                            reinterpret_cast<int32_t*>(base + w.cnt_off),
                            reinterpret_cast<float*>(base + w.acc_off),
                            reinterpret_cast<float*>(base + w.ml_off)};
}

}  // namespace

// ----------------------------------------------------------- no-allocation scratch
// The decode scratch of sas_decode_noalloc: one copy per GPU in the library's
// code object.  In host code `scratch` names a host-side stand-in, not device
// memory; host code uses only the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SAS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`, resolved once
// per device with that device current.
sas_status scratch_of(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return SAS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return from_hip(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return from_hip(e);
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return from_hip(e);
    if (es != hipSuccess) return from_hip(es);
    if (!p) return from_hip(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SAS_OK;
}

// ----------------------------------------------------------- profiling state
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
struct ProfState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<ProfRec> pending;
  std::vector<const char*> names;
  std::vector<double> ms;
  std::vector<int32_t> launches;
  hipEvent_t open = nullptr;
} g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace sas {
void prof_before(const char*, hipStream_t st) {
  if (!g_prof.on) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.open = prof_event();
  if (g_prof.open) hipEventRecord(g_prof.open, st);
}
void prof_after(const char* name, hipStream_t st) {
  if (!g_prof.on) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.open) return;
  hipEvent_t e = prof_event();
  if (!e) return;
  hipEventRecord(e, st);
  g_prof.pending.push_back({name, g_prof.open, e});
  g_prof.open = nullptr;
}
}  // namespace sas

extern "C" {

int32_t sas_abi_version(void) { return 4; }

const char* sas_status_string(sas_status st) {
  switch (st) {
    case SAS_OK: return "SAS_OK";
    case SAS_ERR_ARG: return "SAS_ERR_ARG: invalid pointer, size or shape";
    case SAS_ERR_DTYPE: return "SAS_ERR_DTYPE: dtype must be SAS_F32 or SAS_BF16";
    case SAS_ERR_UNSUPPORTED: return "SAS_ERR_UNSUPPORTED: valid but not implemented";
    case SAS_ERR_WORKSPACE: return "SAS_ERR_WORKSPACE: workspace missing or too small";
    case SAS_ERR_HIP: return "SAS_ERR_HIP: kernel launch failed";
    default: return "SAS: unknown status";
  }
}

size_t sas_pool_workspace_bytes(const sas_shape* s) {
  if (check_shape(s) != SAS_OK) return 0;
  return align_up(2 * sizeof(float) * size_t(s->B) * s->Hkv * size_t(nblocks(s)) * s->d);
}

sas_status sas_pool_scores(const sas_shape* s, const void* q, const void* k, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  sas_status st = check_shape(s);
  if (st != SAS_OK) return st;
  if (!q || !k || !out) return SAS_ERR_ARG;
  if (!ws || ws_bytes < sas_pool_workspace_bytes(s)) return SAS_ERR_WORKSPACE;
  clear_stale_error();
  return from_hip(sas::launch_pool(s->dtype, q, k, out, (float*)ws, s->B, s->Hq, s->Hkv, s->n,
                                   s->d, s->blocks, nblocks(s), stream));
}

sas_status sas_select(const sas_shape* s, const float* sc, int32_t* idx, int32_t* cnt,
                      float* log_gate, float* s_lse, hipStream_t stream) {
  sas_status st = check_shape(s);
  if (st != SAS_OK) return st;
  if (!sc || !cnt || !s_lse) return SAS_ERR_ARG;
  if (s->topk > 0 && (!idx || !log_gate)) return SAS_ERR_ARG;
  const int nb = nblocks(s);
  clear_stale_error();
  return from_hip(sas::launch_select(sc, idx, cnt, log_gate, s_lse, s->B * s->Hkv * nb, nb, nb,
                                     s->topk, nullptr, s->Hkv, s->n, s->gate, stream));
}

sas_status sas_mask_documents(const sas_shape* s, const int32_t* doc_first, float* sc,
                              hipStream_t stream) {
  sas_status st = check_shape(s);
  if (st != SAS_OK) return st;
  if (!doc_first || !sc) return SAS_ERR_ARG;
  clear_stale_error();
  return from_hip(sas::launch_mask_documents(doc_first, sc, s->B, s->Hkv, nblocks(s), stream));
}

sas_status sas_fwd(const sas_shape* s, const void* q, const void* k, const void* v,
                   const int32_t* idx, const int32_t* cnt, const float* log_gate, void* o,
                   float* lse, hipStream_t stream) {
  sas_status st = check_shape(s);
  if (st != SAS_OK) return st;
  if (!q || !k || !v || !cnt || !o || !lse) return SAS_ERR_ARG;
  if (s->topk > 0 && (!idx || !log_gate)) return SAS_ERR_ARG;
  const float tau = tau_of(s->scale, s->d);
  const int G = s->Hq / s->Hkv;
  clear_stale_error();
  if (s->dtype == SAS_BF16 && sas::mfma_supported(s->d, G))
    return from_hip(sas::launch_fwd_mfma(q, k, v, idx, cnt, log_gate, o, lse, s->B, s->Hq, s->Hkv,
                                         s->n, s->d, s->topk, tau, s->gate, s->blocks,
                                         nblocks(s), stream));
  return from_hip(sas::launch_fwd_simt(s->dtype, q, k, v, idx, cnt, log_gate, o, lse, s->B, s->Hq,
                                       s->Hkv, s->n, s->d, s->topk, tau, s->gate, s->blocks,
                                       nblocks(s), stream));
}

size_t sas_bwd_workspace_bytes(const sas_shape* s) {
  if (check_shape(s) != SAS_OK) return 0;
  return bwd_layout(s).total_dz;
}

size_t sas_bwd_min_workspace_bytes(const sas_shape* s) {
  if (check_shape(s) != SAS_OK) return 0;
  return bwd_layout(s).total;
}

sas_status sas_bwd(const sas_shape* s, const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, const int32_t* idx, const int32_t* cnt,
                   const float* log_gate, const float* sc, const float* s_lse, void* dq, void* dk,
                   void* dv, float* ds, void* ws, size_t ws_bytes, hipStream_t stream) {
  sas_status st = check_shape(s);
  if (st != SAS_OK) return st;
  if (!q || !k || !v || !o || !dO || !lse || !cnt || !sc || !s_lse || !dq || !dk || !dv || !ds)
    return SAS_ERR_ARG;
  if (s->topk > 0 && (!idx || !log_gate)) return SAS_ERR_ARG;
  const BwdWs w = bwd_layout(s);
  if (!ws || ws_bytes < w.total) return SAS_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* Dws = reinterpret_cast<float*>(base + w.D_off);
  int32_t* rev_off = reinterpret_cast<int32_t*>(base + w.off_off);
  int32_t* rev_list = reinterpret_cast<int32_t*>(base + w.list_off);
  const int nb = nblocks(s);
  const float tau = tau_of(s->scale, s->d);
  clear_stale_error();
  const int G = s->Hq / s->Hkv;
  const bool mfma = s->dtype == SAS_BF16 && sas::mfma_supported(s->d, G);
  // the dZ-tile path (bf16, a gate other than the external one, tiles within
  // the cap, a workspace that holds them); its statistics pass runs in the
  // reverse-list launch
  void* dz = mfma && w.total_dz > w.total && ws_bytes >= w.total_dz ? base + w.dz_off : nullptr;
  hipError_t e = dz != nullptr
                     ? sas::launch_revidx_stats(idx, cnt, rev_off, rev_list, s->B * s->Hkv, nb,
                                                s->topk, o, dO, lse, Dws, s->B, s->Hq, s->n, s->d,
                                                tau, s->blocks, stream)
                     : sas::launch_revidx(idx, cnt, rev_off, rev_list, s->B * s->Hkv, nb, s->topk,
                                          stream);
  if (e != hipSuccess) return from_hip(e);
  if (mfma) {
    return from_hip(sas::launch_bwd_mfma(
        q, k, v, o, dO, lse, idx, cnt, log_gate, sc, s_lse, dq, dk, dv, ds, Dws, rev_off, rev_list,
        reinterpret_cast<float*>(base + w.dlg_off), dz, s->B, s->Hq, s->Hkv, s->n, s->d, s->topk,
        tau, s->gate, s->blocks, nb, stream));
  }
  return from_hip(sas::launch_bwd_simt(s->dtype, q, k, v, o, dO, lse, idx, cnt, log_gate, sc, s_lse,
                                       dq, dk, dv, ds, Dws, rev_off, rev_list, s->B, s->Hq, s->Hkv,
                                       s->n, s->d, s->topk, tau, s->gate, s->blocks, nb, stream));
}

size_t sas_decode_workspace_bytes(const sas_decode_shape* s) {
  if (check_dshape(s) != SAS_OK) return 0;
  return dec_layout(s).total;
}

sas_status sas_decode(const sas_decode_shape* s, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* seq_lens, const float* sc, void* o,
                      int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  sas_status st = check_dshape(s);
  if (st != SAS_OK) return st;
  if (!q || !k_cache || !v_cache || !seq_lens || !sc || !o) return SAS_ERR_ARG;
  const DecWs w = dec_layout(s);
  if (!ws || ws_bytes < w.total) return SAS_ERR_WORKSPACE;
  clear_stale_error();
  return from_hip(sas::launch_decode(s->dtype, q, k_cache, v_cache, seq_lens, sc, idx_out,
                                     dec_scratch(w, ws), o, s->B, s->Hq, s->Hkv, s->cap, s->d,
                                     s->topk, w.nsplit, tau_of(s->scale, s->d), s->gate, stream));
}

sas_status sas_decode_noalloc(const sas_decode_shape* s, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens, const float* sc,
                              void* o, int32_t* idx_out, hipStream_t stream) {
  sas_status st = check_dshape(s);
  if (st != SAS_OK) return st;
  if (!q || !k_cache || !v_cache || !seq_lens || !sc || !o) return SAS_ERR_ARG;
  const DecWs w = dec_layout(s);
  if (w.total > size_t(SAS_NOALLOC_SCRATCH_BYTES)) return SAS_ERR_WORKSPACE;
  void* base_v = nullptr;
  if ((st = scratch_of(stream, &base_v)) != SAS_OK) return st;
  clear_stale_error();
  return from_hip(sas::launch_decode(s->dtype, q, k_cache, v_cache, seq_lens, sc, idx_out,
                                     dec_scratch(w, base_v), o, s->B, s->Hq, s->Hkv, s->cap, s->d,
                                     s->topk, w.nsplit, tau_of(s->scale, s->d), s->gate, stream));
}

size_t sas_decode_paged_workspace_bytes(const sas_decode_paged_shape* s) {
  if (check_pshape(s) != SAS_OK) return 0;
  const sas_decode_shape d = as_decode_shape(s);
  return dec_layout(&d).total;
}

sas_status sas_decode_paged(const sas_decode_paged_shape* s, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* page_table,
                            const int32_t* seq_lens, const float* sc, void* o, int32_t* idx_out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  sas_status st = check_pshape(s);
  if (st != SAS_OK) return st;
  if (!q || !k_pages || !v_pages || !page_table || !seq_lens || !sc || !o) return SAS_ERR_ARG;
  const sas_decode_shape d = as_decode_shape(s);
  const DecWs w = dec_layout(&d);
  if (!ws || ws_bytes < w.total) return SAS_ERR_WORKSPACE;
  clear_stale_error();
  return from_hip(sas::launch_decode_paged(s->dtype, q, k_pages, v_pages, page_table, s->num_pages,
                                           seq_lens, sc, idx_out, dec_scratch(w, ws), o, s->B,
                                           s->Hq, s->Hkv, s->max_blocks, s->d, s->topk, w.nsplit,
                                           tau_of(s->scale, s->d), s->gate, stream));
}

int32_t sas_blocks_from_cu_seqlens(const int32_t* cu, int32_t ndocs, int32_t* blocks,
                                   int32_t* doc_first, int32_t max_blocks) {
  if (!cu || ndocs < 0 || max_blocks < 0 || (max_blocks > 0 && (!blocks || !doc_first)))
    return -1;
  if (cu[0] != 0) return -1;
  int64_t need = 0;
  for (int32_t j = 0; j < ndocs; ++j) {
    if (cu[j + 1] < cu[j]) return -1;
    need += (int64_t(cu[j + 1]) - cu[j] + SAS_BLOCK - 1) / SAS_BLOCK;
  }
  if (need > max_blocks) return -1;
  int32_t nb = 0;
  for (int32_t j = 0; j < ndocs; ++j) {
    const int32_t first = nb;
    for (int32_t a = cu[j]; a < cu[j + 1]; a += SAS_BLOCK) {
      blocks[2 * nb] = a;
      blocks[2 * nb + 1] = std::min(SAS_BLOCK, cu[j + 1] - a);
      doc_first[nb] = first;
      ++nb;
    }
  }
  return nb;
}

const char* sas_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

sas_status sas_prof_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  return SAS_OK;
}

int32_t sas_prof_collect(const char** names, double* total_ms, int32_t* launches, int32_t max) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (const ProfRec& r : g_prof.pending) {
    float ms = 0.f;
    hipEventSynchronize(r.b);
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) ms = 0.f;
    size_t j = 0;
    for (; j < g_prof.names.size(); ++j)
      if (std::strcmp(g_prof.names[j], r.name) == 0) break;
    if (j == g_prof.names.size()) {
      g_prof.names.push_back(r.name);
      g_prof.ms.push_back(0.0);
      g_prof.launches.push_back(0);
    }
    g_prof.ms[j] += ms;
    g_prof.launches[j] += 1;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.pending.clear();
  const int32_t n = int32_t(g_prof.names.size());
  for (int32_t j = 0; j < n && j < max; ++j) {
    if (names) names[j] = g_prof.names[j];
    if (total_ms) total_ms[j] = g_prof.ms[j];
    if (launches) launches[j] = g_prof.launches[j];
  }
  // reset the accumulators so that the next collect covers a new interval
  g_prof.names.clear();
  g_prof.ms.clear();
  g_prof.launches.clear();
  return n;
}

}  // extern "C"
