/*
 * sas.h - C ABI of libsas: SAS gated block-sparse attention on AMD MI355X (gfx950).
 *
 * What is computed (sources: the Chinese review page "论文综述：SAS——通过端到端
 * 优化上下文排序实现简单的注意力稀疏化" on paper.oopus.info, cited as [Review];
 * the project README on gitee, cited as [README]):
 *
 *   The sequence is cut into blocks of b = 64 tokens [Review §2.1].  For every
 *   (batch b, kv-head kv, 64-query block i) a score row s[b,kv,i,:] rates the
 *   history blocks m < i [Review §2.2, selector equation].  The Top-K history
 *   blocks are kept; each kept block m adds the log-gate
 *       log g_m = s_m - LSE(s over ALL history blocks m' < i)
 *   [Review §2.4, equation for log g_m] to the logits of its 64 keys; the
 *   current block i is always kept, causally masked (key j <= query t), with
 *   no bias (g_0 = 1); every other block is skipped:
 *       o = softmax(tau * q K_S^T + log g_S) V_S      [Review §2.3, equation]
 *   The backward returns dq, dk, dv and ds, where the gate gradient of a kept
 *   block is the sum of its logit gradients [Review §2.6] pushed through the
 *   softmax Jacobian of the normalised gate.  Top-K itself is discrete and gets
 *   no gradient [README, figure caption (b)].
 *
 * Conventions shared by every entry point
 *   - The query heads of a group share one selection: query head h reads
 *     kv-head h / G with G = Hq / Hkv (contiguous grouping).
 *   - tau = shape->scale, or 1/sqrt(d) when scale == 0.  The gate is never scaled.
 *   - All tensors are dense, row-major, contiguous DEVICE buffers that the caller
 *     owns; the library keeps no pointer after a call returns and allocates no
 *     device memory (scratch comes from the caller's workspace argument).
 *   - Every call validates its arguments on the host and then enqueues its
 *     kernels on `stream` (hipStream_t; NULL = the null stream) and returns
 *     without synchronising.  A nonzero status other than SAS_ERR_HIP means
 *     nothing was enqueued.  SAS_ERR_HIP reports a failed launch.
 *   - Outputs take the dtype of the inputs (q, k, v, o, dO, dq, dk, dv, decode
 *     caches); s, log_gate, s_lse, lse and ds are always float32; idx and cnt int32.
 *   - Calls are reentrant; calls on different streams may run concurrently as
 *     long as their output buffers do not overlap.
 *   - A score of -inf marks a history block that is not a candidate (in a
 *     packed batch, a block of an earlier document): it is left out of the
 *     gate's LSE, never kept, and gets ds = 0.  Other scores must be finite
 *     (NaN or +inf in s is undefined behaviour).
 */
#ifndef SAS_H_
#define SAS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sas_status;
#define SAS_OK 0
#define SAS_ERR_ARG 1          /* bad pointer, size or shape */
#define SAS_ERR_DTYPE 2        /* dtype not SAS_F32 / SAS_BF16 */
#define SAS_ERR_UNSUPPORTED 3  /* valid but outside what the kernels implement */
#define SAS_ERR_WORKSPACE 4    /* workspace missing or smaller than required */
#define SAS_ERR_HIP 5          /* a kernel launch failed (hipGetLastError) */

#define SAS_F32 0
#define SAS_BF16 1

#define SAS_BLOCK 64           /* tokens per block [Review §2.1] */

/* Gate kinds (the `gate` field of every shape).  The selection is the same
 * Top-K for all of them; they differ in the gate a kept block m of row i gets
 * and in where it acts.  LSE runs over the row's candidates.
 *   SAS_GATE_SOFTMAX   the method [Review §2.4]: log g_m = s_m - LSE(s), added
 *                      to the logits of block m inside the softmax.
 *   SAS_GATE_SIGMOID   normalisation ablation [Review §2.4, ablation table of
 *                      §4]: log g_m = log sigmoid(s_m), inside the softmax;
 *                      ds[i,m] = [m kept] dlg[i,m] sigmoid(-s[i,m]).
 *   SAS_GATE_HARD      hard-gate ablation [Review §2.5]: g_m = 1 on kept blocks
 *                      (log_gate = 0), trained with a straight-through
 *                      estimator: ds is that of SAS_GATE_SOFTMAX for the bias
 *                      gradients dlg of this forward.
 *   SAS_GATE_EXTERNAL  placement ablation [Review §2.3]: g_m = exp(s_m - LSE(s))
 *                      scales the values of block m after an unbiased softmax
 *                      over the kept and current keys:
 *                        o = sum_j P_j g_block(j) v_j,  P = softmax(tau q K_S^T)
 *                      (g = 1 for the current block; lse is that softmax's);
 *                      dlg[i,m] = sum over block m's keys of P * dP with
 *                      dP = g (dO . v), and ds as for SAS_GATE_SOFTMAX.  Gates
 *                      below e^-60 act as e^-60 (a relative change in o below
 *                      1e-26). */
#define SAS_GATE_SOFTMAX 0
#define SAS_GATE_SIGMOID 1
#define SAS_GATE_HARD 2
#define SAS_GATE_EXTERNAL 3
#define SAS_MAX_BLOCKS 2048    /* most blocks per sequence (n or cap <= 131072) */

/* Training-layer shape.  q [B,Hq,n,d]; k, v [B,Hkv,n,d].
 * Requires B,Hq,Hkv >= 1, Hq % Hkv == 0, 1 <= Hq/Hkv <= 16, d in {64,128},
 * 0 <= topk <= SAS_MAX_BLOCKS (a row with fewer history blocks keeps all of
 * them), scale >= 0 and finite, dtype SAS_F32 or SAS_BF16, gate one of the
 * SAS_GATE_* kinds.  sas_select, sas_fwd, sas_bwd and the decode calls must
 * see the same gate.
 *
 * Blocks.  With blocks == NULL the sequence is cut into nb = n/64 blocks of
 * 64 tokens (n % 64 == 0, 64 <= n <= 64*SAS_MAX_BLOCKS; nb may be given as 0
 * or n/64).  Otherwise blocks is a DEVICE int32 table [B, nb, 2] giving, for
 * block i of batch entry b, its first token and its number of tokens
 * (1..64, or 0 for a padding block that holds none), and 1 <= nb <=
 * SAS_MAX_BLOCKS, 64 <= n <= 64*SAS_MAX_BLOCKS.  This is the layout of packed documents of any
 * length [Review §2.2 and §2.4 applied per document]: each document is cut
 * into 64-token blocks from its own first token, so only its last block may
 * be shorter; blocks are listed in token order; padding blocks come last.
 * sas_blocks_from_cu_seqlens builds the table.  A block's tokens must lie in
 * [0, n) and every block but a document's last must hold 64 tokens; table
 * entries outside these rules are clamped on the device (nothing outside the
 * tensors is read or written) and give unspecified results.  Every row of q,
 * k, v and dO must hold finite values, also rows outside every block; the
 * outputs o, lse, dq, dk and dv are written on the rows of the blocks only.
 * All per-block tensors (s, idx, cnt, log_gate, s_lse, ds and the
 * doc_first table) have nb in place of n/64. */
typedef struct {
  int32_t B, Hq, Hkv, n, d, topk;
  float scale;
  int32_t dtype;
  int32_t gate;
  int32_t nb;             /* number of blocks (0: n/64 when blocks == NULL) */
  const int32_t* blocks;  /* NULL, or device int32 [B, nb, 2] (first token, length) */
} sas_shape;

/* Decode shape.  q [B,Hq,d]; k_cache, v_cache [B,Hkv,cap,d]; same limits with
 * cap in place of n. */
typedef struct {
  int32_t B, Hq, Hkv, cap, d, topk;
  float scale;
  int32_t dtype;
  int32_t gate;
} sas_decode_shape;

#define SAS_MAX_DECODE_BLOCKS 8192  /* most blocks per sequence in paged decode (context <= 524288) */

/* Paged decode shape.  The KV cache is a pool of num_pages pages, each holding
 * one 64-token block of every kv-head: k_pages, v_pages [num_pages,Hkv,64,d].
 * Block m of sequence b lives in page page_table[b,m] (int32 [B,max_blocks]).
 * q [B,Hq,d]; s float32 [B,Hkv,max_blocks].  Same limits as sas_shape with
 * 64*max_blocks in place of n, except 1 <= max_blocks <= SAS_MAX_DECODE_BLOCKS;
 * num_pages >= 1; 0 <= topk <= SAS_MAX_BLOCKS. */
typedef struct {
  int32_t B, Hq, Hkv, max_blocks, num_pages, d, topk;
  float scale;
  int32_t dtype;
  int32_t gate;
} sas_decode_paged_shape;

/* Version of this ABI (bumped on any incompatible change): 4. */
int32_t sas_abi_version(void);

/* Human-readable text of a status code (static storage, never NULL). */
const char* sas_status_string(sas_status st);

/* ---------------------------------------------------------------- pooling
 * Stand-in selector (mean pooling) of the 32K training workload; a score per
 * history block from q and K_{B_m} as in [Review §2.2, selector equation].
 *   s[b,kv,i,m] = qbar[b,kv,i] . kbar[b,kv,m] / sqrt(d)   for ALL i, m
 * qbar = mean of q over the tokens of q-block i (64 rows, or the block's
 * rows of the blocks table) and the G heads of group kv; kbar = mean of k over
 * the tokens of block m; an empty padding block has mean 0.  Means accumulate
 * in float32.
 *   q, k: device, shape->dtype.  s: device float32 [B,Hkv,nb,nb] (written).
 *   ws: device scratch of at least sas_pool_workspace_bytes(shape) bytes. */
size_t sas_pool_workspace_bytes(const sas_shape* shape);
sas_status sas_pool_scores(const sas_shape* shape, const void* q, const void* k, float* s,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- selection
 * LSE-normalise and Top-K block-index builder [Review §2.2, §2.4].
 * For each row (b,kv,i) with candidates C = {m < i : s[b,kv,i,m] > -inf}:
 *   s_lse[b,kv,i]   = log sum_{m in C} exp s[b,kv,i,m]       (-inf when C is empty)
 *   cnt[b,kv,i]     = min(topk, |C|)
 *   idx[b,kv,i,:]   = the cnt candidates with the largest scores, ties to the
 *                     lower index (-0.0 == +0.0), listed in ascending order, then
 *                     padded with -1 up to topk
 *   log_gate[b,kv,i,j] = s[b,kv,i,idx[j]] - s_lse (j < cnt), -inf in the padding
 *                     (for the gate kinds: log sigmoid(s), 0 for SAS_GATE_HARD)
 * s: device float32 [B,Hkv,nb,nb]; entries m >= i are never read.
 * idx: int32 [B,Hkv,nb,topk]; cnt: int32 [B,Hkv,nb];
 * log_gate: float32 [B,Hkv,nb,topk]; s_lse: float32 [B,Hkv,nb] (all written).
 * idx and log_gate may be NULL when topk == 0. */
sas_status sas_select(const sas_shape* shape, const float* s, int32_t* idx, int32_t* cnt,
                      float* log_gate, float* s_lse, hipStream_t stream);

/* ---------------------------------------------------------------- packed batches
 * Several documents packed into one sequence [Review §2.2 and §2.4, applied
 * per document]: with the blocks table of the shape, each document is cut
 * into 64-token blocks from its own first token.  A q-block attends only to
 * blocks of its own document: this call sets, in place,
 *   s[b,kv,i,m] = -inf   for m < doc_first[b,i]
 * and leaves every other entry unchanged; sas_select, sas_fwd, sas_bwd and
 * sas_decode then treat those blocks as non-candidates (see the -inf rule
 * above), so the packed run gives each document what a run over it alone gives.
 *   doc_first: device int32 [B,nb], the first block of the document holding
 *              block i (0 <= doc_first[b,i] <= i; other values are clamped to
 *              that range).
 *   s: device float32 [B,Hkv,nb,nb], modified in place. */
sas_status sas_mask_documents(const sas_shape* shape, const int32_t* doc_first, float* s,
                              hipStream_t stream);

/* Host helper (no device work): the blocks table and doc_first of packed
 * documents.  cu_seqlens: host int32 [ndocs+1], 0 = cu[0] <= cu[1] <= ...,
 * document j holds tokens [cu[j], cu[j+1]) (empty documents are skipped).
 * Writes up to max_blocks entries of blocks (host int32 [max_blocks, 2]) and
 * doc_first (host int32 [max_blocks]) for one batch entry and returns the
 * number of blocks, or -1 when cu_seqlens is not ascending from 0, or when the
 * documents need more than max_blocks blocks (nothing written then).  Pad
 * shorter batch entries with (cu[ndocs], 0) blocks whose doc_first is their
 * own index. */
int32_t sas_blocks_from_cu_seqlens(const int32_t* cu_seqlens, int32_t ndocs, int32_t* blocks,
                                   int32_t* doc_first, int32_t max_blocks);

/* ---------------------------------------------------------------- forward
 * Gated block-sparse attention forward [Review §2.3 equation, §2.6].
 * For each query head h and q-block i: keys = the cnt[b,kv,i] blocks idx[b,kv,i,:]
 * (bias log_gate) plus block i itself (bias 0, key j visible iff j <= query t;
 * positions are tokens, so in a block table the causal rule runs over the
 * block's own tokens).
 *   o   [B,Hq,n,d]  dtype of q (written on the blocks' rows; bf16 rounded to
 *                   nearest even)
 *   lse [B,Hq,n]    float32 natural-log row logsumexp of the biased logits
 * idx/cnt/log_gate as produced by sas_select (idx ascending is NOT required,
 * but every entry j < cnt must be a block in [0, i); this is not checked on the
 * device).  log_gate may be NULL when topk == 0. */
sas_status sas_fwd(const sas_shape* shape, const void* q, const void* k, const void* v,
                   const int32_t* idx, const int32_t* cnt, const float* log_gate,
                   void* o, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------- backward
 * Gradients of sum(dO * o) [Review §2.6 and the chain rule through §2.4]:
 *   dq [B,Hq,n,d], dk, dv [B,Hkv,n,d]  (dtype of q; written, not accumulated)
 *   ds [B,Hkv,nb,nb] float32: for m < i,
 *        ds[i,m] = [m kept] dlg[i,m] - pi_i[m] * sum_{m' kept} dlg[i,m'],
 *        pi_i = softmax of s[i,:] over the row's candidates (0 elsewhere, and
 *        0 in a row without candidates), dlg[i,m] = sum of the logit gradients
 *        of the group's heads over rows of block i and keys of block m;
 *      and ds[i,m] = 0 for m >= i (every entry is written).
 * o and lse must come from sas_fwd on the same inputs; s, idx, cnt, log_gate
 * and s_lse are the sas_select inputs/outputs (idx ascending, as it writes).
 * ws: device scratch, contents on entry irrelevant, of at least
 * sas_bwd_min_workspace_bytes(shape) bytes (SAS_ERR_WORKSPACE otherwise).
 * With sas_bwd_workspace_bytes(shape) bytes or more, a bf16 call with the
 * softmax, sigmoid or hard gate keeps the logit gradient dZ of every kept and
 * own tile (bf16, B*Hq*nb*(topk+1) tiles of 8 KiB) in ws and forms dq from
 * it instead of recomputing the logits and dP: the same results to rounding,
 * faster.  The two sizes are equal where that path does not apply (float32,
 * the external gate, or tiles beyond 16 GiB). */
size_t sas_bwd_workspace_bytes(const sas_shape* shape);
size_t sas_bwd_min_workspace_bytes(const sas_shape* shape);
sas_status sas_bwd(const sas_shape* shape, const void* q, const void* k, const void* v,
                   const void* o, const void* dO, const float* lse, const int32_t* idx,
                   const int32_t* cnt, const float* log_gate, const float* s,
                   const float* s_lse, void* dq, void* dk, void* dv, float* ds, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- decode
 * Single-token decode over a contiguous KV cache (the serving-side use of the
 * same attention, [Review §2.6] and the decode-speed results of [Review §4]).
 * Batch entry b holds seq_lens[b] tokens (1 <= seq_lens[b] <= cap); its query is
 * token T = seq_lens[b]-1, whose current block is i = T/64 holding the tokens
 * [64 i, seq_lens[b]).  Per kv-group: select from s[b,kv,0..i-1] exactly as
 * sas_select; each query head attends to the kept blocks (bias log_gate) and to
 * the current block's tokens (bias 0).
 *   q [B,Hq,d]; k_cache, v_cache [B,Hkv,cap,d]; seq_lens int32 [B] (device);
 *   s float32 [B,Hkv,cap/64]; o [B,Hq,d] (written).
 *   idx_out: NULL, or int32 [B,Hkv,topk] receiving the ascending selection
 *   (-1 padded).  ws: device scratch of sas_decode_workspace_bytes(shape) bytes.
 * seq_lens outside [1, cap] are clamped on the device (host cannot read them). */
size_t sas_decode_workspace_bytes(const sas_decode_shape* shape);
sas_status sas_decode(const sas_decode_shape* shape, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* seq_lens, const float* s, void* o,
                      int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- decode without allocation
 * For callers that cannot allocate device memory or hand in a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and status codes as sas_decode, without
 * ws / ws_bytes: the scratch lives in a library-owned device array of
 * SAS_NOALLOC_SCRATCH_BYTES bytes, one per GPU, which the GPU holds from the
 * library's load until the process ends.  Returns SAS_ERR_WORKSPACE (nothing
 * enqueued) when sas_decode_workspace_bytes(shape) exceeds that size.  Calls
 * no hipMalloc, hipFree or allocating routine.
 *   - Every call on a GPU shares that GPU's array, which keeps the last call's
 *     contents (nothing in it needs to start at zero).  Calls that overlap in
 *     time on one GPU (other streams, other threads) race on it: the caller
 *     must serialise them, e.g. by issuing them on one stream.
 *   - The first call on each GPU resolves the array's device address
 *     (hipGetSymbolAddress, with the stream's device current); make that first
 *     call outside graph capture. */
#define SAS_NOALLOC_SCRATCH_BYTES (16u << 20)
sas_status sas_decode_noalloc(const sas_decode_shape* shape, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens, const float* s,
                              void* o, int32_t* idx_out, hipStream_t stream);

/* ---------------------------------------------------------------- paged decode
 * sas_decode over a paged KV pool, the serving-side cache of [Review §2.6]:
 * the same selection and attention with cap = 64*max_blocks, where the K/V
 * rows of token t of sequence b are k_pages[page_table[b,t/64], kv, t%64, :]
 * (likewise v_pages).  Only the table entries of each row's kept blocks and
 * current block are read.  Entries outside [0, num_pages) are clamped on the
 * device: nothing outside the pool is read, and rows that use such entries get
 * unspecified values.  Rows of more than SAS_MAX_BLOCKS history blocks are
 * selected by a whole workgroup (long contexts up to 512K tokens).
 *   seq_lens int32 [B] (device), clamped into [1, 64*max_blocks];
 *   idx_out: NULL, or int32 [B,Hkv,topk] receiving the ascending block indices
 *   (not pages), -1 padded; o [B,Hq,d] (written).
 *   ws: device scratch of sas_decode_paged_workspace_bytes(shape) bytes. */
size_t sas_decode_paged_workspace_bytes(const sas_decode_paged_shape* shape);
sas_status sas_decode_paged(const sas_decode_paged_shape* shape, const void* q,
                            const void* k_pages, const void* v_pages, const int32_t* page_table,
                            const int32_t* seq_lens, const float* s, void* o, int32_t* idx_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Name of the HIP error behind the last SAS_ERR_HIP returned on this thread
 * ("hipSuccess" if none); static storage. */
const char* sas_last_hip_error(void);

/* ---------------------------------------------------------------- profiling
 * Kernel-level timing for measurement tools.  When enabled, the library records
 * a hipEvent pair around every kernel it launches afterwards (events are
 * created lazily, outside the timed kernels) and accumulates per-kernel elapsed
 * milliseconds when sas_prof_collect is called after the stream has drained.
 * Not thread-safe; off by default. */
sas_status sas_prof_enable(int32_t on);
/* Writes up to `max` entries; returns the number of distinct kernel names seen.
 * names[i] points to static strings; total_ms[i] is summed over launches[i]. */
int32_t sas_prof_collect(const char** names, double* total_ms, int32_t* launches, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* SAS_H_ */
