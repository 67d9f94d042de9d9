/*
 * xattn.h -- C ABI of the MI355X (gfx950) XAttention block-sparse prefill
 * library (libxattn.so).
 *
 * The path has three stages, each with its own entry point plus one that
 * runs them all for one prefill chunk:
 *
 *   xattn_estimate      strided anti-diagonal importance estimate -> block sums
 *                       ("XAttention BSA Policy" design doc, core algorithm
 *                       Steps 1-2; two-pass chunked statistics per "XAttention
 *                       Offload Stream Synchronization Fix", 技术细节)
 *   xattn_select        cumulative-threshold block selection, GQA aggregation,
 *                       forced blocks and majority vote (design doc Steps 3-4)
 *   xattn_sparse_attn   flash attention with LSE over the selected blocks
 *                       (design doc section 2, compute_chunked_prefill)
 *   xattn_merge_attn    LSE merge of two partial attentions
 *                       (design doc section 2, merge_attention_outputs)
 *   xattn_prefill_chunk all of the above; optionally streams the K/V history
 *                       from pinned host memory through a device ring of slots
 *                       ordered by events on one compute stream (stream fix
 *                       page, 根因分析 and Event 同步机制)
 *
 * Conventions (all entry points):
 *  - Pointers are device pointers unless the comment says "host".
 *  - Tensors are row-major, token-major:
 *      Q        [total_q, Hq, d]
 *      K, V     [total_k, Hkv, d]            when shape.block_table == NULL
 *               [num_phys_blocks, 128, Hkv, d] when shape.block_table != NULL
 *    Sequence b owns query rows [cu_q[b], cu_q[b+1]) and keys
 *    [cu_k[b], cu_k[b+1]) (cumulative lengths as in the transformers
 *    paged-attention page, "Caminho Varlen").  With a block table, key y of
 *    sequence b lives in page block_table[b*max_blocks_per_seq + y/128] at row
 *    y%128; -1 marks an unallocated page ("Caminho de decodificação").
 *    Every entry a sequence uses (key block j < Lk/128) must name a page in
 *    [0, num_phys_blocks).  An entry that does not is treated as an absent
 *    page by every kernel (the estimate reads its keys as zero vectors and
 *    the attention skips the block; nothing outside the cache is read),
 *    which silently changes the result.  With the environment variable XATTN_DEBUG set (to anything
 *    but "" or "0") the calls that take a block table first wait for `stream`
 *    to drain, copy the table to the host and return XATTN_ERR_INVALID for
 *    such an entry, before enqueuing anything.
 *  - The queries of a sequence are its LAST Lq = cu_q[b+1]-cu_q[b] positions:
 *    query x sits at absolute position (Lk - Lq) + x and sees keys y <= that.
 *  - Every length must be a multiple of 128 and Lk >= Lq (the design doc's
 *    alignment limit, 限制); block_size must be 128 and stride must divide 128.
 *  - All validation runs on the host BEFORE anything is enqueued: a call that
 *    returns an error has enqueued no work.  Nothing here throws.
 *  - All work is enqueued on `stream`; calls return without synchronising
 *    (exception: ring mode of xattn_prefill_chunk, see there).  The library
 *    never uses the null stream unless `stream` is NULL.
 *  - The library never allocates device memory inside these calls except in
 *    xattn_ring_create; scratch space is the caller's workspace `ws`.
 *  - Calls that use one workspace must not overlap in time: enqueue them on
 *    one stream or order them with events.  A workspace carries state from
 *    call to call (the attention plan, and a work counter that the plan
 *    clears and every attention launch returns to zero as it ends), so two
 *    concurrent launches on one workspace race.  Different workspaces are
 *    independent.
 *  - Outputs are owned by the caller; the library keeps no pointer after a
 *    call returns (the ring keeps only its own slots).
 */
#ifndef XATTN_H_
#define XATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
#define XATTN_OK 0
#define XATTN_ERR_INVALID (-1)     /* bad pointer, size or argument          */
#define XATTN_ERR_UNSUPPORTED (-2) /* valid but not supported (d, stride...) */
#define XATTN_ERR_HIP (-3)         /* a HIP runtime call failed              */
#define XATTN_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than needed  */
#define XATTN_ERR_NOT_PINNED (-5)  /* ring history is not pinned host memory */

#define XATTN_DTYPE_BF16 0
#define XATTN_DTYPE_F32 1

/* select_mode */
#define XATTN_SELECT_PER_KVHEAD 0 /* per (kv head, q block) masks + sink/diagonal */
#define XATTN_SELECT_CHUNK_VOTE 1 /* history majority vote, dense causal current  */
#define XATTN_SELECT_CHUNK_VOTE_SPARSE 2 /* history majority vote, current chunk
                                            per KV head (sink and diagonal kept) */
/* group_agg: how the q heads of one KV group combine their masks */
#define XATTN_GQA_ANY 0      /* any head keeps the block (design doc Step 4)   */
#define XATTN_GQA_MAJORITY 1 /* more than half of the group's heads keep it    */

#define XATTN_BLOCK 128

typedef struct XattnShape {
  int batch;        /* number of sequences (>= 1)                           */
  int num_q_heads;  /* Hq                                                    */
  int num_kv_heads; /* Hkv; Hq % Hkv == 0, q head h uses kv head h/(Hq/Hkv)  */
  int head_dim;     /* d in {64, 128}                                        */
  int dtype;        /* XATTN_DTYPE_BF16 or XATTN_DTYPE_F32 (Q, K, V, out)    */
  const int32_t *cu_q_host; /* host   [batch+1] cumulative query lengths     */
  const int32_t *cu_k_host; /* host   [batch+1] cumulative key lengths       */
  const int32_t *cu_q;      /* device copy of cu_q_host                      */
  const int32_t *cu_k;      /* device copy of cu_k_host                      */
  const int32_t *block_table; /* device [batch, max_blocks_per_seq] or NULL  */
  int max_blocks_per_seq;     /* row length of block_table                   */
  int num_phys_blocks;        /* pages in the K/V cache (block_table != NULL)*/
} XattnShape;

typedef struct XattnParams {
  int stride;          /* s in {4, 8, 16}: reshape stride of the estimate       */
  int block_size;      /* must be 128 (design doc 参数配置: BSA block 128)      */
  float threshold;     /* tau; >= 1 keeps every allowed block                   */
  float est_scale;     /* logit scale of the estimate; 0 => 1/(s*sqrt(d))       */
  float softmax_scale; /* attention scale; 0 => 1/sqrt(d)                       */
  int kv_chunk_tokens; /* estimate KV chunk (ring slot size); multiple of 128   */
  int select_mode;     /* XATTN_SELECT_*                                        */
  int group_agg;       /* XATTN_GQA_*                                           */
  int num_to_choose;   /* > 0: keep the num_to_choose largest allowed blocks of
                          each (q head, q block) row (value desc, index asc)
                          instead of the threshold rule -- the fixed-count
                          argument of find_blocks_chunked (design doc 核心算法
                          Step 3); 0: threshold rule                        */
  int reuse_selection; /* xattn_prefill_chunk only.  1: skip the estimate and
                          the selection and attend over aux->mask_kv (and,
                          in ring mode, stream the blocks aux->hist_sel
                          marks) as produced by an earlier call -- the
                          design doc's sharing of one layer's estimate with
                          the other layers (性能分析, 优化方向 1).  Counts and
                          block sums are not written.  0: full path.       */
} XattnParams;

/* Optional extra outputs of xattn_prefill_chunk (any field may be NULL). */
typedef struct XattnAux {
  float *block_sums; /* [batch, Hq, maxQb, maxKb] fp32                   */
  uint8_t *mask_kv;  /* [batch, Hkv, maxQb, maxKb] effective attention mask */
  uint8_t *hist_sel; /* [batch, maxKb] voted history blocks                */
} XattnAux;

typedef struct XattnRing XattnRing;

/* Bytes of device workspace needed by every call below for this shape and
 * these parameters (one size covers all of them).  Pure host arithmetic;
 * returns 0 if the arguments are invalid (see xattn_last_error). */
size_t xattn_workspace_size(const XattnShape *shape, const XattnParams *params);

/* Strided anti-diagonal estimate ("XAttention BSA Policy" design doc, Steps
 * 1-2; stream-fix page, 三阶段 KV Chunking).  For q head h, reshaped query
 * row r < Lq/s and reshaped key column c < Lk/s:
 *     S[h,r,c] = sum_{t<s} < q[r*s+s-1-t, h], k[c*s+t, h/G] >
 * cell (r,c) is allowed iff c <= r + (Lk-Lq)/s; z = est_scale*S is soft-maxed
 * per row over allowed cells and summed over (128/s)x(128/s) tiles.
 * Out: block_sums [batch, Hq, maxQb, maxKb] fp32, zero outside each
 * sequence's [Qb, Kb] and beyond the causal block diagonal.
 * The key range is processed in chunks of kv_chunk_tokens with per-chunk
 * softmax statistics merged before normalisation; the result does not depend
 * on the chunk size. */
int xattn_estimate(const XattnShape *shape, const XattnParams *params, const void *q,
                   const void *k, float *block_sums, void *ws, size_t ws_bytes,
                   void *stream);

/* Block selection (design doc Steps 3-4).  Per (b, q head h, q block i) over
 * the allowed blocks j <= i + Kh (Kh = (Lk-Lq)/128): order by (value desc,
 * index asc) and keep an item iff the float64 sum of the items before it is
 * below threshold * (float64 sum of all allowed items), both accumulated in
 * that order.  The G q heads of a KV group combine by group_agg.
 *  PER_KVHEAD: the sink block 0 and the diagonal block i+Kh are always kept.
 *  CHUNK_VOTE: history block j < Kh is kept iff more than half of the Hkv*Qb
 *    (kv head, q block) rows keep it; blocks 0 and Kh-1 are always kept; the
 *    current chunk (j >= Kh) stays dense causal.
 *  CHUNK_VOTE_SPARSE: history as CHUNK_VOTE; the current chunk as
 *    PER_KVHEAD (each row keeps its group's selected blocks, the sink and its
 *    diagonal), the per-KV-head selection the GPU-only mode makes over the
 *    whole key range ("XAttention Offload Stream Synchronization Fix",
 *    测试结果).  With no history it equals PER_KVHEAD.
 * Out: mask_kv [batch, Hkv, maxQb, maxKb] uint8 effective attention mask;
 *      hist_sel [batch, maxKb] uint8 (may be NULL; zero in PER_KVHEAD mode);
 *      counts [batch, 2] int32 = {selected, available} (design doc, Density
 *      统计 API): CHUNK_VOTE {sum hist_sel, Kh}; PER_KVHEAD and
 *      CHUNK_VOTE_SPARSE {sum mask_kv, number of allowed (kv head, q block,
 *      block) triples}. */
int xattn_select(const XattnShape *shape, const XattnParams *params,
                 const float *block_sums, uint8_t *mask_kv, uint8_t *hist_sel,
                 int32_t *counts, void *ws, size_t ws_bytes, void *stream);

/* Block-sparse flash attention with LSE (design doc section 2).  Query x of
 * q head h attends to keys y <= (Lk-Lq)+x of kv head h/G whose block y/128
 * has mask_kv[b, h/G, x/128, y/128] != 0, with softmax scale softmax_scale.
 * Out: out [total_q, Hq, d] in shape.dtype; lse [Hq, total_q] fp32 natural
 * log-sum-exp of the scaled logits (may be NULL). */
int xattn_sparse_attn(const XattnShape *shape, const XattnParams *params, const void *q,
                      const void *k, const void *v, const uint8_t *mask_kv, void *out,
                      float *lse, void *ws, size_t ws_bytes, void *stream);

/* The two halves of xattn_sparse_attn, for callers that reuse V and the
 * mask across calls (and to time the attention kernel alone).
 * xattn_attn_plan re-lays V out d-major for the bf16 kernel and builds, in
 * the workspace, each (sequence, kv head, q block) row's list of blocks to
 * visit; it is a no-op for fp32.  xattn_attn_run launches only the attention
 * kernel; its workspace must hold a plan made with the same shape, params,
 * v and mask_kv contents, with no other call on that workspace in between. */
int xattn_attn_plan(const XattnShape *shape, const XattnParams *params, const void *v,
                    const uint8_t *mask_kv, void *ws, size_t ws_bytes, void *stream);
int xattn_attn_run(const XattnShape *shape, const XattnParams *params, const void *q,
                   const void *k, const void *v, const uint8_t *mask_kv, void *out,
                   float *lse, void *ws, size_t ws_bytes, void *stream);

/* LSE merge of two partial attentions over disjoint key sets (design doc
 * section 2, merge_attention_outputs):
 *   lse = max(a,b) + log1p(exp(-|a-b|)),  o = e^(a-lse) o_a + e^(b-lse) o_b;
 * a side whose lse is -inf contributes nothing.  o_* [rows, heads, head_dim]
 * fp32, lse_* [heads, rows] fp32.  Outputs may alias inputs element-wise. */
int xattn_merge_attn(int rows, int heads, int head_dim, const float *o_a,
                     const float *lse_a, const float *o_b, const float *lse_b, float *o,
                     float *lse, void *stream);

/* Whole path for one prefill chunk: estimate -> select -> sparse attention.
 *
 * ring == NULL: K/V are resident (contiguous or paged per `shape`).
 * ring != NULL: batch must be 1 and the block table NULL; k, v hold only the
 *   current chunk [Lq, Hkv, d] (the last Lq keys) and k_hist_host,
 *   v_hist_host are PINNED host arrays [hist_blocks, 128, Hkv, d] with the
 *   history (Lk = hist_blocks*128 + Lq).  History K streams through the ring
 *   once for the estimate; after selection the selected K/V blocks stream
 *   through it again for attention.  Copies run on the ring's transfer
 *   stream; every kernel runs on `stream`; slot reuse is ordered by events
 *   only.  This mode makes ONE blocking wait per call, for the maxKb-byte
 *   selection result that decides which blocks to copy.
 *   The ring's head count, head dim and dtype must match `shape`.
 * out [total_q, Hq, d] shape.dtype; lse [Hq, total_q] fp32 (may be NULL);
 * counts [batch, 2] int32 (may be NULL); aux may be NULL. */
int xattn_prefill_chunk(XattnRing *ring, const XattnShape *shape, const XattnParams *params,
                        const void *q, const void *k, const void *v,
                        const void *k_hist_host, const void *v_hist_host, int hist_blocks,
                        void *out, float *lse, int32_t *counts, const XattnAux *aux,
                        void *ws, size_t ws_bytes, void *stream);

/* Allocation-free variant of xattn_prefill_chunk with resident K/V (ring ==
 * NULL), for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * library's scratch comes from a fixed per-device array of
 * XATTN_STATIC_SCRATCH_BYTES instead of a caller workspace; each GPU the
 * library runs on holds its own copy until the process ends.  The call makes
 * no device allocation; the caller passes inputs and outputs as for
 * xattn_prefill_chunk.  Every call on one GPU shares that GPU's array and
 * leaves its contents behind: calls that overlap in time on one GPU race
 * (enqueue them on one stream or order them with events).  Errors: as
 * xattn_prefill_chunk; a shape and params whose xattn_workspace_size exceeds
 * XATTN_STATIC_SCRATCH_BYTES return XATTN_ERR_UNSUPPORTED (nothing
 * enqueued). */
#define XATTN_STATIC_SCRATCH_BYTES (256u << 20)
int xattn_prefill_chunk_static(const XattnShape *shape, const XattnParams *params, const void *q,
                               const void *k, const void *v, void *out, float *lse,
                               int32_t *counts, const XattnAux *aux, void *stream);

/* Device ring of `num_slots` slots of `slot_blocks` 128-token K and V blocks
 * (the design doc's ring-buffer pipeline; 4 slots as in the layerwise
 * offload plan, 1.1).  Owns its slots, one transfer stream (default
 * priority) and per-slot ready/done events; every done event is recorded
 * once at creation so the first copy into a slot does not wait.  Returns
 * XATTN_OK and *out, or an error (nothing allocated). */
int xattn_ring_create(int num_slots, int slot_blocks, int num_kv_heads, int head_dim,
                      int dtype, XattnRing **out);
/* Staged variant for the same calls (NEXT step of the ring: a zero-copy
 * selected-block gather that removes the host wait of the selection).  Owns
 * one device region for max_blocks 128-token blocks of K and of V -- the
 * history plus the current chunk of a sequence -- a transfer stream and
 * events.  xattn_prefill_chunk with it: history K in one bulk copy on the
 * transfer stream, the chunk copied behind it, estimate and selection over the
 * whole sequence as in resident mode, then a kernel gathers the voted history
 * V blocks straight from the pinned host array (mapped into the device
 * address space; read over the link by the kernel, driven by the device-side
 * selection, no host wait) and one attention launch writes the output.  With
 * reuse_selection it gathers the K and V blocks aux->hist_sel marks and copies
 * no history in bulk.  Errors as xattn_ring_create; a sequence longer than
 * max_blocks is rejected (INVALID) by xattn_prefill_chunk. */
int xattn_ring_create_staged(int max_blocks, int num_kv_heads, int head_dim, int dtype,
                             XattnRing **out);
/* Waits for the ring's pending copies, then frees it.  NULL is a no-op. */
void xattn_ring_destroy(XattnRing *ring);
/* Test hook: sleep `usec` microseconds on the transfer stream before every
 * slot copy, and on the offload stream before every write-back (a host
 * callback), widening any missing-wait race.  0 = off. */
int xattn_ring_set_copy_delay_us(XattnRing *ring, int usec);

/* Write-back of a prefilled chunk's K/V into the pinned host history: the
 * design doc's offload step after prefill (the per-chunk D2H offload of the
 * [Stream fix] stream table, offload_layer_kv_async / wait_layer_offload of
 * the layerwise plan 1.2).  Enqueues on the ring's offload stream (default
 * priority), after everything already enqueued on `stream`, the copies of
 * num_blocks 128-token blocks of k and v (device, [num_blocks*128, Hkv, d]
 * in the ring's dtype) to k_host_dst and v_host_dst (PINNED host memory of
 * the same layout, typically the history arrays at block hist_blocks), and
 * returns without waiting.  Every later slot copy of this ring waits for it,
 * so the next chunk's prefill reads the written-back blocks; the caller keeps
 * k and v unchanged until xattn_ring_offload_wait has ordered a stream after
 * it.  Errors (nothing enqueued): NULL ring or pointers, num_blocks < 0
 * (INVALID); destinations not pinned (NOT_PINNED). */
int xattn_ring_offload_chunk(XattnRing *ring, const void *k, const void *v, void *k_host_dst,
                             void *v_host_dst, int num_blocks, void *stream);
/* Makes `stream` wait for the ring's last write-back. */
int xattn_ring_offload_wait(XattnRing *ring, void *stream);

/* Measurement hook, for callers that time the attention kernel alone (the
 * roofline of the block-sparse attention, a7).  While enabled (on != 0),
 * every attention launch of the library records a pair of events on its
 * stream around the block-sparse attention kernel itself -- not the plan,
 * nor the merges of split rows or fp32 parts that follow it.
 * xattn_kernel_timing_read waits for the recorded events, writes the sum of
 * their elapsed times (ms) and their number, and forgets them.  Off by
 * default; switching it on or off also forgets them.  The library keeps the
 * events (created on first use) until the process ends.  Not for use while a
 * stream is being captured into a graph.  Errors: NULL outputs (INVALID); a
 * HIP error while reading (HIP; the pairs are forgotten). */
int xattn_kernel_timing(int on);
int xattn_kernel_timing_read(double *total_ms, int *launches);

/* Message of the last error on the calling thread ("" if none). */
const char *xattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H_ */
