// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "xattn_device.h"
#include "../../include/xattn.h"

namespace xattn {

// Partial estimate of one launch: for every (sequence b, q head h, key block j
// in [jb0, jb0 + jb_count), reshaped query row r) the base-2 log-sum-exp of
// est_scale*log2(e)*S over the allowed columns of block j.  Stored at
// part[((b*hq + h)*max_kb + j)*max_r + r].
constexpr int kEstMaxSeq = 64;  // sequences of the tile GEMM's active-tile table

struct EstArgs {
  const char* q;
  KvView k;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int hq;
  int group;
  int jb0;
  int jb_count;
  float scale2;
  float* part;
  int max_kb;
  int max_r;
  long long q_bytes;  // bytes addressable from q
  long long k_bytes;  // bytes addressable from k.base
  int tiles_c;        // big-tile GEMM: column tiles per head (set by the launcher)
  int tiles_r;        // big-tile GEMM: row tiles per head
  // > 0: grouped unit order (set by the launcher).  Without a tile table:
  // (sequence, kv group) blocks, each in chunks of group_chunk column tiles
  // holding every row tile and head of the group; with one: within a
  // sequence, the heads of a kv group take each tile one after the other.
  int group_chunk;
  // Host copies of cu_q / cu_k (launcher only).  With them the launcher
  // gives the tile GEMM one workgroup per tile that has work, numbered
  // (sequence, head, row tile, column tile) with tile_base[b] the number of
  // such tiles before sequence b (n_tab = batch + 1 entries; 0: one
  // workgroup per grid tile, the empty ones exit).
  const int32_t* cu_q_host;
  const int32_t* cu_k_host;
  int n_tab;
  int tile_base[kEstMaxSeq + 1];
};

struct BlockSumArgs {
  const float* part;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int hq;
  int stride;
  int max_qb;
  int max_kb;
  int max_r;
  float* block_sums;  // [batch, hq, max_qb, max_kb]
};

struct SelectArgs {
  const float* block_sums;  // [batch, hq, max_qb, max_kb]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int hq;
  int hkv;
  int max_qb;
  int max_kb;
  float threshold;
  int num_to_choose;  // > 0: top-k rule instead of the threshold
  int select_mode;
  int group_agg;
  uint8_t* mask_q;   // [batch, hq, max_qb, max_kb]  (workspace)
  uint8_t* mask_kv;  // [batch, hkv, max_qb, max_kb]
  uint8_t* hist_sel; // [batch, max_kb]
  int32_t* counts;   // [batch, 2]
  // lists != nullptr: the kernel that writes a final mask_kv row also writes
  // that row's attention block list over the whole key range (PlanArgs
  // layout, pages from block_table or contiguous), and the attention's
  // tail-part counter is cleared, so that no plan launch is needed
  int32_t* lists;
  const int32_t* block_table;  // [batch, max_blocks] or nullptr
  int max_blocks;
  int num_pages;  // pages of the K/V arrays; table entries outside [0, num_pages) are absent
  int* tail_ctr;
};

// V re-laid out for the attention kernel: page p (128 keys) of kv head g is a
// [d][128] bf16 block at vt + ((p*hkv + g)*d)*128*2, keys of every 16-key
// group stored in the order the MFMA B operand of P^T consumes them.
struct VtArgs {
  const char* v;  // [num_pages, 128, hkv, d] (a contiguous [total_k, hkv, d] array is the same)
  char* vt;
  int num_pages;
  int hkv;
  int head_dim;
};

// Per (b, kv head g, q block i) list of the key blocks the attention visits,
// in increasing j: lists[row*(max_kb+1)] = count, then entries
// (page << 1) | (j == i + Kh), for selected j in [jb0, min(jb1, i+Kh+1)).
struct PlanArgs {
  const uint8_t* mask;  // [batch, hkv, max_qb, max_kb]
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_table;  // [batch, max_blocks] or nullptr (contiguous)
  int max_blocks;
  int num_pages;  // pages of the K/V arrays; table entries outside [0, num_pages) are absent
  int hkv;
  int max_qb;
  int max_kb;
  int jb0;
  int jb1;
  int32_t* lists;
  int* tail_ctr;  // attention's tail-part counter, cleared by the plan
};

// Attention of one launch.  Keys come from blocks j in [jb0, jb1) whose mask
// byte is set and whose page is present; rows are (b, q head, query).
constexpr int kMaxOrder = 256;

struct AttnArgs {
  const char* q;
  KvView k;
  KvView v;
  const char* vt;         // bf16 path: transposed V pages (VtArgs layout)
  const int32_t* lists;   // bf16 path: block lists (PlanArgs layout)
  int num_pages;          // 128-key pages addressable through k.base / vt
  // bf16 path: work rows in launch order, longest first (n_order == 0: the
  // kernel's default order).  Entry: i | b << 16 | s << 28 | (ns - 1) << 30,
  // part s of ns equal parts of row (b, i)'s block list (see order_entry).
  int n_order;
  int order[kMaxOrder];
  // For an entry with ns == 2: part 0 takes the first (count * cut) / 256
  // entries of the row's block list and part 1 the rest (cut 0: halves).
  uint8_t order_cut[kMaxOrder];
  // 0 < n_static < n_order: one workgroup per (entry, kv slot) of the first
  // n_static entries; after its own unit every workgroup draws units of the
  // remaining entries (entry-major, longest first) from *tail_ctr, which is
  // zero at launch and which the launch's last increment sets back to zero.
  int n_static;
  int* tail_ctr;
  // Rows split into ns > 1 parts write part s as a normalised fp32 output
  // and its natural-log LSE to split_o[s] / split_l[s] (layouts of out_f32 /
  // lse); a split merge then writes the final output.
  float* split_o[3];
  float* split_l[3];
  // A split row whose block list holds at most split_whole entries is done
  // whole by its part 0, which writes the final output (0: never).
  // split_whole < 0: the head length comes from the device (heads from the
  // lists): every workgroup sums the list counts of the launch's
  // cut_rows (sequence, kv head, q block) rows, takes the head length H of
  // the host rule (98% of the per-CU share over cut_cus CUs, plus two
  // blocks) from that total, and a two-part row takes H entries in part 0
  // and the rest in part 1 (whole when it holds at most H); workgroup 0
  // stores H in *cut_head for the split merge.
  int split_whole;
  int cut_rows;
  int cut_cus;
  int* cut_head;
  // set by the caller before planning: the launch may take its head length
  // from the device (its block lists are complete before it starts)
  int device_cut;
  const uint8_t* mask;  // [batch, hkv, max_qb, max_kb]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int hq;
  int group;
  int max_qb;
  int max_kb;
  int jb0;
  int jb1;
  float scale2;       // softmax_scale * log2(e)
  int total_q;
  // Output: final (out in input dtype) or partial fp32 (out_f32).
  void* out;          // [total_q, hq, d] dtype   (nullptr if partial)
  float* out_f32;     // [total_q, hq, d] fp32    (nullptr if final)
  float* lse;         // [hq, total_q] natural log (may be nullptr)
  // fp32 path: f32_splits > 1 workgroups share each (q block, head) row,
  // part s taking a contiguous s-th of the row's candidate key tiles (32
  // keys each); part s writes its normalised output and natural-log LSE to
  // f32_o + s*total_q*hq*d and f32_l + s*hq*total_q, and a merge writes the
  // result.
  int f32_splits;
  float* f32_o;
  float* f32_l;
};

// Key-tile splits of the fp32 attention for a launch of `rows` (q block,
// head, sequence) rows: about 1024 workgroups' worth of parts for a 256-CU
// chip, at most kMaxF32Splits.
constexpr int kMaxF32Splits = 32;
constexpr int f32_attention_splits(long long rows) {
  return rows <= 0 ? 1
                   : (rows >= 512 ? 1 : (int)(1024 / rows < kMaxF32Splits ? 1024 / rows : kMaxF32Splits));
}

// Head length of a split row (host and device rule): ceil(0.98 * share) +
// kHeadPad blocks, share = the launch's blocks per CU.
#ifndef XATTN_HEAD_PAD
#define XATTN_HEAD_PAD 2
#endif
constexpr int kHeadPad = XATTN_HEAD_PAD;

constexpr uint32_t order_entry(int b, int i, int s, int ns) {
  return (uint32_t)i | ((uint32_t)b << 16) | ((uint32_t)s << 28) | ((uint32_t)(ns - 1) << 30);
}

// Final output of the rows an attention launch split: for each listed row
// (first query token / 128, ns) the LSE-weighted sum of its ns partial
// outputs, written to out (bf16) and lse.
struct SplitMergeArgs {
  int n;
  int heads;
  int head_dim;
  int total_q;
  const float* o[3];
  const float* l[3];
  void* out;   // bf16 [total_q, heads, d]
  float* lse;  // [heads, total_q] or nullptr
  int rows[kMaxOrder];  // q block (global) | (ns - 1) << 28
  // rows the attention did whole (list count <= whole) are skipped
  int row_bi[kMaxOrder];  // sequence << 16 | q block of rows[r]
  const int32_t* lists;   // the attention's block lists (PlanArgs layout)
  int group, max_qb, max_kb, whole;
  const int* cut_head;    // whole < 0: the head length the attention stored
};

struct MergeArgs {
  int rows;
  int heads;
  int head_dim;
  const float* o_a;
  const float* lse_a;
  const float* o_b;
  const float* lse_b;
  float* o;        // fp32 out (or nullptr)
  void* o_bf16;    // bf16 out (or nullptr)
  float* lse;      // may be nullptr
};

// Sets the calling thread's xattn_last_error message (printf format) and
// returns `code`.
int fail_message(int code, const char* fmt, ...);
// Workspace bytes of a call (xattn_workspace_size) with make_plan's status.
int workspace_bytes(const XattnShape* shape, const XattnParams* params, size_t* bytes);

hipError_t launch_estimate(const EstArgs& a, int dtype, int head_dim, int stride, int batch,
                           hipStream_t s);
hipError_t launch_block_sums(const BlockSumArgs& a, int batch, hipStream_t s);
// *lists_done (if given) tells whether the kernels wrote a.lists.
hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t s, bool* lists_done = nullptr);
hipError_t launch_vt_transpose(const VtArgs& a, hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, int batch, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int dtype, int head_dim, int batch,
                            hipStream_t s);
// Whether the attention launch for `a` reads the V^T pages (a.vt).
bool attention_reads_vt(const AttnArgs& a, int dtype, int head_dim);
// Whether the bf16 launch runs the ping-pong kernel (the one that draws tail
// units dynamically).
bool attention_uses_pp(const AttnArgs& a, int head_dim);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t s);
// fp32 attention with f32_splits > 1: the merge of the parts (after
// launch_attention)
hipError_t launch_f32_merge(const AttnArgs& a, int head_dim, hipStream_t s);
// Copies block j of src (host memory mapped into the device address space)
// to block j of dst for every j < nblocks with sel[j] != 0.
hipError_t launch_gather_blocks(const uint8_t* sel, int nblocks, const void* src, void* dst, size_t block_bytes,
                                hipStream_t s);

}  // namespace xattn
