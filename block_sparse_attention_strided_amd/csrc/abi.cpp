// C ABI of libxattn: host validation, workspace planning and kernel launches.
// Every entry point validates all of its arguments on the host before it
// enqueues anything, so an error return leaves no partial work behind.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <unistd.h>

#include <cstdlib>

#include <algorithm>
#include <mutex>
#include <utility>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/xattn.h"
#include "xattn_internal.h"

using namespace xattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(XATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace xattn {
int fail_message(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}
}  // namespace xattn

namespace {

constexpr int kMaxKb = 4096;  // select sorts up to this many blocks per row in LDS
constexpr int kStageChunk = 128;  // history blocks per pipeline step of a staged ring

// Everything derived from (shape, params) on the host.
struct Plan {
  int batch, hq, hkv, d, dtype, elem;
  int stride, rb;
  int max_qb, max_kb, max_r;
  int total_q, total_k;
  float est_scale, softmax_scale;
  // workspace layout (byte offsets)
  size_t off_part, off_bs, off_maskq, off_maskkv, off_hist, off_counts;
  size_t off_o[3], off_l[3];
  size_t off_table;
  size_t off_vt, off_lists;
  size_t off_ctr;  // attention's tail-part counter (4 bytes), then the device head length (4 bytes)
  int num_pages;  // 128-key pages of the K/V arrays (contiguous or paged)
  bool reads_vt;  // some attention launch reads V^T pages (off_vt holds them)
  int f32_splits;           // fp32 attention: key-block parts per row (1: none)
  size_t off_f32o, off_f32l;  // their partial outputs and LSEs
  size_t total;
};

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int make_plan(const XattnShape* sh, const XattnParams* pr, Plan* p) {
  if (!sh || !pr) return fail(XATTN_ERR_INVALID, "shape and params must not be NULL");
  if (sh->batch < 1) return fail(XATTN_ERR_INVALID, "batch must be >= 1 (got %d)", sh->batch);
  if (sh->num_q_heads < 1 || sh->num_kv_heads < 1)
    return fail(XATTN_ERR_INVALID, "head counts must be >= 1");
  if (sh->num_q_heads % sh->num_kv_heads != 0)
    return fail(XATTN_ERR_INVALID, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                sh->num_q_heads, sh->num_kv_heads);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(XATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", sh->head_dim);
  if (sh->dtype != XATTN_DTYPE_BF16 && sh->dtype != XATTN_DTYPE_F32)
    return fail(XATTN_ERR_INVALID, "unknown dtype %d", sh->dtype);
  if (!sh->cu_q_host || !sh->cu_k_host)
    return fail(XATTN_ERR_INVALID, "cu_q_host and cu_k_host must not be NULL");
  if (!sh->cu_q || !sh->cu_k) return fail(XATTN_ERR_INVALID, "device cu_q and cu_k must not be NULL");
  if (pr->block_size != XATTN_BLOCK)
    return fail(XATTN_ERR_UNSUPPORTED, "block_size must be 128 (got %d)", pr->block_size);
  if (pr->stride != 4 && pr->stride != 8 && pr->stride != 16)
    return fail(XATTN_ERR_UNSUPPORTED, "stride must be 4, 8 or 16 (got %d)", pr->stride);
  if (!std::isfinite(pr->threshold) || pr->threshold < 0.f)
    return fail(XATTN_ERR_INVALID, "threshold must be finite and >= 0");
  if (pr->num_to_choose < 0) return fail(XATTN_ERR_INVALID, "num_to_choose must be >= 0 (0 = threshold rule)");
  if (pr->reuse_selection != 0 && pr->reuse_selection != 1)
    return fail(XATTN_ERR_INVALID, "reuse_selection must be 0 or 1");
  if (!std::isfinite(pr->est_scale) || pr->est_scale < 0.f)
    return fail(XATTN_ERR_INVALID, "est_scale must be finite and >= 0 (0 = default)");
  if (!std::isfinite(pr->softmax_scale) || pr->softmax_scale < 0.f)
    return fail(XATTN_ERR_INVALID, "softmax_scale must be finite and >= 0 (0 = default)");
  if (pr->kv_chunk_tokens < 0 || pr->kv_chunk_tokens % XATTN_BLOCK != 0)
    return fail(XATTN_ERR_INVALID, "kv_chunk_tokens must be a non-negative multiple of 128");
  if (pr->select_mode != XATTN_SELECT_PER_KVHEAD && pr->select_mode != XATTN_SELECT_CHUNK_VOTE &&
      pr->select_mode != XATTN_SELECT_CHUNK_VOTE_SPARSE)
    return fail(XATTN_ERR_INVALID, "unknown select_mode %d", pr->select_mode);
  if (pr->group_agg != XATTN_GQA_ANY && pr->group_agg != XATTN_GQA_MAJORITY)
    return fail(XATTN_ERR_INVALID, "unknown group_agg %d", pr->group_agg);
  if (sh->cu_q_host[0] != 0 || sh->cu_k_host[0] != 0)
    return fail(XATTN_ERR_INVALID, "cu_q and cu_k must start at 0");
  int max_lq = 0, max_lk = 0;
  for (int b = 0; b < sh->batch; ++b) {
    const long long lq = (long long)sh->cu_q_host[b + 1] - sh->cu_q_host[b];
    const long long lk = (long long)sh->cu_k_host[b + 1] - sh->cu_k_host[b];
    if (lq < 0 || lk < 0) return fail(XATTN_ERR_INVALID, "cu_q / cu_k must be non-decreasing (sequence %d)", b);
    if (lq % XATTN_BLOCK || lk % XATTN_BLOCK)
      return fail(XATTN_ERR_UNSUPPORTED, "sequence %d: Lq=%lld and Lk=%lld must be multiples of 128", b, lq, lk);
    if (lk < lq) return fail(XATTN_ERR_INVALID, "sequence %d: Lk=%lld < Lq=%lld", b, lk, lq);
    if (lq > max_lq) max_lq = (int)lq;
    if (lk > max_lk) max_lk = (int)lk;
  }
  p->batch = sh->batch;
  p->hq = sh->num_q_heads;
  p->hkv = sh->num_kv_heads;
  p->d = sh->head_dim;
  p->dtype = sh->dtype;
  p->elem = sh->dtype == XATTN_DTYPE_BF16 ? 2 : 4;
  p->stride = pr->stride;
  p->rb = XATTN_BLOCK / pr->stride;
  p->max_qb = max_lq / XATTN_BLOCK;
  p->max_kb = max_lk / XATTN_BLOCK;
  p->max_r = max_lq / pr->stride;
  p->total_q = sh->cu_q_host[sh->batch];
  p->total_k = sh->cu_k_host[sh->batch];
  if (p->max_kb > kMaxKb)
    return fail(XATTN_ERR_UNSUPPORTED, "key length %d exceeds the supported %d tokens", max_lk, kMaxKb * XATTN_BLOCK);
  if (sh->block_table) {
    if (sh->max_blocks_per_seq < p->max_kb)
      return fail(XATTN_ERR_INVALID, "max_blocks_per_seq (%d) < longest sequence's blocks (%d)",
                  sh->max_blocks_per_seq, p->max_kb);
    if (sh->num_phys_blocks < 1) return fail(XATTN_ERR_INVALID, "num_phys_blocks must be >= 1 with a block table");
  }
  p->est_scale = pr->est_scale > 0.f ? pr->est_scale : 1.0f / (pr->stride * std::sqrt((float)p->d));
  p->softmax_scale = pr->softmax_scale > 0.f ? pr->softmax_scale : 1.0f / std::sqrt((float)p->d);

  const size_t B = p->batch;
  size_t off = 0;
  p->off_part = off;
  off = align_up(off + B * p->hq * (size_t)p->max_kb * p->max_r * sizeof(float));
  p->off_bs = off;
  off = align_up(off + B * p->hq * (size_t)p->max_qb * p->max_kb * sizeof(float));
  p->off_maskq = off;
  off = align_up(off + B * p->hq * (size_t)p->max_qb * p->max_kb);
  p->off_maskkv = off;
  off = align_up(off + B * p->hkv * (size_t)p->max_qb * p->max_kb);
  p->off_hist = off;
  off = align_up(off + B * (size_t)p->max_kb);
  p->off_counts = off;
  off = align_up(off + B * 2 * sizeof(int32_t));
  for (int x = 0; x < 3; ++x) {
    p->off_o[x] = off;
    off = align_up(off + (size_t)p->total_q * p->hq * p->d * sizeof(float));
    p->off_l[x] = off;
    off = align_up(off + (size_t)p->hq * p->total_q * sizeof(float));
  }
  p->off_table = off;
  off = align_up(off + (size_t)(p->max_kb + 1) * sizeof(int32_t));
  p->num_pages = sh->block_table ? sh->num_phys_blocks : p->total_k / XATTN_BLOCK;
  p->off_vt = off;
  // V^T pages are read only by the single-phase bf16 attention kernel (odd
  // GQA groups, or K/V spans beyond 31-bit buffer offsets); every attention
  // launch of a call addresses at most num_pages pages, so the ping-pong
  // kernel serves all of them when the whole span fits
  const size_t span = (size_t)p->num_pages * p->hkv * p->d * XATTN_BLOCK * 2;
  p->reads_vt = p->dtype == XATTN_DTYPE_BF16 && ((p->hq / p->hkv) % 2 != 0 || span >= ((size_t)1 << 31));
  if (p->reads_vt) off = align_up(off + span);
  p->off_lists = off;
  off = align_up(off + B * p->hkv * (size_t)p->max_qb * (p->max_kb + 1) * sizeof(int32_t));
  p->off_ctr = off;
  off = align_up(off + sizeof(int32_t));
  // fp32 attention: partials of the rows' key-block splits
  p->f32_splits = p->dtype == XATTN_DTYPE_F32 ? f32_attention_splits((long long)p->max_qb * p->hq * p->batch) : 1;
  p->off_f32o = p->off_f32l = off;
  if (p->f32_splits > 1) {
    p->off_f32o = off;
    off = align_up(off + (size_t)p->f32_splits * p->total_q * p->hq * p->d * sizeof(float));
    p->off_f32l = off;
    off = align_up(off + (size_t)p->f32_splits * p->hq * p->total_q * sizeof(float));
  }
  p->total = off;
  return XATTN_OK;
}

int check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(XATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", p.total);
  if (ws_bytes < p.total) return fail(XATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, p.total);
  if (((uintptr_t)ws) & 255) return fail(XATTN_ERR_INVALID, "workspace must be 256-byte aligned");
  return XATTN_OK;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

KvView make_view(const XattnShape* sh, const Plan& p, const void* base) {
  KvView v;
  v.base = (const char*)base;
  v.block_table = sh->block_table;
  v.cu_k = sh->cu_k;
  v.max_blocks = sh->max_blocks_per_seq;
  v.num_pages = p.num_pages;
  v.kv_heads = p.hkv;
  v.head_dim = p.d;
  v.elem_bytes = p.elem;
  v.y_offset = 0;
  return v;
}

// k_pages: 128-key pages addressable from kview.base.
// Host-side roctx range around one stage's enqueue (visible in a
// rocprofv3 --marker-trace next to the kernels it launches).
struct StageRange {
  explicit StageRange(const char* name) { roctxRangePushA(name); }
  ~StageRange() { roctxRangePop(); }
  StageRange(const StageRange&) = delete;
  StageRange& operator=(const StageRange&) = delete;
};

hipError_t run_estimate(const XattnShape* sh, const Plan& p, const void* q, KvView kview, int jb0,
                        int jb_count, int k_pages, float* part, hipStream_t st) {
  const StageRange range("xattn:estimate");
  EstArgs ea{};
  ea.q = (const char*)q;
  ea.k = kview;
  ea.cu_q = sh->cu_q;
  ea.cu_k = sh->cu_k;
  ea.cu_q_host = sh->cu_q_host;
  ea.cu_k_host = sh->cu_k_host;
  ea.hq = p.hq;
  ea.group = p.hq / p.hkv;
  ea.jb0 = jb0;
  ea.jb_count = jb_count;
  ea.scale2 = p.est_scale * kLog2e;
  ea.part = part;
  ea.max_kb = p.max_kb;
  ea.max_r = p.max_r;
  ea.q_bytes = (long long)p.total_q * p.hq * p.d * (p.dtype == XATTN_DTYPE_BF16 ? 2 : 4);
  ea.k_bytes = (long long)k_pages * XATTN_BLOCK * p.hkv * p.d * (p.dtype == XATTN_DTYPE_BF16 ? 2 : 4);
  return launch_estimate(ea, p.dtype == XATTN_DTYPE_BF16 ? 0 : 1, p.d, p.stride, p.batch, st);
}

hipError_t run_block_sums(const XattnShape* sh, const Plan& p, const float* part, float* bs,
                          hipStream_t st) {
  const StageRange range("xattn:block_sums");
  BlockSumArgs ba;
  ba.part = part;
  ba.cu_q = sh->cu_q;
  ba.cu_k = sh->cu_k;
  ba.hq = p.hq;
  ba.stride = p.stride;
  ba.max_qb = p.max_qb;
  ba.max_kb = p.max_kb;
  ba.max_r = p.max_r;
  ba.block_sums = bs;
  return launch_block_sums(ba, p.batch, st);
}

// plan_ws (bf16 only, or nullptr): the workspace whose attention block lists
// the selection should also write, for an attention over the whole key range
// of `kview`; *lists_done tells whether it did.
hipError_t run_select(const XattnShape* sh, const XattnParams* pr, const Plan& p, const float* bs,
                      uint8_t* maskq, uint8_t* maskkv, uint8_t* hist, int32_t* counts, hipStream_t st,
                      void* plan_ws = nullptr, const KvView* kview = nullptr, bool* lists_done = nullptr) {
  const StageRange range("xattn:select");
  SelectArgs sa{};
  sa.block_sums = bs;
  sa.cu_q = sh->cu_q;
  sa.cu_k = sh->cu_k;
  sa.hq = p.hq;
  sa.hkv = p.hkv;
  sa.max_qb = p.max_qb;
  sa.max_kb = p.max_kb;
  sa.threshold = pr->threshold;
  sa.num_to_choose = pr->num_to_choose;
  sa.select_mode = pr->select_mode;
  sa.group_agg = pr->group_agg;
  sa.mask_q = maskq;
  sa.mask_kv = maskkv;
  sa.hist_sel = hist;
  sa.counts = counts;
  if (plan_ws && kview && p.dtype == XATTN_DTYPE_BF16) {
    sa.lists = ws_at<int32_t>(plan_ws, p.off_lists);
    sa.block_table = kview->block_table;
    sa.max_blocks = kview->max_blocks;
    sa.num_pages = kview->num_pages;
    sa.tail_ctr = ws_at<int>(plan_ws, p.off_ctr);
  }
  return launch_select(sa, p.batch, st, lists_done);
}

AttnArgs attn_args(const XattnShape* sh, const Plan& p, const void* q, KvView kv, KvView vv,
                   const uint8_t* mask, int jb0, int jb1) {
  AttnArgs aa{};
  aa.q = (const char*)q;
  aa.k = kv;
  aa.v = vv;
  aa.mask = mask;
  aa.cu_q = sh->cu_q;
  aa.cu_k = sh->cu_k;
  aa.hq = p.hq;
  aa.group = p.hq / p.hkv;
  aa.max_qb = p.max_qb;
  aa.max_kb = p.max_kb;
  aa.jb0 = jb0;
  aa.jb1 = jb1;
  aa.scale2 = p.softmax_scale * kLog2e;
  aa.total_q = p.total_q;
  aa.out = nullptr;
  aa.out_f32 = nullptr;
  aa.lse = nullptr;
  aa.vt = nullptr;
  aa.lists = nullptr;
  aa.num_pages = p.num_pages;
  aa.n_order = 0;
  aa.f32_splits = 1;
  aa.split_whole = 0;
  aa.cut_rows = 0;
  aa.cut_cus = 0;
  aa.cut_head = nullptr;
  aa.device_cut = 0;
  aa.f32_o = nullptr;
  aa.f32_l = nullptr;
  for (int x = 0; x < 3; ++x) {
    aa.split_o[x] = nullptr;
    aa.split_l[x] = nullptr;
  }
  return aa;
}

// bf16 preparation of an attention launch over blocks [jb0, jb1) of
// aa.mask: V^T pages of `v` (num_pages pages; with transpose_v only pages
// [vt_first, vt_first + vt_count), all from vt_first when vt_count < 0) and
// the per-row block lists.
hipError_t plan_attention(const XattnShape* sh, const Plan& p, const AttnArgs& aa, const void* v, int num_pages,
                          void* ws, bool transpose_v, hipStream_t st, bool lists_ready = false, int vt_first = 0,
                          int vt_count = -1) {
  if (p.dtype == XATTN_DTYPE_BF16) {
    AttnArgs probe = aa;
    probe.num_pages = num_pages;
    if (vt_count < 0) vt_count = num_pages - vt_first;
    // make_plan reserves V^T pages whenever a launch of the call can read them
    if (attention_reads_vt(probe, 0, p.d) && !p.reads_vt) return hipErrorInvalidValue;
    if (transpose_v && vt_count > 0 && attention_reads_vt(probe, 0, p.d)) {
      const size_t page_v = (size_t)XATTN_BLOCK * p.hkv * p.d * 2;  // bytes of one page of V (= of V^T)
      VtArgs va;
      va.v = (const char*)v + (size_t)vt_first * page_v;
      va.vt = ws_at<char>(ws, p.off_vt) + (size_t)vt_first * page_v;
      va.num_pages = vt_count;
      va.hkv = p.hkv;
      va.head_dim = p.d;
      hipError_t e = launch_vt_transpose(va, st);
      if (e != hipSuccess) return e;
    }
    if (lists_ready) return hipSuccess;  // written by the selection
    PlanArgs pa;
    pa.mask = aa.mask;
    pa.cu_q = sh->cu_q;
    pa.cu_k = sh->cu_k;
    pa.block_table = aa.k.block_table;
    pa.max_blocks = aa.k.max_blocks;
    pa.num_pages = num_pages;
    pa.hkv = p.hkv;
    pa.max_qb = p.max_qb;
    pa.max_kb = p.max_kb;
    pa.jb0 = aa.jb0;
    pa.jb1 = aa.jb1;
    pa.lists = ws_at<int32_t>(ws, p.off_lists);
    pa.tail_ctr = ws_at<int>(ws, p.off_ctr);
    return launch_plan(pa, p.batch, st);
  }
  return hipSuccess;
}

int device_cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// Whether a final-output launch takes its head length from the block lists
// on the device (set_order): in the chunk-vote modes, where the vote makes
// every row's history the same and rows differ by their causal part, so
// that the rows the host splits are the longest ones whatever the
// selection kept (every launch's lists are written before it starts, by the
// plan kernel or by the selection).  Per-KV-head rows keep the host's head:
// measured, the per-workgroup sum of the list counts cost the 4K layer 2%
// and gave the sparse per-KV-head regime nothing.
bool device_heads(const XattnParams* pr) { return pr->select_mode != XATTN_SELECT_PER_KVHEAD; }

// Launch order of the bf16 attention's rows and the split of long rows.
// A row's length is the number of key blocks it may see in [jb0, jb1) (the
// causal bound; the selection only shortens it).  Rows go longest first
// (ties keep sequence order, q blocks descending), so that the workgroups
// dispatched last are the short ones.  When the launch writes the final
// output and its longest row is well above the per-CU share of the launch
// (total row-blocks x workgroups per row / CUs) -- a single causal sequence
// whose long rows would set the launch time -- rows longer than
// bmax = max(share, longest / 3) are cut into ns = ceil(length / bmax) <= 3
// parts whose partial outputs a split merge combines (the merge rule of
// partial attention results).  Otherwise, when the longest row exceeds the
// share by at least 4 blocks and 2%, rows longer than 98% of the share plus
// two blocks keep a head of that many blocks and move the rest into a tail
// part; the tails
// come after every head and unsplit row, longest first, so they start on
// the CUs that finish first, which evens out the CUs' totals.  When
// the ping-pong kernel runs the launch, the tails are not given workgroups
// of their own: every workgroup draws them from a counter after its head or
// unsplit row, so CUs that run faster (the XCDs differ by a few percent)
// take more of them.  One sequence without splits keeps the kernel's default
// order, which is the same order.
void set_order(const XattnShape* sh, const Plan& p, AttnArgs& aa, void* ws, SplitMergeArgs* sm) {
  sm->n = 0;
  aa.n_order = 0;
  aa.split_whole = 0;
  aa.n_static = 0;
  aa.tail_ctr = nullptr;
  struct Row {
    int len, b, i;
  };
  std::vector<Row> rows;
  long long total = 0;
  int lmax = 0;
  for (int b = 0; b < p.batch; ++b) {
    const int lq = sh->cu_q_host[b + 1] - sh->cu_q_host[b];
    const int lk = sh->cu_k_host[b + 1] - sh->cu_k_host[b];
    const int qb = lq / XATTN_BLOCK, kh = (lk - lq) / XATTN_BLOCK;
    for (int i = qb - 1; i >= 0; --i) {
      const int len = std::max(0, std::min(aa.jb1, i + kh + 1) - aa.jb0);
      rows.push_back({len, b, i});
      total += len;
      lmax = std::max(lmax, len);
    }
  }
  if (rows.empty() || p.batch >= 4096 || p.max_qb >= 65536) return;
  const int group = p.hq / p.hkv;
  const int per_row = p.hkv * (group / ((group % 2 == 0) ? 2 : 1));
  const int cus = device_cu_count();
  int bmax = 0;     // > 0: equal parts of at most bmax blocks
  int head = 0;     // > 0: head + tail parts
  if (aa.out && !aa.out_f32 && cus > 0) {
    const double share = (double)total * per_row / cus;
    // rows more than twice the share: up to three equal parts; else, when
    // the longest row is over the share, head + tail (the tail at most
    // about one head long)
    if (lmax >= 4 && lmax > 2.0 * share) {
      bmax = std::max({(int)std::ceil(share), (lmax + 2) / 3, 2});
    } else if (lmax >= share + 4 && lmax >= 1.02 * share) {
      // heads a little below the share leave the faster XCDs tail work to
      // take over from the slowest one (whose heads set the launch's end);
      // two blocks more pay for the second unit's fixed cost (block list,
      // first copies, output: about 8 us against about 3 us per block) on
      // the CUs that run a short row and then a tail
      head = (int)std::ceil(0.98 * share) + kHeadPad;
    }
  }
  // With the ping-pong kernel the same rule is applied again on the device,
  // to the block lists' lengths (which a sparse selection makes much shorter
  // than the causal bounds): the rows cut here get a head of that length and
  // the rest as their tail, a row that fits it being done whole.
  const bool dev_head = head > 0 && aa.device_cut && attention_uses_pp(aa, p.d) &&
                        (long long)p.batch * p.hkv * p.max_qb <= 8192;
  struct Item {
    int neg_len;
    uint32_t entry;
    uint8_t cut;
  };
  std::vector<Item> items;  // longest part first
  int nsplit = 0;
  for (const Row& r : rows) {
    int ns = 1;
    if (bmax > 0 && r.len > bmax) {
      ns = std::min(3, (r.len + bmax - 1) / bmax);
      for (int x = 0; x < ns; ++x)
        items.push_back({-(((x + 1) * r.len) / ns - (x * r.len) / ns), order_entry(r.b, r.i, x, ns), 0});
    } else if (head > 0 && r.len > head) {
      // cut = 256 * head / len, rounded, so that part 0 holds about `head`
      // of the listed blocks (the selection may list fewer than len)
      const int cut = std::min(255, std::max(1, (int)((256LL * head + r.len / 2) / r.len)));
      ns = 2;
      items.push_back({-head, order_entry(r.b, r.i, 0, 2), (uint8_t)cut});
      items.push_back({-(r.len - head), order_entry(r.b, r.i, 1, 2), (uint8_t)cut});
    } else {
      items.push_back({-r.len, order_entry(r.b, r.i, 0, 1), 0});
    }
    if (ns > 1) {
      if (nsplit < kMaxOrder) {
        sm->rows[nsplit] = (sh->cu_q_host[r.b] / XATTN_BLOCK + r.i) | ((ns - 1) << 28);
        sm->row_bi[nsplit] = (r.b << 16) | r.i;
      }
      ++nsplit;
    }
  }
  if (items.size() > (size_t)kMaxOrder) {
    // too many parts for the order table: no splits, plain rows if they fit
    if (p.batch == 1 || rows.size() > (size_t)kMaxOrder) return;
    items.clear();
    for (const Row& r : rows) items.push_back({-r.len, order_entry(r.b, r.i, 0, 1), 0});
    nsplit = 0;
  }
  if (p.batch == 1 && nsplit == 0) return;
  // heads and unsplit rows first, then the tails, each run longest first;
  // the ping-pong kernel draws the tails dynamically
  const bool dyn = head > 0 && attention_uses_pp(aa, p.d);
  std::stable_sort(items.begin(), items.end(), [head](const Item& x, const Item& y) {
    if (head > 0) {
      const bool tx = ((x.entry >> 28) & 3u) != 0, ty = ((y.entry >> 28) & 3u) != 0;
      if (tx != ty) return !tx;
    }
    return x.neg_len < y.neg_len;
  });
  aa.n_static = 0;
  aa.tail_ctr = nullptr;
  if (dyn) {
    int ns = 0;
    while (ns < (int)items.size() && ((items[ns].entry >> 28) & 3u) == 0) ++ns;
    if (ns < (int)items.size()) {
      aa.n_static = ns;
      aa.tail_ctr = ws_at<int>(ws, p.off_ctr);
    }
  }
  aa.n_order = (int)items.size();
  for (size_t r = 0; r < items.size(); ++r) {
    aa.order[r] = (int)items[r].entry;
    aa.order_cut[r] = items[r].cut;
  }
  if (nsplit > 0) {
    for (int x = 0; x < 3; ++x) {
      aa.split_o[x] = ws_at<float>(ws, p.off_o[x]);
      aa.split_l[x] = ws_at<float>(ws, p.off_l[x]);
      sm->o[x] = aa.split_o[x];
      sm->l[x] = aa.split_l[x];
    }
    sm->n = nsplit;
    sm->lists = ws_at<int32_t>(ws, p.off_lists);
    sm->group = p.hq / p.hkv;
    sm->max_qb = p.max_qb;
    sm->max_kb = p.max_kb;
    // rows whose selection kept no more than a part's share are done whole
    sm->whole = aa.split_whole = bmax > 0 ? bmax : head;
    sm->cut_head = nullptr;
    if (dev_head) {
      sm->whole = aa.split_whole = -1;
      aa.cut_rows = p.batch * p.hkv * p.max_qb;
      aa.cut_cus = cus;
      aa.cut_head = ws_at<int>(ws, p.off_ctr) + 1;
      sm->cut_head = aa.cut_head;
      for (int r = 0; r < aa.n_order; ++r) aa.order_cut[r] = 0;
    }
    sm->heads = p.hq;
    sm->head_dim = p.d;
    sm->total_q = p.total_q;
    sm->out = aa.out;
    sm->lse = aa.lse;
  }
}

// Measurement hook (xattn_kernel_timing): while enabled, every attention
// launch records a pair of events around its block-sparse attention kernel
// on the launch's stream (pairs pooled, never destroyed while the process
// runs).
struct KernelTiming {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> used, pool;
};
KernelTiming& kernel_timing() {
  static KernelTiming t;
  return t;
}
// The event pair for the next launch, or {nullptr, nullptr} when timing is off.
std::pair<hipEvent_t, hipEvent_t> timing_pair() {
  KernelTiming& t = kernel_timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.on) return {nullptr, nullptr};
  if (t.pool.empty()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return {nullptr, nullptr};
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return {nullptr, nullptr};
    }
    t.pool.push_back({a, b});
  }
  const auto pr = t.pool.back();
  t.pool.pop_back();
  t.used.push_back(pr);
  return pr;
}

hipError_t launch_planned(const XattnShape* sh, const Plan& p, AttnArgs aa, void* ws, hipStream_t st) {
  aa.vt = ws_at<char>(ws, p.off_vt);
  aa.lists = ws_at<int32_t>(ws, p.off_lists);
  aa.f32_splits = p.f32_splits;
  aa.f32_o = ws_at<float>(ws, p.off_f32o);
  aa.f32_l = ws_at<float>(ws, p.off_f32l);
  SplitMergeArgs sm;
  sm.n = 0;
  if (p.dtype == XATTN_DTYPE_BF16) set_order(sh, p, aa, ws, &sm);
  const auto tp = timing_pair();
  if (tp.first) (void)hipEventRecord(tp.first, st);
  hipError_t e = launch_attention(aa, p.dtype == XATTN_DTYPE_BF16 ? 0 : 1, p.d, p.batch, st);
  if (tp.second) (void)hipEventRecord(tp.second, st);
  if (e != hipSuccess) return e;
  if (p.dtype != XATTN_DTYPE_BF16) {
    e = launch_f32_merge(aa, p.d, st);
    if (e != hipSuccess) return e;
  }
  if (sm.n == 0) return hipSuccess;
  return launch_split_merge(sm, st);
}

// Attention over blocks [jb0, jb1) of `mask`: prepare (bf16), then attend.
// lists_ready: the block lists are in the workspace already.
hipError_t run_attention(const XattnShape* sh, const Plan& p, AttnArgs aa, const void* v, int num_pages,
                         void* ws, bool transpose_v, hipStream_t st, bool lists_ready = false, int vt_first = 0,
                         int vt_count = -1) {
  const StageRange range("xattn:attention");
  aa.num_pages = num_pages;
  hipError_t e = plan_attention(sh, p, aa, v, num_pages, ws, transpose_v, st, lists_ready, vt_first, vt_count);
  if (e != hipSuccess) return e;
  return launch_planned(sh, p, aa, ws, st);
}

}  // namespace

// ---------------------------------------------------------------------------
// Ring engine: device slots fed from pinned host history on a transfer
// stream.  Per slot s: the transfer stream waits done[s], copies, records
// ready[s]; the caller's compute stream waits ready[s], runs every kernel
// that reads the slot, records done[s].  done[s] is recorded once at
// creation so the first copy into a slot does not wait.
// ---------------------------------------------------------------------------
struct XattnRing {
  int num_slots = 0, slot_blocks = 0, hkv = 0, d = 0, dtype = 0, elem = 0;
  // staged mode: one slot holding a whole sequence (history + chunk); the
  // history K arrives in one bulk copy, the selected V blocks are gathered
  // from the mapped pinned host memory by a kernel
  bool staged = false;
  std::vector<hipEvent_t> stage_k, stage_v;  // per history chunk: K landed, V gathered
  hipEvent_t sel_done = nullptr;             // selection written (gather may start)
  size_t block_bytes = 0;  // one 128-token block of K (or V)
  char* k_slots = nullptr;
  char* v_slots = nullptr;
  hipStream_t xfer = nullptr;
  std::vector<hipEvent_t> ready, done;
  hipEvent_t sel_ready = nullptr;
  uint8_t* host_sel = nullptr;    // pinned staging of the selection result
  int32_t* host_table = nullptr;  // pinned staging of the block -> slot table
  int host_cap = 0;               // entries of both staging buffers
  int next_slot = 0;
  int copy_delay_us = 0;
  // write-back of prefilled chunks to the host history (offload stream)
  hipStream_t offload = nullptr;
  hipEvent_t chunk_ready = nullptr;  // recorded on the caller's stream
  hipEvent_t offload_done = nullptr; // recorded after the last write-back
};

namespace {

void sleep_host_fn(void* arg) { usleep((useconds_t)(*(const int*)arg)); }

int check_pinned(const void* ptr, const char* what) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(XATTN_ERR_NOT_PINNED, "%s is not pinned host memory", what);
  }
  if (attr.type != hipMemoryTypeHost)
    return fail(XATTN_ERR_NOT_PINNED, "%s is not pinned host memory (memory type %d)", what, (int)attr.type);
  return XATTN_OK;
}

// Ring copy of `nb` K/V blocks into slot s, enqueued on the transfer stream;
// `runs` lists (first history block, count) runs laid out back to back.
hipError_t ring_fill(XattnRing* r, int s, const char* kh, const char* vh,
                     const std::vector<std::pair<int, int>>& runs, bool with_v) {
  hipError_t e = hipStreamWaitEvent(r->xfer, r->done[s], 0);
  if (e != hipSuccess) return e;
  // history written back by an earlier call may be among the blocks read
  if ((e = hipStreamWaitEvent(r->xfer, r->offload_done, 0)) != hipSuccess) return e;
  if (r->copy_delay_us > 0) {
    e = hipLaunchHostFunc(r->xfer, sleep_host_fn, &r->copy_delay_us);
    if (e != hipSuccess) return e;
  }
  const size_t slot_bytes = (size_t)r->slot_blocks * r->block_bytes;
  size_t pos = 0;
  for (const auto& run : runs) {
    const size_t off = (size_t)run.first * r->block_bytes, n = (size_t)run.second * r->block_bytes;
    e = hipMemcpyAsync(r->k_slots + s * slot_bytes + pos, kh + off, n, hipMemcpyHostToDevice, r->xfer);
    if (e != hipSuccess) return e;
    if (with_v) {
      e = hipMemcpyAsync(r->v_slots + s * slot_bytes + pos, vh + off, n, hipMemcpyHostToDevice, r->xfer);
      if (e != hipSuccess) return e;
    }
    pos += n;
  }
  return hipEventRecord(r->ready[s], r->xfer);
}

int prefill_ring(XattnRing* r, const XattnShape* sh, const XattnParams* pr, const Plan& p, const void* q,
                 const void* k, const void* v, const void* k_hist, const void* v_hist, int hist_blocks,
                 void* out, float* lse, int32_t* counts, const XattnAux* aux, void* ws, hipStream_t st) {
  const int lq = sh->cu_q_host[1], lk = sh->cu_k_host[1];
  const int qb = lq / XATTN_BLOCK, kb = lk / XATTN_BLOCK, kh = kb - qb;
  if (p.batch != 1 || sh->block_table)
    return fail(XATTN_ERR_INVALID, "ring mode needs batch == 1 and no block table");
  if (hist_blocks != kh)
    return fail(XATTN_ERR_INVALID, "hist_blocks (%d) must equal (Lk - Lq) / 128 = %d", hist_blocks, kh);
  if (r->hkv != p.hkv || r->d != p.d || r->dtype != p.dtype)
    return fail(XATTN_ERR_INVALID, "ring geometry (kv heads %d, head_dim %d, dtype %d) does not match the shape",
                r->hkv, r->d, r->dtype);
  if (pr->select_mode == XATTN_SELECT_PER_KVHEAD)
    return fail(XATTN_ERR_UNSUPPORTED, "ring mode streams the voted history blocks: select_mode must be a chunk vote");
  const bool reuse = pr->reuse_selection == 1;
  if (reuse && (!aux || !aux->mask_kv || !aux->hist_sel))
    return fail(XATTN_ERR_INVALID, "reuse_selection in ring mode needs aux->mask_kv and aux->hist_sel");
  if (kh > 0) {
    if (!k_hist || !v_hist) return fail(XATTN_ERR_INVALID, "k_hist_host and v_hist_host must not be NULL");
    int rc = check_pinned(k_hist, "k_hist_host");
    if (rc) return rc;
    if ((rc = check_pinned(v_hist, "v_hist_host"))) return rc;
  }
  if (r->host_cap < kb) {
    if (r->host_sel) (void)hipHostFree(r->host_sel);
    if (r->host_table) (void)hipHostFree(r->host_table);
    r->host_sel = nullptr;
    r->host_table = nullptr;
    r->host_cap = 0;
    hipError_t e = hipHostMalloc((void**)&r->host_sel, (size_t)kb, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void**)&r->host_table, (size_t)kb * sizeof(int32_t), hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "ring staging allocation");
    r->host_cap = kb;
  }
  g_last_error.clear();
  const char* kh_ptr = (const char*)k_hist;
  const char* vh_ptr = (const char*)v_hist;
  const size_t slot_bytes = (size_t)r->slot_blocks * r->block_bytes;
  float* part = ws_at<float>(ws, p.off_part);
  float* bs = (aux && aux->block_sums) ? aux->block_sums : ws_at<float>(ws, p.off_bs);
  uint8_t* maskkv = (aux && aux->mask_kv) ? aux->mask_kv : ws_at<uint8_t>(ws, p.off_maskkv);
  uint8_t* hist = (aux && aux->hist_sel) ? aux->hist_sel : ws_at<uint8_t>(ws, p.off_hist);
  int32_t* cnt = counts ? counts : ws_at<int32_t>(ws, p.off_counts);
  int32_t* table = ws_at<int32_t>(ws, p.off_table);
  hipError_t e;

  // ---- pass 1: history K through the ring, estimate per slot; then the current chunk
  // (skipped when an earlier selection is reused)
  for (int j0 = 0; !reuse && j0 < kh; j0 += r->slot_blocks) {
    const int nb = std::min(r->slot_blocks, kh - j0);
    const int s = r->next_slot;
    r->next_slot = (s + 1) % r->num_slots;
    if ((e = ring_fill(r, s, kh_ptr, vh_ptr, {{j0, nb}}, false)) != hipSuccess) return hip_fail(e, "ring copy");
    if ((e = hipStreamWaitEvent(st, r->ready[s], 0)) != hipSuccess) return hip_fail(e, "ring wait");
    KvView kv = make_view(sh, p, r->k_slots + s * slot_bytes);
    kv.y_offset = j0 * XATTN_BLOCK;
    if ((e = run_estimate(sh, p, q, kv, j0, nb, nb, part, st)) != hipSuccess) return hip_fail(e, "estimate launch");
    if ((e = hipEventRecord(r->done[s], st)) != hipSuccess) return hip_fail(e, "ring record");
  }
  if (!reuse) {
    KvView kv = make_view(sh, p, k);
    kv.y_offset = kh * XATTN_BLOCK;
    if ((e = run_estimate(sh, p, q, kv, kh, qb, qb, part, st)) != hipSuccess) return hip_fail(e, "estimate launch");
    if ((e = run_block_sums(sh, p, part, bs, st)) != hipSuccess) return hip_fail(e, "block-sum launch");
    if ((e = run_select(sh, pr, p, bs, ws_at<uint8_t>(ws, p.off_maskq), maskkv, hist, cnt, st)) != hipSuccess)
      return hip_fail(e, "select launch");
  }

  // ---- the one host wait: which history blocks were voted in
  if ((e = hipMemcpyAsync(r->host_sel, hist, (size_t)kb, hipMemcpyDeviceToHost, st)) != hipSuccess)
    return hip_fail(e, "selection copy");
  if ((e = hipEventRecord(r->sel_ready, st)) != hipSuccess) return hip_fail(e, "selection record");
  if ((e = hipEventSynchronize(r->sel_ready)) != hipSuccess) return hip_fail(e, "selection wait");
  std::vector<int> sel;
  for (int j = 0; j < kh; ++j)
    if (r->host_sel[j]) sel.push_back(j);
  for (int j = 0; j < kb; ++j) r->host_table[j] = -1;
  for (size_t x = 0; x < sel.size(); ++x) r->host_table[sel[x]] = (int)(x % r->slot_blocks);
  for (int j = kh; j < kb; ++j) r->host_table[j] = j - kh;
  if ((e = hipMemcpyAsync(table, r->host_table, (size_t)kb * sizeof(int32_t), hipMemcpyHostToDevice, st)) != hipSuccess)
    return hip_fail(e, "table copy");

  // the current chunk (qb pages at k / v) or one slot (slot_blocks pages)
  auto paged_view = [&](const void* base, int pages) {
    KvView kv = make_view(sh, p, base);
    kv.block_table = table;
    kv.max_blocks = kb;
    kv.num_pages = pages;
    return kv;
  };
  float* o_acc = ws_at<float>(ws, p.off_o[0]);
  float* l_acc = ws_at<float>(ws, p.off_l[0]);
  float* o_cur = ws_at<float>(ws, p.off_o[1]);
  float* l_cur = ws_at<float>(ws, p.off_l[1]);
  float* o_tmp = ws_at<float>(ws, p.off_o[2]);
  float* l_tmp = ws_at<float>(ws, p.off_l[2]);
  const bool bf16 = p.dtype == XATTN_DTYPE_BF16;

  // ---- current chunk (causal), overlapping the first history copies
  {
    AttnArgs aa = attn_args(sh, p, q, paged_view(k, qb), paged_view(v, qb), maskkv, kh, kb);
    if (sel.empty()) {
      if (bf16) aa.out = out;
      else aa.out_f32 = (float*)out;
      aa.lse = lse;
    } else {
      aa.out_f32 = o_cur;
      aa.lse = l_cur;
    }
    if ((e = run_attention(sh, p, aa, v, qb, ws, true, st)) != hipSuccess) return hip_fail(e, "attention launch");
    if (sel.empty()) return XATTN_OK;
  }
  // ---- selected history blocks, slot by slot; partials merged history-first
  for (size_t x0 = 0; x0 < sel.size(); x0 += r->slot_blocks) {
    const size_t x1 = std::min(sel.size(), x0 + (size_t)r->slot_blocks);
    std::vector<std::pair<int, int>> runs;
    for (size_t x = x0; x < x1; ++x) {
      if (!runs.empty() && runs.back().first + runs.back().second == sel[x]) runs.back().second++;
      else runs.push_back({sel[x], 1});
    }
    const int s = r->next_slot;
    r->next_slot = (s + 1) % r->num_slots;
    if ((e = ring_fill(r, s, kh_ptr, vh_ptr, runs, true)) != hipSuccess) return hip_fail(e, "ring copy");
    if ((e = hipStreamWaitEvent(st, r->ready[s], 0)) != hipSuccess) return hip_fail(e, "ring wait");
    const bool first = (x0 == 0);
    AttnArgs aa = attn_args(sh, p, q, paged_view(r->k_slots + s * slot_bytes, r->slot_blocks),
                            paged_view(r->v_slots + s * slot_bytes, r->slot_blocks),
                            maskkv, sel[x0], sel[x1 - 1] + 1);
    aa.out_f32 = first ? o_acc : o_tmp;
    aa.lse = first ? l_acc : l_tmp;
    if ((e = run_attention(sh, p, aa, r->v_slots + s * slot_bytes, (int)(x1 - x0), ws, true, st)) != hipSuccess)
      return hip_fail(e, "attention launch");
    if ((e = hipEventRecord(r->done[s], st)) != hipSuccess) return hip_fail(e, "ring record");
    if (!first) {
      MergeArgs ma;
      ma.rows = p.total_q;
      ma.heads = p.hq;
      ma.head_dim = p.d;
      ma.o_a = o_acc;
      ma.lse_a = l_acc;
      ma.o_b = o_tmp;
      ma.lse_b = l_tmp;
      ma.o = o_acc;
      ma.o_bf16 = nullptr;
      ma.lse = l_acc;
      if ((e = launch_merge(ma, st)) != hipSuccess) return hip_fail(e, "merge launch");
    }
  }
  // ---- final: history partial, then the current chunk
  MergeArgs ma;
  ma.rows = p.total_q;
  ma.heads = p.hq;
  ma.head_dim = p.d;
  ma.o_a = o_acc;
  ma.lse_a = l_acc;
  ma.o_b = o_cur;
  ma.lse_b = l_cur;
  ma.o = bf16 ? nullptr : (float*)out;
  ma.o_bf16 = bf16 ? out : nullptr;
  ma.lse = lse ? lse : l_tmp;
  if ((e = launch_merge(ma, st)) != hipSuccess) return hip_fail(e, "merge launch");
  return XATTN_OK;
}

// Staged ring prefill: history K in one bulk copy on the transfer stream,
// the current chunk copied behind it, the resident estimate and selection
// over the whole sequence, then a gather kernel reads exactly the voted
// history V blocks from the mapped pinned host memory (no host wait), and one
// resident attention launch writes the final output.
int prefill_staged(XattnRing* r, const XattnShape* sh, const XattnParams* pr, const Plan& p, const void* q,
                   const void* k, const void* v, const void* k_hist, const void* v_hist, int hist_blocks,
                   void* out, float* lse, int32_t* counts, const XattnAux* aux, void* ws, hipStream_t st) {
  const int lq = sh->cu_q_host[1], lk = sh->cu_k_host[1];
  const int qb = lq / XATTN_BLOCK, kb = lk / XATTN_BLOCK, kh = kb - qb;
  if (p.batch != 1 || sh->block_table)
    return fail(XATTN_ERR_INVALID, "ring mode needs batch == 1 and no block table");
  if (hist_blocks != kh)
    return fail(XATTN_ERR_INVALID, "hist_blocks (%d) must equal (Lk - Lq) / 128 = %d", hist_blocks, kh);
  if (r->hkv != p.hkv || r->d != p.d || r->dtype != p.dtype)
    return fail(XATTN_ERR_INVALID, "ring geometry (kv heads %d, head_dim %d, dtype %d) does not match the shape",
                r->hkv, r->d, r->dtype);
  if (pr->select_mode == XATTN_SELECT_PER_KVHEAD)
    return fail(XATTN_ERR_UNSUPPORTED, "ring mode streams the voted history blocks: select_mode must be a chunk vote");
  if (kb > r->slot_blocks)
    return fail(XATTN_ERR_INVALID, "the sequence has %d blocks; the staged ring holds %d", kb, r->slot_blocks);
  const bool reuse = pr->reuse_selection == 1;
  if (reuse && (!aux || !aux->mask_kv || !aux->hist_sel))
    return fail(XATTN_ERR_INVALID, "reuse_selection in ring mode needs aux->mask_kv and aux->hist_sel");
  void* kh_dev = nullptr;
  void* vh_dev = nullptr;
  if (kh > 0) {
    if (!k_hist || !v_hist) return fail(XATTN_ERR_INVALID, "k_hist_host and v_hist_host must not be NULL");
    int rc = check_pinned(k_hist, "k_hist_host");
    if (rc) return rc;
    if ((rc = check_pinned(v_hist, "v_hist_host"))) return rc;
    if (hipHostGetDevicePointer(&kh_dev, const_cast<void*>(k_hist), 0) != hipSuccess ||
        hipHostGetDevicePointer(&vh_dev, const_cast<void*>(v_hist), 0) != hipSuccess) {
      (void)hipGetLastError();
      return fail(XATTN_ERR_NOT_PINNED, "the history arrays are not mapped into the device address space");
    }
  }
  g_last_error.clear();
  const size_t bb = r->block_bytes;
  char* sk = r->k_slots;
  char* sv = r->v_slots;
  float* part = ws_at<float>(ws, p.off_part);
  float* bs = (aux && aux->block_sums) ? aux->block_sums : ws_at<float>(ws, p.off_bs);
  uint8_t* maskkv = (aux && aux->mask_kv) ? aux->mask_kv : ws_at<uint8_t>(ws, p.off_maskkv);
  uint8_t* hist = (aux && aux->hist_sel) ? aux->hist_sel : ws_at<uint8_t>(ws, p.off_hist);
  int32_t* cnt = counts ? counts : ws_at<int32_t>(ws, p.off_counts);
  float* o_acc = ws_at<float>(ws, p.off_o[0]);
  float* l_acc = ws_at<float>(ws, p.off_l[0]);
  float* o_cur = ws_at<float>(ws, p.off_o[1]);
  float* l_cur = ws_at<float>(ws, p.off_l[1]);
  float* o_tmp = ws_at<float>(ws, p.off_o[2]);
  float* l_tmp = ws_at<float>(ws, p.off_l[2]);
  const bool bf16 = p.dtype == XATTN_DTYPE_BF16;
  const int nch = (kh + kStageChunk - 1) / kStageChunk;
  hipError_t e;
  // Pipeline (transfer stream X, caller's stream S):
  //   X: history K chunk c -> stage_k[c], for every c (skipped on reuse)
  //   S: chunk K/V copied in; estimate of K chunk c as it lands; the current
  //      chunk's estimate; block sums; selection -> sel_done
  //   X: after sel_done, gather of the voted V (and, on reuse, K) blocks of
  //      chunk c from mapped host memory -> stage_v[c]
  //   S: current chunk attention (partial), then chunk c's history attention
  //      after stage_v[c], merged history-first, then with the current chunk
  if ((e = hipStreamWaitEvent(r->xfer, r->done[0], 0)) != hipSuccess) return hip_fail(e, "ring wait");
  if ((e = hipStreamWaitEvent(r->xfer, r->offload_done, 0)) != hipSuccess) return hip_fail(e, "ring wait");
  for (int c = 0; !reuse && c < nch; ++c) {
    const int j0 = c * kStageChunk, nb = std::min(kStageChunk, kh - j0);
    if (r->copy_delay_us > 0 && (e = hipLaunchHostFunc(r->xfer, sleep_host_fn, &r->copy_delay_us)) != hipSuccess)
      return hip_fail(e, "ring delay");
    if ((e = hipMemcpyAsync(sk + (size_t)j0 * bb, (const char*)k_hist + (size_t)j0 * bb, (size_t)nb * bb,
                            hipMemcpyHostToDevice, r->xfer)) != hipSuccess)
      return hip_fail(e, "history copy");
    if ((e = hipEventRecord(r->stage_k[c], r->xfer)) != hipSuccess) return hip_fail(e, "ring record");
  }
  if ((e = hipStreamWaitEvent(st, r->done[0], 0)) != hipSuccess) return hip_fail(e, "ring wait");
  if ((e = hipMemcpyAsync(sk + (size_t)kh * bb, k, (size_t)qb * bb, hipMemcpyDeviceToDevice, st)) != hipSuccess ||
      (e = hipMemcpyAsync(sv + (size_t)kh * bb, v, (size_t)qb * bb, hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return hip_fail(e, "chunk copy");
  const KvView kview = make_view(sh, p, sk), vview = make_view(sh, p, sv);
  if (!reuse) {
    for (int c = 0; c < nch; ++c) {
      const int j0 = c * kStageChunk, nb = std::min(kStageChunk, kh - j0);
      if ((e = hipStreamWaitEvent(st, r->stage_k[c], 0)) != hipSuccess) return hip_fail(e, "ring wait");
      if ((e = run_estimate(sh, p, q, kview, j0, nb, kb, part, st)) != hipSuccess) return hip_fail(e, "estimate launch");
    }
    if ((e = run_estimate(sh, p, q, kview, kh, qb, kb, part, st)) != hipSuccess) return hip_fail(e, "estimate launch");
    if ((e = run_block_sums(sh, p, part, bs, st)) != hipSuccess) return hip_fail(e, "block-sum launch");
    if ((e = run_select(sh, pr, p, bs, ws_at<uint8_t>(ws, p.off_maskq), maskkv, hist, cnt, st)) != hipSuccess)
      return hip_fail(e, "select launch");
  }
  if ((e = hipEventRecord(r->sel_done, st)) != hipSuccess) return hip_fail(e, "ring record");
  if ((e = hipStreamWaitEvent(r->xfer, r->sel_done, 0)) != hipSuccess) return hip_fail(e, "ring wait");
  for (int c = 0; c < nch; ++c) {
    const int j0 = c * kStageChunk, nb = std::min(kStageChunk, kh - j0);
    const size_t off = (size_t)j0 * bb;
    if ((e = launch_gather_blocks(hist + j0, nb, (const char*)vh_dev + off, sv + off, bb, r->xfer)) != hipSuccess)
      return hip_fail(e, "gather launch");
    if (reuse &&
        (e = launch_gather_blocks(hist + j0, nb, (const char*)kh_dev + off, sk + off, bb, r->xfer)) != hipSuccess)
      return hip_fail(e, "gather launch");
    if ((e = hipEventRecord(r->stage_v[c], r->xfer)) != hipSuccess) return hip_fail(e, "ring record");
  }
  // ---- current chunk (causal) while the first gathers run
  {
    AttnArgs aa = attn_args(sh, p, q, kview, vview, maskkv, kh, kb);
    if (nch == 0) {
      if (bf16) aa.out = out;
      else aa.out_f32 = (float*)out;
      aa.lse = lse;
    } else {
      aa.out_f32 = o_cur;
      aa.lse = l_cur;
    }
    if ((e = run_attention(sh, p, aa, sv, kb, ws, true, st, false, kh, qb)) != hipSuccess)
      return hip_fail(e, "attention launch");
  }
  MergeArgs ma;
  ma.rows = p.total_q;
  ma.heads = p.hq;
  ma.head_dim = p.d;
  for (int c = 0; c < nch; ++c) {
    const int j0 = c * kStageChunk, j1 = std::min(kh, j0 + kStageChunk);
    if ((e = hipStreamWaitEvent(st, r->stage_v[c], 0)) != hipSuccess) return hip_fail(e, "ring wait");
    AttnArgs aa = attn_args(sh, p, q, kview, vview, maskkv, j0, j1);
    aa.out_f32 = c == 0 ? o_acc : o_tmp;
    aa.lse = c == 0 ? l_acc : l_tmp;
    if ((e = run_attention(sh, p, aa, sv, kb, ws, true, st, false, j0, j1 - j0)) != hipSuccess)
      return hip_fail(e, "attention launch");
    if (c > 0) {
      ma.o_a = o_acc;
      ma.lse_a = l_acc;
      ma.o_b = o_tmp;
      ma.lse_b = l_tmp;
      ma.o = o_acc;
      ma.o_bf16 = nullptr;
      ma.lse = l_acc;
      if ((e = launch_merge(ma, st)) != hipSuccess) return hip_fail(e, "merge launch");
    }
  }
  if (nch > 0) {
    ma.o_a = o_acc;
    ma.lse_a = l_acc;
    ma.o_b = o_cur;
    ma.lse_b = l_cur;
    ma.o = bf16 ? nullptr : (float*)out;
    ma.o_bf16 = bf16 ? out : nullptr;
    ma.lse = lse ? lse : l_tmp;
    if ((e = launch_merge(ma, st)) != hipSuccess) return hip_fail(e, "merge launch");
  }
  if ((e = hipEventRecord(r->done[0], st)) != hipSuccess) return hip_fail(e, "ring record");
  return XATTN_OK;
}

int ring_create(int num_slots, int slot_blocks, int num_kv_heads, int head_dim, int dtype, bool staged,
                XattnRing** out) {
  if (!out) return fail(XATTN_ERR_INVALID, "out must not be NULL");
  *out = nullptr;
  if (num_slots < 1 || slot_blocks < 1 || num_kv_heads < 1)
    return fail(XATTN_ERR_INVALID, "need slot_blocks >= 1, num_kv_heads >= 1");
  if (head_dim != 64 && head_dim != 128) return fail(XATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != XATTN_DTYPE_BF16 && dtype != XATTN_DTYPE_F32) return fail(XATTN_ERR_INVALID, "unknown dtype %d", dtype);
  XattnRing* r = new XattnRing();
  r->staged = staged;
  r->num_slots = num_slots;
  r->slot_blocks = slot_blocks;
  r->hkv = num_kv_heads;
  r->d = head_dim;
  r->dtype = dtype;
  r->elem = dtype == XATTN_DTYPE_BF16 ? 2 : 4;
  r->block_bytes = (size_t)XATTN_BLOCK * num_kv_heads * head_dim * r->elem;
  const size_t bytes = (size_t)num_slots * slot_blocks * r->block_bytes;
  hipError_t e = hipMalloc((void**)&r->k_slots, bytes);
  if (e == hipSuccess) e = hipMalloc((void**)&r->v_slots, bytes);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&r->xfer, hipStreamNonBlocking);
  for (int s = 0; e == hipSuccess && s < num_slots; ++s) {
    hipEvent_t a = nullptr, b = nullptr;
    e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
    if (a) r->ready.push_back(a);
    if (b) r->done.push_back(b);
    if (e == hipSuccess) e = hipEventRecord(b, r->xfer);  // slot free before its first copy
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&r->sel_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&r->offload, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&r->chunk_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&r->offload_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(r->offload_done, r->offload);  // nothing written back yet
  if (e == hipSuccess && staged) {
    e = hipEventCreateWithFlags(&r->sel_done, hipEventDisableTiming);
    const int nch = (slot_blocks + kStageChunk - 1) / kStageChunk;
    for (int c = 0; e == hipSuccess && c < nch; ++c) {
      hipEvent_t a = nullptr, b = nullptr;
      e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
      if (a) r->stage_k.push_back(a);
      if (b) r->stage_v.push_back(b);
    }
  }
  if (e != hipSuccess) {
    int rc = hip_fail(e, "ring creation");
    xattn_ring_destroy(r);
    return rc;
  }
  *out = r;
  return XATTN_OK;
}



// XATTN_DEBUG set to anything but "" or "0": calls with a block table first
// copy it to the host (after the caller's stream has drained) and reject an
// entry that a sequence uses (key block j < Lk/128) but that names no page of
// the cache.  Without it such entries are treated as absent pages by every
// kernel (keys read as missing), which is memory-safe but silently changes
// the result.
bool debug_mode() {
  const char* e = getenv("XATTN_DEBUG");
  return e && *e && strcmp(e, "0") != 0;
}

int validate_block_table(const XattnShape* sh, const Plan& p, hipStream_t st) {
  if (!sh->block_table || !debug_mode()) return XATTN_OK;
  std::vector<int32_t> t((size_t)sh->batch * sh->max_blocks_per_seq);
  hipError_t e = hipMemcpyAsync(t.data(), sh->block_table, t.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "block table copy (XATTN_DEBUG)");
  for (int b = 0; b < sh->batch; ++b) {
    const int nb = (sh->cu_k_host[b + 1] - sh->cu_k_host[b]) / XATTN_BLOCK;
    for (int j = 0; j < nb; ++j) {
      const int page = t[(size_t)b * sh->max_blocks_per_seq + j];
      if (page < 0 || page >= p.num_pages)
        return fail(XATTN_ERR_INVALID,
                    "sequence %d: block_table entry %d is %d, not a page of the cache [0, %d) (XATTN_DEBUG)", b, j,
                    page, p.num_pages);
    }
  }
  return XATTN_OK;
}

// The resident-K/V path of xattn_prefill_chunk on workspace `ws` (validated).
int prefill_resident(const XattnShape* shape, const XattnParams* params, const Plan& p, const void* q,
                     const void* k, const void* v, void* out, float* lse, int32_t* counts, const XattnAux* aux,
                     void* ws, hipStream_t st) {
  g_last_error.clear();
  float* part = ws_at<float>(ws, p.off_part);
  float* bs = (aux && aux->block_sums) ? aux->block_sums : ws_at<float>(ws, p.off_bs);
  uint8_t* maskkv = (aux && aux->mask_kv) ? aux->mask_kv : ws_at<uint8_t>(ws, p.off_maskkv);
  uint8_t* hist = (aux && aux->hist_sel) ? aux->hist_sel : ws_at<uint8_t>(ws, p.off_hist);
  int32_t* cnt = counts ? counts : ws_at<int32_t>(ws, p.off_counts);
  const KvView kview = make_view(shape, p, k), vview = make_view(shape, p, v);
  hipError_t e = hipSuccess;
  bool lists_ready = false;  // block lists written by the selection kernels
  if (params->reuse_selection) {
    if (!aux || !aux->mask_kv) return fail(XATTN_ERR_INVALID, "reuse_selection needs aux->mask_kv");
  } else {
    e = run_estimate(shape, p, q, kview, 0, p.max_kb, p.num_pages, part, st);
    if (e != hipSuccess) return hip_fail(e, "estimate launch");
    e = run_block_sums(shape, p, part, bs, st);
    if (e != hipSuccess) return hip_fail(e, "block-sum launch");
    e = run_select(shape, params, p, bs, ws_at<uint8_t>(ws, p.off_maskq), maskkv, hist, cnt, st, ws, &kview,
                   &lists_ready);
    if (e != hipSuccess) return hip_fail(e, "select launch");
  }
  AttnArgs aa = attn_args(shape, p, q, kview, vview, maskkv, 0, p.max_kb);
  aa.device_cut = device_heads(params);
  if (p.dtype == XATTN_DTYPE_BF16) aa.out = out;
  else aa.out_f32 = (float*)out;
  aa.lse = lse;
  e = run_attention(shape, p, aa, v, p.num_pages, ws, true, st, lists_ready);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return XATTN_OK;
}

}  // namespace

namespace xattn {
int workspace_bytes(const XattnShape* shape, const XattnParams* params, size_t* bytes) {
  Plan p;
  const int rc = make_plan(shape, params, &p);
  *bytes = rc ? 0 : p.total;
  return rc;
}
}  // namespace xattn

extern "C" {

const char* xattn_last_error(void) { return g_last_error.c_str(); }

int xattn_kernel_timing(int on) {
  KernelTiming& t = kernel_timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.on = on != 0;
  for (const auto& pr : t.used) t.pool.push_back(pr);
  t.used.clear();
  return XATTN_OK;
}

int xattn_kernel_timing_read(double* total_ms, int* launches) {
  if (!total_ms || !launches) return fail(XATTN_ERR_INVALID, "xattn_kernel_timing_read: NULL output");
  KernelTiming& t = kernel_timing();
  std::lock_guard<std::mutex> lock(t.mu);
  double sum = 0.0;
  int n = 0;
  int rc = XATTN_OK;
  for (const auto& pr : t.used) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) {
      rc = fail(XATTN_ERR_HIP, "xattn_kernel_timing_read: %s", hipGetErrorString(e));
      break;
    }
    sum += ms;
    ++n;
  }
  for (const auto& pr : t.used) t.pool.push_back(pr);
  t.used.clear();
  *total_ms = sum;
  *launches = n;
  return rc;
}

size_t xattn_workspace_size(const XattnShape* shape, const XattnParams* params) {
  Plan p;
  if (make_plan(shape, params, &p) != XATTN_OK) return 0;
  return p.total;
}

int xattn_estimate(const XattnShape* shape, const XattnParams* params, const void* q, const void* k,
                   float* block_sums, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, params, &p);
  if (rc) return rc;
  if (!q || !k || !block_sums) return fail(XATTN_ERR_INVALID, "q, k and block_sums must not be NULL");
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if ((rc = validate_block_table(shape, p, (hipStream_t)stream))) return rc;
  g_last_error.clear();
  hipStream_t st = (hipStream_t)stream;
  float* part = ws_at<float>(ws, p.off_part);
  hipError_t e = run_estimate(shape, p, q, make_view(shape, p, k), 0, p.max_kb, p.num_pages, part, st);
  if (e != hipSuccess) return hip_fail(e, "estimate launch");
  e = run_block_sums(shape, p, part, block_sums, st);
  if (e != hipSuccess) return hip_fail(e, "block-sum launch");
  return XATTN_OK;
}

int xattn_select(const XattnShape* shape, const XattnParams* params, const float* block_sums,
                 uint8_t* mask_kv, uint8_t* hist_sel, int32_t* counts, void* ws, size_t ws_bytes,
                 void* stream) {
  Plan p;
  int rc = make_plan(shape, params, &p);
  if (rc) return rc;
  if (!block_sums || !mask_kv) return fail(XATTN_ERR_INVALID, "block_sums and mask_kv must not be NULL");
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  g_last_error.clear();
  uint8_t* hist = hist_sel ? hist_sel : ws_at<uint8_t>(ws, p.off_hist);
  int32_t* cnt = counts ? counts : ws_at<int32_t>(ws, p.off_counts);
  hipError_t e = run_select(shape, params, p, block_sums, ws_at<uint8_t>(ws, p.off_maskq), mask_kv, hist,
                            cnt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return XATTN_OK;
}

int xattn_sparse_attn(const XattnShape* shape, const XattnParams* params, const void* q, const void* k,
                      const void* v, const uint8_t* mask_kv, void* out, float* lse, void* ws,
                      size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, params, &p);
  if (rc) return rc;
  if (!q || !k || !v || !mask_kv || !out)
    return fail(XATTN_ERR_INVALID, "q, k, v, mask_kv and out must not be NULL");
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if ((rc = validate_block_table(shape, p, (hipStream_t)stream))) return rc;
  g_last_error.clear();
  AttnArgs aa = attn_args(shape, p, q, make_view(shape, p, k), make_view(shape, p, v), mask_kv, 0, p.max_kb);
  aa.device_cut = device_heads(params);
  if (p.dtype == XATTN_DTYPE_BF16) aa.out = out;
  else aa.out_f32 = (float*)out;
  aa.lse = lse;
  hipError_t e = run_attention(shape, p, aa, v, p.num_pages, ws, true, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return XATTN_OK;
}

int xattn_attn_plan(const XattnShape* shape, const XattnParams* params, const void* v, const uint8_t* mask_kv,
                    void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, params, &p);
  if (rc) return rc;
  if (!v || !mask_kv) return fail(XATTN_ERR_INVALID, "v and mask_kv must not be NULL");
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if ((rc = validate_block_table(shape, p, (hipStream_t)stream))) return rc;
  g_last_error.clear();
  AttnArgs aa = attn_args(shape, p, nullptr, make_view(shape, p, v), make_view(shape, p, v), mask_kv, 0, p.max_kb);
  hipError_t e = plan_attention(shape, p, aa, v, p.num_pages, ws, true, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention plan launch");
  return XATTN_OK;
}

int xattn_attn_run(const XattnShape* shape, const XattnParams* params, const void* q, const void* k, const void* v,
                   const uint8_t* mask_kv, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, params, &p);
  if (rc) return rc;
  if (!q || !k || !v || !mask_kv || !out)
    return fail(XATTN_ERR_INVALID, "q, k, v, mask_kv and out must not be NULL");
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if ((rc = validate_block_table(shape, p, (hipStream_t)stream))) return rc;
  g_last_error.clear();
  AttnArgs aa = attn_args(shape, p, q, make_view(shape, p, k), make_view(shape, p, v), mask_kv, 0, p.max_kb);
  aa.device_cut = device_heads(params);
  if (p.dtype == XATTN_DTYPE_BF16) aa.out = out;
  else aa.out_f32 = (float*)out;
  aa.lse = lse;
  hipError_t e = launch_planned(shape, p, aa, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return XATTN_OK;
}

int xattn_merge_attn(int rows, int heads, int head_dim, const float* o_a, const float* lse_a,
                     const float* o_b, const float* lse_b, float* o, float* lse, void* stream) {
  if (rows < 0 || heads < 1 || head_dim < 4 || head_dim % 4)
    return fail(XATTN_ERR_INVALID, "rows >= 0, heads >= 1 and head_dim a positive multiple of 4 required");
  if (rows == 0) return XATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse)
    return fail(XATTN_ERR_INVALID, "merge pointers must not be NULL");
  g_last_error.clear();
  MergeArgs ma;
  ma.rows = rows;
  ma.heads = heads;
  ma.head_dim = head_dim;
  ma.o_a = o_a;
  ma.lse_a = lse_a;
  ma.o_b = o_b;
  ma.lse_b = lse_b;
  ma.o = o;
  ma.o_bf16 = nullptr;
  ma.lse = lse;
  hipError_t e = launch_merge(ma, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return XATTN_OK;
}

int xattn_prefill_chunk(XattnRing* ring, const XattnShape* shape, const XattnParams* params,
                        const void* q, const void* k, const void* v, const void* k_hist_host,
                        const void* v_hist_host, int hist_blocks, void* out, float* lse,
                        int32_t* counts, const XattnAux* aux, void* ws, size_t ws_bytes,
                        void* stream) {
  const StageRange range("xattn_prefill_chunk");
  Plan p;
  int rc = make_plan(shape, params, &p);
  if (rc) return rc;
  if (!q || !k || !v || !out) return fail(XATTN_ERR_INVALID, "q, k, v and out must not be NULL");
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if (ring && ring->staged)
    return prefill_staged(ring, shape, params, p, q, k, v, k_hist_host, v_hist_host, hist_blocks, out, lse, counts,
                          aux, ws, (hipStream_t)stream);
  if (ring)
    return prefill_ring(ring, shape, params, p, q, k, v, k_hist_host, v_hist_host, hist_blocks, out, lse, counts,
                        aux, ws, (hipStream_t)stream);
  if ((rc = validate_block_table(shape, p, (hipStream_t)stream))) return rc;
  return prefill_resident(shape, params, p, q, k, v, out, lse, counts, aux, ws, (hipStream_t)stream);
}

int xattn_ring_create(int num_slots, int slot_blocks, int num_kv_heads, int head_dim, int dtype,
                      XattnRing** out) {
  if (num_slots < 2) return fail(XATTN_ERR_INVALID, "need num_slots >= 2");
  return ring_create(num_slots, slot_blocks, num_kv_heads, head_dim, dtype, false, out);
}

int xattn_ring_create_staged(int max_blocks, int num_kv_heads, int head_dim, int dtype, XattnRing** out) {
  return ring_create(1, max_blocks, num_kv_heads, head_dim, dtype, true, out);
}

void xattn_ring_destroy(XattnRing* r) {
  if (!r) return;
  if (r->xfer) (void)hipStreamSynchronize(r->xfer);
  for (auto ev : r->ready) (void)hipEventSynchronize(ev), (void)hipEventDestroy(ev);
  for (auto ev : r->done) (void)hipEventSynchronize(ev), (void)hipEventDestroy(ev);
  if (r->sel_ready) (void)hipEventDestroy(r->sel_ready);
  if (r->offload) (void)hipStreamSynchronize(r->offload);
  for (auto ev : r->stage_k) (void)hipEventDestroy(ev);
  for (auto ev : r->stage_v) (void)hipEventDestroy(ev);
  if (r->sel_done) (void)hipEventDestroy(r->sel_done);
  if (r->chunk_ready) (void)hipEventDestroy(r->chunk_ready);
  if (r->offload_done) (void)hipEventDestroy(r->offload_done);
  if (r->offload) (void)hipStreamDestroy(r->offload);
  if (r->xfer) (void)hipStreamDestroy(r->xfer);
  if (r->k_slots) (void)hipFree(r->k_slots);
  if (r->v_slots) (void)hipFree(r->v_slots);
  if (r->host_sel) (void)hipHostFree(r->host_sel);
  if (r->host_table) (void)hipHostFree(r->host_table);
  delete r;
}

int xattn_ring_offload_chunk(XattnRing* ring, const void* k, const void* v, void* k_host_dst, void* v_host_dst,
                             int num_blocks, void* stream) {
  if (!ring) return fail(XATTN_ERR_INVALID, "ring must not be NULL");
  if (num_blocks < 0) return fail(XATTN_ERR_INVALID, "num_blocks must be >= 0");
  if (num_blocks == 0) return XATTN_OK;
  if (!k || !v || !k_host_dst || !v_host_dst) return fail(XATTN_ERR_INVALID, "k, v and the host destinations must not be NULL");
  int rc = check_pinned(k_host_dst, "k_host_dst");
  if (rc) return rc;
  if ((rc = check_pinned(v_host_dst, "v_host_dst"))) return rc;
  g_last_error.clear();
  const size_t bytes = (size_t)num_blocks * ring->block_bytes;
  hipError_t e = hipEventRecord(ring->chunk_ready, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(ring->offload, ring->chunk_ready, 0);
  if (e == hipSuccess && ring->copy_delay_us > 0) e = hipLaunchHostFunc(ring->offload, sleep_host_fn, &ring->copy_delay_us);
  if (e == hipSuccess) e = hipMemcpyAsync(k_host_dst, k, bytes, hipMemcpyDeviceToHost, ring->offload);
  if (e == hipSuccess) e = hipMemcpyAsync(v_host_dst, v, bytes, hipMemcpyDeviceToHost, ring->offload);
  if (e == hipSuccess) e = hipEventRecord(ring->offload_done, ring->offload);
  if (e != hipSuccess) return hip_fail(e, "write-back");
  return XATTN_OK;
}

int xattn_ring_offload_wait(XattnRing* ring, void* stream) {
  if (!ring) return fail(XATTN_ERR_INVALID, "ring must not be NULL");
  hipError_t e = hipStreamWaitEvent((hipStream_t)stream, ring->offload_done, 0);
  if (e != hipSuccess) return hip_fail(e, "write-back wait");
  return XATTN_OK;
}

int xattn_ring_set_copy_delay_us(XattnRing* ring, int usec) {
  if (!ring || usec < 0) return fail(XATTN_ERR_INVALID, "ring must not be NULL and usec >= 0");
  ring->copy_delay_us = usec;
  return XATTN_OK;
}

}  // extern "C"
