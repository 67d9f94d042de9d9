// Block-sparse flash attention with log-sum-exp ("XAttention BSA Policy"
// design doc, section 2: flash_attn_with_lse over the selected blocks) and
// the LSE merge of two partial results (merge_attention_outputs).
//
// bf16 kernel (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//  * a workgroup is HPW q heads of one KV group x one 128-query block; wave
//    w owns 32 queries of head w/4.  The HPW heads share every K/V tile.
//  * key tiles of 64 keys are copied global -> LDS with direct
//    (global_load_lds) 16-byte loads into a 3-stage ring, one barrier per tile;
//    K rows and V^T rows are XOR-swizzled in 16-byte chunks against LDS bank
//    conflicts.  V is read from a d-major copy (VtArgs) so that its tile is a
//    plain copy too.
//  * S^T = K Q^T puts one query per lane (accumulator column) and 32 of the
//    tile's keys in that lane's registers: the online-softmax max and sum are
//    per lane plus one exchange between half-waves.  Its registers, rounded to
//    bf16, are the B operand of O^T += V^T P^T directly (the k-slot order of
//    P^T is matched by the key order of the V^T copy).
//  * the running max is refreshed only when a tile raises it by more than 8
//    (base 2), so the O rescale is rare; probabilities stay below 2^8.
//  * blockIdx -> (kv head, q block) is XCD-aware: the workgroups of one KV
//    head land on one XCD and share its L2.
#include <type_traits>
#include <utility>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();
// Bound on a lane's sum of the probabilities of one tile (32 per lane) taken
// at a running max that has not moved; a larger sum moves the max.
constexpr float kLazySum = 1024.f;
#ifndef XATTN_GATHER_WGS
#define XATTN_GATHER_WGS 16
#endif
#ifndef XATTN_PF
#define XATTN_PF 3
#endif


// Position of key k inside a 16-key group of a V^T row: bits 2 and 3
// swapped, so k-slot group hh of MFMA k-step m holds keys
// {16m + 4hh + 0..3, 16m + 8 + 4hh + 0..3}, the keys a lane's S^T
// accumulator registers 4*i0 .. 4*i0+7 hold.
__host__ __device__ __forceinline__ int vperm(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 2^x with the bare v_exp_f32 (results below 2^-126 flush to zero, which is
// harmless for softmax weights; exp2f would add a denormal range fix-up of
// five more VALU instructions per call).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine the values of lanes l and l ^ 32 with one v_permlane32_swap: after
// the swap, the two results hold {x[l ^ 32], x[l]} in some order on every lane.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer descriptor word 3 for gfx950 (32-bit data format, no swizzle).
constexpr int kBufFlags = 0x00020000;

// 16 bytes per lane, buffer -> LDS (lane L writes lds + 16 L); offsets at or
// beyond the descriptor's byte count read as zero.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
}

// 16-byte and 4-byte LDS reads issued from inline asm.  The compiler does not
// see them as LDS accesses, so it never adds a wait for the pending direct
// (global -> LDS) tile loads in front of them; the kernel orders them itself
// (s_waitcnt vmcnt + s_barrier before a tile is read, lgkm_wait before use).
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
__device__ __forceinline__ int lds_read4_sync(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ int lds_read4(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
// Wait until at most N LDS (lgkm) operations are outstanding; the operands
// tie the values that must have arrived to this point of the program.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 8-byte transposing LDS read (gfx950): within each group of 16 lanes, lane
// i receives 16-bit element i % 4 of the 8-byte chunks addressed by lanes
// i / 4 + 4 e, e = 0..3 (element e of the result).
template <int OFF>
__device__ __forceinline__ u32x2 lds_read8_tr_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2& a, u32x2& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(int& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}

// Empty asm that needs its operand in registers at this point of the
// program: values computed before it stay computed before it.
__device__ __forceinline__ void reg_fence(const f32x16& v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void reg_fence(const bf16x8& v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void reg_fence(float v) { asm volatile("" ::"v"(v)); }

// s_waitcnt with only vmcnt constrained (expcnt, lgkmcnt left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Work unit (sequence b, kv head g, head pair, q block i) of workgroup `id`.
// With a row order from the host (a.order: (b, i) rows, longest causal row
// first) and a multiple of 8 kv slots (g, pair), XCD id % 8 takes the slots
// congruent to it (its L2 serves their K/V) and every XCD walks the same
// longest-first row order, so heavy and light sequences are spread evenly
// over the XCDs.  Otherwise: blocks of consecutive units per XCD, rows of
// each sequence longest first.
// A row may be split into ns parts (part s of ns equal parts of its block
// list); the host splits only rows it lists in the order.
struct WorkUnit {
  int b, g, pair, i, s, ns, cut;
};
// Unit of order entry r in kv slot `slot` (slot = pair * hkv + g).
__device__ __forceinline__ WorkUnit entry_unit(const AttnArgs& a, int hkv, int r, int slot) {
  WorkUnit u;
  const uint32_t e = (uint32_t)a.order[r];
  u.b = (int)((e >> 16) & 0xfffu);
  u.i = (int)(e & 0xffffu);
  u.s = (int)((e >> 28) & 3u);
  u.ns = (int)(e >> 30) + 1;
  u.cut = a.order_cut[r];
  u.g = slot % hkv;
  u.pair = slot / hkv;
  return u;
}
__device__ __forceinline__ WorkUnit work_unit(const AttnArgs& a, int hkv, int npair, int id, int nwg) {
  WorkUnit u;
  const int ns = hkv * npair;
  if (a.n_order > 0) {
    int slot, r;
    if (ns % 8 == 0 && nwg % 8 == 0) {
      const int per = ns / 8, k = id / 8;
      slot = (id % 8) + 8 * (k % per);
      r = k / per;
    } else {
      slot = id % ns;
      r = id / ns;
    }
    return entry_unit(a, hkv, r, slot);
  }
  const int full = (nwg / 8) * 8;
  const int logical = id < full ? (id % 8) * (nwg / 8) + id / 8 : id;
  const int irev = logical % a.max_qb;
  int rest = logical / a.max_qb;
  u.pair = rest % npair;
  rest /= npair;
  u.g = rest % hkv;
  u.b = rest / hkv;
  u.i = a.max_qb - 1 - irev;
  u.s = 0;
  u.ns = 1;
  u.cut = 0;
  return u;
}

// Part s of ns of a row's block list, copied to LDS: list[0] = its count,
// list[1..] its entries.  The parts are consecutive runs of the list, as even
// as integer division makes them, or for two parts with cut > 0 the first
// (count * cut) / 256 entries and the rest; the diagonal block (the last
// entry) falls in the last part.  The caller synchronises before reading
// `list`.
// A row cut into ns > 1 parts whose list holds at most `whole` entries (the
// selection kept few of its blocks) is done whole by part 0, which writes the
// final output; its other parts are empty and the split merge skips the row
// (split_row_whole).
__device__ __forceinline__ bool split_row_whole(int nall, int ns, int whole) { return ns > 1 && nall <= whole; }

// Entries [z0, z0 + n) of a row list of nall entries that part s of ns takes.
// head > 0 (heads from the device): part 0 of two takes the first `head`
// entries, part 1 the rest.
__device__ __forceinline__ void row_part(int nall, int s, int ns, int cut, int whole, int head, int& z0, int& n) {
  if (split_row_whole(nall, ns, whole)) {
    z0 = 0;
    n = s == 0 ? nall : 0;
  } else if (ns == 2 && head > 0) {
    z0 = s ? head : 0;
    n = s ? nall - head : head;
  } else if (ns == 2 && cut > 0) {
    const int c = (nall * cut) >> 8;
    z0 = s ? c : 0;
    n = s ? nall - c : c;
  } else {
    z0 = (s * nall) / ns;
    n = ((s + 1) * nall) / ns - z0;
  }
}

__device__ __forceinline__ int load_row_list(const int32_t* glist, int32_t* list, int s, int ns, int cut, int tid,
                                             int nthreads, int whole, int head = 0, int nall = -1) {
  if (nall < 0) nall = glist[0];
  int z0, n;
  row_part(nall, s, ns, cut, whole, head, z0, n);
  for (int z = tid; z <= n; z += nthreads) list[z] = (z == 0) ? n : glist[z0 + z];
  return n;
}

// ---------------------------------------------------------------------------
// V -> V^T pages.  Workgroup (page, kv head): [128 keys][d] -> [d][128].
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void vt_transpose_kernel(VtArgs a) {
  constexpr int P = kBlock + 2;  // LDS pitch (bf16) of the [d][key] tile
  __shared__ uint16_t t[D * P];
  const int page = blockIdx.x, g = blockIdx.y;
  const char* src = a.v + ((long long)page * kBlock * a.hkv + g) * D * 2;
  const long long row_bytes = (long long)a.hkv * D * 2;
  for (int c = threadIdx.x; c < kBlock * D / 8; c += 256) {
    const int key = c / (D / 8), part = c % (D / 8);
    const u32x4 v = *(const u32x4*)(src + key * row_bytes + part * 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = v[e >> 1];
      t[(part * 8 + e) * P + key] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
  }
  __syncthreads();
  char* dst = a.vt + ((long long)page * a.hkv + g) * D * kBlock * 2;
  for (int c = threadIdx.x; c < D * kBlock / 8; c += 256) {
    const int d = c / (kBlock / 8), chunk = c % (kBlock / 8);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = chunk * 8 + 2 * e;  // storage positions p0, p0+1
      const int k0 = (p0 & ~15) | vperm(p0 & 15), k1 = (p0 & ~15) | vperm((p0 + 1) & 15);
      o[e] = (uint32_t)t[d * P + k0] | ((uint32_t)t[d * P + k1] << 16);
    }
    *(u32x4*)(dst + ((long long)d * kBlock + chunk * 8) * 2) = o;
  }
}

// ---------------------------------------------------------------------------
// Block lists for one attention launch.  One wave per (q block, kv head, b).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void plan_kernel(PlanArgs a) {
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  int32_t* out = a.lists + (((long long)b * a.hkv + g) * a.max_qb + i) * (a.max_kb + 1);
  if (a.tail_ctr && i == 0 && g == 0 && b == 0 && lane == 0) atomicExch(a.tail_ctr, 0);
  if (i >= qb) {
    if (lane == 0) out[0] = 0;
    return;
  }
  const uint8_t* mrow = a.mask + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  const int jend = min(a.jb1, i + kh + 1);
  const int page0 = a.cu_k[b] / kBlock;
  int n = 0;
  for (int j0 = a.jb0; j0 < jend; j0 += 64) {
    const int j = j0 + lane;
    int page = -1;
    if (j < jend && mrow[j]) page = a.block_table ? a.block_table[(long long)b * a.max_blocks + j] : page0 + j;
    const bool take = page >= 0 && page < a.num_pages;
    const unsigned long long bal = __ballot(take);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (take) out[1 + n + before] = (page << 1) | (j == i + kh ? 1 : 0);
    n += __popcll(bal);
  }
  if (lane == 0) out[0] = n;
}

// ---------------------------------------------------------------------------
// bf16 MFMA attention.
// ---------------------------------------------------------------------------
template <int D, int HPW>
__global__ __launch_bounds__(256 * HPW) void attn_mfma(AttnArgs a, int hkv) {
  constexpr int NW = 4 * HPW;          // waves
  constexpr int KT = 64;               // keys per tile
  constexpr int KROW = D * 2;          // bytes per K row in LDS
  constexpr int KCPR = D / 8;          // 16-byte chunks per K row
  constexpr int TILE = KT * KROW;      // bytes of one K (or V^T) tile
  constexpr int CH = TILE / 16;        // 16-byte chunks per tile
  constexpr int LPW = CH / (64 * NW);  // direct loads per wave per operand
  constexpr int STAGES = 3;
  static_assert(LPW >= 1 && CH % (64 * NW) == 0, "tile / workgroup mismatch");
  // LDS: K tiles of the 3 stages, then V^T tiles of the 3 stages; every read
  // address is a per-lane base plus an immediate offset below 64 KiB.
  __shared__ __align__(1024) char tiles[2 * STAGES * TILE];
  extern __shared__ int32_t list[];

  // ---- work unit (XCD-aware: the 8 XCDs take consecutive ids round-robin)
  const int npair = a.group / HPW;
  const WorkUnit wk = work_unit(a, hkv, npair, blockIdx.x, gridDim.x);
  const int pair = wk.pair, g = wk.g, b = wk.b, i = wk.i;
  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  if (i >= lq / kBlock) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int hsub = w >> 2, qs = w & 3;
  const int h = g * a.group + pair * HPW + hsub;
  const int xq = qs * 32 + l32;  // query within the block
  const int x = i * kBlock + xq;

  // Block list of this row, copied to LDS.
  const int32_t* glist = a.lists + (((long long)b * hkv + g) * a.max_qb + i) * (a.max_kb + 1);
  const int nblk = load_row_list(glist, list, wk.s, wk.ns, wk.cut, tid, 64 * NW, a.split_whole);
  const bool whole = split_row_whole(glist[0], wk.ns, a.split_whole);
  __syncthreads();
  if (whole && wk.s > 0) return;  // part 0 does the whole row
  const int ntile = 2 * nblk;
  // The diagonal block, if present, is the last entry: only its two tiles
  // need the causal mask.
  const int first_diag = (nblk > 0 && (list[nblk] & 1)) ? ntile - 2 : ntile;
  const uint32_t list_lds = (uint32_t)(uintptr_t)(lds_ptr_t)list;

  // Q fragments: B operand of S^T (query col = lane%32, d slots 8*hh .. +8).
  bf16x8 qf[D / 16];
  {
    const char* qrow = a.q + ((long long)(q0 + x) * a.hq + h) * D * 2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qrow + (kk * 16 + hh * 8) * 2);
  }

  // Per-thread constant parts of the direct-load addresses.
  const long long k_page_bytes = (long long)kBlock * hkv * D * 2;
  const long long k_row_bytes = (long long)hkv * D * 2;
  const long long vt_page_bytes = (long long)hkv * D * kBlock * 2;
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    const int idx = (w * LPW + n) * 64 + lane;
    const int krow = idx / KCPR, kpch = idx % KCPR;
    const int kc = (KCPR == 16) ? (kpch ^ (krow & 15)) : (kpch ^ ((krow >> 1) & 7));
    koff[n] = (int)(krow * k_row_bytes + kc * 16);
    const int vrow = idx >> 3, vpch = idx & 7;
    const int vc = vpch ^ ((vrow >> 1) & 7);
    voff[n] = (vrow * kBlock + vc * 8) * 2;
  }
  const char* kbase = a.k.base + (long long)g * D * 2;
  const char* vbase = a.vt + (long long)g * D * kBlock * 2;

  auto issue = [&](int t, int e, int stage) {
    const int page = e >> 1, sub = t & 1;
    const char* kp = kbase + page * k_page_bytes + sub * KT * k_row_bytes;
    const char* vp = vbase + page * vt_page_bytes + sub * KT * 2;
    char* kl = tiles + stage * TILE;
    char* vl = tiles + (STAGES + stage) * TILE;
#pragma unroll
    for (int n = 0; n < LPW; ++n) load_lds16(kp + koff[n], kl + (w * LPW + n) * 1024);
#pragma unroll
    for (int n = 0; n < LPW; ++n) load_lds16(vp + voff[n], vl + (w * LPW + n) * 1024);
  };

  // Per-lane LDS addresses of the MFMA A fragments (stage 0; other stages
  // and rows 32.. / d-blocks add immediate offsets).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)tiles;
  const int kswz = (KCPR == 16) ? (l32 & 15) : ((l32 >> 1) & 7);
  const int vswz = (l32 >> 1) & 7;
  uint32_t kaddr[D / 16], vaddr[4];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kaddr[kk] = lds0 + l32 * KROW + (((2 * kk + hh) ^ kswz) * 16);
#pragma unroll
  for (int m = 0; m < 4; ++m) vaddr[m] = lds0 + STAGES * TILE + l32 * (KT * 2) + (((2 * m + hh) ^ vswz) * 16);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[n][e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.scale2;

  auto compute = [&](auto stage_tag, int t) {
    constexpr int S = decltype(stage_tag)::value;
    const bool diag = t >= first_diag;
    const int sub = t & 1;
    // ---- S^T = K Q^T; K fragments read one MFMA pair ahead
    f32x16 s0, s1;
#pragma unroll
    for (int z = 0; z < 16; ++z) {
      s0[z] = 0.f;
      s1[z] = 0.f;
    }
    u32x4 ka0 = lds_read16_at<S * TILE>(kaddr[0]);
    u32x4 ka1 = lds_read16_at<S * TILE + 32 * KROW>(kaddr[0]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 kb0, kb1;
      if (kk + 1 < D / 16) {
        kb0 = lds_read16_at<S * TILE>(kaddr[kk + 1 < D / 16 ? kk + 1 : 0]);
        kb1 = lds_read16_at<S * TILE + 32 * KROW>(kaddr[kk + 1 < D / 16 ? kk + 1 : 0]);
        lgkm_wait<2>(ka0, ka1);
      } else {
        lgkm_wait<0>(ka0, ka1);
      }
      s0 = mfma32(__builtin_bit_cast(bf16x8, ka0), qf[kk], s0);
      s1 = mfma32(__builtin_bit_cast(bf16x8, ka1), qf[kk], s1);
      ka0 = kb0;
      ka1 = kb1;
    }
    // ---- causal mask on the diagonal block only (a real, uniform branch: the
    // empty asm keeps the compiler from evaluating the mask on every tile)
    if (diag) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int z = 0; z < 16; ++z) {
        const int key = sub * KT + 8 * (z >> 2) + 4 * hh + (z & 3);
        if (key > xq) s0[z] = kNegInf;
        if (key + 32 > xq) s1[z] = kNegInf;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int z = 1; z < 16; ++z) mx = fmaxf(mx, fmaxf(s0[z], s1[z]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_tile = mx * c2;
    // lazy rescale: refresh the running max only when it would grow by > 8
    if (__ballot(m_tile > m_run + 8.0f) != 0ull) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int z = 0; z < 16; ++z) oacc[n][z] *= alpha;
      m_run = m_new;
    }
    const float mneg = (m_run == kNegInf) ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int z = 0; z < 16; ++z) {
      s0[z] = fast_exp2(fmaf(s0[z], c2, mneg));
      s1[z] = fast_exp2(fmaf(s1[z], c2, mneg));
      psum += s0[z] + s1[z];
    }
    l_run += psum;
    // ---- P^T fragments: k-step m covers keys 16m .. 16m+15 of the tile
    bf16x8 pb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i0 = 2 * (m & 1);
#pragma unroll
      for (int z = 0; z < 8; ++z) pb[m][z] = (__bf16)((m < 2) ? s0[4 * i0 + z] : s1[4 * i0 + z]);
    }
    // ---- O^T += V^T P^T; V^T fragments read two MFMAs ahead
    constexpr int NV = 4 * (D / 32);
    auto vread = [&](auto j_tag) {
      constexpr int J = decltype(j_tag)::value;
      constexpr int M = J / (D / 32), N = J % (D / 32);
      return lds_read16_at<S * TILE + N * 32 * KT * 2>(vaddr[M]);
    };
    u32x4 va = vread(std::integral_constant<int, 0>{});
    u32x4 vb = vread(std::integral_constant<int, 1>{});
    auto pv_step = [&](auto j_tag) {
      constexpr int J = decltype(j_tag)::value;
      u32x4 vc;
      if constexpr (J + 2 < NV) {
        vc = vread(std::integral_constant<int, J + 2>{});
        lgkm_wait<2>(va);
      } else if constexpr (J + 1 < NV) {
        lgkm_wait<1>(va);
      } else {
        lgkm_wait<0>(va);
      }
      oacc[J % (D / 32)] = mfma32(__builtin_bit_cast(bf16x8, va), pb[J / (D / 32)], oacc[J % (D / 32)]);
      va = vb;
      vb = vc;
    };
    [&]<int... J>(std::integer_sequence<int, J...>) {
      (pv_step(std::integral_constant<int, J>{}), ...);
    }(std::make_integer_sequence<int, NV>{});
  };

  // One tile step with compile-time stage buffers: wait for this wave's loads
  // of tile t (only tile t+1's may remain in flight), barrier to publish all
  // waves' parts (a bare s_barrier: a memory fence would drain the loads of
  // tile t+1 too), refill the stage freed by tile t-1 with tile t+2, compute.
  // The list entry of tile t+2 was read one step earlier (e_next).
  int e_next = 0;
  auto step = [&](auto stage_tag, int t) {
    constexpr int S = decltype(stage_tag)::value;
    if (t + 1 < ntile) wait_vmcnt<2 * LPW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (t + 2 < ntile) {
      lgkm_wait<0>(e_next);
      issue(t + 2, e_next, (S + 2) % STAGES);
    }
    if (t + 3 < ntile) e_next = lds_read4(list_lds + 4 * (1 + ((t + 3) >> 1)));
    compute(stage_tag, t);
  };

  if (ntile > 0) issue(0, list[1], 0);
  if (ntile > 1) issue(1, list[1], 1);
  if (ntile > 2) e_next = list[1 + 1];
  for (int t = 0; t < ntile; t += 3) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntile) step(std::integral_constant<int, 1>{}, t + 1);
    if (t + 2 < ntile) step(std::integral_constant<int, 2>{}, t + 2);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const long long orow = ((long long)(q0 + x) * a.hq + h) * D;
  float* const of32 = (wk.ns > 1 && !whole) ? a.split_o[wk.s] : a.out_f32;
  float* const lsep = (wk.ns > 1 && !whole) ? a.split_l[wk.s] : a.lse;
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d = n * 32 + 8 * ii + 4 * hh;
      const float v0 = oacc[n][4 * ii + 0] * inv, v1 = oacc[n][4 * ii + 1] * inv;
      const float v2 = oacc[n][4 * ii + 2] * inv, v3 = oacc[n][4 * ii + 3] * inv;
      if (of32) {
        f32x4 v = {v0, v1, v2, v3};
        *(f32x4*)(of32 + orow + d) = v;
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 o4;
        o4[0] = (__bf16)v0;
        o4[1] = (__bf16)v1;
        o4[2] = (__bf16)v2;
        o4[3] = (__bf16)v3;
        *(bf16x4*)((char*)a.out + (orow + d) * 2) = o4;
      }
    }
  if (lsep && hh == 0) {
    const float lse = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
    lsep[(long long)h * a.total_q + q0 + x] = lse;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA attention, two heads per workgroup, ping-pong schedule.
//
// Waves 0-3 (group A, first head of the pair) and waves 4-7 (group B, second
// head) share the SIMDs pairwise (wave w and w+4 on one SIMD) and run the same
// per-tile work half a tile apart.  A wave issues nothing but LDS reads and
// MFMAs in its MFMA phase (O^T += V^T P^T of tile u-1, then S^T = K Q^T of
// tile u; a wave's own VALU work would serialise with its MFMAs) while the
// other group runs its softmax on the VALU.  Per tile, A runs MFMA(u) then
// softmax(u) and B runs softmax(u-1) then MFMA(u); one workgroup barrier per
// tile realigns the two halves (a second barrier between the halves cost
// more in waiting than it gained in alignment).
// K and V tiles (both in the caller's [key][kv head][d] layout) live in two
// 4-stage LDS rings (tile t in stage t % 4); V^T fragments of the PV MFMAs
// come from transposing LDS reads.  The softmax phase of tile g also issues
// copy group g: K of tile g+3 and V of tile g+2 (raw buffer loads straight
// to LDS, which count on vmcnt only).  Each wave waits for its own copies of
// a tile before the barrier after which the tile is read; register fences
// keep the compiler from moving phase work between phases.
// ---------------------------------------------------------------------------
template <int D, int PF>
__global__ __launch_bounds__(512) void attn_pp(AttnArgs a, int hkv) {
  constexpr int NW = 8;
  constexpr int KT = 64;               // keys per tile
  constexpr int KROW = D * 2;          // bytes per K row in LDS
  constexpr int KCPR = D / 8;          // 16-byte chunks per K row
  constexpr int TILE = KT * KROW;      // bytes of one K (or V) tile
  constexpr int CH = TILE / 16;        // 16-byte chunks per tile
  constexpr int LPW = CH / (64 * NW);  // direct loads per wave per operand
  constexpr int ST = 4;                // ring stages
  constexpr int NS = 2 * (D / 16);     // S^T MFMAs per tile
  constexpr int NPV = 4 * (D / 32);    // O^T MFMAs per tile
  static_assert(LPW >= 1 && CH % (64 * NW) == 0, "tile / workgroup mismatch");
  static_assert(NS == NPV, "phase interleave assumes equal MFMA counts");
  __shared__ __align__(1024) char tiles[2 * ST * TILE];  // K stages, then V stages
  extern __shared__ int32_t list[];

  // ---- work units.  Unit of workgroup id: XCD-aware (the 8 XCDs take
  // consecutive ids round-robin).  With dynamic tails, every workgroup then
  // draws further units from the launch's counter until they run out.
  const int npair = a.group / 2;
  const int slots = hkv * npair;
  const bool dyn = a.n_static > 0 && a.n_static < a.n_order && a.tail_ctr != nullptr;
  __shared__ int next_unit;
  // Heads from the device (formed before the first unit, below).
  // nall_pre: the first unit's list count, loaded with them.
  int whole_lim = a.split_whole, dev_head = 0, nall_pre = -1;
  auto run_unit = [&](const WorkUnit wk) __attribute__((always_inline)) {
    const int pair = wk.pair, g = wk.g, b = wk.b, i = wk.i;
    const int q0 = a.cu_q[b];
    const int lq = a.cu_q[b + 1] - q0;
    if (i >= lq / kBlock) return;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int grp = __builtin_amdgcn_readfirstlane(w >> 2), qs = w & 3;
    const int h = g * a.group + pair * 2 + grp;
    const int xq = qs * 32 + l32;  // query within the block
    const int x = i * kBlock + xq;

    // Block list of this row, copied to LDS.
    const int32_t* glist = a.lists + (((long long)b * hkv + g) * a.max_qb + i) * (a.max_kb + 1);
    const int nall = nall_pre >= 0 ? nall_pre : glist[0];
    nall_pre = -1;
    const int nblk = __builtin_amdgcn_readfirstlane(
        load_row_list(glist, list, wk.s, wk.ns, wk.cut, tid, 64 * NW, whole_lim, dev_head, nall));
    const bool whole = split_row_whole(__builtin_amdgcn_readfirstlane(nall), wk.ns, whole_lim);
    __syncthreads();
    if (whole && wk.s > 0) return;  // part 0 does the whole row
    const int ntile = 2 * nblk;
    // The diagonal block, if present, is the last entry: only its two tiles
    // need the causal mask.
    const int first_diag = __builtin_amdgcn_readfirstlane((nblk > 0 && (list[nblk] & 1)) ? ntile - 2 : ntile);
    const uint32_t list_lds = (uint32_t)(uintptr_t)(lds_ptr_t)list;

    // Q fragments: B operand of S^T (query col = lane%32, d slots 8*hh .. +8).
    bf16x8 qf[D / 16];
    {
      const char* qrow = a.q + ((long long)(q0 + x) * a.hq + h) * D * 2;
  #pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qrow + (kk * 16 + hh * 8) * 2);
    }

    // Per-thread constant parts of the direct-load addresses.
    const long long k_page_bytes = (long long)kBlock * hkv * D * 2;
    const long long k_row_bytes = (long long)hkv * D * 2;
    // V row swizzle of the transposing reads: the rows one read instruction
    // touches (4hh + c/4 plus a multiple of 8) spread over all 64 banks, two
    // lanes per bank (the minimum for 512 bytes)
    auto vn_swz = [](int row) { return (KCPR == 16) ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };
    int koff[LPW], voff[LPW];
  #pragma unroll
    for (int n = 0; n < LPW; ++n) {
      const int idx = (w * LPW + n) * 64 + lane;
      const int krow = idx / KCPR, kpch = idx % KCPR;
      const int kc = (KCPR == 16) ? (kpch ^ (krow & 15)) : (kpch ^ ((krow >> 1) & 7));
      koff[n] = (int)(krow * k_row_bytes + kc * 16);
      // V in its own layout, 16-byte chunks of a row XOR-swizzled for the
      // transposing reads
      voff[n] = (int)(krow * k_row_bytes + (kpch ^ vn_swz(krow)) * 16);
    }
    const char* kbase = a.k.base + (long long)g * D * 2;
    const char* vbase = a.v.base + (long long)g * D * 2;

    // Tile copies: one raw buffer descriptor per operand for the whole launch
    // (its K and V spans are below 2^31 bytes, checked by the launcher); a
    // tile is a 32-bit byte offset in soffset plus the constant per-lane
    // offsets, its LDS destination goes to m0.  Copy group gi copies K of
    // tile gi+3 into K stage (gi+3)%4 and V of tile gi+2 into V stage
    // (gi+2)%4.  Those stages last held K of tile gi-1 and V of tile gi-2,
    // both last read in the MFMA phases of tile gi-1, which both groups have
    // finished before group gi is issued.  Every group issues all its loads:
    // a tile past the end (or before the start) re-reads an existing tile
    // into its own stage, which no later phase reads, so the number of
    // loads in flight -- and every vmcnt below -- is the same for each group.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)kbase, (short)0, (int)(a.num_pages * k_page_bytes - (long long)g * D * 2), kBufFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)vbase, (short)0, (int)(a.num_pages * k_page_bytes - (long long)g * D * 2), kBufFlags);
    const int kpb = (int)k_page_bytes, khalf = (int)(KT * k_row_bytes);
    char* const kl0 = tiles + wu * LPW * 1024;  // this wave's part of K stage 0 (V stage 0 at + ST * TILE)
    // Copy sources.  Lane j of `eb` holds the byte offset of the page of block
    // eb0 + j (the last block's for lanes past the end), read from the list in
    // LDS by one read that waits for its own result (a read left in flight in
    // an asm output could be copied by the compiler before it lands) and
    // refilled once per 64 blocks; a group takes its offsets with v_readlane.
    // Tile t is half t & 1 of block t >> 1.  A group past the last tile copies
    // a tile of the last block into a stage that no later phase reads.
    int eb = 0, eb0 = 0;
    auto refill = [&](int base) __attribute__((always_inline)) {
      eb0 = base;
      const int z = base + lane < nblk ? base + lane : nblk - 1;
      eb = (lds_read4_sync(list_lds + 4 * (1 + z)) >> 1) * kpb;
    };
    int soff_k = 0, soff_v = 0;
    // The loads of one copy group: K into stage KS, V into stage VS.
    auto issue = [&](int ks, int vs) __attribute__((always_inline)) {
      const uint32_t lk = (uint32_t)(uintptr_t)(lds_ptr_t)kl0 + ks * TILE;
      const uint32_t lv = (uint32_t)(uintptr_t)(lds_ptr_t)kl0 + (ST + vs) * TILE;
      [&]<int... N>(std::integer_sequence<int, N...>) {
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(uintptr_t)(lk + N * 1024), 16, (uint32_t)koff[N],
                                                  soff_k, 0, 0),
         ...);
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(uintptr_t)(lv + N * 1024), 16, (uint32_t)voff[N],
                                                  soff_v, 0, 0),
         ...);
      }(std::make_integer_sequence<int, LPW>{});
    };
    // Groups -3..-1 (G = gi + 3 = 0..2): K of tile G into stage G, V of tile
    // max(G - 1, 0) into stage max(G - 1, 0), tiles clamped to the last one.
    auto copy_prologue = [&](auto g_tag) __attribute__((always_inline)) {
      constexpr int G = decltype(g_tag)::value, GV = G > 1 ? G - 1 : 0;
      const int tk = G < ntile ? G : ntile - 1;
      const int tv = GV < ntile ? GV : ntile - 1;
      soff_k = __builtin_amdgcn_readlane(eb, tk >> 1) + (tk & 1) * khalf;
      soff_v = __builtin_amdgcn_readlane(eb, tv >> 1) + (tv & 1) * khalf;
      issue(G, GV);
    };
    // Group gi >= 0 (P = gi % 2): K of tile gi + 3 into stage (gi + 3) % 4, V
    // of tile gi + 2 into stage (gi + 2) % 4.  For even gi both tiles are the
    // halves of block (gi + 3) >> 1, whose offset the previous group took
    // (e_last); for odd gi the K tile opens the next block and the V tile is
    // the second half of e_last's.  li = ((gi + 3) >> 1) - eb0.
    int e_last = 0, li = 1;
    auto copy_group = [&](auto p_tag, int gi) __attribute__((always_inline)) {
      if constexpr (decltype(p_tag)::value) {
        if (++li == 64) {
          refill(eb0 + 64);
          li = 0;
        }
        const int e = __builtin_amdgcn_readlane(eb, li);
        soff_k = e;
        soff_v = e_last + khalf;
        e_last = e;
      } else {
        soff_k = e_last + khalf;
        soff_v = e_last;
      }
      issue((gi + 3) & (ST - 1), (gi + 2) & (ST - 1));
    };
    // Per-lane LDS addresses of the MFMA A fragments in stage 0.
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)tiles;
    const int kswz = (KCPR == 16) ? (l32 & 15) : ((l32 >> 1) & 7);
    uint32_t kaddr[D / 16], vaddr[4] = {0u, 0u, 0u, 0u};
  #pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kaddr[kk] = lds0 + l32 * KROW + (((2 * kk + hh) ^ kswz) * 16);
    {
      // Transposing reads of V rows: for d block n and read r of key chunk m,
      // lane c of 16-lane group G (c = lane % 16) addresses key row
      // 16m + 8r + 4hh + c/4 at d = 32n + 16 (G % 2) + 4 (c % 4); lane l then
      // holds V[16m + 8r + 4hh + e][32n + l % 32], e = 0..3, in k-slots
      // 8hh + 4r + e: the keys P^T's k-slots hold (see vperm).  The row part
      // 16m + 8r is an immediate offset; vaddr[n] carries the rest.
      const int c = lane & 15, row0 = 4 * hh + (c >> 2);
  #pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        const int d = 32 * n + 16 * ((lane >> 4) & 1) + 4 * (c & 3);
        vaddr[n] = lds0 + ST * TILE + row0 * KROW + (((d >> 3) ^ vn_swz(row0)) * 16) + ((d >> 2) & 1) * 8;
      }
    }

    f32x16 oacc[D / 32];
  #pragma unroll
    for (int n = 0; n < D / 32; ++n)
  #pragma unroll
      for (int e = 0; e < 16; ++e) oacc[n][e] = 0.f;
    f32x16 s0, s1;
    bf16x8 pb[4];
    float m_run = kNegInf, l_run = 0.f;
    float mneg = kPosInf;  // -m_run; +inf while m_run is -inf
    const float c2 = a.scale2;

    // ---- MFMA phase of tile u: O^T += V^T(u-1) P^T(u-1) if PV, S^T(u) = K(u) Q^T
    // if SS.  The two MFMA streams alternate; LDS fragments are read two ahead.
    auto mma = [&](auto pv_tag, auto ss_tag, int u) __attribute__((always_inline)) {
      constexpr bool PV = decltype(pv_tag)::value, SS = decltype(ss_tag)::value;
      constexpr int NOPS = (PV ? NPV : 0) + (SS ? NS : 0);
      // K(u) in stage u % 4, V(u - 1) in stage (u - 1) % 4
      const uint32_t kst = (uint32_t)((u & (ST - 1)) * TILE);
      const uint32_t vst = (uint32_t)(((u + ST - 1) & (ST - 1)) * TILE);
      uint32_t ka[D / 16], va4[4];
      if constexpr (SS) {
  #pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) ka[kk] = kaddr[kk] + kst;
  #pragma unroll
        for (int z = 0; z < 16; ++z) {
          s0[z] = 0.f;
          s1[z] = 0.f;
        }
      }
      if constexpr (PV) {
  #pragma unroll
        for (int m = 0; m < 4; ++m) va4[m] = vaddr[m] + vst;
      }
      // op J: a PV step when PV and (J even or !SS), else an S step
      auto is_pv = [](int j) constexpr { return PV && (!SS || (j % 2 == 0)); };
      auto sub_idx = [](int j) constexpr { return (PV && SS) ? j / 2 : j; };
      // LDS read instructions of op j (a PV step reads two halves when V is
      // read transposed), and those of ops J+1 .. J+PF (issued before op J's
      // wait)
      auto after = [=](int j) constexpr {
        int c = 0;
        for (int x = j + 1; x < NOPS && x <= j + PF; ++x) c += is_pv(x) ? 2 : 1;
        return c < 15 ? c : 15;  // lgkmcnt field limit; a smaller count only waits longer
      };
      // fragment of op J: fr[J] (16-byte read) or fl[J], fh[J] (transposing
      // halves); reads run PF ops ahead of the MFMAs
      u32x4 fr[NOPS];
      u32x2 fl[NOPS], fh[NOPS];
      auto frag = [&](auto j_tag) {
        constexpr int J = decltype(j_tag)::value;
        constexpr int I = sub_idx(J);
        if constexpr (is_pv(J)) {
          constexpr int M = I / (D / 32), N = I % (D / 32);
          fl[J] = lds_read8_tr_at<(16 * M) * KROW>(va4[N]);
          fh[J] = lds_read8_tr_at<(16 * M + 8) * KROW>(va4[N]);
        } else {
          constexpr int KK = I >> 1, HALF = I & 1;
          fr[J] = lds_read16_at<HALF * 32 * KROW>(ka[KK]);
        }
      };
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (frag(std::integral_constant<int, J>{}), ...);
      }(std::make_integer_sequence<int, (PF < NOPS ? PF : NOPS)>{});
      auto op = [&](auto j_tag) {
        constexpr int J = decltype(j_tag)::value;
        constexpr int I = sub_idx(J);
        if constexpr (J + PF < NOPS) frag(std::integral_constant<int, J + PF>{});
        u32x4 fa;
        if constexpr (is_pv(J)) {
          lgkm_wait<after(J)>(fl[J], fh[J]);
          fa = u32x4{fl[J][0], fl[J][1], fh[J][0], fh[J][1]};
        } else {
          lgkm_wait<after(J)>(fr[J]);
          fa = fr[J];
        }
        if constexpr (is_pv(J)) {
          constexpr int M = I / (D / 32), N = I % (D / 32);
          oacc[N] = mfma32(__builtin_bit_cast(bf16x8, fa), pb[M], oacc[N]);
        } else {
          constexpr int KK = I >> 1, HALF = I & 1;
          if constexpr (HALF == 0) s0 = mfma32(__builtin_bit_cast(bf16x8, fa), qf[KK], s0);
          else s1 = mfma32(__builtin_bit_cast(bf16x8, fa), qf[KK], s1);
        }
      };
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (op(std::integral_constant<int, J>{}), ...);
      }(std::make_integer_sequence<int, NOPS>{});
    };

    // ---- softmax of tile u (P = u % 2): S^T registers -> P^T (bf16) in pb
    auto smax = [&](auto p_tag, int u) __attribute__((always_inline)) {
      constexpr int sub = decltype(p_tag)::value;
      const bool diag = u >= first_diag;
      if (diag) {
        // key = kc + 4 hh > xq with kc a constant: compare kc with xq - 4 hh,
        // which passes through an empty asm so that neither the keys nor the
        // compares are hoisted out of the loop into 64 registers or lane masks
        int xt = xq - 4 * hh;
        asm volatile("" : "+v"(xt)::"memory");
  #pragma unroll
        for (int z = 0; z < 16; ++z) {
          const int kc = sub * KT + 8 * (z >> 2) + (z & 3);
          if (kc > xt) s0[z] = kNegInf;
          if (kc + 32 > xt) s1[z] = kNegInf;
        }
      }
      // Probabilities at the running max, packed to bf16 into pb; returns the
      // lane's fp32 sum of them (rounding them to bf16 first would move the
      // LSE of short rows by up to half a bf16 ulp), four chains.
      auto probs = [&](float mc) __attribute__((always_inline)) {
        float ps[4], p0[16], p1[16];
  #pragma unroll
        for (int z = 0; z < 16; ++z) {
          p0[z] = fast_exp2(fmaf(s0[z], c2, mc));
          p1[z] = fast_exp2(fmaf(s1[z], c2, mc));
          if (z < 4) ps[z & 3] = p0[z] + p1[z];
          else ps[z & 3] += p0[z] + p1[z];
        }
  #pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i0 = 2 * (m & 1);
  #pragma unroll
          for (int z = 0; z < 8; ++z) pb[m][z] = (__bf16)((m < 2) ? p0[4 * i0 + z] : p1[4 * i0 + z]);
        }
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
      };
      // Lazy rescale.  The probabilities are first taken at the running max
      // as it stands; that stands when every lane's tile sum is at most
      // kLazySum (so is every probability).  Otherwise -- a score well above
      // the running max, or a row with no max yet (mneg = +inf makes the sum
      // infinite or NaN) -- the tile's max moves the running max and the
      // probabilities are taken again.  The first tile of a unit goes
      // straight to the second path.
      float tsum = 0.f;
      bool moved = u == 0;
      if (!moved) {
        tsum = probs(mneg);
        moved = __ballot(!(tsum <= kLazySum)) != 0ull;
      }
      if (moved) {
        // Row max as a tree of three-input maxima (IEEE maximum lowers to
        // v_maximum3_f32 without operand canonicalisation): 17 instructions
        // for the 32 values of a lane.
        auto mx3 = [](float p, float q, float r) {
          return __builtin_elementwise_maximum(__builtin_elementwise_maximum(p, q), r);
        };
        float t[11];
  #pragma unroll
        for (int k = 0; k < 5; ++k) {
          t[k] = mx3(s0[3 * k], s0[3 * k + 1], s0[3 * k + 2]);
          t[5 + k] = mx3(s1[3 * k], s1[3 * k + 1], s1[3 * k + 2]);
        }
        t[10] = __builtin_elementwise_maximum(s0[15], s1[15]);
        float mx = __builtin_elementwise_maximum(
            mx3(mx3(t[0], t[1], t[2]), mx3(t[3], t[4], t[5]), mx3(t[6], t[7], t[8])),
            __builtin_elementwise_maximum(t[9], t[10]));
        mx = half_max(mx);
        const float m_new = fmaxf(m_run, mx * c2);
        const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
  #pragma unroll
        for (int n = 0; n < D / 32; ++n)
  #pragma unroll
          for (int z = 0; z < 16; ++z) oacc[n][z] *= alpha;
        m_run = m_new;
        const float mc = (m_new == kNegInf) ? 0.f : -m_new;
        mneg = (m_new == kNegInf) ? kPosInf : mc;
        tsum = probs(mc);
      }
      l_run += tsum;
    };

    // Register fences: the compiler would otherwise move the tail of a phase
    // (e.g. the exponentials, whose only consumer is the next MFMA phase)
    // across the barrier into the other phase of the same wave, where it runs
    // serially with that wave's MFMAs instead of beside the other group's.
    auto fence_mma = [&]() __attribute__((always_inline)) {
      reg_fence(s0);
      reg_fence(s1);
  #pragma unroll
      for (int n = 0; n < D / 32; ++n) reg_fence(oacc[n]);
    };
    auto fence_smax = [&]() __attribute__((always_inline)) {
  #pragma unroll
      for (int m = 0; m < 4; ++m) reg_fence(pb[m]);
      reg_fence(l_run);
      reg_fence(m_run);
  #pragma unroll
      for (int n = 0; n < D / 32; ++n) reg_fence(oacc[n]);
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    // Schedule.  Per tile u, group A (waves 0-3) runs the MFMA phase of u
    // (O += V^T(u-1) P(u-1) and S(u)) and then the softmax phase of u (copy
    // group u, P(u) from S(u)); group B runs the softmax phase of u - 1 and
    // then the MFMA phase of u; one workgroup barrier ends the tile.  On each
    // SIMD the A wave's MFMAs thus run beside the B wave's softmax and vice
    // versa; the barrier realigns the two halves once per tile.
    // Copies: before barrier u, every wave has its copy group u - 2 done (A
    // has issued up to group u and waits for all but two groups, B up to
    // u - 1 and waits for all but one), so after it both operands of MFMA
    // phase u + 1 (K(u + 1), V(u), from group u - 2) are in LDS.  Group g
    // overwrites K(g - 1) and V(g - 2), which only MFMA phase g - 1 reads:
    // A issues it after barrier g - 1, B after barrier g, and every wave's
    // MFMA phase g - 1 precedes barrier g - 1.
    // Prologue: copy groups -3..-1 (K of tiles 0..2, V of tiles 0..1); the
    // barrier after it makes group -3 (K(0)) visible.
    if (ntile > 0) {
      refill(0);
      e_last = __builtin_amdgcn_readlane(eb, 1);  // block 1 (or the last)
      copy_prologue(std::integral_constant<int, 0>{});  // V part: tile 0, the same bytes as group -2's
      copy_prologue(std::integral_constant<int, 1>{});
      copy_prologue(std::integral_constant<int, 2>{});
      wait_vmcnt<4 * LPW>();
    }
    __builtin_amdgcn_s_barrier();
    // Tile 0 has no PV part; the loops are unrolled by two so that the tile
    // parity (the copy sources' bookkeeping and the diagonal mask) is a
    // constant.
    auto softmax_phase = [&](auto p_tag, int u) __attribute__((always_inline)) {
      copy_group(p_tag, u);
      smax(p_tag, u);
      fence_smax();
    };
    auto mma_phase = [&](auto pv_tag, int u) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
      mma(pv_tag, T_{}, u);
      fence_mma();
      __builtin_amdgcn_s_setprio(0);
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    if (ntile > 0) {
      if (grp == 0) {
        auto step = [&](auto pv_tag, auto p_tag, int u) __attribute__((always_inline)) {
          mma_phase(pv_tag, u);
          softmax_phase(p_tag, u);
          wait_vmcnt<4 * LPW>();
          __builtin_amdgcn_s_barrier();
        };
        step(F_{}, Even{}, 0);
        int u = 1;
        for (; u + 1 < ntile; u += 2) {
          step(T_{}, Odd{}, u);
          step(T_{}, Even{}, u + 1);
        }
        if (u < ntile) step(T_{}, Odd{}, u);
      } else {
        mma_phase(F_{}, 0);
        wait_vmcnt<2 * LPW>();
        __builtin_amdgcn_s_barrier();
        auto step = [&](auto p_tag, int u) __attribute__((always_inline)) {
          softmax_phase(p_tag, u - 1);  // p_tag: parity of u - 1
          mma_phase(T_{}, u);
          wait_vmcnt<2 * LPW>();
          __builtin_amdgcn_s_barrier();
        };
        int u = 1;
        for (; u + 1 < ntile; u += 2) {
          step(Even{}, u);
          step(Odd{}, u + 1);
        }
        if (u < ntile) step(Even{}, u);
        if (ntile & 1) softmax_phase(Even{}, ntile - 1);
        else softmax_phase(Odd{}, ntile - 1);
      }
      mma(T_{}, F_{}, ntile);  // PV of the last tile
    }
    wait_vmcnt<0>();  // copies of the groups past the end land in LDS before exit

    const float l_tot = half_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* const of32 = (wk.ns > 1 && !whole) ? a.split_o[wk.s] : a.out_f32;
    float* const lsep = (wk.ns > 1 && !whole) ? a.split_l[wk.s] : a.lse;
    // Output rows through LDS.  A lane holds one query (16-byte pieces at
    // d = 32n + 8ii + 4hh), so a store straight from the registers would
    // touch 32 rows, one partial cache line each; instead every wave writes
    // its 32 rows into its own slice of the tile ring (idle once every wave
    // has passed the barrier below: all fragment reads and copies are done),
    // 16-byte pieces XOR-swizzled by the row, and reads them back row-major,
    // so that each store instruction writes whole rows.  The slice is read
    // only by the wave that wrote it (a wave's LDS operations run in order).
    __syncthreads();
    char* const ow = tiles + w * (32 * D * 4);
    // first query row of this wave and the distance between rows, in elements
    const long long obase = ((long long)(q0 + i * kBlock + qs * 32) * a.hq + h) * D;
    int ostride = a.hq * D;
    // The stride and the lane index pass through empty asm statements so that
    // the offsets and LDS addresses below are formed here: hoisted out of the
    // unit loop they would hold registers through the whole kernel.
    int ql = l32, ln = lane;
    asm volatile("" : "+s"(ostride), "+v"(ql), "+v"(ln));
    if (of32) {
      constexpr int CPR = D / 4;            // 16-byte pieces per fp32 row
      constexpr int NR = 32 * CPR / 64;     // reads (and stores) per lane
  #pragma unroll
      for (int n = 0; n < D / 32; ++n)
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int c = 8 * n + 2 * ii + hh;
          const f32x4 v = {oacc[n][4 * ii + 0] * inv, oacc[n][4 * ii + 1] * inv, oacc[n][4 * ii + 2] * inv,
                           oacc[n][4 * ii + 3] * inv};
          *(f32x4*)(ow + ql * (D * 4) + ((c ^ (ql & (CPR - 1))) * 16)) = v;
        }
      asm volatile("" ::: "memory");
      // every piece in its own registers before the first store, so that no
      // store's data registers are rewritten while it is in flight
      constexpr int RPI = 64 / CPR;  // rows per store instruction
      const int r0 = ln / CPR, c = ln % CPR;
      f32x4 rv[NR];
  #pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int r = j * RPI + r0;
        rv[j] = *(const f32x4*)(ow + r * (D * 4) + ((c ^ (r & (CPR - 1))) * 16));
      }
      const __amdgpu_buffer_rsrc_t ro =
          __builtin_amdgcn_make_buffer_rsrc((void*)(of32 + obase), (short)0, 32 * ostride * 4, kBufFlags);
      const int voff = (r0 * ostride + c * 4) * 4;
  #pragma unroll
      for (int j = 0; j < NR; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, rv[j]), ro, voff, j * RPI * ostride * 4, 0);
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      constexpr int GPR = D / 8;            // 16-byte pieces per bf16 row
      constexpr int NR = 32 * GPR / 64;
  #pragma unroll
      for (int n = 0; n < D / 32; ++n)
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int c8 = 8 * n + 2 * ii + hh;  // 8-byte piece of the row
          bf16x4 o4;
  #pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[n][4 * ii + e] * inv);
          *(bf16x4*)(ow + ql * (D * 2) + (((c8 >> 1) ^ (ql & (GPR - 1))) * 16) + (c8 & 1) * 8) = o4;
        }
      asm volatile("" ::: "memory");
      constexpr int RPI = 64 / GPR;
      const int r0 = ln / GPR, gch = ln % GPR;
      u32x4 rv[NR];
  #pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int r = j * RPI + r0;
        rv[j] = *(const u32x4*)(ow + r * (D * 2) + ((gch ^ (r & (GPR - 1))) * 16));
      }
      const __amdgpu_buffer_rsrc_t ro =
          __builtin_amdgcn_make_buffer_rsrc((void*)((char*)a.out + obase * 2), (short)0, 32 * ostride * 2, kBufFlags);
      const int voff = (r0 * ostride + gch * 8) * 2;
  #pragma unroll
      for (int j = 0; j < NR; ++j) __builtin_amdgcn_raw_buffer_store_b128(rv[j], ro, voff, j * RPI * ostride * 2, 0);
    }
    if (lsep && hh == 0) {
      const float lse = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
      lsep[(long long)h * a.total_q + q0 + x] = lse;
    }
  };
  WorkUnit wk = work_unit(a, hkv, npair, blockIdx.x, gridDim.x);
  if (a.split_whole < 0) {
    // Heads from the device: the launch's row blocks are the list counts of
    // its (sequence, kv head, q block) rows (those of q blocks past a
    // sequence's end are never written and not read); the head length is
    // the host rule's, 98% of the per-CU share plus two blocks.  The first
    // unit's list count is loaded in the same round.  Workgroup 0 stores the
    // head length for the split merge whatever its own units are.
    __shared__ int head_red[NW];
    if (wk.i < (a.cu_q[wk.b + 1] - a.cu_q[wk.b]) / kBlock)
      nall_pre = a.lists[(((long long)wk.b * hkv + wk.g) * a.max_qb + wk.i) * (a.max_kb + 1)];
    int part = 0;
    for (int r = threadIdx.x; r < a.cut_rows; r += 64 * NW) {
      const int i = r % a.max_qb, b = r / (hkv * a.max_qb);
      const int cnt = a.lists[(long long)r * (a.max_kb + 1)];
      if (i < (a.cu_q[b + 1] - a.cu_q[b]) / kBlock) part += cnt;
    }
  #pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if ((threadIdx.x & 63) == 0) head_red[threadIdx.x >> 6] = part;
    __syncthreads();
    int tot = 0;
  #pragma unroll
    for (int x = 0; x < NW; ++x) tot += head_red[x];
    const double share = (double)tot * npair / a.cut_cus;
    whole_lim = dev_head = __builtin_amdgcn_readfirstlane((int)ceil(0.98 * share) + kHeadPad);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.cut_head = dev_head;
  }
  for (;;) {
    run_unit(wk);
    if (!dyn) break;
    const int nt = (a.n_order - a.n_static) * slots;
    __syncthreads();  // every wave is done with list[], tiles[] and next_unit
    if (threadIdx.x == 0) {
      const int t = atomicAdd(a.tail_ctr, 1);
      // every workgroup increments once past the last unit, so the launch's
      // last increment returns nt + gridDim.x - 1: reset for the next launch
      if (t == nt + (int)gridDim.x - 1) atomicExch(a.tail_ctr, 0);
      next_unit = t;
    }
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(next_unit);
    if (t >= nt) break;
    wk = entry_unit(a, hkv, a.n_static + t / slots, t % slots);
  }
}

struct BlockIter {
  const uint8_t* mrow;
  const int32_t* table;  // block table row (paged) or nullptr
  int num_pages;         // table entries outside [0, num_pages) are absent
  int jend;
  // First selected block >= j (page present), or jend.
  __device__ __forceinline__ int next(int j) const {
    for (; j < jend; ++j) {
      if (!mrow[j]) continue;
      if (table && (table[j] < 0 || table[j] >= num_pages)) continue;
      return j;
    }
    return jend;
  }
};

// ---------------------------------------------------------------------------
// fp32 inputs: one thread per query, key tiles of 32 staged in LDS.  A tile's
// 32 scores are formed first (independent chains), then one running-max
// update and rescale per tile, then the PV accumulation.  With
// f32_splits = S > 1, blockIdx.z = b * S + s and the workgroup takes the
// s-th contiguous part of the row's candidate key tiles, writing a partial
// (normalised output, LSE) for merge_f32_kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32(AttnArgs a) {
  constexpr int KT = 32;
  constexpr int TPB = kBlock / KT;  // tiles per key block
  __shared__ __align__(16) float ks[KT * D];
  __shared__ __align__(16) float vs[KT * D];
  const int i = a.max_qb - 1 - blockIdx.x;
  const int ns = a.f32_splits;
  const int h = blockIdx.y, b = blockIdx.z / ns, sp = blockIdx.z % ns;
  const int g = h / a.group;
  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  if (i >= qb) return;
  const int o = lk - lq;
  const int tid = threadIdx.x;
  const int x = i * kBlock + tid;
  const int qpos = o + x;
  BlockIter it;
  it.mrow = a.mask + (((long long)b * (a.hq / a.group) + g) * a.max_qb + i) * a.max_kb;
  it.table = a.k.block_table ? a.k.block_table + (long long)b * a.k.max_blocks : nullptr;
  it.num_pages = a.k.num_pages;
  const int jend = min(a.jb1, i + kh + 1);
  it.jend = jend;
  // this part's candidate tiles [ta, tb), numbered from block jb0
  const int nt = TPB * max(0, jend - a.jb0);
  int ta = 0, tb = nt;
  if (ns > 1) {
    ta = (int)(((long long)sp * nt) / ns);
    tb = (int)(((long long)(sp + 1) * nt) / ns);
  }

  if (ns > 1 && ta >= tb) {
    // an empty part: LSE -inf marks it for the merge, which then reads none
    // of its output
    a.f32_l[(long long)sp * a.hq * a.total_q + (long long)h * a.total_q + q0 + x] = kNegInf;
    return;
  }
  float qv[D];
  const float* qrow = (const float*)a.q + ((long long)(q0 + x) * a.hq + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) qv[e] = qrow[e];
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  for (int tt = ta; tt < tb; ++tt) {
    // skip to the first selected block at or after the tile's block
    const int jc = a.jb0 + tt / TPB;
    const int j = it.next(jc);
    if (j >= jend) break;
    if (j != jc) {
      tt = (j - a.jb0) * TPB;
      if (tt >= tb) break;
    }
    const int t0 = (tt % TPB) * KT;
    __syncthreads();
    for (int c = tid; c < KT * D / 4; c += 128) {
      const int key = c / (D / 4), part = c % (D / 4);
      *(f32x4*)(&ks[key * D + part * 4]) =
          *(const f32x4*)((const float*)a.k.row(b, j * kBlock + t0 + key, g) + part * 4);
      *(f32x4*)(&vs[key * D + part * 4]) =
          *(const f32x4*)((const float*)a.v.row(b, j * kBlock + t0 + key, g) + part * 4);
    }
    __syncthreads();
    float sc[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4 kv = *(const f32x4*)(&ks[kk * D + e]);
        d0 = fmaf(qv[e], kv[0], d0);
        d1 = fmaf(qv[e + 1], kv[1], d1);
        d0 = fmaf(qv[e + 2], kv[2], d0);
        d1 = fmaf(qv[e + 3], kv[3], d1);
      }
      sc[kk] = (d0 + d1) * a.scale2;
    }
    if (j == i + kh) {  // diagonal block: keys after the query are masked
#pragma unroll
      for (int kk = 0; kk < KT; ++kk)
        if (j * kBlock + t0 + kk > qpos) sc[kk] = kNegInf;
    }
    float mx = sc[0];
#pragma unroll
    for (int kk = 1; kk < KT; ++kk) mx = fmaxf(mx, sc[kk]);
    const float m_new = fmaxf(m_run, mx);
    // reference for this tile's weights: 0 while every score so far is -inf
    // (weights 0), else the running max; alpha rescales what came before
    const float mc = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - mc);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      const float p = exp2f(sc[kk] - mc);
      l_run += p;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4 vv = *(const f32x4*)(&vs[kk * D + e]);
        acc[e] = fmaf(p, vv[0], acc[e]);
        acc[e + 1] = fmaf(p, vv[1], acc[e + 1]);
        acc[e + 2] = fmaf(p, vv[2], acc[e + 2]);
        acc[e + 3] = fmaf(p, vv[3], acc[e + 3]);
      }
    }
  }
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  const long long orow = ((long long)(q0 + x) * a.hq + h) * D;
  float* out = ns > 1 ? a.f32_o + (long long)sp * a.total_q * a.hq * D : (a.out_f32 ? a.out_f32 : (float*)a.out);
  float* lse = ns > 1 ? a.f32_l + (long long)sp * a.hq * a.total_q : a.lse;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const f32x4 v = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
    *(f32x4*)(out + orow + e) = v;
  }
  if (lse) lse[(long long)h * a.total_q + q0 + x] = (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
}

// Merge of the f32_splits partials of the fp32 attention: one thread per 4
// consecutive d of one (query, head) row, over the query rows of every q
// block the launch covered (rows of sequences' q blocks only; others are
// never written).  lse = M + log(sum_s e^(lse_s - M)),
// out = sum_s e^(lse_s - lse) o_s; a row whose parts all saw no key gets out
// 0 and lse -inf, as unsplit.  Every part's LSE and output are loaded before
// any is used (fixed trip counts, part indices clamped to the launch's
// count), so the loads overlap; a part with LSE -inf (empty parts write no
// output) is excluded by a select, whatever its output memory holds.
template <int D>
__global__ __launch_bounds__(256) void merge_f32_kernel(AttnArgs a) {
  constexpr int DV = D / 4;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)a.total_q * a.hq * DV) return;
  const int dv = (int)(t % DV);
  const long long row = t / DV;
  const int h = (int)(row % a.hq);
  const long long xq = row / a.hq;
  const int ns = a.f32_splits;
  const long long plane_o = (long long)a.total_q * a.hq * D, plane_l = (long long)a.hq * a.total_q;
  const float* lp = a.f32_l + (long long)h * a.total_q + xq;
  const long long off = xq * a.hq * D + (long long)h * D + 4 * dv;
  float ls[kMaxF32Splits];
  f32x4 os[kMaxF32Splits];
#pragma unroll
  for (int s = 0; s < kMaxF32Splits; ++s) {
    const int sc = s < ns ? s : ns - 1;
    ls[s] = lp[sc * plane_l];
    os[s] = *(const f32x4*)(a.f32_o + sc * plane_o + off);
  }
  float mx = kNegInf;
#pragma unroll
  for (int s = 0; s < kMaxF32Splits; ++s) mx = fmaxf(mx, ls[s]);
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxF32Splits; ++s) {
    const bool use = s < ns && ls[s] != kNegInf;
    const float w = use ? expf(ls[s] - mx) : 0.f;
    tot += w;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    acc += use ? os[s] * w : z;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  float* out = a.out_f32 ? a.out_f32 : (float*)a.out;
  *(f32x4*)(out + off) = acc * inv;
  if (a.lse && dv == 0) a.lse[(long long)h * a.total_q + xq] = tot > 0.f ? mx + logf(tot) : kNegInf;
}

// ---------------------------------------------------------------------------
// LSE merge: one thread per 4 consecutive d of one (row, head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const long long nvec = (long long)a.rows * a.heads * (a.head_dim / 4);
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= nvec) return;
  const int dv = (int)(t % (a.head_dim / 4));
  const long long rh = t / (a.head_dim / 4);
  const int h = (int)(rh % a.heads);
  const long long r = rh / a.heads;
  const float la = a.lse_a[(long long)h * a.rows + r];
  const float lb = a.lse_b[(long long)h * a.rows + r];
  const float mx = fmaxf(la, lb);
  float lse, wa, wb;
  if (mx == kNegInf) {
    lse = kNegInf;
    wa = 0.f;
    wb = 0.f;
  } else {
    const float mn = fminf(la, lb);
    lse = mx + log1pf(expf(mn - mx));
    wa = (la == kNegInf) ? 0.f : expf(la - lse);
    wb = (lb == kNegInf) ? 0.f : expf(lb - lse);
  }
  const long long off = rh * a.head_dim + dv * 4;
  f32x4 oa = *(const f32x4*)(a.o_a + off);
  f32x4 ob = *(const f32x4*)(a.o_b + off);
  f32x4 res;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xa = (wa == 0.f) ? 0.f : wa * oa[e];
    const float xb = (wb == 0.f) ? 0.f : wb * ob[e];
    res[e] = xa + xb;
  }
  if (a.o) *(f32x4*)(a.o + off) = res;
  if (a.o_bf16) {
    uint32_t* p = (uint32_t*)((char*)a.o_bf16 + off * 2);
    p[0] = pack_bf16x2(res[0], res[1]);
    p[1] = pack_bf16x2(res[2], res[3]);
  }
  if (a.lse && dv == 0) a.lse[(long long)h * a.rows + r] = lse;
}

// Split rows: one thread per 8 consecutive d of one (query, head) of a
// listed row (grid y: the row; 8 rather than 4 per thread: 4K merge 0.5 us
// shorter, same bits); the ns partial LSEs give the weights exp(lse_s - lse) with
// lse = m + log(sum_s exp(lse_s - m)), m the largest partial LSE.
// d values per thread of the split merge (head_dim is a multiple of it)
#ifndef XATTN_MERGE_V
#define XATTN_MERGE_V 8
#endif
constexpr int kMergeV = XATTN_MERGE_V;

// One row's merge with its part count NS (2 or 3) fixed, so that no part is
// loaded twice.  The combine is the same arithmetic for either count: parts
// past NS would enter as -inf LSEs with zero weight.
template <int NS>
__device__ __forceinline__ void split_merge_row(const SplitMergeArgs& a, int r, int rem) {
  constexpr int V = kMergeV;
  const int dq = a.head_dim / V;
  const int dv = rem % dq, qh = rem / dq;
  const int h = qh % a.heads, xq = qh / a.heads;
  const uint32_t e = (uint32_t)a.rows[r];
  const long long tok = (long long)(e & 0x0fffffffu) * kBlock + xq;
  const long long li = (long long)h * a.total_q + tok;
  const long long off = (tok * a.heads + h) * a.head_dim + dv * V;
  // The row's list count and the parts' LSEs are loaded together, then (for
  // a row not done whole) every part's output at once: two rounds of loads
  // instead of four.
  const int rb = a.row_bi[r], g = h / a.group;
  const int nall =
      a.lists[(((long long)(rb >> 16) * (a.heads / a.group) + g) * a.max_qb + (rb & 0xffff)) * (a.max_kb + 1)];
  int whole = a.whole >= 0 ? a.whole : *a.cut_head;
  float l[NS], w[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) l[s] = a.l[s][li];
  // (empty asm statements that take the loaded values keep the compiler from
  // sinking the loads past the branch, which would make them a round of
  // their own)
#pragma unroll
  for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(l[s]));
  asm volatile("" : "+v"(whole));
  // a row the attention did whole (few selected blocks) already holds its output
  if (split_row_whole(nall, NS, whole)) return;
  f32x4 ov[NS][V / 4];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int u = 0; u < V / 4; ++u) ov[s][u] = *(const f32x4*)(a.o[s] + off + 4 * u);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int u = 0; u < V / 4; ++u) asm volatile("" : "+v"(ov[s][u]));
  float mx = kNegInf;
#pragma unroll
  for (int s = 0; s < NS; ++s) mx = fmaxf(mx, l[s]);
  float lse = kNegInf;
  float res[V];
#pragma unroll
  for (int c = 0; c < V; ++c) res[c] = 0.f;
  if (mx != kNegInf) {
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) sum += (l[s] == kNegInf) ? 0.f : expf(l[s] - mx);
    lse = mx + logf(sum);
#pragma unroll
    for (int s = 0; s < NS; ++s) w[s] = (l[s] == kNegInf) ? 0.f : expf(l[s] - lse);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (w[s] != 0.f) {
#pragma unroll
        for (int u = 0; u < V / 4; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) res[4 * u + c] = fmaf(w[s], ov[s][u][c], res[4 * u + c]);
      }
    }
  }
  uint32_t* p = (uint32_t*)((char*)a.out + off * 2);
#pragma unroll
  for (int c = 0; c < V / 2; ++c) p[c] = pack_bf16x2(res[2 * c], res[2 * c + 1]);
  if (a.lse && dv == 0) a.lse[(long long)h * a.total_q + tok] = lse;
}

__global__ __launch_bounds__(256) void split_merge_kernel(SplitMergeArgs a) {
  const int per_row = kBlock * a.heads * (a.head_dim / kMergeV);
  const int r = blockIdx.y;
  const int rem = blockIdx.x * 256 + threadIdx.x;
  if (rem >= per_row) return;
  const int ns = (int)((uint32_t)a.rows[r] >> 28) + 1;  // uniform per workgroup
  if (ns == 2) split_merge_row<2>(a, r, rem);
  else split_merge_row<3>(a, r, rem);
}

// The ping-pong kernel serves even GQA groups whose K/V spans fit 32-bit
// buffer offsets.
bool uses_attn_pp(const AttnArgs& a, int head_dim) {
  const int hkv = a.hq / a.group;
  const long long span = (long long)a.num_pages * kBlock * hkv * head_dim * 2;
  return a.group % 2 == 0 && span < (1ll << 31);
}

template <int D>
hipError_t attn_dispatch(const AttnArgs& a, int dtype, int batch, hipStream_t s) {
  if (dtype == 0) {
    const int hkv = a.hq / a.group;
    const int hpw = (a.group % 2 == 0) ? 2 : 1;
    const bool dyn = a.n_static > 0 && a.n_static < a.n_order && a.tail_ctr && uses_attn_pp(a, D);
    const int nwg = (dyn ? a.n_static : a.n_order > 0 ? a.n_order : batch * a.max_qb) * hkv * (a.group / hpw);
    const size_t shm = (size_t)(a.max_kb + 1) * sizeof(int32_t);
    if (uses_attn_pp(a, D)) hipLaunchKernelGGL((attn_pp<D, XATTN_PF>), dim3(nwg), dim3(512), shm, s, a, hkv);
    else if (hpw == 2) hipLaunchKernelGGL((attn_mfma<D, 2>), dim3(nwg), dim3(512), shm, s, a, hkv);
    else hipLaunchKernelGGL((attn_mfma<D, 1>), dim3(nwg), dim3(256), shm, s, a, hkv);
  } else {
    dim3 grid(a.max_qb, a.hq, batch * max(1, a.f32_splits));
    hipLaunchKernelGGL((attn_f32<D>), grid, dim3(128), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

bool attention_reads_vt(const AttnArgs& a, int dtype, int head_dim) {
  return dtype == 0 && !uses_attn_pp(a, head_dim);
}

bool attention_uses_pp(const AttnArgs& a, int head_dim) { return uses_attn_pp(a, head_dim); }

hipError_t launch_attention(const AttnArgs& a, int dtype, int head_dim, int batch,
                            hipStream_t s) {
  if (a.max_qb <= 0 || batch <= 0) return hipSuccess;
  if (head_dim == 128) return attn_dispatch<128>(a, dtype, batch, s);
  if (head_dim == 64) return attn_dispatch<64>(a, dtype, batch, s);
  return hipErrorInvalidValue;
}

hipError_t launch_f32_merge(const AttnArgs& a, int head_dim, hipStream_t s) {
  if (a.f32_splits <= 1 || a.total_q <= 0) return hipSuccess;
  const long long n = (long long)a.total_q * a.hq * (head_dim / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (head_dim == 128) hipLaunchKernelGGL((merge_f32_kernel<128>), grid, dim3(256), 0, s, a);
  else if (head_dim == 64) hipLaunchKernelGGL((merge_f32_kernel<64>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_vt_transpose(const VtArgs& a, hipStream_t s) {
  if (a.num_pages <= 0) return hipSuccess;
  dim3 grid(a.num_pages, a.hkv);
  if (a.head_dim == 128) hipLaunchKernelGGL((vt_transpose_kernel<128>), grid, dim3(256), 0, s, a);
  else if (a.head_dim == 64) hipLaunchKernelGGL((vt_transpose_kernel<64>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, int batch, hipStream_t s) {
  if (a.max_qb <= 0 || batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(a.max_qb, a.hkv, batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Selected-block gather: block j of `src` (host memory mapped into the
// device address space, read over the link by the kernel itself) is copied
// to block j of `dst` when sel[j] is set.  A small grid (kGatherWgs
// workgroups) walks the 16 KiB pieces of all blocks, four 16-byte loads per
// thread in flight before their stores: 256 KiB of outstanding reads keep
// the link busy, and the CUs stay with the attention kernels running beside
// it (a workgroup per piece filled the CUs with waves stalled on the link
// and slowed the concurrent attention launches several-fold).
constexpr int kGatherWgs = XATTN_GATHER_WGS;  // 16: 13.8 ms per 128K staged step; 32: 14.4; 64: 15.2; 128: 15.8
__global__ __launch_bounds__(256) void gather_blocks_kernel(const uint8_t* sel, int nblocks, const char* src,
                                                            char* dst, long long block_bytes) {
  const long long parts = (block_bytes + 16383) / 16384;
  for (long long it = blockIdx.x; it < (long long)nblocks * parts; it += gridDim.x) {
    const int j = (int)(it / parts);
    if (!sel[j]) continue;
    const long long piece = it - (long long)j * parts;
    const long long base = (long long)j * block_bytes + piece * 16384;
    const u32x4* s = (const u32x4*)(src + base);
    u32x4* d = (u32x4*)(dst + base);
    const long long n = min(16384ll, block_bytes - piece * 16384) / 16;
    u32x4 v[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const long long i = threadIdx.x + 256 * x;
      if (i < n) v[x] = __builtin_nontemporal_load(s + i);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const long long i = threadIdx.x + 256 * x;
      if (i < n) d[i] = v[x];
    }
  }
}

hipError_t launch_gather_blocks(const uint8_t* sel, int nblocks, const void* src, void* dst, size_t block_bytes,
                                hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  if (block_bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_blocks_kernel, dim3(kGatherWgs), dim3(256), 0, s, sel, nblocks, (const char*)src,
                     (char*)dst, (long long)block_bytes);
  return hipGetLastError();
}

hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t s) {
  const long long per_row = (long long)kBlock * a.heads * (a.head_dim / kMergeV);
  if (a.head_dim % kMergeV) return hipErrorInvalidValue;
  if (a.n <= 0 || per_row <= 0) return hipSuccess;
  if (per_row >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)((per_row + 255) / 256), a.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const long long nvec = (long long)a.rows * a.heads * (a.head_dim / 4);
  if (nvec <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace xattn
