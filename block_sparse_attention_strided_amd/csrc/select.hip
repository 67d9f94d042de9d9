// Block selection ("XAttention BSA Policy" design doc, core algorithm Steps 3
// and 4): cumulative-threshold selection per (sequence, q head, q block) row,
// GQA aggregation over the q heads of a KV group, forced blocks, the majority
// vote over history blocks, and the density counts of the Density API section.
//
// Threshold rule, per row over the allowed blocks j <= i + Kh: order the
// blocks by (value desc, index asc); keep the k-th iff the float64 sum of the
// k items before it, accumulated in that order, is below tau * T, with T the
// float64 sum of all of them in the same order.  The sort is a bitonic sort of
// 64-bit keys in LDS; the float64 scan runs in one lane, so the rounding of
// every partial sum is fixed by the order alone.
#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kSelMaxWaves = 16;           // q heads per KV group in the fused kernel
constexpr size_t kSelMaxLds = 64 * 1024;  // dynamic LDS limit of the fused kernel

// Order-preserving map of a float to uint32 (-0 canonicalised to +0).
__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_orderable(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// One workgroup per (q block i, q head h, sequence b).  Dynamic LDS holds
// n2 = next power of two >= max_kb sort keys and n2 float64 prefix sums.
__global__ __launch_bounds__(256) void select_rows_kernel(SelectArgs a, int n2) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* keys = (uint64_t*)smem;
  double* before = (double*)(smem + (size_t)n2 * sizeof(uint64_t));
  __shared__ double thr_s;

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  uint8_t* out = a.mask_q + (((long long)b * a.hq + h) * a.max_qb + i) * a.max_kb;
  const int tid = threadIdx.x;
  if (i >= qb) {
    for (int j = tid; j < a.max_kb; j += 256) out[j] = 0;
    return;
  }
  const int n = i + kh + 1;
  const float* row = a.block_sums + (((long long)b * a.hq + h) * a.max_qb + i) * a.max_kb;
  if (a.num_to_choose > 0 ? a.num_to_choose >= n : a.threshold >= 1.0f) {
    for (int j = tid; j < a.max_kb; j += 256) out[j] = (j < n) ? 1 : 0;
    return;
  }
  for (int x = tid; x < n2; x += 256) {
    uint64_t key = 0;
    if (x < n) key = ((uint64_t)orderable(row[x]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)x);
    keys[x] = key;
  }
  __syncthreads();
  // Bitonic sort, descending.
  for (int k = 2; k <= n2; k <<= 1) {
    for (int js = k >> 1; js > 0; js >>= 1) {
      for (int idx = tid; idx < (n2 >> 1); idx += 256) {
        const int lo = 2 * idx - (idx & (js - 1));
        const int hi = lo + js;
        const bool desc = (lo & k) == 0;
        const uint64_t x = keys[lo], y = keys[hi];
        if ((x < y) == desc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) thr_s = 0.0;
  if (tid == 0 && a.num_to_choose == 0) {
    double acc = 0.0;
    int x = 0;
    for (; x + 4 <= n; x += 4) {
      const uint64_t k0 = keys[x], k1 = keys[x + 1], k2 = keys[x + 2], k3 = keys[x + 3];
      before[x] = acc;
      acc += (double)from_orderable((uint32_t)(k0 >> 32));
      before[x + 1] = acc;
      acc += (double)from_orderable((uint32_t)(k1 >> 32));
      before[x + 2] = acc;
      acc += (double)from_orderable((uint32_t)(k2 >> 32));
      before[x + 3] = acc;
      acc += (double)from_orderable((uint32_t)(k3 >> 32));
    }
    for (; x < n; ++x) {
      before[x] = acc;
      acc += (double)from_orderable((uint32_t)(keys[x] >> 32));
    }
    thr_s = (double)a.threshold * acc;
  }
  __syncthreads();
  const double thr = thr_s;
  for (int x = tid; x < a.max_kb; x += 256) {
    if (x < n) {
      const int j = (int)(0xffffffffu - (uint32_t)(keys[x] & 0xffffffffu));
      out[j] = (a.num_to_choose > 0 ? x < a.num_to_choose : before[x] < thr) ? 1 : 0;
    } else {
      out[x] = 0;  // not allowed (positions >= n hold only padding keys)
    }
  }
}

// Orders LDS accesses of one wave: its LDS instructions execute in issue
// order, so only the compiler has to be kept from moving them across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Attention block list of row (b, g, i) in the plan kernel's layout: the
// count, then (page << 1) | (j is the diagonal block i + kh) for every j <
// jend whose mask byte flag(j) is set and whose page is present, in
// increasing j (pages from the block table, else contiguous from the
// sequence's first key).  All threads of the workgroup call it; wcnt holds
// one int per wave.  Clears the attention's tail-part counter once per
// launch (workgroup (0, 0, 0)).
template <typename F>
__device__ void emit_row_list(const SelectArgs& a, int b, int g, int i, int kh, int jend, F flag, int* wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nthr = blockDim.x, nw = nthr >> 6;
  int32_t* out = a.lists + (((long long)b * a.hkv + g) * a.max_qb + i) * (a.max_kb + 1);
  if (a.tail_ctr && i == 0 && g == 0 && b == 0 && tid == 0) atomicExch(a.tail_ctr, 0);
  const int page0 = a.cu_k[b] / kBlock;
  int n = 0;
  for (int j0 = 0; j0 < jend; j0 += nthr) {
    const int j = j0 + tid;
    int page = -1;
    if (j < jend && flag(j)) page = a.block_table ? a.block_table[(long long)b * a.max_blocks + j] : page0 + j;
    const bool take = page >= 0 && page < a.num_pages;
    const unsigned long long bal = __ballot(take);
    if (lane == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    int before = n, total = n;
    for (int x = 0; x < nw; ++x) {
      const int c = wcnt[x];
      before += (x < w) ? c : 0;
      total += c;
    }
    if (take) out[1 + before + __popcll(bal & ((1ull << lane) - 1ull))] = (page << 1) | (j == i + kh ? 1 : 0);
    n = total;
    __syncthreads();  // wcnt reused
  }
  if (tid == 0) out[0] = n;
}

// Threshold selection and GQA aggregation fused.  One workgroup per (q block
// i, kv head g, sequence b) with one wave per q head of the group; wave w
// works on row (b, h = g*G + w, i) in its own LDS region (the aggregated row
// goes to mask_kv, or in chunk-vote mode to the mask_q scratch):
//   keys   (orderable(v_j) << 32) | ~j for the allowed j (descending order =
//          value desc, index asc); zero keys pad to n2 and sort last
//   sort   bitonic, wave-synchronous (no workgroup barriers)
//   scan   the values as float64 in sorted order (converted by all lanes in
//          place of their keys, indices kept aside); one lane accumulates
//          them in that order, so before[x] and the total T round exactly
//          as a left-to-right float64 cumulative sum
//   keep   before[x] < tau * T
// After one workgroup barrier every thread combines the waves' flags for its
// columns (ANY or MAJORITY), ORs in the forced blocks in per-KV-head mode,
// and writes the mask_kv row.  In per-KV-head mode workgroup (0, 0, b) also
// clears hist_sel[b].  Dynamic LDS per wave: n2 8-byte keys (then values)
// and n2 16-bit indices; then G * max_kb flag bytes.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m, 64);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// The 32-bit value of lane ^ JS without an LDS round trip where the
// hardware has a direct lane exchange: DPP quad permutes for 1 and 2,
// ds_swizzle's xor mode (within 32 lanes, no address register) for 4, 8 and
// 16, v_permlane32_swap for 32.  permlane32_swap of v with itself returns the
// lane's own value and its partner's in an order that depends on the half;
// the one that differs from the own value is the partner's (when both are
// equal either is).
template <int JS>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  if constexpr (JS == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (JS == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (JS == 4 || JS == 8 || JS == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (JS << 10));  // and 0x1f, or 0, xor JS
  } else if constexpr (JS == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (uint32_t)p[0] == v ? (uint32_t)p[1] : (uint32_t)p[0];
  } else {
    return (uint32_t)__shfl_xor((int)v, JS, 64);
  }
}
template <int JS>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v) {
  const uint32_t lo = xor_lane_u32<JS>((uint32_t)v);
  const uint32_t hi = xor_lane_u32<JS>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v, int js) {
  switch (js) {
    case 1: return xor_lane_u64<1>(v);
    case 2: return xor_lane_u64<2>(v);
    case 4: return xor_lane_u64<4>(v);
    case 8: return xor_lane_u64<8>(v);
    case 16: return xor_lane_u64<16>(v);
    case 32: return xor_lane_u64<32>(v);
    default: return shfl_xor_u64(v, js);
  }
}

// The same bitonic network on KPL keys per lane held in registers (key x =
// p * 64 + lane in k[p]): compare-exchange partners 64 or more apart sit in
// the same lane, closer ones in lane ^ js of the same register, swapped with
// lane shuffles.  64 * KPL >= n2 keys are sorted (the extra ones are zero
// padding and end up last); keys[0 .. n2) receive the result.
template <int KPL>
__device__ __forceinline__ void sort_keys_in_registers(uint64_t* keys, const float* row, int n, int n2, int lane) {
  constexpr int N = 64 * KPL;
  uint64_t k[KPL];
#pragma unroll
  for (int p = 0; p < KPL; ++p) {
    const int x = lane + 64 * p;
    k[p] = (x < n) ? (((uint64_t)orderable(row[x]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)x)) : 0ull;
  }
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int js = size >> 1; js > 0; js >>= 1) {
      if (js >= 64) {
        const int pj = js >> 6;
#pragma unroll
        for (int p = 0; p < KPL; ++p) {
          if ((p & pj) == 0) {
            const int q = p | pj;
            const bool desc = (((p << 6) | lane) & size) == 0;
            const uint64_t lo = k[p], hi = k[q];
            const bool sw = (lo < hi) == desc;
            k[p] = sw ? hi : lo;
            k[q] = sw ? lo : hi;
          }
        }
      } else {
#pragma unroll
        for (int p = 0; p < KPL; ++p) {
          const uint64_t o = xor_lane_u64(k[p], js);
          const bool desc = (((p << 6) | lane) & size) == 0, lower = (lane & js) == 0;
          // the lower position of a pair keeps the larger key in a
          // descending run, the smaller in an ascending one
          const bool keep_larger = lower == desc;
          k[p] = ((k[p] < o) == keep_larger) ? o : k[p];
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < KPL; ++p) {
    const int x = lane + 64 * p;
    if (x < n2) keys[x] = k[p];
  }
  wave_lds_sync();
}

// Wave-synchronous bitonic sort of one row's keys in LDS: key x < n is
// (orderable(row[x]) << 32) | ~x, keys n..n2-1 are 0; descending order =
// value desc, index asc, padding last.  Rows of up to 512 keys are sorted in
// registers (sort_keys_in_registers), longer ones in LDS.
template <int PPL>
__device__ __forceinline__ void sort_row_keys(uint64_t* keys, const float* row, int n, int n2, int lane) {
  if constexpr (PPL <= 4) {
    sort_keys_in_registers<2 * PPL>(keys, row, n, n2, lane);
    return;
  }
  // all of a lane's row loads in flight at once
#pragma unroll
  for (int p = 0; p < 2 * PPL; ++p) {
    const int x = lane + 64 * p;
    if (x < n2) {
      uint64_t key = 0;
      if (x < n) key = ((uint64_t)orderable(row[x]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)x);
      keys[x] = key;
    }
  }
  wave_lds_sync();
  // a step's pairs are disjoint: every read of the step is issued before
  // its first write
  for (int k = 2; k <= n2; k <<= 1) {
    for (int js = k >> 1; js > 0; js >>= 1) {
      uint64_t xs[PPL], ys[PPL];
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        const int idx = lane + 64 * p;
        const int lo = 2 * idx - (idx & (js - 1));
        if (idx < (n2 >> 1)) {
          xs[p] = keys[lo];
          ys[p] = keys[lo + js];
        }
      }
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        const int idx = lane + 64 * p;
        const int lo = 2 * idx - (idx & (js - 1));
        const bool desc = (lo & k) == 0;
        if (idx < (n2 >> 1) && (xs[p] < ys[p]) == desc) {
          keys[lo] = ys[p];
          keys[lo + js] = xs[p];
        }
      }
      wave_lds_sync();
    }
  }
}

template <int PPL>  // compare-exchange pairs per lane and sort step: max(1, n2 / 128)
__global__ __launch_bounds__(64 * kSelMaxWaves) void select_group_kernel(SelectArgs a, int n2) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = a.hq / a.hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  const int nthr = 64 * G;
  if (a.select_mode == 0 && i == 0 && g == 0)
    for (int j = tid; j < a.max_kb; j += nthr) a.hist_sel[(long long)b * a.max_kb + j] = 0;
  // chunk-vote modes: the per-KV-head rows go to the mask_q scratch (same
  // layout), which chunk_vote_mask_kernel turns into the effective mask_kv
  uint8_t* const dst = a.select_mode != 0 ? a.mask_q : a.mask_kv;
  uint8_t* out = dst + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  __shared__ int wcnt[kSelMaxWaves];
  const bool emit = a.lists && a.select_mode == 0;
  if (i >= qb) {
    for (int j = tid; j < a.max_kb; j += nthr) out[j] = 0;
    if (emit) emit_row_list(a, b, g, i, kh, 0, [](int) { return false; }, wcnt);
    return;
  }
  const int n = i + kh + 1;
  uint64_t* keys = (uint64_t*)(smem + (size_t)w * n2 * 8);
  double* vals = (double*)keys;  // values replace the keys after the sort
  uint16_t* idx = (uint16_t*)(smem + (size_t)G * n2 * 8) + (size_t)w * n2;
  uint8_t* fl = smem + (size_t)G * n2 * 10 + (size_t)w * a.max_kb;
  const int h = g * G + w;
  const float* row = a.block_sums + (((long long)b * a.hq + h) * a.max_qb + i) * a.max_kb;
  if (a.num_to_choose > 0 ? a.num_to_choose >= n : a.threshold >= 1.0f) {
    for (int j = lane; j < a.max_kb; j += 64) fl[j] = (j < n) ? 1 : 0;
  } else if (a.num_to_choose > 0) {
    // top-k rule: the first num_to_choose keys of the sorted order
    sort_row_keys<PPL>(keys, row, n, n2, lane);
    for (int j = n + lane; j < a.max_kb; j += 64) fl[j] = 0;
    for (int x = lane; x < n; x += 64) {
      const uint64_t key = keys[x];
      fl[0xffffffffu - (uint32_t)(key & 0xffffffffu)] = (x < a.num_to_choose) ? 1 : 0;
    }
  } else {
    sort_row_keys<PPL>(keys, row, n, n2, lane);
    // exponent range of the row's nonzero values: 2^me <= v < 2^(me+1), and v
    // a multiple of 2^qe (its fp32 ulp; denormals 2^-149)
    int me_max = -1000, qe_min = 1000;
    for (int x = lane; x < n; x += 64) {
      const uint64_t key = keys[x];
      idx[x] = (uint16_t)(0xffffffffu - (uint32_t)(key & 0xffffffffu));
      const float v = from_orderable((uint32_t)(key >> 32));
      vals[x] = (double)v;
      const uint32_t vb = __float_as_uint(v);
      if ((vb & 0x7fffffffu) != 0u) {
        const int ef = (int)((vb >> 23) & 0xffu);
        me_max = max(me_max, ef - 127);
        qe_min = min(qe_min, max(ef, 1) - 150);
      }
    }
    for (int j = n + lane; j < a.max_kb; j += 64) fl[j] = 0;
    for (int o = 32; o > 0; o >>= 1) {
      me_max = max(me_max, __shfl_xor(me_max, o, 64));
      qe_min = min(qe_min, __shfl_xor(qe_min, o, 64));
    }
    // Every partial sum of these values is a multiple of 2^qe_min below
    // n * 2^(me_max+1); when that bound is at most 2^(qe_min+53) every
    // float64 addition is exact, so any order of the additions -- here a
    // wave-parallel scan -- gives the bits of the left-to-right sum.
    const int lg_n = n > 1 ? 32 - __clz(n - 1) : 0;
    const bool exact = me_max + 1 + lg_n <= qe_min + 53;
    wave_lds_sync();
    double total = 0.0;
    if (exact) {
      const int c = (n + 63) / 64;  // values per lane, contiguous in sorted order
      const int x0 = lane * c;
      double loc = 0.0;
      for (int k = 0; k < c; ++k)
        if (x0 + k < n) loc += vals[x0 + k];
      double inc = loc;
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      double run = __shfl_up(inc, 1, 64);
      if (lane == 0) run = 0.0;
      for (int k = 0; k < c; ++k) {
        if (x0 + k < n) {
          const double v0 = vals[x0 + k];
          vals[x0 + k] = run;
          run += v0;
        }
      }
      total = __shfl(inc, 63, 64);
    } else if (lane == 0) {
      // blocks of 16 values, the next block's loads issued before the
      // current block's additions (the additions are the serial chain);
      // each value's slot takes the sum before it as soon as it is read
      constexpr int SB = 16;
      double acc = 0.0;
      const int nfull = n & ~(SB - 1);
      double cur[SB] = {}, nxt[SB] = {};
      if (nfull > 0)
#pragma unroll
        for (int k = 0; k < SB; ++k) cur[k] = vals[k];
      for (int x0 = 0; x0 < nfull; x0 += SB) {
        if (x0 + SB < nfull)
#pragma unroll
          for (int k = 0; k < SB; ++k) nxt[k] = vals[x0 + SB + k];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          vals[x0 + k] = acc;
          acc += cur[k];
        }
#pragma unroll
        for (int k = 0; k < SB; ++k) cur[k] = nxt[k];
      }
      for (int x = nfull; x < n; ++x) {
        const double v0 = vals[x];
        vals[x] = acc;
        acc += v0;
      }
      total = acc;
    }
    // lane 0's total to every lane (every lane holds it already when exact)
    const uint64_t tb = (uint64_t)__double_as_longlong(total);
    const uint32_t t_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tb);
    const uint32_t t_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tb >> 32));
    const double thr = (double)a.threshold * __longlong_as_double((long long)(((uint64_t)t_hi << 32) | t_lo));
    wave_lds_sync();
    for (int x = lane; x < n; x += 64) fl[idx[x]] = vals[x] < thr ? 1 : 0;
  }
  __syncthreads();
  const uint8_t* flags = smem + (size_t)G * n2 * 10;
  uint8_t* rowf = smem + (size_t)G * n2 * 10 + (size_t)G * a.max_kb;  // the row, for the block list
  for (int j = tid; j < a.max_kb; j += nthr) {
    uint8_t val = 0;
    if (j < n) {
      int cnt = 0;
      for (int x = 0; x < G; ++x) cnt += flags[x * a.max_kb + j];
      bool keep = (a.group_agg == 1) ? (2 * cnt > G) : (cnt > 0);
      if (a.select_mode == 0) keep = keep || j == 0 || j == i + kh;
      val = keep ? 1 : 0;
    }
    out[j] = val;
    if (emit) rowf[j] = val;
  }
  if (emit) {
    __syncthreads();
    emit_row_list(a, b, g, i, kh, n, [&](int j) { return rowf[j] != 0; }, wcnt);
  }
}

// GQA aggregation (+ per-KV-head forced sink and diagonal), per (i, g, b).
__global__ __launch_bounds__(256) void aggregate_kernel(SelectArgs a) {
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int group = a.hq / a.hkv;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  uint8_t* out = a.mask_kv + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  for (int j = threadIdx.x; j < a.max_kb; j += 256) {
    uint8_t val = 0;
    if (i < qb && j <= i + kh) {
      int cnt = 0;
      for (int x = 0; x < group; ++x)
        cnt += a.mask_q[(((long long)b * a.hq + g * group + x) * a.max_qb + i) * a.max_kb + j];
      bool keep = (a.group_agg == 1) ? (2 * cnt > group) : (cnt > 0);
      if (a.select_mode == 0) keep = keep || j == 0 || j == i + kh;
      val = keep ? 1 : 0;
    }
    out[j] = val;
  }
}

// Votes of history column j over the Hkv*Qb (kv head, q block) rows and the
// chunk-vote hist_sel (per-KV-head mode: hist_sel cleared).  Workgroup = 64
// columns x 16 row lanes; the 16 partial counts of a column meet in LDS.
__global__ __launch_bounds__(1024) void vote_kernel(SelectArgs a) {
  __shared__ int part[16][64];
  const int c = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  const int b = blockIdx.y;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  int votes = 0;
  if (a.select_mode != 0 && j < kh) {
    const int nrows = a.hkv * qb;
#pragma unroll 8
    for (int r = rl; r < nrows; r += 16) {
      const int g = r / qb, i = r - (r / qb) * qb;
      votes += a.mask_kv[(((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb + j];
    }
  }
  part[rl][c] = votes;
  __syncthreads();
  if (rl == 0 && j < a.max_kb) {
    uint8_t sel = 0;
    if (a.select_mode != 0 && qb > 0 && j < kh) {
      int v = 0;
#pragma unroll
      for (int x = 0; x < 16; ++x) v += part[x][c];
      sel = (2 * v > a.hkv * qb || j == 0 || j == kh - 1) ? 1 : 0;
    }
    a.hist_sel[(long long)b * a.max_kb + j] = sel;
  }
}

// Chunk-vote modes: effective mask row (g, i): voted history; current chunk
// dense causal (mode 1) or the row's own per-KV-head selection with the sink
// and the diagonal forced (mode 2, read in place from the aggregated row).
// One workgroup per (i, g, b).
__global__ __launch_bounds__(256) void effective_mask_kernel(SelectArgs a) {
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kb = lk / kBlock, kh = (lk - lq) / kBlock;
  uint8_t* row = a.mask_kv + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  const uint8_t* hs = a.hist_sel + (long long)b * a.max_kb;
  for (int j = threadIdx.x; j < a.max_kb; j += 256) {
    uint8_t v = 0;
    if (i < qb && j < kb) {
      if (j < kh) v = hs[j];
      else if (j <= i + kh) v = (a.select_mode == 1 || row[j] || j == i + kh || j == 0) ? 1 : 0;
    }
    row[j] = v;
  }
}

// counts[b] = {selected, available}; one workgroup of 1024 threads per
// sequence.  Mask bytes are 0 or 1, so a 16-byte word's selected count is
// the population count of its bits.
__global__ __launch_bounds__(1024) void counts_kernel(SelectArgs a) {
  __shared__ long long red[16];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  long long sel = 0;
  if (qb > 0) {
    if (a.select_mode == 1) {
      for (int j = tid; j < kh; j += 1024) sel += a.hist_sel[(long long)b * a.max_kb + j];
    } else {
      const long long n = (long long)a.hkv * a.max_qb * a.max_kb;
      const uint8_t* m = a.mask_kv + (long long)b * n;
      const int head = (int)min(n, (long long)((16 - ((uintptr_t)m & 15)) & 15));
      if (tid < head) sel += m[tid];
      const long long nw = (n - head) / 16;
      const u32x4* wp = (const u32x4*)(m + head);
#pragma unroll 4
      for (long long x = tid; x < nw; x += 1024) {
        const u32x4 v = wp[x];
        sel += __popc(v[0]) + __popc(v[1]) + __popc(v[2]) + __popc(v[3]);
      }
      for (long long x = head + nw * 16 + tid; x < n; x += 1024) sel += m[x];
    }
  }
  for (int off = 32; off > 0; off >>= 1) sel += __shfl_xor(sel, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = sel;
  __syncthreads();
  if (tid == 0) {
    long long tot = 0;
    for (int x = 0; x < 16; ++x) tot += red[x];
    long long avail = 0;
    if (qb > 0) {
      if (a.select_mode == 1) avail = kh;
      else avail = (long long)a.hkv * ((long long)qb * (kh + 1) + (long long)qb * (qb - 1) / 2);
    }
    a.counts[2 * b] = (int32_t)tot;
    a.counts[2 * b + 1] = (int32_t)avail;
  }
}

// Chunk-vote modes after select_group_kernel, which left the per-KV-head
// rows in the mask_q scratch: one workgroup per (q block i, kv head g,
// sequence b) counts the votes of every history column over the sequence's
// Hkv*Qb rows itself (16 row lanes x 16 chunks of 16 columns per pass,
// partial counts met in LDS; the rows are 57 KiB at 32K, read from L2 by
// every workgroup), then writes its effective mask_kv row (voted history;
// current chunk dense causal in mode 1, the row's own per-KV-head selection
// with sink and diagonal forced in mode 2; zeros past the sequence).
// Workgroup (0, 0, b) also writes hist_sel, and in mode 1 counts =
// {selected history blocks, history blocks}.  One launch instead of vote +
// effective mask (+ counts).
__global__ __launch_bounds__(256) void chunk_vote_mask_kernel(SelectArgs a) {
  extern __shared__ uint8_t hs[];  // max_kb voted history flags
  __shared__ int part[16][256];
  __shared__ int nsel[4];
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kb = lk / kBlock, kh = (lk - lq) / kBlock;
  const bool lead = (i == 0 && g == 0);
  uint8_t* out = a.mask_kv + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  __shared__ int wcnt[4];
  if (i >= qb && !lead) {
    for (int j = tid; j < a.max_kb; j += 256) out[j] = 0;
    if (a.lists) emit_row_list(a, b, g, i, kh, 0, [](int) { return false; }, wcnt);
    return;
  }
  const int nrows = a.hkv * qb;
  const uint8_t* sel = a.mask_q + (long long)b * a.hkv * a.max_qb * a.max_kb;
  const bool vec = (a.max_kb & 15) == 0 && ((uintptr_t)a.mask_q & 15) == 0;
  const int rl = tid >> 4, cc = tid & 15;
  int mine = 0;  // this thread's selected history columns (lead workgroup)
  for (int j0 = 0; j0 < a.max_kb; j0 += 256) {
    int cnt[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) cnt[e] = 0;
    const int jc = j0 + 16 * cc;
    if (jc < kh) {
#pragma unroll 4
      for (int r = rl; r < nrows; r += 16) {
        const int gg = r / qb, ii = r - gg * qb;
        const uint8_t* row = sel + ((long long)gg * a.max_qb + ii) * a.max_kb + jc;
        if (vec) {
          const u32x4 w = *(const u32x4*)row;
#pragma unroll
          for (int e = 0; e < 16; ++e) cnt[e] += (w[e >> 2] >> (8 * (e & 3))) & 0xffu;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (jc + e < a.max_kb) cnt[e] += row[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) part[rl][16 * cc + e] = cnt[e];
    __syncthreads();
    const int j = j0 + tid;
    if (j < a.max_kb) {
      uint8_t v = 0;
      if (qb > 0 && j < kh) {
        int votes = 0;
#pragma unroll
        for (int x = 0; x < 16; ++x) votes += part[x][tid];
        v = (2 * votes > nrows || j == 0 || j == kh - 1) ? 1 : 0;
      }
      hs[j] = v;
      if (lead) {
        a.hist_sel[(long long)b * a.max_kb + j] = v;
        mine += v;
      }
    }
    __syncthreads();  // part[] reused; hs[] complete after the last pass
  }
  // mode 2: this row's per-KV-head selection (un-forced) for the current chunk
  const uint8_t* own = a.mask_q + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  const bool dense_cur = a.select_mode == 1;
  auto keep = [&](int j) -> bool {
    if (j < kh) return hs[j] != 0;
    return j <= i + kh && (dense_cur || own[j] != 0 || j == i + kh || j == 0);
  };
  for (int j = tid; j < a.max_kb; j += 256) out[j] = (i < qb && j < kb && keep(j)) ? 1 : 0;
  if (a.lists) emit_row_list(a, b, g, i, kh, i < qb ? i + kh + 1 : 0, keep, wcnt);
  if (lead && a.counts && dense_cur) {
    for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off, 64);
    if ((tid & 63) == 0) nsel[tid >> 6] = mine;
    __syncthreads();
    if (tid == 0) {
      a.counts[2 * b] = nsel[0] + nsel[1] + nsel[2] + nsel[3];
      a.counts[2 * b + 1] = qb > 0 ? kh : 0;
    }
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t s, bool* lists_done) {
  if (lists_done) *lists_done = false;
  if (a.max_kb <= 0 || batch <= 0) return hipSuccess;
  int n2 = 1;
  while (n2 < a.max_kb) n2 <<= 1;
  const int group = a.hq / a.hkv;
  const size_t fused_lds = (size_t)group * n2 * 10 + (size_t)(group + (a.lists ? 1 : 0)) * a.max_kb;
  const bool fused = group <= kSelMaxWaves && fused_lds <= kSelMaxLds;
  // the fused kernels write the attention block lists when asked to
  if (lists_done) *lists_done = a.lists && fused && a.max_qb > 0;
  hipError_t e = hipSuccess;
  if (a.max_qb > 0) {
    if (fused) {
      const dim3 grid(a.max_qb, a.hkv, batch), block(64 * group);
      switch (n2 <= 128 ? 1 : n2 / 128) {
        case 1: hipLaunchKernelGGL(select_group_kernel<1>, grid, block, fused_lds, s, a, n2); break;
        case 2: hipLaunchKernelGGL(select_group_kernel<2>, grid, block, fused_lds, s, a, n2); break;
        case 4: hipLaunchKernelGGL(select_group_kernel<4>, grid, block, fused_lds, s, a, n2); break;
        case 8: hipLaunchKernelGGL(select_group_kernel<8>, grid, block, fused_lds, s, a, n2); break;
        case 16: hipLaunchKernelGGL(select_group_kernel<16>, grid, block, fused_lds, s, a, n2); break;
        default: hipLaunchKernelGGL(select_group_kernel<32>, grid, block, fused_lds, s, a, n2); break;
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (a.select_mode != 0) {
        hipLaunchKernelGGL(chunk_vote_mask_kernel, dim3(a.max_qb, a.hkv, batch), dim3(256), (size_t)a.max_kb, s, a);
        if ((e = hipGetLastError()) != hipSuccess || a.select_mode == 1 || !a.counts) return e;
        // mode 2: counts over the effective mask (per-KV-head statistics)
        hipLaunchKernelGGL(counts_kernel, dim3(batch), dim3(1024), 0, s, a);
        return hipGetLastError();
      }
    } else {
      const size_t shm = (size_t)n2 * (sizeof(uint64_t) + sizeof(double));
      hipLaunchKernelGGL(select_rows_kernel, dim3(a.max_qb, a.hq, batch), dim3(256), shm, s, a, n2);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(aggregate_kernel, dim3(a.max_qb, a.hkv, batch), dim3(256), 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  // the fused kernel clears hist_sel itself in per-KV-head mode
  if (a.select_mode != 0 || !fused || a.max_qb == 0) {
    hipLaunchKernelGGL(vote_kernel, dim3((a.max_kb + 63) / 64, batch), dim3(1024), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.select_mode != 0 && a.max_qb > 0) {
    hipLaunchKernelGGL(effective_mask_kernel, dim3(a.max_qb, a.hkv, batch), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.counts) {
    hipLaunchKernelGGL(counts_kernel, dim3(batch), dim3(1024), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace xattn
