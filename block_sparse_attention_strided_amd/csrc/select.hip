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
  if (a.threshold >= 1.0f) {
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
  if (tid == 0) {
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
      out[j] = before[x] < thr ? 1 : 0;
    } else {
      out[x] = 0;  // not allowed (positions >= n hold only padding keys)
    }
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

// Chunk-vote mode: votes of history column j over the Hkv*Qb (kv head,
// q block) rows.  Workgroup = 64 columns x 4 row lanes; per-KV-head mode
// clears hist_sel.
__global__ __launch_bounds__(256) void vote_kernel(SelectArgs a) {
  __shared__ int part[4][64];
  const int c = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  const int b = blockIdx.y;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  int votes = 0;
  if (a.select_mode == 1 && j < kh) {
    const int nrows = a.hkv * qb;
#pragma unroll 8
    for (int r = rl; r < nrows; r += 4) {
      const int g = r / qb, i = r - (r / qb) * qb;
      votes += a.mask_kv[(((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb + j];
    }
  }
  part[rl][c] = votes;
  __syncthreads();
  if (rl == 0 && j < a.max_kb) {
    uint8_t sel = 0;
    if (a.select_mode == 1 && qb > 0 && j < kh) {
      const int v = part[0][c] + part[1][c] + part[2][c] + part[3][c];
      sel = (2 * v > a.hkv * qb || j == 0 || j == kh - 1) ? 1 : 0;
    }
    a.hist_sel[(long long)b * a.max_kb + j] = sel;
  }
}

// Chunk-vote mode: effective mask row (g, i): voted history, dense causal
// current chunk.  One workgroup per (i, g, b).
__global__ __launch_bounds__(256) void effective_mask_kernel(SelectArgs a) {
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kb = lk / kBlock, kh = (lk - lq) / kBlock;
  uint8_t* row = a.mask_kv + (((long long)b * a.hkv + g) * a.max_qb + i) * a.max_kb;
  const uint8_t* hs = a.hist_sel + (long long)b * a.max_kb;
  for (int j = threadIdx.x; j < a.max_kb; j += 256) {
    uint8_t v = 0;
    if (i < qb && j < kb) v = (j < kh) ? hs[j] : (j <= i + kh ? 1 : 0);
    row[j] = v;
  }
}

// counts[b] = {selected, available}; one workgroup per sequence.
__global__ __launch_bounds__(256) void counts_kernel(SelectArgs a) {
  __shared__ long long red[256];
  const int b = blockIdx.x;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  long long sel = 0;
  if (qb > 0) {
    if (a.select_mode == 1) {
      for (int j = threadIdx.x; j < kh; j += 256) sel += a.hist_sel[(long long)b * a.max_kb + j];
    } else {
      const long long n = (long long)a.hkv * a.max_qb * a.max_kb;
      const uint8_t* m = a.mask_kv + (long long)b * n;
      for (long long x = threadIdx.x; x < n; x += 256) sel += m[x];
    }
  }
  red[threadIdx.x] = sel;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    long long avail = 0;
    if (qb > 0) {
      if (a.select_mode == 1) avail = kh;
      else avail = (long long)a.hkv * ((long long)qb * (kh + 1) + (long long)qb * (qb - 1) / 2);
    }
    a.counts[2 * b] = (int32_t)red[0];
    a.counts[2 * b + 1] = (int32_t)avail;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t s) {
  if (a.max_kb <= 0 || batch <= 0) return hipSuccess;
  int n2 = 1;
  while (n2 < a.max_kb) n2 <<= 1;
  if (a.max_qb > 0) {
    const size_t shm = (size_t)n2 * (sizeof(uint64_t) + sizeof(double));
    hipLaunchKernelGGL(select_rows_kernel, dim3(a.max_qb, a.hq, batch), dim3(256), shm, s, a, n2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(aggregate_kernel, dim3(a.max_qb, a.hkv, batch), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(vote_kernel, dim3((a.max_kb + 63) / 64, batch), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.select_mode == 1 && a.max_qb > 0) {
    hipLaunchKernelGGL(effective_mask_kernel, dim3(a.max_qb, a.hkv, batch), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.counts) {
    hipLaunchKernelGGL(counts_kernel, dim3(batch), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace xattn
