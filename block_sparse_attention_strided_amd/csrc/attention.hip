// Block-sparse flash attention with log-sum-exp ("XAttention BSA Policy"
// design doc, section 2: flash_attn_with_lse over the selected blocks) and
// the LSE merge of two partial results (merge_attention_outputs).
//
// bf16 kernel layout (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//  * workgroup = one (sequence, q head, 128-query block); wave w owns queries
//    32w .. 32w+31 of the block.
//  * key tiles of 64 keys: K staged row-major in LDS, V staged transposed
//    (d-major) so that both MFMA operands read 16 contiguous bytes per lane.
//  * S^T = K Q^T: the accumulator puts one query per lane (column) and 32 of
//    the tile's keys in its registers, so the running max/sum of the online
//    softmax are per lane, with one exchange between the two half-waves.
//  * O^T += V^T P^T reuses the S^T accumulator registers as the B operand
//    directly: the k-slots of P^T are a fixed permutation of the tile's keys,
//    and V^T is written to LDS in the same permuted key order.
#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kKT = 64;  // keys per tile

// Position of key k (0..63) inside a V^T LDS row: bits 2 and 3 swapped, so
// the 8 keys of k-slot group (16m + 8hh .. +8) are {16m+4hh+0..3, 16m+8+4hh+0..3}.
__device__ __forceinline__ int vperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

struct BlockIter {
  const uint8_t* mrow;
  const int32_t* table;  // block table row (paged) or nullptr
  int jend;
  // First selected block >= j (page present), or jend.
  __device__ __forceinline__ int next(int j) const {
    for (; j < jend; ++j) {
      if (!mrow[j]) continue;
      if (table && table[j] < 0) continue;
      return j;
    }
    return jend;
  }
};

template <int D>
__global__ __launch_bounds__(256) void attn_bf16(AttnArgs a) {
  constexpr int KP = D + 8;    // K LDS pitch (bf16)
  constexpr int VP = kKT + 8;  // V^T LDS pitch (bf16)
  constexpr int CPR = D / 8;   // 16-byte chunks per key row
  constexpr int KLOADS = kKT * CPR / 256;       // K chunks per thread
  constexpr int VPAIRS = (kKT / 2) * CPR / 256;  // V key-pair chunks per thread
  __shared__ __align__(16) uint16_t ks[kKT * KP];
  __shared__ __align__(16) uint16_t vts[D * VP];

  const int i = a.max_qb - 1 - blockIdx.x;  // heaviest causal rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / a.group;
  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  if (i >= qb) return;
  const int o = lk - lq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int x = i * kBlock + w * 32 + l32;  // this lane's query (sequence-relative)
  const int qpos = o + x;

  BlockIter it;
  it.mrow = a.mask + (((long long)b * (a.hq / a.group) + g) * a.max_qb + i) * a.max_kb;
  it.table = a.k.block_table ? a.k.block_table + (long long)b * a.k.max_blocks : nullptr;
  it.jend = min(a.jb1, i + kh + 1);

  // Q fragments: B operand of S^T = K Q^T (query col = lane%32, d slots 8*hh..).
  bf16x8 qf[D / 16];
  {
    const char* qrow = a.q + ((long long)(q0 + x) * a.hq + h) * D * 2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qrow + (kk * 16 + hh * 8) * 2);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[n][e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  u32x4 kreg[KLOADS];
  u32x4 vreg[VPAIRS][2];

  auto fetch = [&](int j, int sub) {
    const int key0 = j * kBlock + sub * kKT;
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int c = tid + 256 * n;
      const int key = c / CPR, part = c % CPR;
      kreg[n] = *(const u32x4*)(a.k.row(b, key0 + key, g) + part * 16);
    }
#pragma unroll
    for (int n = 0; n < VPAIRS; ++n) {
      const int p = tid + 256 * n;
      const int kp = p % (kKT / 2), part = p / (kKT / 2);
      vreg[n][0] = *(const u32x4*)(a.v.row(b, key0 + 2 * kp, g) + part * 16);
      vreg[n][1] = *(const u32x4*)(a.v.row(b, key0 + 2 * kp + 1, g) + part * 16);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int c = tid + 256 * n;
      const int key = c / CPR, part = c % CPR;
      *(u32x4*)(&ks[key * KP + part * 8]) = kreg[n];
    }
#pragma unroll
    for (int n = 0; n < VPAIRS; ++n) {
      const int p = tid + 256 * n;
      const int kp = p % (kKT / 2), part = p / (kKT / 2);
      const int pos = vperm(2 * kp);  // even; key 2kp+1 lands at pos+1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = vreg[n][0][e >> 1], w1 = vreg[n][1][e >> 1];
        const uint32_t lo = (e & 1) ? (w0 >> 16) : (w0 & 0xffffu);
        const uint32_t hi = (e & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
        *(uint32_t*)(&vts[(part * 8 + e) * VP + pos]) = lo | hi;
      }
    }
  };

  int j = it.next(a.jb0);
  int sub = 0;
  if (j < it.jend) fetch(j, 0);
  while (j < it.jend) {
    stage();
    __syncthreads();
    const int cj = j, csub = sub;
    if (sub == 0) {
      sub = 1;
    } else {
      sub = 0;
      j = it.next(j + 1);
    }
    if (j < it.jend) fetch(j, sub);

    // ---- S^T = K Q^T over this 64-key tile
    f32x16 s[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[cb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const bf16x8 af = *(const bf16x8*)(&ks[(cb * 32 + l32) * KP + kk * 16 + hh * 8]);
        s[cb] = mfma32(af, qf[kk], s[cb]);
      }
    }
    // ---- online softmax (base 2), causal mask on the diagonal block only
    const int key0 = cj * kBlock + csub * kKT;
    const bool diag = (cj == i + kh);
    float mx = kNegInf;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[cb][e] * a.scale2;
        if (diag) {
          const int key = key0 + cb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key > qpos) v = kNegInf;
        }
        s[cb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(s[cb][e] - m_use);
        s[cb][e] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[n][e] *= alpha;
    // ---- P^T fragments (B operand), k-step m covers keys 16m .. 16m+15
    bf16x8 pb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int cb = m >> 1, i0 = 2 * (m & 1);
      u32x4 u;
      u[0] = pack_bf16x2(s[cb][4 * i0 + 0], s[cb][4 * i0 + 1]);
      u[1] = pack_bf16x2(s[cb][4 * i0 + 2], s[cb][4 * i0 + 3]);
      u[2] = pack_bf16x2(s[cb][4 * i0 + 4], s[cb][4 * i0 + 5]);
      u[3] = pack_bf16x2(s[cb][4 * i0 + 6], s[cb][4 * i0 + 7]);
      pb[m] = __builtin_bit_cast(bf16x8, u);
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        const bf16x8 av = *(const bf16x8*)(&vts[(n * 32 + l32) * VP + m * 16 + hh * 8]);
        oacc[n] = mfma32(av, pb[m], oacc[n]);
      }
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const long long orow = ((long long)(q0 + x) * a.hq + h) * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d = n * 32 + 8 * ii + 4 * hh;
      const float v0 = oacc[n][4 * ii + 0] * inv, v1 = oacc[n][4 * ii + 1] * inv;
      const float v2 = oacc[n][4 * ii + 2] * inv, v3 = oacc[n][4 * ii + 3] * inv;
      if (a.out_f32) {
        f32x4 v = {v0, v1, v2, v3};
        *(f32x4*)(a.out_f32 + orow + d) = v;
      } else {
        uint32_t* p = (uint32_t*)((char*)a.out + (orow + d) * 2);
        p[0] = pack_bf16x2(v0, v1);
        p[1] = pack_bf16x2(v2, v3);
      }
    }
  if (a.lse && hh == 0) {
    const float lse = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
    a.lse[(long long)h * a.total_q + q0 + x] = lse;
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: one thread per query, key tiles of 32 staged in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32(AttnArgs a) {
  constexpr int KT = 32;
  __shared__ __align__(16) float ks[KT * D];
  __shared__ __align__(16) float vs[KT * D];
  const int i = a.max_qb - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
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
  it.jend = min(a.jb1, i + kh + 1);

  float qv[D];
  const float* qrow = (const float*)a.q + ((long long)(q0 + x) * a.hq + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) qv[e] = qrow[e];
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  for (int j = it.next(a.jb0); j < it.jend; j = it.next(j + 1)) {
    const bool diag = (j == i + kh);
    for (int t0 = 0; t0 < kBlock; t0 += KT) {
      __syncthreads();
      for (int c = tid; c < KT * D / 4; c += 128) {
        const int key = c / (D / 4), part = c % (D / 4);
        *(f32x4*)(&ks[key * D + part * 4]) =
            *(const f32x4*)((const float*)a.k.row(b, j * kBlock + t0 + key, g) + part * 4);
        *(f32x4*)(&vs[key * D + part * 4]) =
            *(const f32x4*)((const float*)a.v.row(b, j * kBlock + t0 + key, g) + part * 4);
      }
      __syncthreads();
      for (int kk = 0; kk < KT; ++kk) {
        const int key = j * kBlock + t0 + kk;
        if (diag && key > qpos) continue;
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) sdot = fmaf(qv[e], ks[kk * D + e], sdot);
        const float z = sdot * a.scale2;
        if (z > m_run) {
          const float alpha = exp2f(m_run - z);
          l_run = l_run * alpha + 1.f;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] = acc[e] * alpha + vs[kk * D + e];
          m_run = z;
        } else {
          const float p = exp2f(z - m_run);
          l_run += p;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vs[kk * D + e], acc[e]);
        }
      }
    }
  }
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  const long long orow = ((long long)(q0 + x) * a.hq + h) * D;
  float* out = a.out_f32 ? a.out_f32 : (float*)a.out;
#pragma unroll
  for (int e = 0; e < D; ++e) out[orow + e] = acc[e] * inv;
  if (a.lse) a.lse[(long long)h * a.total_q + q0 + x] = (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
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

template <int D>
hipError_t attn_dispatch(const AttnArgs& a, int dtype, int batch, hipStream_t s) {
  dim3 grid(a.max_qb, a.hq, batch);
  if (dtype == 0) hipLaunchKernelGGL((attn_bf16<D>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((attn_f32<D>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int dtype, int head_dim, int batch,
                            hipStream_t s) {
  if (a.max_qb <= 0 || batch <= 0) return hipSuccess;
  if (head_dim == 128) return attn_dispatch<128>(a, dtype, batch, s);
  if (head_dim == 64) return attn_dispatch<64>(a, dtype, batch, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const long long nvec = (long long)a.rows * a.heads * (a.head_dim / 4);
  if (nvec <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace xattn
