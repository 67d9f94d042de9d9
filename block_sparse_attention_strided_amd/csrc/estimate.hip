// Strided anti-diagonal estimate ("XAttention BSA Policy" design doc, core
// algorithm Steps 1-2) and the chunked softmax statistics of the stream-fix
// page (技术细节, 三阶段 KV Chunking).
//
// For q head h the reshaped query row r is the s tokens r*s+s-1 .. r*s (in
// that order) concatenated, and the reshaped key column c is the tokens
// c*s .. c*s+s-1; S = Qr Kr^T is a GEMM with reduction length s*d.  Instead
// of writing the fp32 score matrix (Lq*Lk/s^2 floats) and re-reading it, the
// GEMM epilogue reduces every (row, 128-token key block) to its base-2
// log-sum-exp over the block's allowed columns: a per-block form of the
// pages' per-chunk partial statistics, 128/s times smaller than the scores.
// The block-sum kernel then merges those partials per row (merge of the
// softmax statistics) and normalises them into block sums.  The result does
// not depend on how the key range is chunked.
#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kEstTile = 128;  // reshaped rows and columns per workgroup
// Raw buffer descriptor word 3 for gfx950 (32-bit data format, no swizzle).
constexpr int kEstBufFlags = 0x00020000;

// ---------------------------------------------------------------------------
// bf16 MFMA score tile + per-block log-sum-exp epilogue.
// Workgroup: 4 waves, tile 128 (c) x 128 (r); wave w owns the 64 x 64 quarter
// (c half w&1, r half w>>1) as 2 x 2 MFMA 32x32 accumulators of S^T, so each
// lane holds one query row r and 16 key columns of every accumulator.
// ---------------------------------------------------------------------------
template <int D, int S>
__global__ __launch_bounds__(256) void est_partial_bf16(EstArgs a) {
  constexpr int RB = kBlock / S;  // reshaped block
  constexpr int PITCH = D + 8;    // bf16 per LDS row (padding against bank conflicts)
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  __shared__ __align__(16) uint16_t qs[kEstTile * PITCH];
  __shared__ __align__(16) uint16_t ks[kEstTile * PITCH];

  const int bh = blockIdx.z;
  const int b = bh / a.hq, h = bh % a.hq, g = h / a.group;
  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int R = lq / S, C = lk / S, o_s = (lk - lq) / S;
  const int r0 = blockIdx.y * kEstTile;
  if (r0 >= R) return;
  const int c0 = a.jb0 * RB + blockIdx.x * kEstTile;
  const int c_end = min((a.jb0 + a.jb_count) * RB, C);
  if (c0 >= c_end) return;
  const int r_last = min(r0 + kEstTile, R) - 1;
  if (c0 > r_last + o_s) return;  // whole tile beyond the causal block diagonal

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wc = w & 1, wr = w >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

  const long long q_tok_bytes = (long long)a.hq * D * 2;
  const char* qbase = a.q + (long long)q0 * q_tok_bytes + (long long)h * D * 2;

  for (int t = 0; t < S; ++t) {
    for (int it = tid; it < kEstTile * CPR; it += 256) {
      const int row = it / CPR, part = it - (it / CPR) * CPR;
      u32x4 vq = {0u, 0u, 0u, 0u};
      const int r = r0 + row;
      if (r < R) vq = *(const u32x4*)(qbase + (long long)(r * S + S - 1 - t) * q_tok_bytes + part * 16);
      *(u32x4*)(&qs[row * PITCH + part * 8]) = vq;
      u32x4 vk = {0u, 0u, 0u, 0u};
      const int c = c0 + row;
      if (c < c_end) {
        const char* p = a.k.row(b, c * S + t, g);
        if (p) vk = *(const u32x4*)(p + part * 16);
      }
      *(u32x4*)(&ks[row * PITCH + part * 8]) = vk;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      bf16x8 af[2], bq[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
        af[x] = *(const bf16x8*)(&ks[(wc * 64 + x * 32 + l32) * PITCH + kk * 16 + hh * 8]);
#pragma unroll
      for (int y = 0; y < 2; ++y)
        bq[y] = *(const bf16x8*)(&qs[(wr * 64 + y * 32 + l32) * PITCH + kk * 16 + hh * 8]);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = mfma32(af[x], bq[y], acc[x][y]);
    }
    __syncthreads();
  }

  constexpr int NBLK = 32 / RB;  // key blocks per 32-column accumulator
  constexpr int IPB = RB / 8;    // accumulator row groups per key block
  const int j_end = a.jb0 + a.jb_count;
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int r = r0 + wr * 64 + y * 32 + l32;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int cblk = c0 + wc * 64 + x * 32;
      float z[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = cblk + 8 * (e >> 2) + 4 * hh + (e & 3);
        const bool ok = (r < R) && (c < c_end) && (c <= r + o_s);
        z[e] = ok ? acc[x][y][e] * a.scale2 : kNegInf;
      }
#pragma unroll
      for (int m = 0; m < NBLK; ++m) {
        float mx = kNegInf;
#pragma unroll
        for (int ii = 0; ii < IPB; ++ii)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) mx = fmaxf(mx, z[(m * IPB + ii) * 4 + jj]);
        float sm = 0.f;
        if (mx != kNegInf) {
#pragma unroll
          for (int ii = 0; ii < IPB; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sm += exp2f(z[(m * IPB + ii) * 4 + jj] - mx);
        }
        const float mo = __shfl_xor(mx, 32, 64);
        const float so = __shfl_xor(sm, 32, 64);
        const float M = fmaxf(mx, mo);
        float lse = kNegInf;
        if (M != kNegInf) lse = M + log2f(sm * exp2f(mx - M) + so * exp2f(mo - M));
        const int j = cblk / RB + m;
        const bool writer = (NBLK == 1) ? (hh == 0) : (hh == (m & 1));
        if (writer && r < R && j < j_end && j * RB < C)
          a.part[((long long)bh * a.max_kb + j) * a.max_r + r] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA score GEMM for large launches.  Workgroup: 8 waves, tile 256
// reshaped key columns x 256 reshaped query rows; wave w owns 128 columns
// (half w&1) x 64 rows (quarter w>>1) as 4 x 2 MFMA 32x32 accumulators of
// S^T.  The reduction (s tokens x d) runs in stages of 64 elements (one
// token offset t, one half or quarter of d), double-buffered in LDS and
// filled by direct buffer -> LDS loads: a row's token goes into a per-lane
// offset computed once, the stage's (t, d) position into the scalar offset,
// and rows past the end (or unallocated pages) read zeros through the
// descriptor's byte bound.  LDS rows are 128 B with 16-byte chunks
// XOR-swizzled by the row's low 3 bits (no bank conflicts for the fragment
// reads, which are inline asm retired by explicit lgkmcnt waits so that the
// compiler adds no wait for the in-flight copies).
// ---------------------------------------------------------------------------
template <int OFF>
__device__ __forceinline__ u32x4 est_lds_read16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int N>
__device__ __forceinline__ void est_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most N LDS operations are outstanding; ties the M fragments
template <int N, int M>
__device__ __forceinline__ void est_lgkm_wait_arr(u32x4* f) {
  if constexpr (M == 2) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(f[0]), "+v"(f[1]) : "n"(N));
  } else if constexpr (M == 3) {
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]) : "n"(N));
  } else if constexpr (M == 4) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]) : "n"(N));
  } else {
    static_assert(M == 6, "fragment count");
    asm volatile("s_waitcnt lgkmcnt(%6)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]) : "n"(N));
  }
}

// LPW buffer -> LDS copies of 1 KiB (16 B per lane) to consecutive KiB of LDS
template <int LPW>
__device__ __forceinline__ void est_copy_rows(__amdgpu_buffer_rsrc_t r, char* lds, const uint32_t* voff, int soff) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
  for (int n = 0; n < LPW; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(lds + n * 1024), 16, voff[n], soff, 0, 0);
}

// Maximum and sum of v over the lane pair (l, l ^ 32) -- the two halves of a
// 32-column MFMA accumulator row.  v_permlane32_swap of v with itself leaves
// one lane's own value and its partner's in the two results (which is which
// depends on the half); max and sum treat them alike, and a + b == b + a
// exactly, so both lanes get identical bits.
__device__ __forceinline__ float pair_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// 128 x 128 tiles: 8 waves (two per SIMD, each 64 x 32), 4 stage buffers of
// 32 reduction elements (64 KiB of LDS).  Measured on the 4K layer: 4 waves
// with 4 buffers of 64 19.5 us; 8 waves with 4 x 64 17.5, 2 x 64 17.5,
// 2 x 32 18.0, 4 x 32 17.0 us (same bits).
#ifndef XATTN_EST_NBUF
#define XATTN_EST_NBUF 4
#endif
#ifndef XATTN_EST_BK
#define XATTN_EST_BK 32
#endif
constexpr int kEstSmallWaves = 8;
constexpr int kEstSmallPerCu = 2;  // 128 x 128 workgroups per CU (64 KiB of LDS each)
// Big tiles: 256 x 256 over 8 waves, 2 stage buffers of 64 reduction
// elements (measured at 32K: 4 buffers of 32 elements 0.082 ms, 2 of 32
// 0.088, 2 of 64 0.078)
#ifndef XATTN_EST_BIG_TR
#define XATTN_EST_BIG_TR 256
#endif
#ifndef XATTN_EST_BIG_TC
#define XATTN_EST_BIG_TC 256
#endif
#ifndef XATTN_EST_BIG_NW
#define XATTN_EST_BIG_NW 8
#endif
#ifndef XATTN_EST_BIG_NBUF
#define XATTN_EST_BIG_NBUF 2
#endif
#ifndef XATTN_EST_BIG_BK
#define XATTN_EST_BIG_BK 64
#endif
#ifndef XATTN_EST_BIG_WPE
#define XATTN_EST_BIG_WPE 1
#endif
// workgroups of big tiles that share a CU (by their LDS and registers)
constexpr int kEstBigPerCu =
    std::min((160 * 1024) / (XATTN_EST_BIG_NBUF * (XATTN_EST_BIG_TR + XATTN_EST_BIG_TC) * XATTN_EST_BIG_BK * 2),
             std::max(1, 4 * XATTN_EST_BIG_WPE / XATTN_EST_BIG_NW));

// TR x TC tile (reshaped rows x columns) over NW waves: wave w owns TC/2
// columns (half w&1) x 2*TR/NW rows (part w>>1); XT x YT accumulators.  A
// stage covers BK reduction elements (LDS rows of 2*BK bytes); NBUF LDS stage
// buffers: NBUF - 1 stages of copies are in flight while one is computed.
// TAB: workgroups numbered over the tiles with work (a.tile_base), else over
// the whole (sequence, head, row tile, column tile) grid.  WPE: waves per SIMD
// the register allocation must leave room for (2 lets two 4-wave workgroups
// share a CU, so that one's epilogue runs under the other's MFMAs).
template <int D, int S, int TR, int TC, int NW, int NBUF, int BK, bool TAB, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE))) void est_gemm_bf16(EstArgs a) {
  constexpr int RB = kBlock / S;
  constexpr int KTB = TC * BK * 2;   // bytes of the K operand tile
  constexpr int BUFB = (TR + TC) * BK * 2;  // one stage buffer: K tile, then Q tile
  constexpr int CPR = BK / 8;        // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPR;      // rows per copy instruction (1 KiB)
  constexpr int KS = BK / 16;        // MFMA k-steps per stage
  constexpr int DQ = D / BK;         // stages per token offset
  constexpr int NST = S * DQ;        // stages
  constexpr int WR = NW / 2;         // wave rows
  constexpr int XT = TC / 2 / 32;    // 32-column accumulator tiles per wave
  constexpr int YT = TR / WR / 32;   // 32-row accumulator tiles per wave
  constexpr int LPK = TC / (RPI * NW); // K copy instructions per wave and stage
  constexpr int LPQ = TR / (RPI * NW); // Q copy instructions per wave and stage
  static_assert(BK == 32 || BK == 64, "stage width");
  static_assert(NBUF >= 2, "stage ring");
  static_assert(XT >= 1 && YT >= 1 && LPK >= 1 && LPQ >= 1 && TC % (RPI * NW) == 0 && TR % (RPI * NW) == 0,
                "tile / wave split");
  // 16-byte chunk swizzle of LDS row `row`.  A ds_read_b128 serves 16 lanes
  // (256 bytes, all banks) at a time, here 16 consecutive rows at one logical
  // chunk: the rows sharing a 256-byte bank window position (same parity for
  // 128-byte rows, same row % 4 for 64-byte rows) need distinct swizzles.
  // (row & 7 for 128-byte rows gave rows r and r + 8 the same banks: half of
  // the fragment reads' LDS cycles were bank-conflict stalls.)
  auto swz = [](int row) { return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3); };
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __shared__ __align__(1024) char lds[NBUF * BUFB];

  // XCD-aware work unit: the 8 XCDs take consecutive workgroup ids
  // round-robin, so logical unit (id % 8) * (n / 8) + id / 8 gives each XCD a
  // contiguous range of (head, row tile, column tile) units -- with the
  // column tile fastest, an XCD holds whole heads (typically one KV group),
  // and its L2 fetches their Q and K once.
  const int ntx = a.tiles_c, nty = a.tiles_r;
  const int nwg = gridDim.x, id = blockIdx.x;
  const int full = (nwg / 8) * 8;
  const int logical = id < full ? (id % 8) * (nwg / 8) + id / 8 : id;
  int bx, by, b, h;
  if (TAB) {
    // the logical-th tile with work: its sequence by binary search of
    // tile_base, then head, row tile and column tile (est_active_tiles)
    int lo = 0, hi = a.n_tab - 1;  // tile_base[lo] <= logical < tile_base[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_base[mid] <= logical) lo = mid;
      else hi = mid;
    }
    b = lo;
    const int per_head = (a.tile_base[b + 1] - a.tile_base[b]) / a.hq;
    int rem = logical - a.tile_base[b];
    if (a.group_chunk > 0) {
      // grouped order: the heads of a kv group take the same tile one after
      // the other, so that they read its K tile in the same round
      const int G = a.group;
      const int gi = rem / (per_head * G);
      rem -= gi * (per_head * G);
      const int t = rem / G;
      h = gi * G + (rem - t * G);
      rem = t;
    } else {
      h = rem / per_head;
      rem -= h * per_head;
    }
    const int lq_ = a.cu_q[b + 1] - a.cu_q[b], lk_ = a.cu_k[b + 1] - a.cu_k[b];
    const int R_ = lq_ / S, C_ = lk_ / S, os_ = (lk_ - lq_) / S;
    const int cbase = a.jb0 * RB, cend = min((a.jb0 + a.jb_count) * RB, C_);
    by = 0;
    bx = 0;
    for (int r0 = 0; r0 < R_; r0 += TR, ++by) {
      const int lim = min(cend, min(r0 + TR, R_) + os_);
      const int nbx = lim > cbase ? (lim - cbase + TC - 1) / TC : 0;
      if (rem < nbx) {
        bx = rem;
        break;
      }
      rem -= nbx;
    }
  } else if (a.group_chunk > 0) {
    // (sequence, kv group) blocks of units; inside a block, chunks of CC
    // column tiles with every row tile and every head of the group, so that
    // the units reading one K column tile run in the same round on one XCD
    // (with head-major units a launch of several rounds read each K tile
    // once per head: 146 instead of 96 MiB at 32K)
    const int G = a.group, hkv_ = a.hq / a.group;
    const int CC = a.group_chunk;
    const int per_group = ntx * nty * G;
    const int bg = logical / per_group;
    const int rem = logical - bg * per_group;
    const int full = (ntx / CC) * CC * nty * G;
    int c, r2, width;
    if (rem < full) {
      c = rem / (CC * nty * G);
      r2 = rem - c * (CC * nty * G);
      width = CC;
    } else {
      c = ntx / CC;
      r2 = rem - full;
      width = ntx - c * CC;
    }
    by = r2 / (G * width);
    const int r3 = r2 - by * (G * width);
    const int hg = r3 / width;
    bx = c * CC + (r3 - hg * width);
    b = bg / hkv_;
    h = (bg - b * hkv_) * G + hg;
  } else {
    bx = logical % ntx;
    by = (logical / ntx) % nty;
    const int bh = logical / (ntx * nty);
    b = bh / a.hq;
    h = bh % a.hq;
  }
  const int g = h / a.group, bh = b * a.hq + h;
  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int R = lq / S, C = lk / S, o_s = (lk - lq) / S;
  const int r0 = by * TR;
  if (r0 >= R) return;
  const int c0 = a.jb0 * RB + bx * TC;
  const int c_end = min((a.jb0 + a.jb_count) * RB, C);
  if (c0 >= c_end) return;
  const int r_last = min(r0 + TR, R) - 1;
  if (c0 > r_last + o_s) return;  // whole tile beyond the causal block diagonal

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int wc = w & 1, wr = w >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- copies: instruction n of wave w fills K tile rows (LPK*w+n)*RPI ..
  // +RPI and Q tile rows (LPQ*w+n)*RPI .. +RPI
  const long long q_tok = (long long)a.hq * D * 2;
  const long long k_row = (long long)a.k.kv_heads * D * 2;
  constexpr uint32_t kOut = 0x80000000u;  // beyond either descriptor's bound
  uint32_t kvo[LPK], qvo[LPQ];
#pragma unroll
  for (int n = 0; n < LPK; ++n) {
    const int row = (w * LPK + n) * RPI + lane / CPR;
    const int lc = (lane % CPR) ^ swz(row);  // logical chunk stored at this lane's position
    const int c = c0 + row;
    kvo[n] = kOut;
    if (c < c_end) {
      const char* p = a.k.row(b, c * S, g);
      if (p) kvo[n] = (uint32_t)(p - a.k.base) + lc * 16;
    }
  }
#pragma unroll
  for (int n = 0; n < LPQ; ++n) {
    const int row = (w * LPQ + n) * RPI + lane / CPR;
    const int lc = (lane % CPR) ^ swz(row);
    const int r = r0 + row;
    qvo[n] = kOut;
    if (r < R) qvo[n] = (uint32_t)(((long long)(q0 + r * S) * a.hq + h) * D * 2) + lc * 16;
  }
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.k.base, (short)0, (int)a.k_bytes, kEstBufFlags);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.q, (short)0, (int)a.q_bytes, kEstBufFlags);
  auto issue = [&](int st, int bf) {
    const int t = st / DQ, dq = st - (st / DQ) * DQ;
    const int so_k = (int)(t * k_row) + dq * BK * 2;
    const int so_q = (int)((S - 1 - t) * q_tok) + dq * BK * 2;
    char* kd = lds + bf * BUFB + wu * LPK * 1024;
    char* qd = lds + bf * BUFB + KTB + wu * LPQ * 1024;
    est_copy_rows<LPK>(rk, kd, kvo, so_k);
    est_copy_rows<LPQ>(rq, qd, qvo, so_q);
  };

  // ---- fragment addresses: every tile row a lane reads has the swizzle of
  // row l32 (rows differ by multiples of 32)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)lds;
  uint32_t ka[NBUF][KS], qa[NBUF][KS];
#pragma unroll
  for (int bf = 0; bf < NBUF; ++bf)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint32_t ch = (uint32_t)(((2 * kk + hh) ^ swz(l32)) * 16);
      ka[bf][kk] = lds0 + bf * BUFB + (wc * (TC / 2) + l32) * (BK * 2) + ch;
      qa[bf][kk] = lds0 + bf * BUFB + KTB + (wr * (YT * 32) + l32) * (BK * 2) + ch;
    }

  f32x16 acc[XT][YT];
#pragma unroll
  for (int x = 0; x < XT; ++x)
#pragma unroll
    for (int y = 0; y < YT; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

  // one stage: KS k-steps of 16; k-step kk+1's XT + YT fragments are read
  // while k-step kk's XT * YT MFMAs issue
  constexpr int NF = XT + YT;
  auto compute = [&](auto bf_tag) {
    constexpr int BF = decltype(bf_tag)::value;
    u32x4 f[NF], gq[NF];
    auto rd = [&](u32x4* dst, int kk) {
      [&]<int... X>(std::integer_sequence<int, X...>) {
        ((dst[X] = est_lds_read16<X * 32 * BK * 2>(ka[BF][kk])), ...);
      }(std::make_integer_sequence<int, XT>{});
      [&]<int... Y>(std::integer_sequence<int, Y...>) {
        ((dst[XT + Y] = est_lds_read16<Y * 32 * BK * 2>(qa[BF][kk])), ...);
      }(std::make_integer_sequence<int, YT>{});
    };
    rd(f, 0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 1 < KS) {
        rd(gq, kk + 1 < KS ? kk + 1 : 0);
        est_lgkm_wait_arr<NF, NF>(f);
      } else {
        est_lgkm_wait_arr<0, NF>(f);
      }
#pragma unroll
      for (int x = 0; x < XT; ++x)
#pragma unroll
        for (int y = 0; y < YT; ++y)
          acc[x][y] = mfma32(__builtin_bit_cast(bf16x8, f[x]), __builtin_bit_cast(bf16x8, f[XT + y]), acc[x][y]);
      if (kk + 1 < KS) {
#pragma unroll
        for (int z = 0; z < NF; ++z) f[z] = gq[z];
      }
    }
  };

  // ---- stage loop: wait for this wave's copies of stage st (the copies of
  // the NBUF - 2 later stages may stay in flight), barrier (every wave's
  // copies of stage st visible; buffer (st - 1) % NBUF, computed in the
  // previous step, free), copy stage st + NBUF - 1 into it, compute st
  constexpr int PER = LPK + LPQ;  // copy instructions per wave and stage
#pragma unroll
  for (int x = 0; x < NBUF - 1; ++x) issue(x, x);
  for (int st0 = 0; st0 < NST; st0 += NBUF) {
    [&]<int... B>(std::integer_sequence<int, B...>) {
      ([&] {
        const int st = st0 + B;
        if (NST % NBUF == 0 || st < NST) {
          if (st + NBUF - 2 < NST) est_wait_vmcnt<(NBUF - 2) * PER>();
          else est_wait_vmcnt<0>();
          __builtin_amdgcn_s_barrier();
          if (st + NBUF - 1 < NST) issue(st + NBUF - 1, (B + NBUF - 1) % NBUF);
          compute(std::integral_constant<int, B>{});
        }
      }(), ...);
    }(std::make_integer_sequence<int, NBUF>{});
  }

  // ---- epilogue: per (query row, key block) base-2 log-sum-exp over the
  // block's allowed columns.  A block's columns are split between lanes l and
  // l ^ 32: the pair first agrees on the block's maximum (one swap of the two
  // halves' maxima), each lane sums 2^(z - max) over its half, and one more
  // swap adds the two sums, so lse = max + log2(sum of both halves).
  constexpr int NBLK = 32 / RB;  // key blocks per 32-column accumulator
  constexpr int EPB = 16 / NBLK; // accumulator values per lane and block
  static_assert(EPB % 2 == 0, "max tree pairs");
  const int j_end = a.jb0 + a.jb_count;
  // Whole tile inside the rows, the launch's columns and the causal bound
  // (the common case): no per-element masks.  Exponentials and logarithm
  // are the bare hardware instructions (v_exp_f32 / v_log_f32): every term
  // is 2^(z - max) <= 1 and the sum is >= 1, so flushing terms below 2^-126
  // to zero changes nothing at fp32 resolution.
  const bool unmasked = (r0 + TR <= R) && (c0 + TC <= c_end) && (c0 + TC - 1 <= r0 + o_s);
  const float sc = a.scale2;
  auto mx3 = [](float p, float q, float r) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(p, q), r);
  };
#pragma unroll
  for (int y = 0; y < YT; ++y) {
    const int r = r0 + wr * (YT * 32) + y * 32 + l32;
#pragma unroll
    for (int x = 0; x < XT; ++x) {
      const int cblk = c0 + wc * (TC / 2) + x * 32;
#pragma unroll
      for (int m = 0; m < NBLK; ++m) {
        float lse = kNegInf;
        if (unmasked) {
          // max of the lane's EPB raw scores (sc > 0 keeps the order), then of the pair
          float am = acc[x][y][m * EPB];
          int q = 1;
#pragma unroll
          for (; q + 1 < EPB; q += 2) am = mx3(am, acc[x][y][m * EPB + q], acc[x][y][m * EPB + q + 1]);
#pragma unroll
          for (; q < EPB; ++q) am = __builtin_elementwise_maximum(am, acc[x][y][m * EPB + q]);
          const float mxs = pair_max(am) * sc;
          float sm = 0.f;
#pragma unroll
          for (int e = 0; e < EPB; ++e) sm += __builtin_amdgcn_exp2f(fmaf(acc[x][y][m * EPB + e], sc, -mxs));
          lse = mxs + __builtin_amdgcn_logf(pair_sum(sm));
        } else {
          float z[EPB];
          float mx = kNegInf;
#pragma unroll
          for (int q = 0; q < EPB; ++q) {
            const int e = m * EPB + q;
            const int c = cblk + 8 * (e >> 2) + 4 * hh + (e & 3);
            const bool ok = (r < R) && (c < c_end) && (c <= r + o_s);
            z[q] = ok ? acc[x][y][e] * sc : kNegInf;
            mx = fmaxf(mx, z[q]);
          }
          const float M = pair_max(mx);
          float sm = 0.f;
          if (M != kNegInf) {
#pragma unroll
            for (int q = 0; q < EPB; ++q) sm += __builtin_amdgcn_exp2f(z[q] - M);
          }
          const float tot = pair_sum(sm);
          if (M != kNegInf) lse = M + __builtin_amdgcn_logf(tot);
        }
        const int j = cblk / RB + m;
        if (hh == 0 && r < R && j < j_end && j * RB < C)
          a.part[((long long)bh * a.max_kb + j) * a.max_r + r] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: plain VALU dot products (tiny workloads; fp32 accuracy).
// Workgroup = one key block j x 4 reshaped rows, one wave per row; within a
// wave, lane = cx * PT + pt: PT = 64 / RB lanes share column cx, each summing
// S / PT of the S token offsets (two chains), and the parts are added with
// cross-lane shuffles (fixed order, so every launch of the same cell gives
// the same bits); the RB columns of the row are then reduced to the block's
// log-sum-exp with shuffles as well.
// ---------------------------------------------------------------------------
template <int D, int S>
__global__ __launch_bounds__(256) void est_partial_f32(EstArgs a) {
  constexpr int RB = kBlock / S;
  constexpr int PT = 64 / RB;  // lanes per column
  constexpr int TP = S / PT;   // token offsets per lane
  static_assert(PT >= 1 && S % PT == 0, "stride / lane split");
  const int lane = threadIdx.x & 63;
  const int cx = lane / PT, pt = lane % PT;
  const int bh = blockIdx.z;
  const int b = bh / a.hq, h = bh % a.hq, g = h / a.group;
  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int R = lq / S, C = lk / S, o_s = (lk - lq) / S;
  const int j = a.jb0 + blockIdx.x;
  const int r = blockIdx.y * 4 + (int)(threadIdx.x >> 6);
  if (r >= R || j * RB >= C) return;  // whole waves: r is uniform in a wave
  const int c = j * RB + cx;
  const bool allowed = c <= r + o_s;
  float s0 = 0.f, s1 = 0.f;
  if (allowed) {
#pragma unroll
    for (int u = 0; u < TP; ++u) {
      const int t = pt * TP + u;
      const float* qp = (const float*)(a.q) + ((long long)(q0 + r * S + S - 1 - t) * a.hq + h) * D;
      const float* kp = (const float*)a.k.row(b, c * S + t, g);
      if (!kp) continue;
#pragma unroll 4
      for (int e = 0; e < D; e += 4) {
        const f32x4 qv = *(const f32x4*)(qp + e);
        const f32x4 kv = *(const f32x4*)(kp + e);
        s0 = fmaf(qv[0], kv[0], s0);
        s1 = fmaf(qv[1], kv[1], s1);
        s0 = fmaf(qv[2], kv[2], s0);
        s1 = fmaf(qv[3], kv[3], s1);
      }
    }
  }
  float sd = s0 + s1;
#pragma unroll
  for (int off = 1; off < PT; off <<= 1) sd += __shfl_xor(sd, off, 64);
  const float z = allowed ? sd * a.scale2 : kNegInf;
  float mx = z;
#pragma unroll
  for (int off = PT; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  // each column is held by PT lanes: count it once
  float e = (mx == kNegInf || pt != 0) ? 0.f : exp2f(z - mx);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) e += __shfl_xor(e, off, 64);
  if (lane == 0)
    a.part[((long long)bh * a.max_kb + j) * a.max_r + r] = (mx == kNegInf) ? kNegInf : mx + log2f(e);
}

// ---------------------------------------------------------------------------
// Merge of the softmax statistics + normalise + block sum.
// Workgroup (i, h, b): rows r in [i*RB, (i+1)*RB), allowed blocks j <= i+Kh.
// Phase 1 merges the per-block partial log-sum-exps of each row into its row
// log-sum-exp; phase 2 writes block_sums[b,h,i,j] = sum_r 2^(part - row).
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256) void block_sums_kernel(BlockSumArgs a) {
  constexpr int JL = 256 / RB;
  __shared__ float sm_m[JL][RB];
  __shared__ float sm_l[JL][RB];
  __shared__ float row_lse[RB];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  float* out = a.block_sums + (((long long)b * a.hq + h) * a.max_qb + i) * a.max_kb;
  if (i >= qb) {
    for (int j = threadIdx.x; j < a.max_kb; j += 256) out[j] = 0.f;
    return;
  }
  const int nj = i + kh + 1;
  const float* base = a.part + ((long long)(b * a.hq + h) * a.max_kb) * a.max_r + i * RB;
  const int rr = threadIdx.x % RB, jl = threadIdx.x / RB;
  float m = kNegInf, l = 0.f;
  for (int j = jl; j < nj; j += JL) {
    const float v = base[(long long)j * a.max_r + rr];
    if (v == kNegInf) continue;
    if (v > m) {
      l = l * exp2f(m - v) + 1.f;
      m = v;
    } else {
      l += exp2f(v - m);
    }
  }
  sm_m[jl][rr] = m;
  sm_l[jl][rr] = l;
  __syncthreads();
  if (threadIdx.x < RB) {
    float M = kNegInf;
    for (int x = 0; x < JL; ++x) M = fmaxf(M, sm_m[x][threadIdx.x]);
    float L = 0.f;
    if (M != kNegInf)
      for (int x = 0; x < JL; ++x)
        if (sm_m[x][threadIdx.x] != kNegInf) L += sm_l[x][threadIdx.x] * exp2f(sm_m[x][threadIdx.x] - M);
    row_lse[threadIdx.x] = (M == kNegInf) ? kNegInf : M + log2f(L);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.max_kb; j += 256) {
    float s = 0.f;
    if (j < nj) {
      const float* p = base + (long long)j * a.max_r;
#pragma unroll
      for (int x = 0; x < RB; ++x) {
        const float v = p[x];
        if (v != kNegInf) s += exp2f(v - row_lse[x]);
      }
    }
    out[j] = s;
  }
}

// The same in one read: workgroup (i, h, b) of 1024 threads, thread (jl, rr)
// holds the partial log-sum-exps of row rr for blocks jl, jl + JL, ... in
// registers (NV * JL >= max_kb).  Row maxima and row sums meet in LDS; then
// each thread scales its 2^(part - max) by 1 / row sum and the RB lanes of a
// block add them with cross-lane shuffles.
template <int RB, int NV>
__global__ __launch_bounds__(1024) void block_sums_reg_kernel(BlockSumArgs a) {
  constexpr int JL = 1024 / RB;
  __shared__ float red[JL][RB];
  __shared__ float row_v[RB];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lq = a.cu_q[b + 1] - a.cu_q[b];
  const int lk = a.cu_k[b + 1] - a.cu_k[b];
  const int qb = lq / kBlock, kh = (lk - lq) / kBlock;
  const int tid = threadIdx.x;
  float* out = a.block_sums + (((long long)b * a.hq + h) * a.max_qb + i) * a.max_kb;
  if (i >= qb) {
    for (int j = tid; j < a.max_kb; j += 1024) out[j] = 0.f;
    return;
  }
  const int nj = i + kh + 1;
  const float* base = a.part + ((long long)(b * a.hq + h) * a.max_kb) * a.max_r + i * RB;
  const int rr = tid % RB, jl = tid / RB;
  float v[NV];
  float m = kNegInf;
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    const int j = jl + t * JL;
    v[t] = (j < nj) ? base[(long long)j * a.max_r + rr] : kNegInf;
    m = fmaxf(m, v[t]);
  }
  red[jl][rr] = m;
  __syncthreads();
  if (tid < RB) {
    float M = kNegInf;
    for (int x = 0; x < JL; ++x) M = fmaxf(M, red[x][tid]);
    row_v[tid] = M;
  }
  __syncthreads();
  const float M = row_v[rr];
  float l = 0.f;
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    v[t] = (v[t] == kNegInf) ? 0.f : exp2f(v[t] - M);
    l += v[t];
  }
  red[jl][rr] = l;
  __syncthreads();
  if (tid < RB) {
    float L = 0.f;
    for (int x = 0; x < JL; ++x) L += red[x][tid];
    row_v[tid] = (L > 0.f) ? 1.f / L : 0.f;
  }
  __syncthreads();
  const float inv = row_v[rr];
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    float sb = v[t] * inv;
#pragma unroll
    for (int off = RB / 2; off > 0; off >>= 1) sb += __shfl_xor(sb, off, RB);
    const int j = jl + t * JL;
    if (rr == 0 && j < a.max_kb) out[j] = (j < nj) ? sb : 0.f;
  }
}

// Tiles of a sequence's head that have work for tile size tt over the
// launch's key blocks [jb0, jb0 + jb_count): row tile r0 keeps the column
// tiles whose first column c0 lies before both the key range's end and the
// causal bound of its last row (c0 <= r_last + (Lk - Lq)/s), the same rules
// by which est_gemm_bf16 skips a tile.
int est_active_tiles(int lq, int lk, int S, int tr, int tc, int jb0, int jb_count) {
  const int RB = kBlock / S;
  const int R = lq / S, C = lk / S, o_s = (lk - lq) / S;
  const int cbase = jb0 * RB, cend = std::min((jb0 + jb_count) * RB, C);
  int n = 0;
  for (int r0 = 0; r0 < R; r0 += tr) {
    const int lim = std::min(cend, std::min(r0 + tr, R) + o_s);
    if (lim > cbase) n += (lim - cbase + tc - 1) / tc;
  }
  return n;
}

// Fills a.tile_base / a.n_tab for tr x tc tiles; false (and n_tab 0) when
// the batch is beyond the table or a count overflows.
bool est_tile_table(EstArgs& a, int S, int tr, int tc, int batch) {
  a.n_tab = 0;
  if (!a.cu_q_host || !a.cu_k_host || batch > kEstMaxSeq) return false;
  long long acc = 0;
  for (int b = 0; b < batch; ++b) {
    a.tile_base[b] = (int)acc;
    const int lq = a.cu_q_host[b + 1] - a.cu_q_host[b], lk = a.cu_k_host[b + 1] - a.cu_k_host[b];
    acc += (long long)a.hq * est_active_tiles(lq, lk, S, tr, tc, a.jb0, a.jb_count);
    if (acc >= (1ll << 31)) return false;
  }
  a.tile_base[batch] = (int)acc;
  a.n_tab = batch + 1;
  return true;
}

// Column tiles per chunk of the grouped unit order (EstArgs::group_chunk)
// for a launch of n workgroups, per_cu of which share a CU: 0 (head-major
// units) when every XCD's units fit one round, else enough column tiles
// that one chunk -- all row tiles of all heads of a kv group -- fills one
// XCD's 32 CUs.
int est_group_chunk(long long n, int per_cu, int tiles_r, int group) {
  if (n <= 256ll * per_cu) return 0;
  return std::max(1, 32 * per_cu / (tiles_r * group));
}

template <int D, int S>
hipError_t est_dispatch(const EstArgs& a, int dtype, int batch, hipStream_t st) {
  constexpr int RB = kBlock / S;
  if (dtype == 0) {
    // big tiles when they still fill the chip, else 128 x 128 tiles (8
    // waves); both need Q and K spans within 31-bit buffer offsets.
    if (a.q_bytes < (1ll << 31) && a.k_bytes < (1ll << 31)) {
      // several sequences: one workgroup per tile with work when the batch
      // fits the table, so that every XCD gets the same number of tiles
      // whatever the sequences' lengths (one per grid tile otherwise: for a
      // single sequence that measured 1-2 us faster)
      constexpr int TR = XATTN_EST_BIG_TR, TC = XATTN_EST_BIG_TC, NW = XATTN_EST_BIG_NW;
      dim3 big((a.jb_count * RB + TC - 1) / TC, (a.max_r + TR - 1) / TR, batch * a.hq);
      EstArgs a2 = a;
      long long nbig = (long long)big.x * big.y * big.z;
      if (batch > 1 && est_tile_table(a2, S, TR, TC, batch)) nbig = a2.tile_base[batch];
      if (nbig >= 256 * kEstBigPerCu) {
        a2.tiles_c = (int)big.x;
        a2.tiles_r = (int)big.y;
        a2.group_chunk = est_group_chunk(nbig, kEstBigPerCu, a2.tiles_r, a.group);  // (with a table: > 0 = grouped)
        if (a2.n_tab > 0)
          hipLaunchKernelGGL((est_gemm_bf16<D, S, TR, TC, NW, XATTN_EST_BIG_NBUF, XATTN_EST_BIG_BK, true, XATTN_EST_BIG_WPE>),
                             dim3((unsigned)nbig), dim3(64 * NW), 0, st, a2);
        else
          hipLaunchKernelGGL((est_gemm_bf16<D, S, TR, TC, NW, XATTN_EST_BIG_NBUF, XATTN_EST_BIG_BK, false, XATTN_EST_BIG_WPE>),
                             dim3((unsigned)nbig), dim3(64 * NW), 0, st, a2);
      } else {
        a2.tiles_c = (a.jb_count * RB + kEstTile - 1) / kEstTile;
        a2.tiles_r = (a.max_r + kEstTile - 1) / kEstTile;
        long long n = (long long)a2.tiles_c * a2.tiles_r * batch * a.hq;
        a2.group_chunk = est_group_chunk(n, kEstSmallPerCu, a2.tiles_r, a.group);
        if (batch > 1 && est_tile_table(a2, S, kEstTile, kEstTile, batch)) n = a2.tile_base[batch];
        else a2.n_tab = 0;
        if (n > 0 && a2.n_tab > 0)
          hipLaunchKernelGGL((est_gemm_bf16<D, S, kEstTile, kEstTile, kEstSmallWaves, XATTN_EST_NBUF, XATTN_EST_BK, true, 1>),
                             dim3((unsigned)n), dim3(64 * kEstSmallWaves), 0, st, a2);
        else if (n > 0)
          hipLaunchKernelGGL((est_gemm_bf16<D, S, kEstTile, kEstTile, kEstSmallWaves, XATTN_EST_NBUF, XATTN_EST_BK, false, 1>),
                             dim3((unsigned)n), dim3(64 * kEstSmallWaves), 0, st, a2);
      }
      return hipGetLastError();
    }
    dim3 grid((a.jb_count * RB + kEstTile - 1) / kEstTile, (a.max_r + kEstTile - 1) / kEstTile,
              batch * a.hq);
    hipLaunchKernelGGL((est_partial_bf16<D, S>), grid, dim3(256), 0, st, a);
  } else {
    dim3 grid(a.jb_count, (a.max_r + 3) / 4, batch * a.hq);
    hipLaunchKernelGGL((est_partial_f32<D, S>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_estimate(const EstArgs& a, int dtype, int head_dim, int stride, int batch,
                           hipStream_t s) {
  if (a.jb_count <= 0 || a.max_r <= 0 || batch <= 0) return hipSuccess;
#define XATTN_EST_CASE(D_, S_) \
  if (head_dim == D_ && stride == S_) return est_dispatch<D_, S_>(a, dtype, batch, s);
  XATTN_EST_CASE(128, 8)
  XATTN_EST_CASE(128, 16)
  XATTN_EST_CASE(128, 4)
  XATTN_EST_CASE(64, 8)
  XATTN_EST_CASE(64, 16)
  XATTN_EST_CASE(64, 4)
#undef XATTN_EST_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_block_sums(const BlockSumArgs& a, int batch, hipStream_t s) {
  if (a.max_qb <= 0 || a.max_kb <= 0 || batch <= 0) return hipSuccess;
  dim3 grid(a.max_qb, a.hq, batch);
  const int rb = kBlock / a.stride;
  const int jl = 1024 / rb;
  int nv = 1;
  while (nv * jl < a.max_kb) nv <<= 1;
#define XATTN_BS_CASE(RB_, NV_)                                                                  \
  if (rb == RB_ && nv == NV_) {                                                                  \
    hipLaunchKernelGGL((block_sums_reg_kernel<RB_, NV_>), grid, dim3(1024), 0, s, a);           \
    return hipGetLastError();                                                                    \
  }
  XATTN_BS_CASE(8, 1) XATTN_BS_CASE(8, 2) XATTN_BS_CASE(8, 4) XATTN_BS_CASE(8, 8) XATTN_BS_CASE(8, 16)
  XATTN_BS_CASE(16, 1) XATTN_BS_CASE(16, 2) XATTN_BS_CASE(16, 4) XATTN_BS_CASE(16, 8) XATTN_BS_CASE(16, 16)
  XATTN_BS_CASE(32, 1) XATTN_BS_CASE(32, 2) XATTN_BS_CASE(32, 4) XATTN_BS_CASE(32, 8) XATTN_BS_CASE(32, 16)
#undef XATTN_BS_CASE
  switch (rb) {
    case 8: hipLaunchKernelGGL((block_sums_kernel<8>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((block_sums_kernel<16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((block_sums_kernel<32>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace xattn
