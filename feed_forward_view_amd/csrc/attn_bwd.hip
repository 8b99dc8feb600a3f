// Gradients of bf16 softmax attention on gfx950 matrix cores.
//
// With s_ij = scale <q_i, k_j> (q, k rotated by RoPE), p_ij = 2^(s_ij log2(e)
// - lse2_i) from the forward pass's log-normaliser, D_i = sum_d dO_id O_id:
//   dV_j = sum_i p_ij dO_i
//   dS_ij = p_ij (<dO_i, V_j> - D_i)
//   dQ_i = scale sum_j dS_ij K_j        dK_j = scale sum_i dS_ij Q_i
// (the chain rule through softmax(Q K^T / sqrt(d)) V, "VGGT 論文報告" slide
// deck, Section V, slide 5/10; D_i = sum_j p_ij <dO_i, V_j> because
// O_i = sum_j p_ij V_j).  dQ and dK are rotated back by the transpose of the
// position's rotation.
//
// Two kernels, no atomics:
//   attn_bwd_dq_kernel    one wave per 32 queries, keys streamed in 64-key
//                         tiles (K rows, V rows, K^T) through LDS:
//                           S^T  = K Q^T - lse2      (accumulator input -lse2)
//                           dP^T = V dO^T - D        (accumulator input -D)
//                           dS^T = 2^(S^T) * dP^T
//                           dQ^T += K^T dS^T
//   attn_bwd_dkdv_kernel  one wave per 32 keys, queries streamed in 64-query
//                         tiles (Q rows, dO rows, Q^T, dO^T, lse2, D):
//                           S  = Q K^T - lse2,  dP = dO V^T - D
//                           dV^T += dO^T P,      dK^T += Q^T dS
// Both use v_mfma_f32_32x32x16_bf16 with the layout tricks of the forward
// kernel: row tiles hold their 64 rows in the order rho (bits 2 and 3
// swapped), so the accumulator registers of a score block are, in order, the
// bf16 operand of the next product; transposed tiles hold 8-row units per
// 16-byte slot.  The query operand of the scores carries scale*log2(e) and is
// rounded exactly as in the forward kernel, so the recomputed probabilities
// match the saved log-normaliser.  Rows past the end are zero in every tile
// and their -lse2 is -inf, so they contribute nothing.
#include "common.h"

namespace vggt {
namespace {

constexpr int D = kHeadDim;
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = NW * 64;
constexpr int BW = 32;       // queries (dQ) or keys (dK/dV) per wave
constexpr int BWG = NW * BW;  // per workgroup
constexpr float kLog2e = 1.44269504088896340736f;


typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
}

__device__ __forceinline__ f32x16 splat(float x) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x;
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Rotate a dim pair back (transpose of the RoPE rotation), scale, store 4 dims of one row.
__device__ __forceinline__ void store4(uint16_t* dst, const float* x, const f32x2* trow, int d0, float scale) {
  float y[4] = {x[0], x[1], x[2], x[3]};
  if (trow) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x2 cs = trow[(d0 >> 1) + e];
      const float a = y[2 * e], b = y[2 * e + 1];
      y[2 * e] = __builtin_fmaf(a, cs[0], b * cs[1]);
      y[2 * e + 1] = __builtin_fmaf(b, cs[0], -a * cs[1]);
    }
  }
  const u32x2 w = {pack_bf16x2(y[0] * scale, y[1] * scale), pack_bf16x2(y[2] * scale, y[3] * scale)};
  *(u32x2*)(dst + d0) = w;
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

struct SmemDq {
  u32x4 k[2][64][8];   // K rows
  u32x4 v[2][64][8];   // V rows
  u32x4 kt[2][64][8];  // K^T
};

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(AttnBwdProblem p) {
  __shared__ SmemDq sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int ntq = (p.n + BWG - 1) / BWG;
  const int nwg = ntq * p.H * p.nseq;
  int logical;
  xcd_remap(blockIdx.x, nwg, logical);
  const int qt = logical % ntq;
  const int head = (logical / ntq) % p.H;
  const int seq = logical / (ntq * p.H);
  const int64_t tok0 = (int64_t)seq * p.seq_stride;
  const int64_t tbase = ((int64_t)seq * p.H + head) * p.ntile * 512;
  const u32x4* kg = (const u32x4*)p.k_rows + tbase;
  const u32x4* vg = (const u32x4*)p.v_rows + tbase;
  const u32x4* ktg = (const u32x4*)p.k_trans + tbase;
  const int64_t sbase = ((int64_t)seq * p.H + head) * p.ntile * 64;

  auto issue = [&](int stage, int tile) {
    const int64_t off = (int64_t)tile * 512 + wave * 128 + lane;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = (2 * wave + c) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(kg + off + 64 * c), (lds_void*)&sm.k[stage][row][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vg + off + 64 * c), (lds_void*)&sm.v[stage][row][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(ktg + off + 64 * c), (lds_void*)&sm.kt[stage][row][0], 16, 0,
                                       0);
    }
  };
  issue(0, 0);

  // this lane's query, its rotated and scaled Q fragments and its dO fragments
  const int qi = qt * BWG + wave * BW + l32;
  const bool ok = qi < p.n;
  const int64_t tok = tok0 + (ok ? qi : 0);
  const f32x2* trow = p.rope_tab ? p.rope_tab + (int)(tok % p.rope_T) * 32 : nullptr;
  bf16x8 qf[4], df[4];
#pragma unroll
  for (int dc = 0; dc < 4; ++dc) {
    const int d0 = 16 * dc + 8 * hi;
    u32x4 w = *(const u32x4*)((const uint16_t*)p.q + tok * p.tok_stride + head * D + d0);
    u32x4 g = *(const u32x4*)((const uint16_t*)p.dout + tok * p.tok_stride + head * D + d0);
    if (!ok) w = g = u32x4{0u, 0u, 0u, 0u};
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = lo_bf16(w[e]), y = hi_bf16(w[e]);
      if (trow) {
        const f32x2 cs = trow[(d0 >> 1) + e];
        const float x2 = __builtin_fmaf(x, cs[0], -y * cs[1]);
        const float y2 = __builtin_fmaf(x, cs[1], y * cs[0]);
        x = x2;
        y = y2;
      }
      r[e] = pack_bf16x2(x * p.scale_log2, y * p.scale_log2);
    }
    qf[dc] = as_bf16x8(r);
    df[dc] = as_bf16x8(g);
  }
  const f32x16 nl = splat(ok ? p.lse2[sbase + qi] : -INFINITY);
  const f32x16 nd = splat(ok ? p.dsum[sbase + qi] : 0.0f);

  f32x16 acc[2] = {splat(0.0f), splat(0.0f)};  // dQ^T [db]: dims 32db + ..., this lane's query
  for (int t = 0; t < p.ntile; ++t) {
    const int stage = t & 1;
    if (t + 1 < p.ntile) {
      __syncthreads();  // every wave is done with the stage tile t+1 goes to
      issue(stage ^ 1, t + 1);
      wait_vmcnt<6>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * kb + l32;
      s[kb] = nl;
      dp[kb] = nd;
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        const int slot = (2 * dc + hi) ^ row_swz(row);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.k[stage][row][slot]), qf[dc], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.v[stage][row][slot]), df[dc], dp[kb], 0, 0, 0);
      }
    }
    if (t == p.ntile - 1 && 64 * p.ntile > p.n) {
      // keys past the end are zero rows, so their score would be the bare
      // -lse2, whose exponential overflows when the row's log-normaliser lies
      // far below zero (and then meets the zero K^T row as inf * 0)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (64 * t + 32 * kb + 16 * (r >> 3) + 8 * hi + (r & 7) >= p.n) s[kb][r] = -INFINITY;
    }
    // dS^T as bf16 pairs: registers 8j..8j+7 of block kb are keys 32kb + 16j + 8hi + 0..7
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * j + 2 * e;
          w[e] = pack_bf16x2(__builtin_amdgcn_exp2f(s[kb][r]) * dp[kb][r],
                             __builtin_amdgcn_exp2f(s[kb][r + 1]) * dp[kb][r + 1]);
        }
        const int u = 4 * kb + 2 * j + hi;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int d = 32 * db + l32;
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.kt[stage][d][u ^ col_swz(d)]), as_bf16x8(w),
                                                            acc[db], 0, 0, 0);
        }
      }
  }
  if (!ok) return;
  uint16_t* dst = (uint16_t*)p.dq + tok * p.tok_stride + head * D;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float x[4] = {acc[db][4 * a], acc[db][4 * a + 1], acc[db][4 * a + 2], acc[db][4 * a + 3]};
      store4(dst, x, trow, 32 * db + 8 * a + 4 * hi, p.scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

struct SmemDkv {
  u32x4 q[2][64][8];   // Q rows (scaled)
  u32x4 d[2][64][8];   // dO rows
  u32x4 qt[2][64][8];  // Q^T
  u32x4 dt[2][64][8];  // dO^T
  float st[2][2][64];  // lse2, D of the tile's 64 queries
};

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(AttnBwdProblem p) {
  __shared__ SmemDkv sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int ntk = (p.n + BWG - 1) / BWG;
  const int nwg = ntk * p.H * p.nseq;
  int logical;
  xcd_remap(blockIdx.x, nwg, logical);
  const int kt = logical % ntk;
  const int head = (logical / ntk) % p.H;
  const int seq = logical / (ntk * p.H);
  const int64_t tok0 = (int64_t)seq * p.seq_stride;
  const int64_t tbase = ((int64_t)seq * p.H + head) * p.ntile * 512;
  const u32x4* qg = (const u32x4*)p.q_rows + tbase;
  const u32x4* dg = (const u32x4*)p.do_rows + tbase;
  const u32x4* qtg = (const u32x4*)p.q_trans + tbase;
  const u32x4* dtg = (const u32x4*)p.do_trans + tbase;
  const int64_t sbase = ((int64_t)seq * p.H + head) * p.ntile * 64;

  auto issue = [&](int stage, int tile) {
    const int64_t off = (int64_t)tile * 512 + wave * 128 + lane;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = (2 * wave + c) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(qg + off + 64 * c), (lds_void*)&sm.q[stage][row][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(dg + off + 64 * c), (lds_void*)&sm.d[stage][row][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(qtg + off + 64 * c), (lds_void*)&sm.qt[stage][row][0], 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds((const void*)(dtg + off + 64 * c), (lds_void*)&sm.dt[stage][row][0], 16, 0,
                                       0);
    }
    // 512 bytes of statistics: waves 0-1 bring lse2, waves 2-3 bring D (8 lanes x 16 bytes each)
    if (lane < 8) {
      const float* src = (wave < 2 ? p.lse2 : p.dsum) + sbase + (int64_t)tile * 64 + 32 * (wave & 1) + 4 * lane;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)&sm.st[stage][wave >> 1][32 * (wave & 1)], 16, 0,
                                       0);
    }
  };
  issue(0, 0);

  // this lane's key: rotated K and V fragments (B operands of S = Q K^T and dP = dO V^T)
  const int kj = kt * BWG + wave * BW + l32;
  const bool ok = kj < p.n;
  const int64_t tok = tok0 + (ok ? kj : 0);
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int dc = 0; dc < 4; ++dc) {
    const int d0 = 16 * dc + 8 * hi;
    u32x4 a = *(const u32x4*)((const uint16_t*)p.kr + tok * p.tok_stride + head * D + d0);
    u32x4 b = *(const u32x4*)((const uint16_t*)p.v + tok * p.tok_stride + head * D + d0);
    if (!ok) a = b = u32x4{0u, 0u, 0u, 0u};
    kf[dc] = as_bf16x8(a);
    vf[dc] = as_bf16x8(b);
  }

  f32x16 dka[2] = {splat(0.0f), splat(0.0f)};  // dK^T [db], this lane's key
  f32x16 dva[2] = {splat(0.0f), splat(0.0f)};  // dV^T [db]
  for (int t = 0; t < p.ntile; ++t) {
    const int stage = t & 1;
    if (t + 1 < p.ntile) {
      __syncthreads();
      issue(stage ^ 1, t + 1);
      wait_vmcnt<9>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // accumulator inputs: -lse2 and -D of the queries of registers r: 32qb + 16(r/8) + 8hi + r%8
      f32x16 s, dp;
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int q0 = 32 * qb + 16 * h8 + 8 * hi;
        const f32x4 l0 = *(const f32x4*)&sm.st[stage][0][q0], l1 = *(const f32x4*)&sm.st[stage][0][q0 + 4];
        const f32x4 d0 = *(const f32x4*)&sm.st[stage][1][q0], d1 = *(const f32x4*)&sm.st[stage][1][q0 + 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[8 * h8 + e] = l0[e];
          s[8 * h8 + 4 + e] = l1[e];
          dp[8 * h8 + e] = d0[e];
          dp[8 * h8 + 4 + e] = d1[e];
        }
      }
      const int row = 32 * qb + l32;
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        const int slot = (2 * dc + hi) ^ row_swz(row);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.q[stage][row][slot]), kf[dc], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.d[stage][row][slot]), vf[dc], dp, 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 pw, sw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * c + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(s[r]), p1 = __builtin_amdgcn_exp2f(s[r + 1]);
          pw[e] = pack_bf16x2(p0, p1);
          sw[e] = pack_bf16x2(p0 * dp[r], p1 * dp[r + 1]);
        }
        const int u = 4 * qb + 2 * c + hi;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int d = 32 * db + l32;
          const int slot = u ^ col_swz(d);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.dt[stage][d][slot]), as_bf16x8(pw), dva[db],
                                                            0, 0, 0);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sm.qt[stage][d][slot]), as_bf16x8(sw), dka[db],
                                                            0, 0, 0);
        }
      }
    }
  }
  if (!ok) return;
  const f32x2* trow = p.rope_tab ? p.rope_tab + (int)(tok % p.rope_T) * 32 : nullptr;
  uint16_t* dkp = (uint16_t*)p.dk + tok * p.tok_stride + head * D;
  uint16_t* dvp = (uint16_t*)p.dv + tok * p.tok_stride + head * D;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * db + 8 * a + 4 * hi;
      const float xk[4] = {dka[db][4 * a], dka[db][4 * a + 1], dka[db][4 * a + 2], dka[db][4 * a + 3]};
      const float xv[4] = {dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2], dva[db][4 * a + 3]};
      store4(dkp, xk, trow, d0, p.scale);
      store4(dvp, xv, nullptr, d0, 1.0f);
    }
}

// ---------------------------------------------------------------------------
// Pre-pass and fp32 debug kernels
// ---------------------------------------------------------------------------

// -lse * log2(e) and -rowsum(dO * O) per (sequence, head, row), rows padded to ntile*64 with
// (-inf, 0); stored negated because both enter the products as accumulator inputs.
template <bool BF16>
__global__ __launch_bounds__(NT) void bwd_pre_kernel(const void* o, const void* dout, const float* __restrict__ lse,
                                                     float* __restrict__ lse2, float* __restrict__ dsum, int nseq,
                                                     int n, int64_t seq_stride, int H, int npad) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= (int64_t)nseq * H * npad) return;
  const int r = (int)(i % npad);
  const int h = (int)((i / npad) % H);
  const int sq = (int)(i / ((int64_t)npad * H));
  if (r >= n) {
    lse2[i] = -INFINITY;
    dsum[i] = 0.0f;
    return;
  }
  const int64_t tok = (int64_t)sq * seq_stride + r;
  const int64_t off = (tok * H + h) * D;
  float acc = 0.0f;
  if (BF16) {
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      const u32x4 a = *(const u32x4*)((const uint16_t*)o + off + c);
      const u32x4 b = *(const u32x4*)((const uint16_t*)dout + off + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(lo_bf16(a[e]), lo_bf16(b[e]), acc);
        acc = __builtin_fmaf(hi_bf16(a[e]), hi_bf16(b[e]), acc);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const f32x4 a = *(const f32x4*)((const float*)o + off + c);
      const f32x4 b = *(const f32x4*)((const float*)dout + off + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
    }
  }
  lse2[i] = -lse[tok * H + h] * kLog2e;
  dsum[i] = -acc;
}

// fp32: one thread per (sequence, row, head).  DQ: row = query, loop over keys;
// otherwise row = key, loop over queries.  Gradients stay in the rotated frame.
template <bool DQ>
__global__ __launch_bounds__(NT) void attn_bwd_f32_kernel(const float* __restrict__ qr, const float* __restrict__ kr,
                                                          const float* __restrict__ v, const float* __restrict__ dout,
                                                          const float* __restrict__ lse2,
                                                          const float* __restrict__ dsum, float* __restrict__ g0,
                                                          float* __restrict__ g1, int nseq, int n, int64_t seq_stride,
                                                          int H, int npad, float c, float scale) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= (int64_t)nseq * n * H) return;
  const int h = (int)(i % H);
  const int r = (int)((i / H) % n);
  const int sq = (int)(i / ((int64_t)H * n));
  const int64_t tok0 = (int64_t)sq * seq_stride;
  const int64_t sb = ((int64_t)sq * H + h) * npad;
  const int64_t rs = (int64_t)H * D;
  const float* own_a = (DQ ? qr : kr) + (tok0 + r) * rs + h * D;  // q_i or k_j
  const float* own_b = (DQ ? dout : v) + (tok0 + r) * rs + h * D;  // dO_i or v_j
  float a[D], b[D], x[D], y[D];
  for (int d = 0; d < D; ++d) {
    a[d] = own_a[d];
    b[d] = own_b[d];
    x[d] = 0.0f;
    y[d] = 0.0f;
  }
  for (int m = 0; m < n; ++m) {
    const float* oa = (DQ ? kr : qr) + (tok0 + m) * rs + h * D;    // k_j or q_i
    const float* ob = (DQ ? v : dout) + (tok0 + m) * rs + h * D;   // v_j or dO_i
    const int qrow = DQ ? r : m;
    float sdot = 0.0f, pdot = 0.0f;
    for (int d = 0; d < D; ++d) {
      sdot = __builtin_fmaf(a[d], oa[d], sdot);
      pdot = __builtin_fmaf(b[d], ob[d], pdot);
    }
    const float pr = __builtin_amdgcn_exp2f(sdot * c + lse2[sb + qrow]);  // lse2, dsum hold the negated values
    const float ds = pr * (pdot + dsum[sb + qrow]);
    for (int d = 0; d < D; ++d) {
      x[d] = __builtin_fmaf(ds, oa[d], x[d]);        // dq += ds k_j  |  dk += ds q_i
      if (!DQ) y[d] = __builtin_fmaf(pr, ob[d], y[d]);  // dv += p dO_i
    }
  }
  float* out0 = g0 + (tok0 + r) * rs + h * D;
  for (int d = 0; d < D; ++d) out0[d] = x[d] * scale;
  if (!DQ) {
    float* out1 = g1 + (tok0 + r) * rs + h * D;
    for (int d = 0; d < D; ++d) out1[d] = y[d];
  }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnBwdProblem& p, bool dq, hipStream_t stream) {
  const int64_t nwg = (int64_t)((p.n + BWG - 1) / BWG) * p.H * p.nseq;
  if (nwg <= 0) return hipSuccess;
  if (dq)
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)nwg), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)nwg), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_pre(const void* o, const void* dout, bool bf16, const float* lse, float* lse2,
                               float* dsum, int nseq, int n, int64_t seq_stride, int H, int ntile,
                               hipStream_t stream) {
  const int64_t total = (int64_t)nseq * H * ntile * 64;
  if (total <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + NT - 1) / NT);
  if (bf16)
    hipLaunchKernelGGL(bwd_pre_kernel<true>, dim3(blocks), dim3(NT), 0, stream, o, dout, lse, lse2, dsum, nseq, n,
                       seq_stride, H, ntile * 64);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<false>, dim3(blocks), dim3(NT), 0, stream, o, dout, lse, lse2, dsum, nseq, n,
                       seq_stride, H, ntile * 64);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float* qr, const float* kr, const float* v, const float* dout,
                               const float* lse2, const float* dsum, float* dqr, float* dkr, float* dv, int nseq,
                               int n, int64_t seq_stride, int H, int ntile, float scale_log2, float scale,
                               hipStream_t stream) {
  const int64_t total = (int64_t)nseq * n * H;
  if (total <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + NT - 1) / NT);
  hipLaunchKernelGGL(attn_bwd_f32_kernel<true>, dim3(blocks), dim3(NT), 0, stream, qr, kr, v, dout, lse2, dsum, dqr,
                     (float*)nullptr, nseq, n, seq_stride, H, ntile * 64, scale_log2, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_f32_kernel<false>, dim3(blocks), dim3(NT), 0, stream, qr, kr, v, dout, lse2, dsum, dkr,
                     dv, nseq, n, seq_stride, H, ntile * 64, scale_log2, scale);
  return hipGetLastError();
}

}  // namespace vggt
