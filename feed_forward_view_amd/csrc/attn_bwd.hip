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
//   attn_bwd_dq_kernel    one wave per 32 queries (two 16-query blocks), keys
//                         streamed in 64-key tiles (K rows, V rows) through
//                         LDS:
//                           S^T  = K Q^T - lse2      (accumulator input -lse2)
//                           dP^T = V dO^T - D        (accumulator input -D)
//                           dS^T = 2^(S^T) * dP^T
//                           dQ^T += K^T dS^T
//   attn_bwd_dkdv_kernel  one wave per 32 keys (two 16-key blocks), queries
//                         streamed in 64-query tiles (Q rows, dO rows, lse2,
//                         D):
//                           S  = Q K^T - lse2,  dP = dO V^T - D
//                           dV^T += dO^T P,      dK^T += Q^T dS
// Both use v_mfma_f32_16x16x32_bf16 with the layout of the forward kernel:
// the accumulator registers of two 16-row score blocks are, in order, the
// bf16 B operand of the next product for their 32-row chunk.  The A operands
// of those products (K^T, dO^T, Q^T) are read from the row tiles in LDS with
// transposing reads (ds_read_b64_tr_b16) that deliver each chunk's rows in
// that operand order, so no transposed copy is made in memory.  (Under
// sustained load this shape keeps a higher clock than 32x32x16 at the same
// work.)  The query operand of the scores carries scale*log2(e) and is
// rounded exactly as in the forward kernel, so the recomputed probabilities
// match the saved log-normaliser.  Rows past the end are zero in every tile
// and their -lse2 is -inf, so they contribute nothing; keys past the end are
// masked in the dQ kernel's last tile.
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
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Workgroup barrier for the tile ring.  __syncthreads() would make the compiler drain every
// outstanding copy first, including the next tile's, which was issued just before; the
// explicit counter waits already cover the copies each barrier needs.  The empty asm keeps
// LDS reads from being moved or merged across it (the copies write LDS unseen).
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

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
  u32x4 k[3][64][8];   // K rows (also read transposed: the A operand of dQ^T += K^T dS^T)
  u32x4 v[3][64][8];   // V rows
};

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(AttnBwdProblem p) {
  __shared__ SmemDq sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
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
  const int64_t sbase = ((int64_t)seq * p.H + head) * p.ntile * 64;

  auto issue = [&](int stage, int tile) {
    const int64_t off = (int64_t)tile * 512 + wave * 128 + lane;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = (2 * wave + c) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(kg + off + 64 * c), (lds_void*)&sm.k[stage][row][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vg + off + 64 * c), (lds_void*)&sm.v[stage][row][0], 16, 0, 0);
    }
  };
  issue(0, 0);

  // the wave's 32 queries as two 16-query blocks: this lane holds query 16qb + l16 of the
  // wave, channels 32dc + 8g .. +7 of its rotated and scaled Q and of its dO
  const int qw = qt * BWG + wave * BW;
  bf16x8 qf[2][2], df[2][2];
  f32x4 nl[2], nd[2];
  const f32x2* trow[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 16 * qb + l16;
    const bool ok = qi < p.n;
    const int64_t tok = tok0 + (ok ? qi : 0);
    trow[qb] = p.rope_tab ? p.rope_tab + (int)(tok % p.rope_T) * 32 : nullptr;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const int d0 = 32 * dc + 8 * g;
      u32x4 w = *(const u32x4*)((const uint16_t*)p.q + tok * p.tok_stride + head * D + d0);
      u32x4 gr = *(const u32x4*)((const uint16_t*)p.dout + tok * p.tok_stride + head * D + d0);
      if (!ok) w = gr = u32x4{0u, 0u, 0u, 0u};
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = lo_bf16(w[e]), y = hi_bf16(w[e]);
        if (trow[qb]) {
          const f32x2 cs = trow[qb][(d0 >> 1) + e];
          const float x2 = __builtin_fmaf(x, cs[0], -y * cs[1]);
          const float y2 = __builtin_fmaf(x, cs[1], y * cs[0]);
          x = x2;
          y = y2;
        }
        r[e] = pack_bf16x2(x * p.scale_log2, y * p.scale_log2);
      }
      qf[qb][dc] = as_bf16x8(r);
      df[qb][dc] = as_bf16x8(gr);
    }
    const float l2 = ok ? p.lse2[sbase + qi] : -INFINITY, ds = ok ? p.dsum[sbase + qi] : 0.0f;
    nl[qb] = f32x4{l2, l2, l2, l2};
    nd[qb] = f32x4{ds, ds, ds, ds};
  }

  f32x4 acc[2][4];  // dQ^T [qb][db]: channels 16db + 4g + r of the lane's query
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Three-slot ring, one barrier per tile.  Tile t+2 is issued in the middle of tile t, after the
  // barrier that shows tile t+1 landed in every wave; its slot held tile t-1, whose reads every
  // wave completed in tile t-1.  The K and V fragments of tile t+1 are read at that point too,
  // into the registers tile t's fragments leave free after its last S/dP product.
  bf16x8 kf[4][2], vf[4][2];
  auto read_kv = [&](int stage) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = 16 * kb + l16;
#pragma unroll
      for (int dc = 0; dc < 2; ++dc) {
        const int slot = (4 * dc + g) ^ row_swz(row);
        kf[kb][dc] = as_bf16x8(sm.k[stage][row][slot]);
        vf[kb][dc] = as_bf16x8(sm.v[stage][row][slot]);
      }
    }
  };
  issue(1, min(1, p.ntile - 1));
  wait_vmcnt<4>();  // tile 0 has landed (tile 1 may still be in flight) ...
  tile_barrier();   // ... in every wave's copies
  read_kv(0);
  int stage = 0;  // ring slot of tile t
  for (int t = 0; t < p.ntile; ++t) {
    const int next = stage == 2 ? 0 : stage + 1;
    bf16x8 ktf[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < 4; ++db) ktf[c][db] = read_tr_rows(sm.k[stage], c, db, lane);
    const bool tail = t == p.ntile - 1 && 64 * p.ntile > p.n;
    // S^T and dP^T of a query block (lane holds keys 16kb + 4g + r of its query), and
    // dS^T = P dP^T as the bf16 B operand of dQ^T += K^T dS^T for 32-key chunk c.  The tile is
    // four phases, so that each block's exponentials, products and packs run beside the
    // other block's independent MFMAs:  S,dP(0) | S,dP(1) + dS(0) | dQ(0) + dS(1) | dQ(1)
    f32x4 s[2][4], dp[2][4];
    auto sdp = [&](int qb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[qb][kb] = mfma16(kf[kb][0], qf[qb][0], nl[qb]);
        dp[qb][kb] = mfma16(vf[kb][0], df[qb][0], nd[qb]);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[qb][kb] = mfma16(kf[kb][1], qf[qb][1], s[qb][kb]);
        dp[qb][kb] = mfma16(vf[kb][1], df[qb][1], dp[qb][kb]);
      }
    };
    auto mask = [&](int qb) {
      if (tail) {
        // keys past the end are zero rows, so their score would be the bare
        // -lse2, whose exponential overflows when the row's log-normaliser lies
        // far below zero (and then meets the zero K^T row as inf * 0)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (64 * t + 16 * kb + 4 * g + r >= p.n) s[qb][kb][r] = -INFINITY;
      }
    };
    auto dsw = [&](int qb, int c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = 2 * c + (e >> 1), r = 2 * (e & 1);
        w[e] = pack_bf16x2(__builtin_amdgcn_exp2f(s[qb][kb][r]) * dp[qb][kb][r],
                           __builtin_amdgcn_exp2f(s[qb][kb][r + 1]) * dp[qb][kb][r + 1]);
      }
      return w;
    };
    auto dq = [&](int qb, const u32x4 (&w)[2]) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[qb][db] = mfma16(ktf[c][db], as_bf16x8(w[c]), acc[qb][db]);
    };
    u32x4 w0[2], w1[2];
    sdp(0);
    mask(0);
    __builtin_amdgcn_sched_barrier(0);
    sdp(1);
    w0[0] = dsw(0, 0);
    w0[1] = dsw(0, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);  // exponential
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // other VALU
    }
    // the phase's weights are complete here: without this use the compiler sinks their
    // exponentials and packs past the phase boundary, next to their first use in the next
    // phase, and the hints above find no VALU work to place beside the MFMAs
    asm volatile("" ::"v"(w0[0]), "v"(w0[1]));
    __builtin_amdgcn_sched_barrier(0);
    {
      // past the last tile the copies repeat the last tile into free slots and the
      // fragments read from them go unused, so the loop body has no branch here
      wait_vmcnt<0>();  // tile t+1 has landed in this wave's copies ...
      // the K^T reads of tile t have returned long ago; a counted wait the compiler sees lets
      // the dQ products below go without waiting for the K and V reads issued next
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      tile_barrier();   // ... and in every wave's; every wave is done with tile t-1's slot
      issue(next == 2 ? 0 : next + 1, min(t + 2, p.ntile - 1));
      read_kv(next);
    }
    __builtin_amdgcn_sched_barrier(0);
    mask(1);
    dq(0, w0);
    w1[0] = dsw(1, 0);
    w1[1] = dsw(1, 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    asm volatile("" ::"v"(w1[0]), "v"(w1[1]));
    __builtin_amdgcn_sched_barrier(0);
    dq(1, w1);
    stage = next;
  }
  wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup ends
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 16 * qb + l16;
    if (qi >= p.n) continue;
    uint16_t* dst = (uint16_t*)p.dq + (tok0 + qi) * p.tok_stride + head * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const float x[4] = {acc[qb][db][0], acc[qb][db][1], acc[qb][db][2], acc[qb][db][3]};
      store4(dst, x, trow[qb], 16 * db + 4 * g, p.scale);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

struct SmemDkv {
  u32x4 q[2][64][8];   // Q rows, scaled (also read transposed: dK^T += Q^T dS)
  u32x4 d[2][64][8];   // dO rows (also read transposed: dV^T += dO^T P)
  float st[2][2][64];  // lse2, D of the tile's 64 queries
};

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(AttnBwdProblem p) {
  __shared__ SmemDkv sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
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
  const int64_t sbase = ((int64_t)seq * p.H + head) * p.ntile * 64;

  auto issue = [&](int stage, int tile) {
    const int64_t off = (int64_t)tile * 512 + wave * 128 + lane;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = (2 * wave + c) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(qg + off + 64 * c), (lds_void*)&sm.q[stage][row][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(dg + off + 64 * c), (lds_void*)&sm.d[stage][row][0], 16, 0, 0);
    }
    // 512 bytes of statistics: waves 0-1 bring lse2, waves 2-3 bring D (8 lanes x 16 bytes each)
    if (lane < 8) {
      const float* src = (wave < 2 ? p.lse2 : p.dsum) + sbase + (int64_t)tile * 64 + 32 * (wave & 1) + 4 * lane;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)&sm.st[stage][wave >> 1][32 * (wave & 1)], 16, 0,
                                       0);
    }
  };
  issue(0, 0);

  // the wave's 32 keys as two 16-key blocks: this lane holds key 16kb + l16 of the wave,
  // channels 32dc + 8g .. +7 of its rotated K and of its V (B operands of S = Q K^T and
  // dP = dO V^T)
  const int kw = kt * BWG + wave * BW;
  bf16x8 kf[2][2], vf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kj = kw + 16 * kb + l16;
    const bool ok = kj < p.n;
    const int64_t tok = tok0 + (ok ? kj : 0);
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const int d0 = 32 * dc + 8 * g;
      u32x4 a = *(const u32x4*)((const uint16_t*)p.kr + tok * p.tok_stride + head * D + d0);
      u32x4 b = *(const u32x4*)((const uint16_t*)p.v + tok * p.tok_stride + head * D + d0);
      if (!ok) a = b = u32x4{0u, 0u, 0u, 0u};
      kf[kb][dc] = as_bf16x8(a);
      vf[kb][dc] = as_bf16x8(b);
    }
  }

  f32x4 dka[2][4], dva[2][4];  // dK^T, dV^T [kb][db]: channels 16db + 4g + r of the lane's key
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) dka[kb][db] = dva[kb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int t = 0; t < p.ntile; ++t) {
    const int stage = t & 1;
    if (t + 1 < p.ntile) {
      tile_barrier();  // every wave is done with the stage tile t+1 goes to
      issue(stage ^ 1, t + 1);
      wait_vmcnt<5>();  // tile t has landed (tile t+1 may still be in flight)
    } else {
      wait_vmcnt<0>();
    }
    tile_barrier();  // ... in every wave's copies
    // The tile's 64 queries are two 32-query chunks c, each two 16-query blocks.  Four
    // phases, so that each chunk's exponentials, products and packs run beside the other
    // chunk's independent MFMAs:  S,dP(0) | S,dP(1) + P,dS(0) | dV,dK(0) + P,dS(1) | dV,dK(1).
    // Each phase reads the LDS operands of the next one.
    struct RowOps {
      bf16x8 qr[2][2], dr[2][2];  // [block i][dc]: Q and dO rows of the chunk's blocks
      f32x4 nl[2], nd[2];         // -lse2 and -D of the register's queries
    };
    auto read_rows = [&](int c, RowOps& r) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int qb = 2 * c + i, row = 16 * qb + l16;
        r.nl[i] = *(const f32x4*)&sm.st[stage][0][16 * qb + 4 * g];
        r.nd[i] = *(const f32x4*)&sm.st[stage][1][16 * qb + 4 * g];
#pragma unroll
        for (int dc = 0; dc < 2; ++dc) {
          const int slot = (4 * dc + g) ^ row_swz(row);
          r.qr[i][dc] = as_bf16x8(sm.q[stage][row][slot]);
          r.dr[i][dc] = as_bf16x8(sm.d[stage][row][slot]);
        }
      }
    };
    // dO^T and Q^T of chunk c: the A operands of dV^T += dO^T P and dK^T += Q^T dS
    auto read_tr = [&](int c, bf16x8 (&dtf)[4], bf16x8 (&qtf)[4]) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dtf[db] = read_tr_rows(sm.d[stage], c, db, lane);
        qtf[db] = read_tr_rows(sm.q[stage], c, db, lane);
      }
    };
    // S and dP of the chunk's blocks: [block i][kb], queries 16(2c+i) + 4g + r, the lane's key
    auto sdp = [&](const RowOps& r, f32x4 (&sc)[2][2], f32x4 (&dpc)[2][2]) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sc[i][kb] = mfma16(r.qr[i][0], kf[kb][0], r.nl[i]);
          dpc[i][kb] = mfma16(r.dr[i][0], vf[kb][0], r.nd[i]);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sc[i][kb] = mfma16(r.qr[i][1], kf[kb][1], sc[i][kb]);
          dpc[i][kb] = mfma16(r.dr[i][1], vf[kb][1], dpc[i][kb]);
        }
    };
    // P and dS = P dP as the bf16 B operands (the chunk's queries in operand order)
    auto pds = [&](const f32x4 (&sc)[2][2], const f32x4 (&dpc)[2][2], u32x4 (&pw)[2], u32x4 (&sw)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = e >> 1, r = 2 * (e & 1);
          const float p0 = __builtin_amdgcn_exp2f(sc[i][kb][r]), p1 = __builtin_amdgcn_exp2f(sc[i][kb][r + 1]);
          pw[kb][e] = pack_bf16x2(p0, p1);
          sw[kb][e] = pack_bf16x2(p0 * dpc[i][kb][r], p1 * dpc[i][kb][r + 1]);
        }
    };
    auto dvdk = [&](const bf16x8 (&dtf)[4], const bf16x8 (&qtf)[4], const u32x4 (&pw)[2], const u32x4 (&sw)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dva[kb][db] = mfma16(dtf[db], as_bf16x8(pw[kb]), dva[kb][db]);
          dka[kb][db] = mfma16(qtf[db], as_bf16x8(sw[kb]), dka[kb][db]);
        }
    };
    RowOps r0, r1;
    f32x4 s0[2][2], dp0[2][2], s1[2][2], dp1[2][2];
    bf16x8 dtf0[4], qtf0[4], dtf1[4], qtf1[4];
    u32x4 pw0[2], sw0[2], pw1[2], sw1[2];
    read_rows(0, r0);
    sdp(r0, s0, dp0);
    read_rows(1, r1);
    __builtin_amdgcn_sched_barrier(0);
    read_tr(0, dtf0, qtf0);
    sdp(r1, s1, dp1);
    pds(s0, dp0, pw0, sw0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);  // exponential
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // other VALU
    }
    // the phase's weights are complete here: without this use the compiler sinks their
    // exponentials and packs next to their first use in the next phase
    asm volatile("" ::"v"(pw0[0]), "v"(pw0[1]), "v"(sw0[0]), "v"(sw0[1]));
    __builtin_amdgcn_sched_barrier(0);
    read_tr(1, dtf1, qtf1);
    dvdk(dtf0, qtf0, pw0, sw0);
    pds(s1, dp1, pw1, sw1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    asm volatile("" ::"v"(pw1[0]), "v"(pw1[1]), "v"(sw1[0]), "v"(sw1[1]));
    __builtin_amdgcn_sched_barrier(0);
    dvdk(dtf1, qtf1, pw1, sw1);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kj = kw + 16 * kb + l16;
    if (kj >= p.n) continue;
    const int64_t tok = tok0 + kj;
    const f32x2* trow = p.rope_tab ? p.rope_tab + (int)(tok % p.rope_T) * 32 : nullptr;
    uint16_t* dkp = (uint16_t*)p.dk + tok * p.tok_stride + head * D;
    uint16_t* dvp = (uint16_t*)p.dv + tok * p.tok_stride + head * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d0 = 16 * db + 4 * g;
      const float xk[4] = {dka[kb][db][0], dka[kb][db][1], dka[kb][db][2], dka[kb][db][3]};
      const float xv[4] = {dva[kb][db][0], dva[kb][db][1], dva[kb][db][2], dva[kb][db][3]};
      store4(dkp, xk, trow, d0, p.scale / p.scale_log2);  // the Q rows carry scale * log2(e)
      store4(dvp, xv, nullptr, d0, 1.0f);
    }
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
