// Flash attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// Computes softmax(scale * Q K^T) V per head (the "VGGT 論文報告" slide deck,
// Section V, slides 5/10-9/10) without ever forming the score matrix: keys
// stream through LDS in tiles of 64 and each query row keeps a running sum
// against a reference offset, so a row costs O(1) memory for any key count.
//
// Work split.  A workgroup of 4 waves (one per SIMD) owns 256 queries of one
// head; each wave owns 64 of them as four 16-query MFMA column blocks (qb),
// taken as two halves of 32.  Per 64-key tile and half:
//   S^T = K Q^T - m   16 x v_mfma_f32_16x16x32_bf16 (4 key blocks of 16 x 2
//                     channel halves x 2 query blocks); keys are the M
//                     dimension, so lane l holds 4 scores (keys 16kb + 4(l/16)
//                     + 0..3) of query l % 16, and the row reference m enters
//                     through the accumulator input;
//   P = 2^(S^T)       one v_exp_f32 per score, rounded to bf16 in pairs; the
//                     row sum adds the rounded pairs with v_dot2_f32_bf16, so
//                     it uses exactly the weights of the P V product;
//   O^T += V^T P^T    16 x v_mfma_f32_16x16x32_bf16 (4 channel blocks x 2
//                     32-key chunks x 2 query blocks); head dim is M and the
//                     lane again holds one query, so per-row scaling stays
//                     in-lane.
// Q is rotated (2D RoPE, fp32, from the per-position cos/sin table) and
// multiplied by scale*log2(e) once in the prologue, so scores come out in log2
// units.  The score registers of key blocks 2c and 2c+1 are, in order, the
// bf16 B operand of the P V product for 32-key chunk c: that operand's key
// index 8g + i stands for key 4g + i (i < 4) or 16 + 4g + i - 4 of the chunk,
// and the V^T tiles store their keys in that order.
//
// Why 16x16x32: under sustained load this chip holds its clock with the
// 16x16x32 shape where the 32x32x16 shape runs into the power limit (same
// cycles per tile, measured ~8 % more clock at this kernel's MFMA density).
//
// Overlap.  While an MFMA runs, plain VALU work (fma, add, cvt) hides almost
// completely, from the same wave or the other wave on the SIMD; v_exp_f32 (8
// clocks per wave instruction) hides about half behind the wave's own MFMAs
// and fully behind the other wave's; v_dot2_f32_bf16 never overlaps an MFMA.
// The loop therefore keeps VALU work per tile to one exp per score and one cvt
// and one dot2 per score pair, and interleaves each half's exponentials with
// the other half's MFMAs.
//
// Softmax reference.  m starts at 0 and stays there while a row's scores stay
// within 2^32 of it.  The first tile, and any tile whose partial row sum
// leaves [0, 2^64], takes a slow path that computes the tile maximum, moves m
// (rescaling O and the running sum exactly by 2^(m_old - m_new), except on
// the first tile, where both are still zero) and redoes the tile; from then on
// the wave subtracts m before the exponential.  The final O / l is the same
// softmax whatever m is.
//
// Operands.  A pre-pass lays K (rotated when RoPE is on) and V^T out in
// tiles of 64 keys, each tile 8 KiB in exactly the order the LDS tile uses
// (K rows in key order, V^T rows holding each 32-key chunk in the operand
// order above, 16-byte units XOR-swizzled per row so that the 16 lanes of an
// operand read hit distinct banks; keys past the end are zero).  Tiles are
// then copied linearly into a 4-stage LDS ring with global_load_lds_dwordx4,
// three tiles ahead of use; one barrier per tile.  The last (partial) tile of
// a key range is peeled out of the loop and its missing keys are masked to
// -inf.
//
// Workgroup order is XCD-aware: the hardware deals workgroups round-robin to
// the 8 XCDs, so the linear id is remapped to give each XCD a contiguous run
// of (query tile, head) work; the workgroups resident on one XCD then stream
// the same head's keys and values through that XCD's L2.
#include <type_traits>

#include "common.h"

namespace vggt {
namespace {

constexpr int D = kHeadDim;
constexpr int BK = kAttnKeyTile;  // 64 keys per tile
constexpr int NW = 4;             // waves per workgroup
#ifndef VGGT_ATTN_NSTAGE
#define VGGT_ATTN_NSTAGE 4
#endif
#ifndef VGGT_ATTN_WPE
#define VGGT_ATTN_WPE 2
#endif
constexpr int NT = NW * 64;
constexpr int QW = 64;            // queries per wave: four 16-query MFMA column blocks
constexpr int BQ = NW * QW;       // queries per workgroup
constexpr int NSTAGE = VGGT_ATTN_NSTAGE;  // LDS ring depth (tiles in flight = NSTAGE - 1)
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64
constexpr float kRaise = 32.0f;   // move m when a tile max exceeds it by this
constexpr float kLow = -64.0f;    // first tile: move m down when the max is below this
constexpr float kLn2 = 0.693147180559945309f;

typedef __attribute__((address_space(3))) void lds_void;

// K tile:   row r holds key r of the tile, 8 units of 8 dims; unit u at slot u ^ row_swz(r).
// V^T tile: row d holds channel d of the 64 keys; unit u holds operand keys 8(u%4)..+7 of
//           32-key chunk u/4 (see the header for their key order), at slot u ^ col_swz(d).
struct Smem {
  u32x4 k[NSTAGE][BK][8];
  u32x4 vt[NSTAGE][D][8];
};

__device__ __forceinline__ float dot2_acc(uint32_t pk, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// interleave hint for the scheduler: n x (1 MFMA, v VALU)
#ifndef VGGT_IL_N
#define VGGT_IL_N 16
#endif
#ifndef VGGT_IL_V
#define VGGT_IL_V 6
#endif
#define VGGT_INTERLEAVE(n, v)                                  \
  _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {         \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x002, (v), 0);       \
  }

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(VGGT_ATTN_WPE, VGGT_ATTN_WPE)))
void attn_fwd_bf16_kernel(AttnProblem p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;  // query within a 16-query block
  const int g = lane >> 4;    // which 4 keys (S^T) / 8 channels (operands) of a block

  // ---- which (query tile, head, sequence, split) this workgroup owns
  const int ntq = (p.nq + BQ - 1) / BQ;
  const int nwg = ntq * p.H * p.nseq * p.splits;
  int logical;
  xcd_remap(blockIdx.x, nwg, logical);
  const int qt = logical % ntq;
  int rest = logical / ntq;
  int head, split, seq;
  if (p.nk_step > 0) {
    // growing key prefixes: each XCD's contiguous range holds whole heads, and
    // within a head the longest sequences come first (balanced XCDs, long
    // workgroups dispatched early)
    seq = p.nseq - 1 - rest % p.nseq;
    rest /= p.nseq;
    split = rest % p.splits;
    head = rest / p.splits;
  } else {
    head = rest % p.H;
    rest /= p.H;
    split = rest % p.splits;
    seq = rest / p.splits;
  }
  const int nq_seq = (int)min((int64_t)p.nq, p.nq_total - (int64_t)seq * p.nq);
  const int nk_seq = p.nk_step > 0 ? (int)min((int64_t)p.nk, (int64_t)(seq + 1) * p.nk_step) : p.nk;

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + (seq * p.q_seq_stride) * p.tok_stride + head * D;
  // K and V^T tiles of this (sequence, head): 512 16-byte units per tile
  const int64_t kseq = p.k_seq_stride != 0 ? seq : 0;
  const u32x4* __restrict__ ktg = (const u32x4*)p.k + (kseq * p.H + head) * p.ktiles_seq * 512;
  const u32x4* __restrict__ vtg = (const u32x4*)p.vt + (kseq * p.H + head) * p.ktiles_seq * 512;

  const int kbeg = split * p.keys_per_split;
  const int kend = min(nk_seq, kbeg + p.keys_per_split);
  const int ntiles = (kend - kbeg + BK - 1) / BK;

  const int q0 = qt * BQ + wave * QW;  // first query of this wave
  const bool active = q0 < nq_seq;

  // ---- tile loads: each wave copies two 1 KiB blocks of the K tile and two of the V^T tile
  const int ktile0 = kbeg / BK;
  auto issue = [&](int stage, int tile) {
    const u32x4* ks = ktg + (int64_t)(ktile0 + tile) * 512 + wave * 128 + lane;
    const u32x4* vs = vtg + (int64_t)(ktile0 + tile) * 512 + wave * 128 + lane;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      __builtin_amdgcn_global_load_lds((const void*)(ks + 64 * c), (lds_void*)&sm.k[stage][(2 * wave + c) * 8][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vs + 64 * c), (lds_void*)&sm.vt[stage][(2 * wave + c) * 8][0], 16, 0, 0);
    }
  };

#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles) issue(i, i);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query q0 + 16qb + l16,
  //      channels 32dc + 8g .. +7 (the other 48 sit in the lanes of the same l16),
  //      after an optional per-head LayerNorm, rotated and scaled by scale*log2(e).
  bf16x8 qf[4][2];
  {
    const f32x2* __restrict__ tab = p.rope_tab;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int qi = q0 + 16 * qb + l16;
      const bool ok = qi < nq_seq;
      const int qrow = ok ? qi : 0;
      const int tpos = tab ? (int)((seq * p.q_seq_stride + qrow) % p.rope_T) : 0;
      const f32x2* trow = tab ? tab + tpos * 32 : nullptr;
      float x[2][4], y[2][4];  // [dc][pair]: channels 32dc + 8g + 2e, +1
#pragma unroll
      for (int dc = 0; dc < 2; ++dc) {
        u32x4 w = *(const u32x4*)(qg + (int64_t)qrow * p.tok_stride + 32 * dc + 8 * g);
        if (!ok) w = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[dc][e] = lo_bf16(w[e]);
          y[dc][e] = hi_bf16(w[e]);
        }
      }
      if (p.q_ln_g) {
        float sum = 0.0f;
#pragma unroll
        for (int dc = 0; dc < 2; ++dc)
#pragma unroll
          for (int e = 0; e < 4; ++e) sum += x[dc][e] + y[dc][e];
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        const float mu = sum * (1.0f / D);
        float dev = 0.0f;
#pragma unroll
        for (int dc = 0; dc < 2; ++dc)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dev = __builtin_fmaf(x[dc][e] - mu, x[dc][e] - mu, dev);
            dev = __builtin_fmaf(y[dc][e] - mu, y[dc][e] - mu, dev);
          }
        dev += __shfl_xor(dev, 16);
        dev += __shfl_xor(dev, 32);
        const float inv = 1.0f / __builtin_sqrtf(dev * (1.0f / D) + p.ln_eps);
#pragma unroll
        for (int dc = 0; dc < 2; ++dc)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = 32 * dc + 8 * g + 2 * e;
            x[dc][e] = __builtin_fmaf((x[dc][e] - mu) * inv, p.q_ln_g[c], p.q_ln_b[c]);
            y[dc][e] = __builtin_fmaf((y[dc][e] - mu) * inv, p.q_ln_g[c + 1], p.q_ln_b[c + 1]);
          }
      }
#pragma unroll
      for (int dc = 0; dc < 2; ++dc) {
        if (trow) {
          // rotation pairs 16dc + 4g + e of the 32 of this position
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x2 cs = trow[16 * dc + 4 * g + e];
            const float x2 = __builtin_fmaf(x[dc][e], cs[0], -y[dc][e] * cs[1]);
            const float y2 = __builtin_fmaf(x[dc][e], cs[1], y[dc][e] * cs[0]);
            x[dc][e] = x2;
            y[dc][e] = y2;
          }
        }
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(x[dc][e] * p.scale_log2, y[dc][e] * p.scale_log2);
        qf[qb][dc] = __builtin_bit_cast(bf16x8, r);
      }
    }
  }

  // ---- running state
  f32x4 o[4][4];  // [qb][db]: O^T rows 16db + 4g + r, column = the lane's query of block qb
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float mref[4], lsum[4];  // reference (log2 units) and this lane's partial row sums
  f32x4 negm[4];           // -m of the lane's query, replicated: accumulator input of S^T
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    mref[qb] = lsum[qb] = 0.0f;
    negm[qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  f32x4 s0[2][4], s1[2][4];  // scores of query blocks (0, 1) and (2, 3): [block][kb], keys 16kb + 4g + r
  u32x4 p0[2][2], p1[2][2];  // [block][chunk]: bf16 pairs, B operand of P V
  bf16x8 kf[4][2];           // K fragments of the tile [kb][dc]
  bf16x8 vf[2][4];           // V^T fragments [chunk][db]

  auto read_k = [&](int stage) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = 16 * kb + l16;
#pragma unroll
      for (int dc = 0; dc < 2; ++dc) {
        const int u = 4 * dc + g;
        kf[kb][dc] = __builtin_bit_cast(bf16x8, sm.k[stage][row][u ^ row_swz(row)]);
      }
    }
  };
  auto read_v = [&](int stage) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 16 * db + l16;
        const int u = 4 * c + g;
        vf[c][db] = __builtin_bit_cast(bf16x8, sm.vt[stage][d][u ^ col_swz(d)]);
      }
  };
  // S^T - m for query blocks 2h, 2h+1 (the reference enters as the accumulator input)
  auto qk = [&](f32x4 (&s)[2][4], int h) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[i][kb] = mfma(kf[kb][0], qf[2 * h + i][0], negm[2 * h + i]);
        s[i][kb] = mfma(kf[kb][1], qf[2 * h + i][1], s[i][kb]);
      }
  };
  auto pv = [&](const u32x4 (&pf)[2][2], int h) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[2 * h + i][db] = mfma(vf[c][db], __builtin_bit_cast(bf16x8, pf[i][c]), o[2 * h + i][db]);
  };
  // P = 2^(S - shift) of one query block as the bf16 B operand of P V (S already has m
  // subtracted, up to `shift`); returns this lane's partial row sum
  auto soft = [&](const f32x4 (&s)[4], bool sub, float shift, u32x4 (&pf)[2]) -> float {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4& sb = s[2 * c + (e >> 1)];
        float a = sb[2 * (e & 1)], b = sb[2 * (e & 1) + 1];
        if (sub) {
          a -= shift;
          b -= shift;
        }
        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(a), __builtin_amdgcn_exp2f(b));
        pf[c][e] = w;
        acc = dot2_acc(w, acc);
      }
    return acc;
  };
  // slow path of one query block: move the reference if needed and redo its exponentials
  auto slow = [&](const f32x4 (&s)[4], int qb, bool first, u32x4 (&pf)[2]) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // mx is relative to the current reference
    float delta = 0.0f;
    if (first) {
      if (mx < kLow || mx > kRaise) delta = mx;
    } else if (mx > kRaise) {
      delta = mx;
    }
    if (__any(delta != 0.0f)) {
      mref[qb] += delta;
      if (!first) {
        // before the first tile O and l are still zero: only the reference
        // moves (2^-delta overflows when the first tile moves it far down)
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
      }
      negm[qb] = f32x4{-mref[qb], -mref[qb], -mref[qb], -mref[qb]};
    }
    return soft(s, true, delta, pf);
  };
  auto mask = [&](f32x4 (&s)[2][4], int kt) {
    // lane/register -> key kt + 16kb + 4g + r
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt + 16 * kb + 4 * g + r >= kend) s[i][kb][r] = -INFINITY;
  };

  // wait until tile `tile` has landed in LDS (later tiles may still be in flight), then barrier
  auto land = [&](int tile) {
    const int ahead = min(NSTAGE - 2, ntiles - 1 - tile);  // tiles issued after `tile`
    if (ahead >= 2)
      wait_vmcnt<8>();
    else if (ahead == 1)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  };

  // One tile: S^T of query blocks 2-3 || exponentials of blocks 0-1, then P V of blocks 0-1 ||
  // exponentials of blocks 2-3.  FIRST: the reference is set by the slow path; LAST: keys past
  // the end are masked.
  auto tile_body = [&](int t, auto first_c, auto last_c) {
    constexpr bool first = decltype(first_c)::value;
    constexpr bool masked = decltype(last_c)::value;
    const int stage = t % NSTAGE;
    read_k(stage);
    qk(s0, 0);
    if constexpr (masked) mask(s0, kbeg + t * BK);
    qk(s1, 1);
    float a0 = soft(s0[0], false, 0.0f, p0[0]);
    float a1 = soft(s0[1], false, 0.0f, p0[1]);
    VGGT_INTERLEAVE(VGGT_IL_N, VGGT_IL_V);
    if constexpr (masked) mask(s1, kbeg + t * BK);
    if (first || __any(!(a0 <= kSumLimit) || !(a1 <= kSumLimit))) {
      a0 = slow(s0[0], 0, first, p0[0]);
      a1 = slow(s0[1], 1, first, p0[1]);
    }
    lsum[0] += a0;
    lsum[1] += a1;
    read_v(stage);
    pv(p0, 0);
    float b0 = soft(s1[0], false, 0.0f, p1[0]);
    float b1 = soft(s1[1], false, 0.0f, p1[1]);
    VGGT_INTERLEAVE(VGGT_IL_N, VGGT_IL_V);
    if (first || __any(!(b0 <= kSumLimit) || !(b1 <= kSumLimit))) {
      b0 = slow(s1[0], 2, first, p1[0]);
      b1 = slow(s1[1], 3, first, p1[1]);
    }
    lsum[2] += b0;
    lsum[3] += b1;
    pv(p1, 1);
  };
  using yes = std::true_type;
  using no = std::false_type;
  auto advance = [&](int t) {
    land(t);
    if (t + NSTAGE - 1 < ntiles) issue((t + NSTAGE - 1) % NSTAGE, t + NSTAGE - 1);
  };

  if (active) {
    if (ntiles == 1) {
      advance(0);
      tile_body(0, yes{}, yes{});
    } else {
      advance(0);
      tile_body(0, yes{}, no{});
      for (int t = 1; t + 1 < ntiles; ++t) {
        advance(t);
        tile_body(t, no{}, no{});
      }
      advance(ntiles - 1);
      tile_body(ntiles - 1, no{}, yes{});
    }
  } else {
    // keep the workgroup's barrier and load sequence
    for (int t = 0; t < ntiles; ++t) advance(t);
    return;
  }

  // ---- epilogue: the 4 lanes of a query (g = 0..3) hold its 64 channels, 16 each
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float ltot = lsum[qb] + __shfl_xor(lsum[qb], 16);
    ltot += __shfl_xor(ltot, 32);
    const int qi = q0 + 16 * qb + l16;
    if (qi >= nq_seq) continue;
    if (p.splits == 1) {
      const float inv = 1.0f / ltot;
      if (p.lse && g == 0) p.lse[(seq * p.q_seq_stride + qi) * p.H + head] = (mref[qb] + log2f(ltot)) * kLn2;
      uint16_t* og = (uint16_t*)p.o + (seq * p.q_seq_stride + qi) * p.tok_stride + head * D;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 w = {pack_bf16x2(o[qb][db][0] * inv, o[qb][db][1] * inv),
                         pack_bf16x2(o[qb][db][2] * inv, o[qb][db][3] * inv)};
        *(u32x2*)(og + 16 * db + 4 * g) = w;
      }
    } else {
      const int64_t row = ((int64_t)split * p.nq_total + (int64_t)seq * p.nq + qi) * p.H + head;
      float* po = p.part_o + row * D;
#pragma unroll
      for (int db = 0; db < 4; ++db) *(f32x4*)(po + 16 * db + 4 * g) = o[qb][db];
      if (g == 0) {
        const f32x2 ml = {mref[qb], ltot};
        *(f32x2*)(p.part_ml + row * 2) = ml;
      }
    }
  }
}

}  // namespace

int attn_bf16_query_tile() { return BQ; }

hipError_t launch_attn_bf16(const AttnProblem& p, hipStream_t stream) {
  const int ntq = (p.nq + BQ - 1) / BQ;
  const int64_t nwg = (int64_t)ntq * p.H * p.nseq * p.splits;
  if (nwg <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)nwg), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vggt
