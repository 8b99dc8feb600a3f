// Flash attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// Computes softmax(scale * Q K^T) V per head (the "VGGT 論文報告" slide deck,
// Section V, slides 5/10-9/10) without ever forming the score matrix: keys
// stream through LDS in tiles of 64 and each query row keeps a running sum
// against a reference offset, so a row costs O(1) memory for any key count.
//
// Work split.  A workgroup of 4 waves (one per SIMD) owns 256 queries of one
// head; each wave owns 64 of them as four 16-query MFMA column blocks (qb).
// Per 64-key tile and query block:
//   S^T = K Q^T       8 x v_mfma_f32_16x16x32_bf16 (4 key blocks of 16 x 2
//                     channel halves); keys are the M dimension, so lane l
//                     holds 4 scores (keys 16kb + 4(l/16) + 0..3) of query
//                     l % 16;
//   P = 2^(S^T - m)   one v_exp_f32 per score, rounded to bf16 in pairs;
//   O^T += V^T P^T    8 x v_mfma_f32_16x16x32_bf16 (4 channel blocks x 2
//                     32-key chunks); head dim is M and the lane again holds
//                     one query, so per-row scaling stays in-lane;
//   l += 1 P^T        2 x v_mfma_f32_16x16x32_bf16 with an all-ones A
//                     operand: the row sum uses exactly the bf16 weights of
//                     the P V product (a single key returns its V row
//                     bit-exactly), and every register of the result holds
//                     the lane's query's sum.
// Q is rotated (2D RoPE, fp32, from the per-position cos/sin table) and
// multiplied by scale*log2(e) once in the prologue, so scores come out in log2
// units.  The score registers of key blocks 2c and 2c+1 are, in order, the
// bf16 B operand of the P V product for 32-key chunk c: that operand's key
// index 8g + i stands for key 4g + i (i < 4) or 16 + 4g + i - 4 of the chunk,
// and the V^T operand must hold its keys in that order (see Operands).
//
// Why 16x16x32: under sustained load this chip holds its clock with the
// 16x16x32 shape where the 32x32x16 shape runs into the power limit.
//
// Issue costs that shape the loop (measured on gfx950).  Plain VALU work and
// v_exp_f32 hide behind a running MFMA as long as the SIMD's VALU issue
// budget lasts; with one exponential and half a conversion per score that
// budget is nearly used up.  v_dot2_f32_bf16 and its VOP3P form do not
// overlap MFMAs at all: a row sum in dot2 costs as much MFMA-pipe time as an
// MFMA per instruction, four times the ones x P product above.  The loop is
// software-pipelined over query blocks so that every block's exponentials run
// beside sixteen independent MFMAs (see the step schedule below).
//
// Softmax reference, optimistic.  The first pass keeps m = 0 for every row
// and checks nothing per tile.  At the end a row is accepted when its sum l
// lies in [2^-64, 2^100] and its un-normalised output is finite: then no
// weight or product overflowed and the largest weight is at least 2^-64 / N,
// far inside the normal range of bf16 and fp32, so the pass computed the same
// softmax as any other reference up to rounding.  If any row
// of the workgroup fails (logits in the hundreds, or rows whose scores all lie
// far below zero), the workgroup reruns its key range exactly: the first tile
// sets a per-row m, every block's largest score is checked against it, and a
// slow path moves m (rescaling O and l exactly by 2^(m_old - m_new)) and
// redoes the block.  The final O / l is the same softmax whatever m is.
//
// Operands.  A pre-pass lays K (rotated when RoPE is on) out in tiles of 64
// keys, each tile 8 KiB in exactly the order the LDS tile uses (rows in key
// order, 16-byte units XOR-swizzled per row so that the lanes of an operand
// read hit distinct banks; keys past the end are zero), and the tiles are
// copied linearly into a 4-stage LDS ring with global_load_lds_dwordx4, three
// tiles ahead of use; one barrier per tile.  V comes in one of two forms:
//   V^T tiles   a second pre-pass writes V^T tiles whose rows hold each 32-key
//               chunk in the operand order above; eight ds_read_b128 per tile
//               and wave read the operand;
//   V in place  the copies gather V rows straight from the [token][head][64]
//               tensor into a row tile laid out as the K tile (each lane
//               fetches the 16-byte unit that its LDS slot holds; rows past the
//               key range arrive as zeros), and sixteen transposing reads
//               (ds_read_b64_tr_b16) per tile and wave form the operand.
// The transposing form saves the V pre-pass (one read and one write of V) but
// issues twice the LDS reads, which costs about 2% of a long kernel's time; the
// host picks it where few query tiles share a key set (frame attention).  The
// last (partial) tile of a key range is peeled out of the loop and its missing
// keys are masked to -inf.
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
#ifndef VGGT_ATTN_NW
#define VGGT_ATTN_NW 4
#endif
constexpr int NW = VGGT_ATTN_NW;  // waves per workgroup
constexpr int CPW = 8 / NW;       // 1 KiB blocks of each tile that a wave copies
constexpr int LPT = 2 * CPW;      // copies (K + V) per wave per tile
#ifndef VGGT_ATTN_NSTAGE
#define VGGT_ATTN_NSTAGE 4
#endif
#ifndef VGGT_ATTN_WPE
#define VGGT_ATTN_WPE 2
#endif
constexpr int NT = NW * 64;
#ifndef VGGT_ATTN_NQB
#define VGGT_ATTN_NQB 4
#endif
constexpr int NQB = VGGT_ATTN_NQB;  // 16-query MFMA column blocks per wave
constexpr int QW = 16 * NQB;        // queries per wave
constexpr int BQ = NW * QW;       // queries per workgroup
constexpr int NSTAGE = VGGT_ATTN_NSTAGE;  // LDS ring depth (tiles in flight = NSTAGE - 1)
// NQB >= 4: a tile's V fragments are read in step 0 and its ring slot is refilled after the
// barrier of step NQB - 2; with NQB = 2 these would be the same step, and a faster wave's
// refill could overwrite the slot while a slower wave's fragment reads are in flight
static_assert(NQB >= 4 && NQB % 2 == 0, "scores and weights are double-buffered by step parity");
static_assert(NSTAGE >= 2 && NSTAGE <= 4, "the tile waits cover at most two later tiles in flight");
static_assert(NW == 4 || NW == 8, "a tile is copied as 8 blocks of 1 KiB, split evenly over the waves");
// exact pass: move m when a block's largest score exceeds it by kRaise; on the first tile
// also when that score lies below kLow
constexpr float kRaise = 32.0f;
constexpr float kLow = -64.0f;
constexpr float kLn2 = 0.693147180559945309f;

typedef __attribute__((address_space(3))) void lds_void;
// word 3 of a raw (untyped) buffer descriptor on gfx950: 32-bit data format, no swizzle
constexpr int kBufferFlags = 0x00020000;

// K tile:   row r holds key r of the tile, 8 units of 8 dims; unit u at slot u ^ row_swz(r).
// V tile:   V^T tile: row d holds channel d of the 64 keys; unit u holds operand keys
//           8(u%4)..+7 of 32-key chunk u/4 (see the header for their key order), at slot
//           u ^ col_swz(d); or (V in place) a row tile laid out as the K tile.
struct Smem {
  u32x4 k[NSTAGE][BK][8];
  u32x4 v[NSTAGE][BK][8];
  int redo;  // some row of the optimistic pass is out of range: rerun the workgroup exactly
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Interleave hints for the scheduler: the first half of a step takes 8 x (1 MFMA, 1
// exponential, 1 other VALU op); the second half is two quarters of 4 x (...), the first of
// which also takes the step's LDS fragment reads (two per MFMA) when it has any.
#define VGGT_INTERLEAVE8()                                     \
  _Pragma("unroll") for (int _i = 0; _i < 8; ++_i) {           \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);         \
  }
#define VGGT_INTERLEAVE4()                                     \
  _Pragma("unroll") for (int _i = 0; _i < 4; ++_i) {           \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);         \
  }
#define VGGT_INTERLEAVE4_DS2()                                 \
  _Pragma("unroll") for (int _i = 0; _i < 4; ++_i) {           \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);         \
    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);         \
  }

// kVDirect: V rows are read in place from p.v, else V^T tiles from p.vt.
template <bool kVDirect>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(VGGT_ATTN_WPE, VGGT_ATTN_WPE)))
void attn_fwd_bf16_kernel(AttnProblem p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  if (tid == 0) sm.redo = 0;  // read only after the first pass, many barriers later
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
  } else if (p.k_seq_stride == 0) {
    // sequences sharing one key set: each XCD's contiguous range holds one head's
    // (and key split's) work over all sequences, so its L2 streams that head's keys only
    seq = rest % p.nseq;
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
  // or V in place: key j of this sequence at vg + j * vrow bytes
  const char* __restrict__ vg = (const char*)p.v + ((seq * p.k_seq_stride) * p.tok_stride + head * D) * 2;
  const int vrow = (int)p.tok_stride * 2;  // at most 128 heads of 128 bytes (host check)

  const int kbeg = split * p.keys_per_split;
  const int kend = min(nk_seq, kbeg + p.keys_per_split);
  const int ntiles = (kend - kbeg + BK - 1) / BK;

  const int q0 = qt * BQ + wave * QW;  // first query of this wave
  const bool active = q0 < nq_seq;

  // ---- tile loads: each wave copies CPW 1 KiB blocks (8 rows) of the K tile and CPW of the
  //      V tile.  Lane l of a block fills slot l % 8 of its row l / 8; for V rows read in
  //      place that slot holds unit (l % 8) ^ row_swz(row), and row_swz(row) = (l / 8) & 6
  //      because blocks start at multiples of 8 rows.  A V block is a raw buffer load whose
  //      descriptor (scalar registers) starts at the block's first key and ends after the
  //      last key of the range: the lanes of rows past that end fall outside the descriptor,
  //      and such a load writes zeros to LDS, so the padding rows hold zeros as in the K tiles.
  const int ktile0 = kbeg / BK;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int v_lane_off = (lane >> 3) * vrow + 16 * ((lane & 7) ^ ((lane >> 3) & 6));
  auto issue = [&](int stage, int tile) {
    // wave-uniform base (scalar registers) + the lane's 16-byte unit
    const u32x4* ks = ktg + (int64_t)(ktile0 + tile) * 512 + wave_u * (64 * CPW);
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      __builtin_amdgcn_global_load_lds((const void*)(ks + 64 * c + lane), (lds_void*)&sm.k[stage][(CPW * wave_u + c) * 8][0], 16, 0, 0);
    if constexpr (!kVDirect) {
      const u32x4* vs = vtg + (int64_t)(ktile0 + tile) * 512 + wave_u * (64 * CPW);
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        __builtin_amdgcn_global_load_lds((const void*)(vs + 64 * c + lane), (lds_void*)&sm.v[stage][(CPW * wave_u + c) * 8][0], 16, 0, 0);
    } else {
      const int key0 = (ktile0 + tile) * BK + 8 * CPW * wave_u;  // first key of the wave's blocks
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int kb = key0 + 8 * c;
        // uniform by construction; readfirstlane keeps the descriptor in scalar registers
        const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(8, kend - kb)) * vrow);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vg + (int64_t)kb * vrow), 0, bytes, kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&sm.v[stage][(CPW * wave_u + c) * 8][0], 16,
                                                 v_lane_off, 0, 0, 0);
      }
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query q0 + 16qb + l16,
  //      channels 32dc + 8g .. +7 (the other 48 sit in the lanes of the same l16),
  //      after an optional per-head LayerNorm, rotated and scaled by scale*log2(e).
  //      Every global operand of this prologue (Q words, cos/sin pairs, LayerNorm
  //      parameters) is loaded before the first tile copies are issued: loads complete in
  //      issue order, so the wait for them then leaves the copies in flight, and the tile
  //      latency overlaps the prologue's arithmetic instead of adding to it.
  const f32x2* __restrict__ tab = p.rope_tab;
  u32x4 qw[NQB][2];  // raw bf16 words [qb][dc]
  f32x4 cs[NQB][2][2];  // (cos, sin) of rotation pairs 16dc + 4g + 2h + 0, 1 [qb][dc][h]
  float lng[2][4][2], lnb[2][4][2];  // LayerNorm gamma / beta of channels 32dc + 8g + 2e + 0, 1
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = q0 + 16 * qb + l16;
    const bool ok = qi < nq_seq;
    const int qrow = ok ? qi : 0;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      qw[qb][dc] = *(const u32x4*)(qg + (int64_t)qrow * p.tok_stride + 32 * dc + 8 * g);
      if (!ok) qw[qb][dc] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tab) {
      const int tpos = (int)((seq * p.q_seq_stride + qrow) % p.rope_T);
      const f32x4* trow = (const f32x4*)(tab + tpos * 32);
#pragma unroll
      for (int dc = 0; dc < 2; ++dc)
#pragma unroll
        for (int h = 0; h < 2; ++h) cs[qb][dc][h] = trow[8 * dc + 2 * g + h];
    }
  }
  if (p.q_ln_g) {
#pragma unroll
    for (int dc = 0; dc < 2; ++dc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 32 * dc + 8 * g + 2 * e;  // the parameters need only 4-byte alignment
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          lng[dc][e][j] = p.q_ln_g[c + j];
          lnb[dc][e][j] = p.q_ln_b[c + j];
        }
      }
  }

#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles) issue(i, i);

  bf16x8 qf[NQB][2];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float x[2][4], y[2][4];  // [dc][pair]: channels 32dc + 8g + 2e, +1
#pragma unroll
    for (int dc = 0; dc < 2; ++dc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[dc][e] = lo_bf16(qw[qb][dc][e]);
        y[dc][e] = hi_bf16(qw[qb][dc][e]);
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
          x[dc][e] = __builtin_fmaf((x[dc][e] - mu) * inv, lng[dc][e][0], lnb[dc][e][0]);
          y[dc][e] = __builtin_fmaf((y[dc][e] - mu) * inv, lng[dc][e][1], lnb[dc][e][1]);
        }
    }
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      if (tab) {
        // rotation pairs 16dc + 4g + e of the 32 of this position
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = cs[qb][dc][e >> 1][2 * (e & 1)], sn = cs[qb][dc][e >> 1][2 * (e & 1) + 1];
          const float x2 = __builtin_fmaf(x[dc][e], c, -y[dc][e] * sn);
          const float y2 = __builtin_fmaf(x[dc][e], sn, y[dc][e] * c);
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

  // ---- running state
  f32x4 o[NQB][4];  // [qb][db]: O^T rows 16db + 4g + r, column = the lane's query of block qb
  f32x4 lrow[NQB];  // [qb]: row sums (ones x P); all four registers hold the lane's query's sum
  float mrow[NQB];  // [qb]: reference m of the lane's query (log2 units)
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lrow[qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    mrow[qb] = 0.0f;
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // Scores and weights of one query block, double-buffered by step parity: step j reads
  // s[j & 1] and writes pp[j & 1] while its MFMAs fill s[~j & 1] and read pp[~j & 1].
  f32x4 s[2][4];     // [buffer][kb]: keys 16kb + 4g + r of the lane's query
  u32x4 pp[2][2];    // [buffer][chunk]: bf16 pairs, B operand of P V
  bf16x8 kf[4][2];   // K fragments of one tile [kb][dc]
  bf16x8 vf[2][4];   // V^T fragments of one tile [chunk][db]

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
  // 32-key chunk c of the V^T operand: 4 reads of the V^T tile or 8 transposing reads
  auto read_v = [&](int stage, int c) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      if constexpr (kVDirect) {
        vf[c][db] = read_tr_rows(sm.v[stage], c, db, lane);
      } else {
        const int d = 16 * db + l16;
        vf[c][db] = __builtin_bit_cast(bf16x8, sm.v[stage][d][(4 * c + g) ^ col_swz(d)]);
      }
    }
  };
  // S^T of query block qb; the two products of a key block are four MFMAs apart
  auto qk = [&](f32x4 (&sd)[4], int qb) {
#pragma unroll
    for (int dc = 0; dc < 2; ++dc)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sd[kb] = mfma(kf[kb][dc], qf[qb][dc], dc == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : sd[kb]);
  };
  // channel half dc of S^T of query block qb (four independent products)
  auto qk_dc = [&](f32x4 (&sd)[4], int qb, int dc) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sd[kb] = mfma(kf[kb][dc], qf[qb][dc], dc == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : sd[kb]);
  };
  // O^T += V^T P^T and the row sums += 1 P^T of query block qb; the two row-sum products,
  // which accumulate into one register, are issued eight MFMAs apart
  auto pv = [&](const u32x4 (&pf)[2], int qb) {
    lrow[qb] = mfma(ones, __builtin_bit_cast(bf16x8, pf[0]), lrow[qb]);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < 4; ++db) o[qb][db] = mfma(vf[c][db], __builtin_bit_cast(bf16x8, pf[c]), o[qb][db]);
    lrow[qb] = mfma(ones, __builtin_bit_cast(bf16x8, pf[1]), lrow[qb]);
  };
  // P = 2^(S - m) of 32-key chunk c of one query block as the bf16 B operand of P V, its
  // register pairs e0 .. e1-1 (GEN: m of the lane's query is subtracted; else m = 0)
  auto soft_e = [&](const f32x4 (&sc)[4], int c, auto gen_c, float m, u32x4& pf, int e0, int e1) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const f32x4& sb = sc[2 * c + (e >> 1)];
      float a = sb[2 * (e & 1)], b = sb[2 * (e & 1) + 1];
      if constexpr (decltype(gen_c)::value) {
        a -= m;
        b -= m;
      }
      pf[e] = pack_bf16x2(__builtin_amdgcn_exp2f(a), __builtin_amdgcn_exp2f(b));
    }
  };
  auto soft_c = [&](const f32x4 (&sc)[4], int c, auto gen_c, float m, u32x4& pf) {
    soft_e(sc, c, gen_c, m, pf, 0, 4);
  };
  // largest of the lane's 16 scores of one query block
  auto smax = [&](const f32x4 (&sc)[4]) -> float {
    float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[i >> 2][i & 3]), sc[(i + 1) >> 2][(i + 1) & 3]);
    return fmaxf(mx, sc[3][3]);
  };
  using yes = std::true_type;
  using no = std::false_type;
  // slow path of one query block: move the reference if needed, rescale O and the row sum
  // exactly, and redo the block's exponentials against the new reference
  auto slow = [&](const f32x4 (&sc)[4], int qb, bool first, u32x4 (&pf)[2]) {
    float mx = smax(sc);
    {
      // the query's other three lanes are l ^ 16, l ^ 32 and l ^ 48
      const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
      const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    }
    mx -= mrow[qb];  // relative to the current reference
    float delta = 0.0f;
    if (first) {
      if (mx < kLow || mx > kRaise) delta = mx;
    } else if (mx > kRaise) {
      delta = mx;
    }
    if (__any(delta != 0.0f)) {
      mrow[qb] += delta;
      if (!first) {
        // before the first tile O and l are still zero: only the reference
        // moves (2^-delta overflows when the first tile moves it far down)
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        lrow[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
      }
    }
    soft_c(sc, 0, yes{}, mrow[qb], pf[0]);
    soft_c(sc, 1, yes{}, mrow[qb], pf[1]);
  };
  auto mask = [&](f32x4 (&sc)[4], int kt) {
    // lane/register -> key kt + 16kb + 4g + r
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kt + 16 * kb + 4 * g + r >= kend) sc[kb][r] = -INFINITY;
  };

  // wait until tile `tile` has landed in LDS (later tiles may still be in flight), then
  // barrier: each wave's counter wait covers its own copies of the tile and the barrier
  // covers every wave's, so the barrier itself waits for nothing else (a __syncthreads
  // would also drain the copies of later tiles)
  auto land = [&](int tile) {
    const int ahead = min(NSTAGE - 2, ntiles - 1 - tile);  // tiles issued after `tile`
    if (ahead >= 2)
      wait_vmcnt<2 * LPT>();
    else if (ahead == 1)
      wait_vmcnt<LPT>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // the copies wrote LDS behind the compiler's back: no LDS value read before this point
    // may stand in for a read after it
    asm volatile("" ::: "memory");
  };
  // tile `tile` lands; the ring slot of tile `tile` - 1 (no wave reads it any more) takes
  // tile `tile` + NSTAGE - 1
  auto advance = [&](int tile) {
    land(tile);
    if (tile + NSTAGE - 1 < ntiles) issue((tile + NSTAGE - 1) % NSTAGE, tile + NSTAGE - 1);
  };

  // Software pipeline over steps j = NQB t + b (tile t, query block b; shown for NQB = 4).  Step j exponentiates
  // block b's scores of tile t while its MFMAs finish the previous step's block (P V and
  // row sums) and start the next one (S^T), so the exponentials of a block always run
  // beside independent MFMAs:
  //   b = 0:  P V (t-1, 3) | V(t) fragments, S^T (t, 1)
  //   b = 1:  P V (t, 0)   | S^T (t, 2)
  //   b = 2:  P V (t, 1)   | S^T (t, 3); then tile t+1 lands and its K fragments are read
  //   b = 3:  P V (t, 2)   | S^T (t+1, 0)
  // Each step is two halves, each interleaving its MFMAs with one 32-key chunk of the
  // block's exponentials.  FIRST: tile 0 (no P V of a previous tile); LAST: keys past the
  // end are masked and no next tile is touched.
  // EXACT: the per-row reference m of the exact pass: the first tile sets it, every block's
  // largest score is checked against it, and the slow path moves it (the exponentials
  // subtract it).  Otherwise m = 0 throughout and nothing is checked.
  // (the first tile takes LAST at run time: a key range of one tile)
  auto step = [&](int t, auto b_c, auto first_c, auto last_c, auto exact_c) {
    constexpr int b = decltype(b_c)::value;
    constexpr bool first = decltype(first_c)::value;
    constexpr bool exact = decltype(exact_c)::value;
    const bool last = first ? ntiles == 1 : decltype(last_c)::value;
    constexpr int cur = b & 1, nxt = cur ^ 1;
    const int stage = t % NSTAGE;
    if (last) mask(s[cur], kbeg + t * BK);
    // first half: P V of the previous step's block
    if constexpr (b == 0) {
      if constexpr (!first) pv(pp[nxt], NQB - 1);
    } else {
      pv(pp[nxt], b - 1);
    }
    if constexpr (!(exact && first)) {
      soft_c(s[cur], 0, exact_c, mrow[b], pp[cur][0]);
      VGGT_INTERLEAVE8();
    }
    __builtin_amdgcn_sched_barrier(0);
    // second half: S^T of the next step's block; in step 0 also the tile's V fragments (the
    // sixteen transposing reads split over both quarters)
    if constexpr (b == 0) {
      read_v(stage, 0);
      if constexpr (!kVDirect) read_v(stage, 1);
    }
    constexpr int nb = b < NQB - 1 ? b + 1 : 0;
    const bool has_next = b < NQB - 1 || !last;
    if constexpr (exact && first) {
      if constexpr (b == 0 && kVDirect) read_v(stage, 1);
      if (has_next) qk(s[nxt], nb);
      slow(s[cur], b, true, pp[cur]);
    } else {
      // split again, so that each key block's second channel half is issued four MFMAs
      // after its first (left to itself the scheduler pairs some of them back to back)
      if (has_next) qk_dc(s[nxt], nb, 0);
      soft_e(s[cur], 1, exact_c, mrow[b], pp[cur][1], 0, 2);
      if constexpr (b == 0) {
        VGGT_INTERLEAVE4_DS2();
      } else {
        VGGT_INTERLEAVE4();
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (b == 0 && kVDirect) read_v(stage, 1);
      if (has_next) qk_dc(s[nxt], nb, 1);
      soft_e(s[cur], 1, exact_c, mrow[b], pp[cur][1], 2, 4);
      if constexpr (b == 0 && kVDirect) {
        VGGT_INTERLEAVE4_DS2();
      } else {
        VGGT_INTERLEAVE4();
      }
      if constexpr (exact) {
        if (__any(smax(s[cur]) - mrow[b] > kRaise)) slow(s[cur], b, false, pp[cur]);
      }
    }
    // the step's weights are complete here: without this use the compiler sinks their
    // exponentials past the tile wait and barrier below, next to their first use in the
    // following step, which then starts with a run of VALU work and no MFMA beside it
    asm volatile("" ::"v"(pp[cur][0]), "v"(pp[cur][1]));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (b == NQB - 2) {
      if (!last) {
        advance(t + 1);
        read_k((t + 1) % NSTAGE);
      }
    }
  };
  auto tile = [&](int t, auto first_c, auto last_c, auto exact_c) {
    static_for<0, NQB>([&](auto b_c) { step(t, b_c, first_c, last_c, exact_c); });
  };
  // one pass over the key range (the first NSTAGE - 1 tiles are already issued)
  auto pass = [&](auto exact_c) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      lrow[qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      mrow[qb] = 0.0f;
    }
    advance(0);
    read_k(0);
    qk(s[0], 0);
    tile(0, yes{}, no{}, exact_c);
    for (int t = 1; t + 1 < ntiles; ++t) tile(t, no{}, no{}, exact_c);
    if (ntiles > 1) tile(ntiles - 1, no{}, yes{}, exact_c);
    pv(pp[(NQB - 1) & 1], NQB - 1);
  };

  // Optimistic pass: m = 0 for every row, so 2^s must neither overflow nor vanish.  A row
  // whose sum lies in [2^-64, 2^100] had every weight finite and its largest weight at
  // least 2^-64 / N, which bf16 and fp32 hold at full precision, so the pass is exact up to
  // rounding.  Otherwise the whole workgroup (its barrier and copy sequence is shared)
  // reruns the key range with the exact per-row reference.
  if (active) {
    pass(no{});
    // and its un-normalised output must be finite: weights up to 2^100 times values
    // beyond about 2^28 overflow the float32 accumulators even when l is in range
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float l = lrow[qb][0];
      float omax = 0.0f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) omax = fmaxf(omax, __builtin_fabsf(o[qb][db][r]));
      // a NaN fails both comparisons
      const bool ok = l >= 0x1p-64f && l <= 0x1p100f && omax <= 0x1p127f;
      if (q0 + 16 * qb + l16 < nq_seq && !ok) bad = true;
    }
    if (__any(bad) && lane == 0) sm.redo = 1;
  } else {
    // keep the workgroup's barrier and load sequence
    for (int t = 0; t < ntiles; ++t) advance(t);
  }
  __syncthreads();
  if (sm.redo) {
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i)
      if (i < ntiles) issue(i, i);
    if (active) {
      pass(yes{});
    } else {
      for (int t = 0; t < ntiles; ++t) advance(t);
    }
  }
  if (!active) return;

  // ---- epilogue: the 4 lanes of a query (g = 0..3) hold its 64 channels, 16 each
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float ltot = lrow[qb][0];
    const int qi = q0 + 16 * qb + l16;
    if (qi >= nq_seq) continue;
    if (p.splits == 1) {
      const float inv = 1.0f / ltot;
      if (p.lse && g == 0) p.lse[(seq * p.q_seq_stride + qi) * p.H + head] = (mrow[qb] + log2f(ltot)) * kLn2;
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
        const f32x2 ml = {mrow[qb], ltot};
        *(f32x2*)(p.part_ml + row * 2) = ml;
      }
    }
  }
}

}  // namespace

int attn_bf16_query_tile() { return BQ; }
int attn_bf16_workgroups_per_cu() { return VGGT_ATTN_WPE * 4 / NW; }  // waves per SIMD x 4 SIMDs

hipError_t launch_attn_bf16(const AttnProblem& p, hipStream_t stream) {
  const int ntq = (p.nq + BQ - 1) / BQ;
  const int64_t nwg = (int64_t)ntq * p.H * p.nseq * p.splits;
  if (nwg <= 0) return hipSuccess;
  if (p.vt)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, dim3((unsigned)nwg), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, dim3((unsigned)nwg), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vggt
