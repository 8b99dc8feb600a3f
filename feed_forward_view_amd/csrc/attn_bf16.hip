// Flash attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// Computes softmax(scale * Q K^T) V per head (the "VGGT 論文報告" slide
// deck, Section V, slides 5/10-9/10) without ever forming the score matrix:
// keys stream through LDS in tiles of 64 and each query row keeps a running
// sum against a reference offset, so a row costs O(1) memory for any key
// count.
//
// Work split.  A workgroup of 4 waves owns 256 queries of one head; each wave
// owns 64 of them (two 32-query MFMA column blocks).  Per 64-key tile:
//   S^T = K Q^T   16 x v_mfma_f32_32x32x16_bf16 (keys are the M dimension, so
//                 one lane holds 32 scores of a single query);
//   P = 2^(S^T - m) in fp32, rounded to bf16; the row sum adds the rounded
//                 P pairs with v_dot2_f32_bf16, i.e. exactly the weights the
//                 P V product uses;
//   O^T += V^T P^T  16 x v_mfma_f32_32x32x16_bf16 (head dim is M, the lane
//                 again holds one query, so per-row scaling stays in-lane).
// Q is rotated (2D RoPE, fp32, from the per-position cos/sin table) and
// multiplied by scale*log2(e) once in the prologue, so scores come out of the
// MFMA in log2 units.  The score-tile rows are taken in the key order rho
// (bits 2 and 3 of the key index swapped) so that the S^T accumulator
// registers are, in order, exactly the bf16 B operand of the P V product.
//
// Softmax reference.  The reference m of a row starts at 0 and is left there
// while the row's scores stay within 2^32 of it: then 2^s needs no subtraction
// at all, and each score costs one v_exp_f32, half a v_cvt_pk_bf16_f32 and
// half a v_dot2.  The first tile, and any tile whose partial row sum leaves
// [0, 2^64], takes a slow path that computes the tile maximum, moves m
// (rescaling O and the sum exactly by 2^(m_old - m_new)) and redoes the
// tile; from then on the wave subtracts m before the exponential.  The final
// O / l is the same softmax whatever m is.
//
// Operands.  K rows (rotated by a pre-pass when RoPE is on) and V^T rows
// (transposed by a pre-pass, every sequence starting at a multiple of 64
// columns) are copied straight from global memory into LDS with
// global_load_lds_dwordx4, 16-byte units XOR-swizzled per row so that the
// 16-byte MFMA operand reads are free of bank conflicts; two stages, one
// barrier per tile.  Keys past the end of a range are masked to -inf.
//
// Workgroup order is XCD-aware: the hardware deals workgroups round-robin to
// the 8 XCDs, so the linear id is remapped to give each XCD a contiguous run
// of (query tile, head) work; the workgroups resident on one XCD then stream
// the same head's keys and values through that XCD's L2.
#include "common.h"

namespace vggt {
namespace {

constexpr int D = kHeadDim;
constexpr int BK = kAttnKeyTile;  // 64 keys per tile
constexpr int NW = 4;             // waves per workgroup
constexpr int NT = NW * 64;
constexpr int BQ = NW * 64;       // 64 queries per wave
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64
constexpr float kRaise = 32.0f;   // move m when a tile max exceeds it by this
constexpr float kLow = -64.0f;    // first tile: move m down when the max is below this

__device__ __forceinline__ int rho(int i) { return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1); }
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

typedef __attribute__((address_space(3))) void lds_void;

// K tile:   row r holds key rho(r) of the tile, 8 units of 8 dims; unit u at slot u ^ (r & 7).
// V^T tile: row d holds channel d of the 64 keys; unit u (keys 8u..8u+7) at slot u ^ vt_swz(d).
struct Smem {
  u32x4 k[2][BK][8];
  u32x4 vt[2][D][8];
};

__device__ __forceinline__ void xcd_remap(int w, int nwg, int& logical) {
  const int q = nwg >> 3, r = nwg & 7;
  const int xcd = w & 7, k = w >> 3;
  logical = (xcd < r) ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

__device__ __forceinline__ float dot2_acc(uint32_t pk, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(AttnProblem p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- which (query tile, head, sequence, split) this workgroup owns
  const int ntq = (p.nq + BQ - 1) / BQ;
  const int nwg = ntq * p.H * p.nseq * p.splits;
  int logical;
  xcd_remap(blockIdx.x, nwg, logical);
  const int qt = logical % ntq;
  int rest = logical / ntq;
  const int head = rest % p.H;
  rest /= p.H;
  const int split = rest % p.splits;
  const int seq = rest / p.splits;

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + (seq * p.q_seq_stride) * p.tok_stride + head * D;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + (seq * p.k_seq_stride) * p.tok_stride + head * D;
  const uint16_t* __restrict__ vtg = (const uint16_t*)p.vt + (int64_t)head * D * p.vt_cols + seq * p.vt_seq_stride;

  const int kbeg = split * p.keys_per_split;
  const int kend = min(p.nk, kbeg + p.keys_per_split);
  const int ntiles = (kend - kbeg + BK - 1) / BK;

  const int q0 = qt * BQ + wave * 64;  // first query of this wave
  const bool active = q0 < p.nq;

  // ---- tile loads: each wave moves two 1 KiB blocks of K and two of V^T
  auto issue = [&](int stage, int kt) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int blk = 2 * wave + c;
      const int r = blk * 8 + (lane >> 3);
      const int s = lane & 7;
      const int key = min(kt + rho(r), kend - 1);
      const uint16_t* ksrc = kg + (int64_t)key * p.tok_stride + 8 * (s ^ (r & 7));
      __builtin_amdgcn_global_load_lds((const void*)ksrc, (lds_void*)&sm.k[stage][blk * 8][0], 16, 0, 0);
      const uint16_t* vsrc = vtg + (int64_t)r * p.vt_cols + kt + 8 * (s ^ vt_swz(r));
      __builtin_amdgcn_global_load_lds((const void*)vsrc, (lds_void*)&sm.vt[stage][blk * 8][0], 16, 0, 0);
    }
  };

  issue(0, kbeg);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query q0+32*qb+l32,
  //      dims 16*dc + 8*hi .. +7, rotated and scaled by scale*log2(e).
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = q0 + 32 * qb + l32;
    const bool ok = qi < p.nq;
    const int tpos = p.rope_tab ? (int)((seq * p.q_seq_stride + qi) % p.rope_T) : 0;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *(const u32x4*)(qg + (int64_t)qi * p.tok_stride + 16 * dc + 8 * hi);
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = lo_bf16(w[e]), y = hi_bf16(w[e]);
        if (p.rope_tab && ok) {
          const f32x2 cs = p.rope_tab[tpos * 32 + 8 * dc + 4 * hi + e];
          const float x2 = __builtin_fmaf(x, cs[0], -y * cs[1]);
          const float y2 = __builtin_fmaf(x, cs[1], y * cs[0]);
          x = x2;
          y = y2;
        }
        r[e] = pack_bf16x2(x * p.scale_log2, y * p.scale_log2);
      }
      qf[qb][dc] = __builtin_bit_cast(bf16x8, r);
    }
  }

  // ---- running state
  f32x16 o[2][2];  // [db][qb]: O^T rows 32*db + 8*(r/4) + 4*hi + r%4, column = query
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[a][b][r] = 0.0f;
  float mref[2] = {0.0f, 0.0f};  // log2 units
  float lsum[2] = {0.0f, 0.0f};  // this lane's partial row sums
  bool offs = false;             // some row of the wave has m != 0

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = kbeg + t * BK;
    if (t + 1 < ntiles) issue(buf ^ 1, kt + BK);

    if (active) {
      // S^T = K Q^T for two 32-key blocks
      f32x16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + l32;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const int u = 2 * dc + hi;
          const bf16x8 kf = __builtin_bit_cast(bf16x8, sm.k[buf][row][u ^ (row & 7)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            if (dc == 0) {
              const f32x16 z = {};
              s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][0], z, 0, 0, 0);
            } else {
              s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][dc], s[kb][qb], 0, 0, 0);
            }
          }
        }
      }
      // mask keys past the end (only the last tile of a range has them);
      // lane/reg -> key kt + 32*kb + 16*(r/8) + 8*hi + r%8
      if (kt + BK > kend) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * kb + 16 * (r >> 3) + 8 * hi + (r & 7);
            if (key >= kend) {
              s[kb][0][r] = -INFINITY;
              s[kb][1][r] = -INFINITY;
            }
          }
      }
      // P = 2^(S - m) as bf16 pairs; tile partial row sums
      uint32_t pf[2][2][2][4];  // [qb][kb][j] bf16 pairs of keys 32kb+16j+8hi+0..7
      float ls[2];
      auto exps = [&](bool sub) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float acc = 0.0f;
          const float m = sub ? mref[qb] : 0.0f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float a = s[kb][qb][8 * j + 2 * e], b = s[kb][qb][8 * j + 2 * e + 1];
                if (sub) {
                  a -= m;
                  b -= m;
                }
                const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(a), __builtin_amdgcn_exp2f(b));
                pf[qb][kb][j][e] = w;
                acc = dot2_acc(w, acc);
              }
          ls[qb] = acc;
        }
      };
      if (offs)
        exps(true);
      else
        exps(false);
      const bool bad = !(ls[0] <= kSumLimit) || !(ls[1] <= kSumLimit);
      if (t == 0 || __any(bad)) {
        // slow path: move the reference where needed, then redo the tile
        bool any_m = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float mx = s[0][qb][0];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          float mnew = mref[qb];
          if (t == 0) {
            if (mx < kLow || mx > kRaise) mnew = mx;
          } else if (mx - mref[qb] > kRaise) {
            mnew = mx;
          }
          if (mnew != mref[qb]) {
            const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mnew);
            lsum[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
            mref[qb] = mnew;
          }
          any_m = any_m || (mref[qb] != 0.0f);
        }
        offs = __any(any_m);
        exps(true);
      }
      lsum[0] += ls[0];
      lsum[1] += ls[1];
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int u = 4 * kb + 2 * j + hi;
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const int d = 32 * db + l32;
            const bf16x8 vf = __builtin_bit_cast(bf16x8, sm.vt[buf][d][u ^ vt_swz(d)]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              const u32x4 w = {pf[qb][kb][j][0], pf[qb][kb][j][1], pf[qb][kb][j][2], pf[qb][kb][j][3]};
              o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, w), o[db][qb], 0, 0, 0);
            }
          }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (!active) return;

  // ---- epilogue
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const int qi = q0 + 32 * qb + l32;
    if (qi >= p.nq) continue;
    if (p.splits == 1) {
      const float inv = 1.0f / ltot;
      uint16_t* og = (uint16_t*)p.o + (seq * p.q_seq_stride + qi) * p.tok_stride + head * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * db + 8 * a + 4 * hi;
          const u32x2 w = {pack_bf16x2(o[db][qb][4 * a] * inv, o[db][qb][4 * a + 1] * inv),
                           pack_bf16x2(o[db][qb][4 * a + 2] * inv, o[db][qb][4 * a + 3] * inv)};
          *(u32x2*)(og + d) = w;
        }
    } else {
      const int64_t row = ((int64_t)split * p.nq_total + (int64_t)seq * p.nq + qi) * p.H + head;
      float* po = p.part_o + row * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * db + 8 * a + 4 * hi;
          const f32x4 w = {o[db][qb][4 * a], o[db][qb][4 * a + 1], o[db][qb][4 * a + 2], o[db][qb][4 * a + 3]};
          *(f32x4*)(po + d) = w;
        }
      if (hi == 0) {
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
