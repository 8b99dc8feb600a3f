// Flash attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// Computes softmax(scale * Q K^T) V per head (the "VGGT 論文報告" slide
// deck, Section V, slides 5/10-9/10) without ever forming the score matrix:
// keys stream through LDS in tiles of 64 and each query row keeps a running
// maximum and sum (online softmax), so a row costs O(1) memory for any key
// count.
//
// Work split.  A workgroup of 4 waves owns 256 queries of one head; each wave
// owns 64 of them (two 32-query MFMA column blocks).  Per 64-key tile:
//   S^T = K Q^T   16 x v_mfma_f32_32x32x16_bf16 (keys are the M dimension, so
//                 one lane holds 32 scores of a single query and row
//                 reductions stay inside the lane plus one lane^32 exchange);
//   P = exp2(S^T * scale*log2e - m) in fp32, rounded to bf16;
//   O^T += V^T P^T  16 x v_mfma_f32_32x32x16_bf16 (head dim is M, the lane
//                 again holds one query, so the per-row rescale is in-lane).
// The score-tile rows are taken in the key order rho (bits 2 and 3 of the key
// index swapped) so that the accumulator registers of S^T are, in order,
// exactly the bf16 B-operand of the P V product: no register shuffles.
//
// Lazy rescaling: the reference maximum m of a row only moves when a tile's
// maximum exceeds it by more than 8 (log2 units), so exp2 arguments stay <= 8
// and the O rescale runs on few tiles.  The final O / l is exact.
//
// LDS: K and V^T tiles, double buffered (32 KiB), 16-byte units XOR-swizzled
// per row so that the 16-byte MFMA operand reads and the tile writes are free
// of bank conflicts.  Global loads of tile t+1 are in flight while tile t is
// computed; one barrier per tile.
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
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ int rho(int i) { return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1); }

// K tile:   row r holds key rho(r) of the tile, 8 units of 8 dims; unit u at u ^ (r & 7).
// V^T tile: row d holds dim d of the 64 keys, unit u = keys 8u..8u+7 at u ^ ((d ^ (d >> 3)) & 7).
struct Smem {
  u32x4 k[2][BK][8];
  u32x4 vt[2][D][8];
};

__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

__device__ __forceinline__ void xcd_remap(int w, int nwg, int& logical) {
  const int q = nwg >> 3, r = nwg & 7;
  const int xcd = w & 7, k = w >> 3;
  logical = (xcd < r) ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

__global__ __launch_bounds__(NT) void attn_fwd_bf16_kernel(AttnProblem p) {
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
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + (seq * p.k_seq_stride) * p.tok_stride + head * D;

  const int kbeg = split * p.keys_per_split;
  const int kend = min(p.nk, kbeg + p.keys_per_split);
  const int ntiles = (kend - kbeg + BK - 1) / BK;

  const int q0 = qt * BQ + wave * 64;          // first query of this wave
  const bool active = q0 < p.nq;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query q0+32*qb+l32,
  //      dims 16*dc + 8*hi .. +7.
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = q0 + 32 * qb + l32;
    const bool ok = qi < p.nq;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *(const u32x4*)(qg + (int64_t)qi * p.tok_stride + 16 * dc + 8 * hi);
      qf[qb][dc] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- tile loaders
  // K: 512 16-byte chunks per tile, two per thread: chunk i -> key i/8, unit i%8.
  // V: thread -> unit vu = tid%8 (dims 8vu..8vu+7) of keys 2*vp, 2*vp+1, vp = tid/8.
  const int vu = tid & 7, vp = tid >> 3;
  u32x4 kreg[2], va, vb;
  auto gload = [&](int kt) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = tid + c * NT;
      const int key = kt + (i >> 3);
      kreg[c] = (key < kend) ? *(const u32x4*)(kg + (int64_t)key * p.tok_stride + 8 * (i & 7)) : u32x4{0u, 0u, 0u, 0u};
    }
    const int k0 = kt + 2 * vp;
    va = (k0 < kend) ? *(const u32x4*)(vg + (int64_t)k0 * p.tok_stride + 8 * vu) : u32x4{0u, 0u, 0u, 0u};
    vb = (k0 + 1 < kend) ? *(const u32x4*)(vg + (int64_t)(k0 + 1) * p.tok_stride + 8 * vu) : u32x4{0u, 0u, 0u, 0u};
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = tid + c * NT;
      const int r = rho(i >> 3);
      sm.k[buf][r][(i & 7) ^ (r & 7)] = kreg[c];
    }
    // transpose the 2 x 8 block: row d = 8*vu + e gets keys (2vp, 2vp+1)
    uint32_t* vt = (uint32_t*)&sm.vt[buf][0][0];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = va[e >> 1], b = vb[e >> 1];
      const uint32_t w = (e & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      const int d = 8 * vu + e;
      vt[d * 32 + 4 * ((vp >> 2) ^ vt_swz(d)) + (vp & 3)] = w;
    }
  };

  // ---- running state
  f32x16 o[2][2];  // [db][qb]: O^T rows 32*db + 8*(r/4) + 4*hi + r%4, column = query
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[a][b][r] = 0.0f;
  float mref[2] = {-INFINITY, -INFINITY};  // log2 units
  float lsum[2] = {0.0f, 0.0f};            // this lane's partial row sums
  const float c = p.scale_log2;

  gload(kbeg);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = kbeg + t * BK;
    if (t + 1 < ntiles) gload(kt + BK);

    if (active) {
      // S^T = K Q^T for two 32-key blocks
      f32x16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
        const int row = 32 * kb + l32;
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const int u = 2 * dc + hi;
          const bf16x8 kf = __builtin_bit_cast(bf16x8, sm.k[buf][row][u ^ (row & 7)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][dc], s[kb][qb], 0, 0, 0);
        }
      }
      // mask keys past the end (only the last tile can have them);
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
      // online softmax per query block
      uint32_t pf[2][2][2][4];  // [qb][kb][j] bf16 pairs of keys 32kb+16j+8hi+0..7
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mx2 = mx * c;
        if (__any(mx2 > mref[qb] + kRescaleThreshold)) {
          const float mnew = fmaxf(mref[qb], mx2);
          const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mnew);
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
          mref[qb] = mnew;
        }
        const float neg = -mref[qb];
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * j + 2 * e], c, neg));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * j + 2 * e + 1], c, neg));
              ls += p0 + p1;
              pf[qb][kb][j][e] = pack_bf16x2(p0, p1);
            }
        lsum[qb] += ls;
      }
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
    if (t + 1 < ntiles) swrite(buf ^ 1);
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
