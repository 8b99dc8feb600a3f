// Operand preparation for the bf16 attention kernel (all HBM-bound, one pass).
//
//  rope_table_kernel  cos/sin of the 32 rotation angles of every in-frame
//                     position: table[t][k], k < 16 turns with the row and
//                     k >= 16 with the column, angle p * base^(-2(k%16)/32)
//                     formed in fp64 and rounded to fp32 (frequency schedule
//                     of the "VGGT 論文報告" slide deck, Section IV, slide
//                     4/6, per axis; rope_base of the VGGT-Omega-1B-512-bf16
//                     config article).
//  rope_apply_kernel  rotated copy of K (bf16) using the table; a pair whose
//                     angle is 0 is copied unchanged.
//  vt_kernel          V [seq][len][H][64] -> V^T [H][64][nseq * pad]: for each
//                     head and channel, the keys of a sequence are contiguous
//                     and every sequence starts at a multiple of 64 columns
//                     (pad columns are zero), so the attention kernel can
//                     stream 16-byte key units of V^T straight into LDS.
#include "common.h"

namespace vggt {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void rope_table_kernel(const int32_t* __restrict__ pos, int T, double base,
                                                        f32x2* __restrict__ table) {
  const int i = blockIdx.x * NT + threadIdx.x;
  if (i >= T * 32) return;
  const int t = i >> 5, k = i & 31;
  const double theta = (double)pos[2 * t + (k >> 4)] * pow(base, -(double)(k & 15) / 16.0);
  table[i] = f32x2{(float)cos(theta), (float)sin(theta)};
}

// one thread per 16-byte unit (8 bf16 = 4 rotation pairs)
__global__ __launch_bounds__(NT) void rope_apply_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n_units, int H, int T,
                                                        const f32x2* __restrict__ table) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= n_units) return;
  const int u = (int)(i & 7);                // unit within a head row
  const int64_t tok = i / (8 * (int64_t)H);
  const int t = (int)(tok % T);
  const u32x4 w = src[i];
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 cs = table[t * 32 + 4 * u + e];
    if (cs[1] != 0.0f) {
      const float x = lo_bf16(w[e]), y = hi_bf16(w[e]);
      r[e] = pack_bf16x2(__builtin_fmaf(x, cs[0], -y * cs[1]), __builtin_fmaf(x, cs[1], y * cs[0]));
    } else {
      r[e] = w[e];
    }
  }
  dst[i] = r;
}

// grid (pad/64, H, nseq); tile = 64 keys x 64 channels through LDS
__global__ __launch_bounds__(NT) void vt_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt, int len,
                                                int pad, int H, int64_t cols) {
  __shared__ uint16_t tile[64][64 + 2];
  const int j0 = blockIdx.x * 64, h = blockIdx.y, sq = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t tok_stride = (int64_t)H * kHeadDim;
  // load: 64 keys x 8 units of 16 bytes; thread -> (key = i / 8, unit = i % 8)
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = tid + c * NT;
    const int j = i >> 3, u = i & 7;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (j0 + j < len) w = *(const u32x4*)(v + ((int64_t)sq * len + j0 + j) * tok_stride + h * kHeadDim + 8 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[j][8 * u + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      tile[j][8 * u + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  // store: 64 channel rows x 8 units of 8 keys
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = tid + c * NT;
    const int d = i >> 3, u = i & 7;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[8 * u + 2 * e][d] | ((uint32_t)tile[8 * u + 2 * e + 1][d] << 16);
    *(u32x4*)(vt + ((int64_t)h * kHeadDim + d) * cols + (int64_t)sq * pad + j0 + 8 * u) = w;
  }
}

}  // namespace

hipError_t launch_rope_table(const int32_t* pos_yx, int T, double base, void* table, hipStream_t stream) {
  const unsigned blocks = (unsigned)((T * 32 + NT - 1) / NT);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(NT), 0, stream, pos_yx, T, base, (f32x2*)table);
  return hipGetLastError();
}

hipError_t launch_rope_apply_bf16(const void* src, void* dst, int64_t n_tok, int H, int T, const void* table,
                                  hipStream_t stream) {
  const int64_t units = n_tok * H * 8;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_apply_kernel, dim3((unsigned)((units + NT - 1) / NT)), dim3(NT), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, units, H, T, (const f32x2*)table);
  return hipGetLastError();
}

hipError_t launch_vt_bf16(const void* v, void* vt, int nseq, int len, int pad, int H, hipStream_t stream) {
  if (nseq <= 0 || len <= 0) return hipSuccess;
  const int64_t cols = (int64_t)nseq * pad;
  hipLaunchKernelGGL(vt_kernel, dim3((unsigned)(pad / 64), (unsigned)H, (unsigned)nseq), dim3(NT), 0, stream,
                     (const uint16_t*)v, (uint16_t*)vt, len, pad, H, cols);
  return hipGetLastError();
}

}  // namespace vggt
