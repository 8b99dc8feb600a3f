// 2D rotary position embedding over [tokens, H, 64] (HBM-bound, one pass).
//
// Channels 0..31 of every head turn with the token's patch row, 32..63 with
// its column; pair (2k, 2k+1) of a half turns by p * base^(-2k/32)
// (frequency schedule of the "VGGT 論文報告" slide deck, Section IV, slide
// 4/6, applied per axis; rope_base from the VGGT-Omega-1B-512-bf16 config
// article).  A workgroup handles 8 tokens: it first forms the 8 x 32 angles
// in fp64 and keeps cos/sin as fp32 in LDS (the frequency buffers of the
// model are fp32), then streams the 8 tokens' 16-byte units through a fp32
// rotation.  A pair whose angle is 0 is passed through unchanged, so
// position (0, 0) is the identity bit for bit.
#include "common.h"

namespace vggt {
namespace {

constexpr int D = kHeadDim;
constexpr int NT = 256;
constexpr int TOK = 8;

__device__ __forceinline__ void rot(float& x, float& y, float c, float s) {
  if (s != 0.0f) {
    const float x2 = __builtin_fmaf(x, c, -y * s);
    const float y2 = __builtin_fmaf(x, s, y * c);
    x = x2;
    y = y2;
  }
}

// INVERSE: rotate by the negated angles (the transpose of the rotation).
template <bool BF16, bool INVERSE>
__global__ __launch_bounds__(NT) void rope_kernel(const void* src, void* dst, int64_t n_tok, int T, int H,
                                                  const int32_t* __restrict__ pos, double base) {
  __shared__ f32x2 cs[TOK][32];
  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * TOK;
  {
    const int lt = tid >> 5, k = tid & 31;
    const int64_t g = tok0 + lt;
    float cv = 1.0f, sv = 0.0f;
    if (g < n_tok) {
      const int t = (int)(g % T);
      const int axis = k >> 4, pair = k & 15;
      const double pp = (double)pos[2 * t + axis];
      const double theta = pp * pow(base, -(double)pair / 16.0);
      cv = (float)cos(theta);
      sv = INVERSE ? -(float)sin(theta) : (float)sin(theta);
    }
    cs[lt][k] = f32x2{cv, sv};
  }
  __syncthreads();

  const int esz = BF16 ? 2 : 4;
  const int units_per_head = D * esz / 16;  // 8 (bf16) or 16 (fp32)
  const int units_per_tok = H * units_per_head;
  const int64_t ntok_here = min((int64_t)TOK, n_tok - tok0);
  const int total = (int)ntok_here * units_per_tok;
  for (int i = tid; i < total; i += NT) {
    const int lt = i / units_per_tok;
    const int u = i % units_per_head;
    const int64_t off16 = (tok0 + lt) * units_per_tok + (i % units_per_tok);  // in 16-byte units
    const u32x4 w = ((const u32x4*)src)[off16];
    u32x4 r;
    if (BF16) {
      // unit u holds dims 8u..8u+7 = pairs 4u..4u+3
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = lo_bf16(w[e]), y = hi_bf16(w[e]);
        const f32x2 a = cs[lt][4 * u + e];
        rot(x, y, a[0], a[1]);
        r[e] = (a[1] != 0.0f) ? pack_bf16x2(x, y) : w[e];
      }
    } else {
      // unit u holds dims 4u..4u+3 = pairs 2u, 2u+1
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float x = __uint_as_float(w[2 * e]), y = __uint_as_float(w[2 * e + 1]);
        const f32x2 a = cs[lt][2 * u + e];
        rot(x, y, a[0], a[1]);
        r[2 * e] = (a[1] != 0.0f) ? __float_as_uint(x) : w[2 * e];
        r[2 * e + 1] = (a[1] != 0.0f) ? __float_as_uint(y) : w[2 * e + 1];
      }
    }
    ((u32x4*)dst)[off16] = r;
  }
}

// Per-head LayerNorm of fp32 head vectors (the fp32 debug path's Q/K prologue):
// one thread per (token, head) row of 64 channels, two passes over registers.
__global__ __launch_bounds__(NT) void layer_norm_f32_kernel(const float* src, float* dst, int64_t rows,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ b, float eps) {
  const int64_t r = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (r >= rows) return;
  float f[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const f32x4 w = *(const f32x4*)(src + r * D + c);
    f[c] = w[0]; f[c + 1] = w[1]; f[c + 2] = w[2]; f[c + 3] = w[3];
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < D; ++c) sum += f[c];
  const float mu = sum * (1.0f / D);
  float dev = 0.0f;
#pragma unroll
  for (int c = 0; c < D; ++c) dev = __builtin_fmaf(f[c] - mu, f[c] - mu, dev);
  const float inv = 1.0f / __builtin_sqrtf(dev * (1.0f / D) + eps);
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __builtin_fmaf((f[c + j] - mu) * inv, g[c + j], b[c + j]);
    *(f32x4*)(dst + r * D + c) = w;
  }
}

}  // namespace

hipError_t launch_layer_norm_f32(const float* src, float* dst, int64_t n_tok, int H, const float* g, const float* b,
                                 float eps, hipStream_t stream) {
  const int64_t rows = n_tok * H;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(layer_norm_f32_kernel, dim3((unsigned)((rows + NT - 1) / NT)), dim3(NT), 0, stream, src, dst,
                     rows, g, b, eps);
  return hipGetLastError();
}

hipError_t launch_rope(const void* src, void* dst, bool bf16, int64_t n_tok, int T, int H, const int32_t* pos_yx,
                       double base, hipStream_t stream, bool inverse) {
  if (n_tok <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n_tok + TOK - 1) / TOK);
  if (bf16 && !inverse)
    hipLaunchKernelGGL((rope_kernel<true, false>), dim3(blocks), dim3(NT), 0, stream, src, dst, n_tok, T, H, pos_yx, base);
  else if (bf16)
    hipLaunchKernelGGL((rope_kernel<true, true>), dim3(blocks), dim3(NT), 0, stream, src, dst, n_tok, T, H, pos_yx, base);
  else if (!inverse)
    hipLaunchKernelGGL((rope_kernel<false, false>), dim3(blocks), dim3(NT), 0, stream, src, dst, n_tok, T, H, pos_yx, base);
  else
    hipLaunchKernelGGL((rope_kernel<false, true>), dim3(blocks), dim3(NT), 0, stream, src, dst, n_tok, T, H, pos_yx, base);
  return hipGetLastError();
}

}  // namespace vggt
