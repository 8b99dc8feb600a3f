// FlashVGGT descriptor pooling (HBM-bound, one pass over K and V).
//
// Per frame, the special tokens (outside the patch grid) are copied first, in
// order, then each ph x pw window of the gh x gw patch grid (windows that
// overhang the last row/column keep only their valid cells) becomes one
// descriptor holding the mean of its cells (FlashVGGT README, "Overview" and
// "Key Arguments" --kv_downfactor).  Sums are fp32; the mean is one
// correctly rounded fp32 division, stored with round-to-nearest-even.
//
// One thread moves one 16-byte unit of one output token; consecutive threads
// cover consecutive units of a token row, so every read and write of a token
// row is a contiguous, coalesced 2 KiB (bf16, 16 heads) segment.  blockIdx.y
// selects K (0) or V (1).
#include "common.h"

namespace vggt {
namespace {

constexpr int NT = 256;

template <bool BF16>
__global__ __launch_bounds__(NT) void pool_kernel(const void* k, const void* v, void* kd, void* vd, int S, int T,
                                                  int H, int gh, int gw, int pb, int ph, int pw, int Dn) {
  const u32x4* __restrict__ src = (const u32x4*)(blockIdx.y == 0 ? k : v);
  u32x4* __restrict__ dst = (u32x4*)(blockIdx.y == 0 ? kd : vd);
  const int upt = H * kHeadDim * (BF16 ? 2 : 4) / 16;  // 16-byte units per token
  const int64_t total = (int64_t)S * Dn * upt;
  const int nspec = T - gh * gw;
  const int cw = (gw + pw - 1) / pw;
  for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * NT) {
    const int64_t ot = idx / upt;
    const int u = (int)(idx % upt);
    const int s = (int)(ot / Dn), w = (int)(ot % Dn);
    const int64_t fbase = (int64_t)s * T;
    if (w < nspec) {
      const int t = (w < pb) ? w : w + gh * gw;
      dst[idx] = src[(fbase + t) * upt + u];
      continue;
    }
    const int ci = w - nspec;
    const int a = ci / cw, b = ci % cw;
    const int r0 = a * ph, r1 = min(r0 + ph, gh);
    const int c0 = b * pw, c1 = min(c0 + pw, gw);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = r0; r < r1; ++r)
      for (int c = c0; c < c1; ++c) {
        const u32x4 x = src[(fbase + pb + (int64_t)r * gw + c) * upt + u];
        if (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += lo_bf16(x[e]);
            acc[2 * e + 1] += hi_bf16(x[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(x[e]);
        }
      }
    const float cnt = (float)((r1 - r0) * (c1 - c0));
    u32x4 y;
    if (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = pack_bf16x2(acc[2 * e] / cnt, acc[2 * e + 1] / cnt);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __float_as_uint(acc[e] / cnt);
    }
    dst[idx] = y;
  }
}

}  // namespace

hipError_t launch_pool(const void* k, const void* v, void* kd, void* vd, bool bf16, int S, int T, int H, int gh,
                       int gw, int patch_begin, int ph, int pw, int Dn, hipStream_t stream) {
  const int upt = H * kHeadDim * (bf16 ? 2 : 4) / 16;
  const int64_t total = (int64_t)S * Dn * upt;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + NT - 1) / NT;
  if (blocks > 65535) blocks = 65535;
  if (bf16)
    hipLaunchKernelGGL(pool_kernel<true>, dim3((unsigned)blocks, 2), dim3(NT), 0, stream, k, v, kd, vd, S, T, H, gh,
                       gw, patch_begin, ph, pw, Dn);
  else
    hipLaunchKernelGGL(pool_kernel<false>, dim3((unsigned)blocks, 2), dim3(NT), 0, stream, k, v, kd, vd, S, T, H, gh,
                       gw, patch_begin, ph, pw, Dn);
  return hipGetLastError();
}

}  // namespace vggt
