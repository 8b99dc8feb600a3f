// Exact merge of split-key attention partials.
//
// Split s of a row left an un-normalised output O_s = sum_j 2^(x_j - m_s) v_j,
// its reference maximum m_s (log2 units) and sum l_s = sum_j 2^(x_j - m_s).
// With M = max_s m_s and w_s = 2^(m_s - M):
//   O = sum_s w_s O_s / sum_s w_s l_s,
// which equals the softmax over the union of the key ranges exactly (up to
// rounding): the split only reorders the sum in the softmax denominator and
// the weighted sum of values.
#include "common.h"

namespace vggt {
namespace {

constexpr int D = kHeadDim;
constexpr int NT = 256;

template <bool OUT_BF16>
__global__ __launch_bounds__(NT) void attn_merge_kernel(AttnProblem p) {
  // one thread per (row, head, 8-dim chunk)
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t rows = p.nq_total * p.H;
  if (gid >= rows * 8) return;
  const int64_t rh = gid >> 3;      // row * H + head
  const int dc = (int)(gid & 7);
  const int64_t row = rh / p.H;
  const int head = (int)(rh % p.H);

  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_ml[((int64_t)s * rows + rh) * 2]);
  float L = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.splits; ++s) {
    const int64_t r = (int64_t)s * rows + rh;
    const f32x2 ml = *(const f32x2*)(p.part_ml + r * 2);
    const float w = __builtin_amdgcn_exp2f(ml[0] - M);
    L = __builtin_fmaf(w, ml[1], L);
    const f32x4 a = *(const f32x4*)(p.part_o + r * D + 8 * dc);
    const f32x4 b = *(const f32x4*)(p.part_o + r * D + 8 * dc + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = __builtin_fmaf(w, a[e], acc[e]);
      acc[e + 4] = __builtin_fmaf(w, b[e], acc[e + 4]);
    }
  }
  const int64_t seq = row / p.nq, qi = row % p.nq;
  const int64_t off = (seq * p.q_seq_stride + qi) * p.tok_stride + (int64_t)head * D + 8 * dc;
  if (p.lse && dc == 0) p.lse[(seq * p.q_seq_stride + qi) * p.H + head] = (M + log2f(L)) * 0.693147180559945309f;
  if (OUT_BF16) {
    const u32x4 w = {pack_bf16x2(acc[0] / L, acc[1] / L), pack_bf16x2(acc[2] / L, acc[3] / L),
                     pack_bf16x2(acc[4] / L, acc[5] / L), pack_bf16x2(acc[6] / L, acc[7] / L)};
    *(u32x4*)((uint16_t*)p.o + off) = w;
  } else {
    const f32x4 a = {acc[0] / L, acc[1] / L, acc[2] / L, acc[3] / L};
    const f32x4 b = {acc[4] / L, acc[5] / L, acc[6] / L, acc[7] / L};
    *(f32x4*)((float*)p.o + off) = a;
    *(f32x4*)((float*)p.o + off + 4) = b;
  }
}

}  // namespace

hipError_t launch_attn_merge(const AttnProblem& p, bool out_bf16, hipStream_t stream) {
  const int64_t threads = p.nq_total * p.H * 8;
  if (threads <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + NT - 1) / NT);
  if (out_bf16)
    hipLaunchKernelGGL(attn_merge_kernel<true>, dim3(blocks), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_merge_kernel<false>, dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vggt
