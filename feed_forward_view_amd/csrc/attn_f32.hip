// Attention forward in fp32 (the library's debug precision mode).
//
// Same problem and same partial-output format as the bf16 matrix-core
// kernel, but every product and sum is an fp32 FMA on the vector ALU: one
// thread owns one query row (64 query values and 64 output accumulators in
// registers) and walks the keys of its range, staged 64 at a time in LDS,
// with an exact online softmax (slide deck "VGGT 論文報告", Section V, slides
// 4/10 and 5/10): on a new row maximum the running sum and output are
// rescaled before the key is added.
#include "common.h"

namespace vggt {
namespace {

constexpr int D = kHeadDim;
constexpr int BK = kAttnKeyTile;
constexpr int NT = 256;
constexpr int BQ = NT;  // one query per thread

__global__ __launch_bounds__(NT) void attn_fwd_f32_kernel(AttnProblem p) {
  __shared__ float ks[BK][D];
  __shared__ float vs[BK][D];
  const int tid = threadIdx.x;

  const int ntq = (p.nq + BQ - 1) / BQ;
  int rest = blockIdx.x;
  const int qt = rest % ntq;
  rest /= ntq;
  const int head = rest % p.H;
  rest /= p.H;
  const int split = rest % p.splits;
  const int seq = p.nk_step > 0 ? p.nseq - 1 - rest / p.splits : rest / p.splits;
  const int nq_seq = (int)min((int64_t)p.nq, p.nq_total - (int64_t)seq * p.nq);
  const int nk_seq = p.nk_step > 0 ? (int)min((int64_t)p.nk, (int64_t)(seq + 1) * p.nk_step) : p.nk;

  const float* __restrict__ qg = (const float*)p.q + (seq * p.q_seq_stride) * p.tok_stride + head * D;
  const float* __restrict__ kg = (const float*)p.k + (seq * p.k_seq_stride) * p.tok_stride + head * D;
  const float* __restrict__ vg = (const float*)p.v + (seq * p.k_seq_stride) * p.tok_stride + head * D;

  const int kbeg = split * p.keys_per_split;
  const int kend = min(nk_seq, kbeg + p.keys_per_split);
  const int qi = qt * BQ + tid;
  const bool valid = qi < nq_seq;

  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (valid) w = *(const f32x4*)(qg + (int64_t)qi * p.tok_stride + d);
    q[d] = w[0]; q[d + 1] = w[1]; q[d + 2] = w[2]; q[d + 3] = w[3];
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const float c = p.scale_log2;

  for (int kt = kbeg; kt < kend; kt += BK) {
    __syncthreads();
    // 64 keys x 64 dims of K and V: 1024 float4 each, 4 per thread
#pragma unroll
    for (int i = tid; i < BK * D / 4; i += NT) {
      const int key = kt + i / (D / 4);
      const int d = 4 * (i % (D / 4));
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (key < kend) {
        a = *(const f32x4*)(kg + (int64_t)key * p.tok_stride + d);
        b = *(const f32x4*)(vg + (int64_t)key * p.tok_stride + d);
      }
      *(f32x4*)&ks[i / (D / 4)][d] = a;
      *(f32x4*)&vs[i / (D / 4)][d] = b;
    }
    __syncthreads();
    const int nvalid = min(BK, kend - kt);
    for (int j = 0; j < nvalid; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], ks[j][d], s);
      const float s2 = s * c;
      if (s2 > m) {
        const float alpha = __builtin_amdgcn_exp2f(m - s2);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        m = s2;
      }
      const float pj = __builtin_amdgcn_exp2f(s2 - m);
      l += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(pj, vs[j][d], acc[d]);
    }
  }

  if (!valid) return;
  if (p.splits == 1) {
    if (p.lse) p.lse[(seq * p.q_seq_stride + qi) * p.H + head] = (m + log2f(l)) * 0.693147180559945309f;
    float* og = (float*)p.o + (seq * p.q_seq_stride + qi) * p.tok_stride + head * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const f32x4 w = {acc[d] / l, acc[d + 1] / l, acc[d + 2] / l, acc[d + 3] / l};
      *(f32x4*)(og + d) = w;
    }
  } else {
    const int64_t row = ((int64_t)split * p.nq_total + (int64_t)seq * p.nq + qi) * p.H + head;
    float* po = p.part_o + row * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const f32x4 w = {acc[d], acc[d + 1], acc[d + 2], acc[d + 3]};
      *(f32x4*)(po + d) = w;
    }
    const f32x2 ml = {m, l};
    *(f32x2*)(p.part_ml + row * 2) = ml;
  }
}

}  // namespace

int attn_f32_query_tile() { return BQ; }

hipError_t launch_attn_f32(const AttnProblem& p, hipStream_t stream) {
  const int ntq = (p.nq + BQ - 1) / BQ;
  const int64_t nwg = (int64_t)ntq * p.H * p.nseq * p.splits;
  if (nwg <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)nwg), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vggt
