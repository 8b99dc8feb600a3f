// Operand preparation for the bf16 attention kernel (HBM-bound passes).
//
//  rope_table_kernel  cos/sin of the 32 rotation angles of every in-frame
//                     position: table[t][k], k < 16 turns with the row and
//                     k >= 16 with the column, angle p * base^(-2(k%16)/32)
//                     formed in fp64 and rounded to fp32 (frequency schedule
//                     of the "VGGT 論文報告" slide deck, Section IV, slide
//                     4/6, per axis; rope_base of the VGGT-Omega-1B-512-bf16
//                     config article).
//  k_tiles_kernel     K -> 64-key tiles in an attention kernel's LDS order,
//                     after an optional per-head LayerNorm and rotated by the
//                     table when RoPE is on.
//  v_tiles_kernel     V -> 64-key tiles of V^T in an attention kernel's LDS
//                     order.
// Each tile is 8 KiB and the attention kernels copy it linearly into LDS.
// The order serves their 16x16x32 MFMA operands: row tiles hold their rows in
// order; a transposed tile's unit of 8 rows holds rows 4g..4g+3 and
// 16+4g..16+4g+3 of a 32-row chunk, the order in which a 16x16x32 score block
// pair, read register by register, forms the next product's B operand.
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

// Row of key j of sequence sq in src.main (>= 0), or -1 - (row in src.extra).
__device__ __forceinline__ int64_t key_row(const KeySrc& src, int sq, int64_t j) {
  if (j >= src.n_main) return -1 - (j - src.n_main);
  // keys stay below 2^28 (host check): 32-bit division
  const int64_t r = src.frame_len > 0 ? (int64_t)((int)j / src.frame_len) * src.frame_stride + (int)j % src.frame_len : j;
  return (int64_t)sq * src.seq_rows + r;
}

template <typename T>
__device__ __forceinline__ const T* key_ptr(const KeySrc& src, int64_t row, int64_t row_elems) {
  return row >= 0 ? (const T*)src.main + row * row_elems : (const T*)src.extra + (-1 - row) * row_elems;
}

// Tile key of the first of the two keys that 32-bit word e (0..3) of V^T unit u (0..7) holds:
// unit u holds operand keys 8g .. 8g+7 of chunk c = u / 4 (g = u % 4), which stand for chunk
// keys 4g .. 4g+3 and 16+4g .. 16+4g+3.
__device__ __forceinline__ int vt_word_key(int u, int e) {
  return 32 * (u >> 2) + 4 * (u & 3) + 2 * (e & 1) + 16 * (e >> 1);
}

// K (key j of sequence q at the row given by the KeySrc) -> KT [nseq][H][ntile][64 rows]
// [8 slots of 16 bytes]: row r of tile
// kt holds key 64*kt + r, slot s holds its channels 8u..8u+7 with u = s ^ row_swz(r).
// Source key j lands on tile key key0 + j; tile keys below key0 keep what the buffer
// holds (appending to a filled prefix), tile keys at or past key0 + len become zero.
// With a table, pairs are rotated as in rope_apply_kernel (the position of a key on main
// row r is r % rope_T; extra keys are not rotated).  grid (tiles written, H, nseq); the first
// tile written is key0 / 64 and each (sequence, head) owns dst_ntile tiles.
//
// With ln_g, every key's head vector is first centred and scaled by its per-head
// LayerNorm (gamma ln_g, beta ln_b, eps ln_eps; the 8 lanes that hold one key row
// reduce its 64 channels by xor shuffles), then rotated, then multiplied by out_scale
// and rounded once to bf16.
__global__ __launch_bounds__(NT) void k_tiles_kernel(KeySrc k, u32x4* __restrict__ kt_out,
                                                     int len, int H, const f32x2* __restrict__ table, int rope_T,
                                                     int key0, int dst_ntile, const float* __restrict__ ln_g,
                                                     const float* __restrict__ ln_b, float ln_eps,
                                                     float out_scale) {
  const int tile = key0 / 64 + blockIdx.x, h = blockIdx.y, sq = blockIdx.z;
  u32x4* dst = kt_out + (((int64_t)sq * H + h) * dst_ntile + tile) * 512;
  const int64_t tok_stride = (int64_t)H * kHeadDim;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + c * NT;
    const int r = i >> 3, slot = i & 7;
    const int key = tile * 64 + r - key0;  // source key
    if (key < 0) continue;
    const int u = slot ^ row_swz(r);
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < len) {
      const int64_t row = key_row(k, sq, key);
      w = *(const u32x4*)(key_ptr<uint16_t>(k, row, tok_stride) + h * kHeadDim + 8 * u);
      if (ln_g || (table && row >= 0) || out_scale != 1.0f) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = lo_bf16(w[e]);
          f[2 * e + 1] = hi_bf16(w[e]);
        }
        if (ln_g) {
          // the 8 lanes of this row hold its 8 units: sums over lanes xor 1, 2, 4
          float sum = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) sum += f[j];
          sum += __shfl_xor(sum, 1);
          sum += __shfl_xor(sum, 2);
          sum += __shfl_xor(sum, 4);
          const float mu = sum * (1.0f / kHeadDim);
          float dev = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) dev = __builtin_fmaf(f[j] - mu, f[j] - mu, dev);
          dev += __shfl_xor(dev, 1);
          dev += __shfl_xor(dev, 2);
          dev += __shfl_xor(dev, 4);
          const float inv = 1.0f / __builtin_sqrtf(dev * (1.0f / kHeadDim) + ln_eps);
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = __builtin_fmaf((f[j] - mu) * inv, ln_g[8 * u + j], ln_b[8 * u + j]);
        }
        if (table && row >= 0) {
          // rows stay below 2^28 (host check), so the position is taken in 32 bits
          const int t = (int)row % rope_T;
          const f32x4* tq = (const f32x4*)(table + t * 32 + 4 * u);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x4 cs2 = tq[h2];  // (cos, sin) of pairs 4u + 2h2 and 4u + 2h2 + 1
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              const int e = 2 * h2 + e2;
              const float c = cs2[2 * e2], sn = cs2[2 * e2 + 1];
              if (sn != 0.0f) {
                const float x = f[2 * e], y = f[2 * e + 1];
                f[2 * e] = __builtin_fmaf(x, c, -y * sn);
                f[2 * e + 1] = __builtin_fmaf(x, sn, y * c);
              }
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(f[2 * e] * out_scale, f[2 * e + 1] * out_scale);
      }
    }
    dst[i] = w;
  }
}

// V (rows as for k_tiles_kernel) -> VT [nseq][H][ntile][64 channel rows][8 slots]: slot s of row d
// holds the 8 tile keys of unit u = s ^ col_swz(d) (vt_word_key) of channel d.  Source key j
// lands on tile key key0 + j; tile keys below key0 keep their contents (a slot holding keys on
// both sides of key0 is merged with what the buffer holds), tile keys at or past key0 + len
// become zero.
// grid (tiles written, H, nseq) as for k_tiles_kernel; the 64 x 64 tile is transposed
// through LDS.
__global__ __launch_bounds__(NT) void v_tiles_kernel(KeySrc v, u32x4* __restrict__ vt_out,
                                                     int len, int H, int key0, int dst_ntile) {
  __shared__ uint32_t tile_s[64][33];  // [key][channel pair], padded
  const int tile = key0 / 64 + blockIdx.x, h = blockIdx.y, sq = blockIdx.z;
  const int64_t tok_stride = (int64_t)H * kHeadDim;
  const int kfirst = tile * 64 - key0;  // source key of tile key 0
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + c * NT;
    const int j = i >> 3, u = i & 7;  // tile key, unit of 8 channels
    const int key = kfirst + j;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key >= 0 && key < len)
      w = *(const u32x4*)(key_ptr<uint16_t>(v, key_row(v, sq, key), tok_stride) + h * kHeadDim + 8 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) tile_s[j][4 * u + e] = w[e];
  }
  __syncthreads();
  u32x4* dst = vt_out + (((int64_t)sq * H + h) * dst_ntile + tile) * 512;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = threadIdx.x + c * NT;
    const int d = i >> 3, slot = i & 7;
    const int u = slot ^ col_swz(d);
    const int kept = -kfirst;  // tile keys below this stay as they are
    u32x4 w, keep;
    bool all_kept = true, any_kept = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = vt_word_key(u, e);  // keys j0, j0+1 of channel d
      const uint32_t a = tile_s[j0][d >> 1], b = tile_s[j0 + 1][d >> 1];
      w[e] = (d & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      keep[e] = (j0 + 1 < kept) ? 0xFFFFFFFFu : (j0 < kept ? 0x0000FFFFu : 0u);
      all_kept = all_kept && keep[e] == 0xFFFFFFFFu;
      any_kept = any_kept || keep[e] != 0u;
    }
    if (all_kept) continue;
    if (any_kept) {
      const u32x4 old = dst[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (old[e] & keep[e]) | (w[e] & ~keep[e]);
    }
    dst[i] = w;
  }
}

// fp32 key rows -> contiguous copy [nseq*len][H][64]; one thread per 16-byte unit.
__global__ __launch_bounds__(NT) void gather_keys_f32_kernel(KeySrc src, float* __restrict__ dst, int len, int H,
                                                             int64_t units) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= units) return;
  const int64_t row_units = (int64_t)H * 16;
  const int64_t key = i / row_units;  // over nseq*len
  const int64_t within = i % row_units;
  const int sq = (int)(key / len);
  const int64_t row = key_row(src, sq, key % len);
  const f32x4 w = *(const f32x4*)(key_ptr<float>(src, row, (int64_t)H * kHeadDim) + 4 * within);
  *(f32x4*)(dst + 4 * i) = w;
}

}  // namespace

hipError_t launch_rope_table(const int32_t* pos_yx, int T, double base, void* table, hipStream_t stream) {
  const unsigned blocks = (unsigned)((T * 32 + NT - 1) / NT);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(NT), 0, stream, pos_yx, T, base, (f32x2*)table);
  return hipGetLastError();
}

hipError_t launch_k_tiles_bf16(const KeySrc& k, void* kt, int nseq, int len, int H, const void* table, int rope_T,
                               const float* ln_g, const float* ln_b, float ln_eps, hipStream_t stream,
                               float out_scale) {
  if (nseq <= 0 || len <= 0) return hipSuccess;
  const int ntile = (len + 63) / 64;
  hipLaunchKernelGGL(k_tiles_kernel, dim3((unsigned)ntile, (unsigned)H, (unsigned)nseq), dim3(NT), 0, stream, k,
                     (u32x4*)kt, len, H, (const f32x2*)table, rope_T, 0, ntile, ln_g, ln_b, ln_eps, out_scale);
  return hipGetLastError();
}

hipError_t launch_v_tiles_bf16(const KeySrc& v, void* vt, int nseq, int len, int H, hipStream_t stream) {
  if (nseq <= 0 || len <= 0) return hipSuccess;
  const int ntile = (len + 63) / 64;
  hipLaunchKernelGGL(v_tiles_kernel, dim3((unsigned)ntile, (unsigned)H, (unsigned)nseq), dim3(NT), 0, stream, v,
                     (u32x4*)vt, len, H, 0, ntile);
  return hipGetLastError();
}

hipError_t launch_gather_keys_f32(const KeySrc& src, float* dst, int nseq, int len, int H, hipStream_t stream) {
  const int64_t units = (int64_t)nseq * len * H * 16;  // 16-byte units
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_keys_f32_kernel, dim3((unsigned)((units + NT - 1) / NT)), dim3(NT), 0, stream, src, dst,
                     len, H, units);
  return hipGetLastError();
}

hipError_t launch_tiles_append_bf16(const void* k, const void* v, void* kt, void* vt, int dst_ntile, int key0, int n,
                                    int H, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int tiles = (key0 + n - 1) / 64 - key0 / 64 + 1;
  hipLaunchKernelGGL(k_tiles_kernel, dim3((unsigned)tiles, (unsigned)H, 1u), dim3(NT), 0, stream,
                     contiguous_keys(k, n), (u32x4*)kt, n, H, (const f32x2*)nullptr, 1, key0, dst_ntile,
                     (const float*)nullptr, (const float*)nullptr, 0.0f, 1.0f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v_tiles_kernel, dim3((unsigned)tiles, (unsigned)H, 1u), dim3(NT), 0, stream,
                     contiguous_keys(v, n), (u32x4*)vt, n, H, key0, dst_ntile);
  return hipGetLastError();
}

}  // namespace vggt
