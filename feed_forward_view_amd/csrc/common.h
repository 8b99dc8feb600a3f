// Internal declarations shared by the HIP sources of libvggt_attn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vggt {

constexpr int kHeadDim = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 16-byte slot swizzles of the 8 KiB tile images (64 rows of 8 x 16-byte units) that the
// attention kernels copy linearly into LDS: unit u of row r sits at slot u ^ row_swz(r) in
// row tiles (rows are keys or queries) and at slot u ^ col_swz(d) in transposed tiles (rows
// are channels).  The LDS of gfx950 has 64 four-byte banks (two 128-byte rows of the tile per
// bank line).  It serves a ds_read_b128 in four passes of 16 lanes, each pass four 4-lane
// blocks (lanes 4b..4b+3) whose block numbers b share bit 3 and the parity of bits 0-2, and a
// ds_read_b64_tr_b16 in two passes of 32 lanes (the two half-waves); both lane groupings
// were measured with a bank-conflict counter.  The operand reads are
//   * ds_read_b128: lane l reads unit 4c + l/16 of row base + l % 16;
//   * ds_read_b64_tr_b16 (gradient kernels, and the forward kernel's V operand when it reads
//     V rows in place): the lanes of a half-wave read 32 bytes (units 2db, 2db + 1) of each
//     of 8 consecutive rows.
// row_swz = r & 6 makes both conflict-free: in a b128 pass the four blocks cover rows
// {4i..4i+3} of two units of opposite parity, and (r & 1, u ^ (r & 6)) differs for all 16
// lanes; in a transposing half-wave, (r & 1, (r >> 1) & 3) differs for all 8 rows.  col_swz
// serves only b128 reads.
__device__ __forceinline__ int row_swz(int r) { return r & 6; }
__device__ __forceinline__ int col_swz(int d) { return (d >> 1) & 7; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The A operand of a 16x16x32 product whose M dimension is the 64 channels of a row tile
// (rows are keys or queries, 8 x 16-byte units per row, unit u at slot u ^ row_swz(row)):
// channel block db (16 channels) of 32-row chunk c, the chunk's rows in operand order (lane l
// holds channel 16db + l%16 of rows 4(l/16) + 0..3 and 16 + 4(l/16) + 0..3).  Two transposing
// LDS reads: within each 16-lane group, lane 4r + q reads the 8 bytes of channels
// 16db + 4q .. +3 of one row, and lane j of the group receives element j % 4 of lane
// 4r' + j / 4's bytes as its element r', i.e. channel 16db + j of the four rows the group read.
__device__ __forceinline__ bf16x8 read_tr_rows(const u32x4 (&tile)[64][8], int c, int db, int lane) {
  const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int u = 2 * db + (q >> 1);
  u32x2 half[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 32 * c + 16 * h + 4 * g + r;
    const char* src = (const char*)&tile[row][u ^ row_swz(row)] + 8 * (q & 1);
    half[h] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
  }
  return __builtin_bit_cast(bf16x8, u32x4{half[0][0], half[0][1], half[1][0], half[1][1]});
}

// Workgroups are dealt round-robin to the 8 XCDs; this maps the hardware id w
// of nwg workgroups to a logical id such that each XCD receives a contiguous
// run of logical ids (consecutive work shares that XCD's L2).
__device__ __forceinline__ void xcd_remap(int w, int nwg, int& logical) {
  const int q = nwg >> 3, r = nwg & 7;
  const int xcd = w & 7, k = w >> 3;
  logical = (xcd < r) ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// One attention problem as the kernels see it.  Q/K/V/O are [tokens][H][64];
// queries of sequence `s` are tokens [s*q_seq_stride, s*q_seq_stride + nq),
// its keys are tokens [s*k_seq_stride, s*k_seq_stride + nk).  With
// splits > 1 each workgroup covers keys_per_split keys of its sequence and
// writes un-normalised fp32 partial outputs plus (max, sum) per row; a merge
// kernel then combines them.
struct AttnProblem {
  const void* q;
  const void* k;
  const void* v;           // V [tokens][H][64]: fp32 kernel, and bf16 kernel when vt is null
  const void* vt;          // bf16 kernel: V^T tiles [nseq][H][ntile][64][64], or null (V rows
                           // are then read from v in place); K is in p.k as K tiles
  int ktiles_seq;          // bf16 kernel: key tiles per sequence in the tile layouts
  const f32x2* rope_tab;   // [rope_T][32] (cos, sin) applied to Q in the bf16 kernel, or null
  int rope_T;              // token positions repeat every rope_T tokens
  void* o;                 // final output (dtype of the call)
  float* part_o;           // [splits][nq_total][H][64]
  float* part_ml;          // [splits][nq_total][H][2]: (max in log2 units, sum)
  int64_t tok_stride;      // elements between consecutive tokens (= H*64)
  int64_t q_seq_stride;    // tokens between sequence starts of q / o
  int64_t k_seq_stride;    // tokens between sequence starts of k / v (0: all sequences
                           // share one key set, and in the bf16 kernel one set of tiles)
  int64_t nq_total;        // query tokens over all sequences; the last sequence may hold
                           // fewer than nq
  int nq;                  // queries per sequence
  int nk;                  // keys per sequence
  int nk_step;             // > 0: sequence s sees only its first min(nk, (s+1)*nk_step) keys
  int nseq;                // sequences
  int H;                   // heads
  int splits;              // key ranges per sequence
  int keys_per_split;      // multiple of the key tile
  float scale_log2;        // softmax scale * log2(e)
  const float* q_ln_g;     // bf16 kernel: per-head LayerNorm of Q before RoPE (gamma [64]), or null
  const float* q_ln_b;     // beta [64]
  float ln_eps;
  float* lse;              // or null: natural log-normaliser of every query row, [token][H]
};

// Attention gradients (bf16).  Sequences, strides and counts as in
// AttnProblem with nq == nk and q/k sequences T tokens apart (frame) or one
// sequence (global).  Tile buffers: [nseq][H][ntile][64 x 64] row tiles in
// the layout of the forward kernel's K tiles; the kernels read the transposed
// operands they need from these tiles in LDS.
struct AttnBwdProblem {
  const void* q;           // [tokens][H][64] bf16: Q fragments of the dQ kernel
  const void* dout;        // [tokens][H][64] bf16: dO fragments of the dQ kernel
  const void* kr;          // K rotated (bf16): key fragments of the dK/dV kernel
  const void* v;           // V: value fragments of the dK/dV kernel
  const f32x2* rope_tab;   // [rope_T][32] cos/sin or null
  int rope_T;
  const void* k_rows;      // K rotated, row tiles (the forward's K tiles)
  const void* v_rows;      // V, row tiles
  const void* q_rows;      // Q rotated and scaled by scale*log2(e), row tiles
  const void* do_rows;     // dO, row tiles
  const float* lse2;       // [nseq][H][ntile*64]: minus the log2-normaliser of each query row (-inf past the end)
  const float* dsum;       // [nseq][H][ntile*64]: minus rowsum(dO * O) (0 past the end)
  void* dq;                // [tokens][H][64] bf16 outputs
  void* dk;
  void* dv;
  int64_t tok_stride;      // H*64
  int64_t seq_stride;      // tokens between sequence starts (0 for one sequence)
  int nseq, n, H, ntile;   // n tokens per sequence, ntile = ceil(n / 64)
  float scale_log2;        // scale * log2(e)
  float scale;
};

// dq: the dQ kernel, else the dK/dV kernel.
hipError_t launch_attn_bwd_bf16(const AttnBwdProblem& p, bool dq, hipStream_t stream);
// Negated lse2 / dsum of the backward pass from the forward's lse and rowsum(dO * O);
// rows [nseq][H][ntile*64] padded with (-inf, 0).
hipError_t launch_attn_bwd_pre(const void* o, const void* dout, bool bf16, const float* lse, float* lse2,
                               float* dsum, int nseq, int n, int64_t seq_stride, int H, int ntile,
                               hipStream_t stream);
// fp32 debug gradients: one thread per (row, head); q/k already rotated.
hipError_t launch_attn_bwd_f32(const float* qr, const float* kr, const float* v, const float* dout,
                               const float* lse2, const float* dsum, float* dqr, float* dkr, float* dv, int nseq,
                               int n, int64_t seq_stride, int H, int ntile, float scale_log2, float scale,
                               hipStream_t stream);

// Launchers (stream-ordered, no synchronisation).  Return hipSuccess or the
// launch error.
hipError_t launch_attn_bf16(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_merge(const AttnProblem& p, bool out_bf16, hipStream_t stream);
hipError_t launch_rope(const void* src, void* dst, bool bf16, int64_t n_tok, int T, int H, const int32_t* pos_yx,
                       double base, hipStream_t stream, bool inverse = false);
hipError_t launch_rope_table(const int32_t* pos_yx, int T, double base, void* table, hipStream_t stream);
// Where key j (0 <= j < len) of sequence s lives: keys [0, n_main) are rows of
// `main` -- row s*seq_rows + j, or, with frame_len > 0, row s*seq_rows +
// (j / frame_len) * frame_stride + j % frame_len -- and keys [n_main, len) are
// rows j - n_main of `extra`.  Rows are [H][64] elements.
struct KeySrc {
  const void* main = nullptr;
  const void* extra = nullptr;
  int64_t seq_rows = 0;
  int frame_len = 0;
  int64_t frame_stride = 0;
  int64_t n_main = 0;
};
inline KeySrc contiguous_keys(const void* k, int len) {
  KeySrc s;
  s.main = k;
  s.seq_rows = len;
  s.n_main = len;
  return s;
}

// K -> tiles for nseq sequences of len keys (RoPE position of a main row r is
// r % rope_T; extra rows are not rotated), with an optional per-head LayerNorm.
hipError_t launch_k_tiles_bf16(const KeySrc& k, void* kt, int nseq, int len, int H, const void* table, int rope_T,
                               const float* ln_g, const float* ln_b, float ln_eps, hipStream_t stream,
                               float out_scale = 1.0f);
// Per-head LayerNorm of fp32 [n_tok][H][64] (src may equal dst).
hipError_t launch_layer_norm_f32(const float* src, float* dst, int64_t n_tok, int H, const float* g, const float* b,
                                 float eps, hipStream_t stream);
hipError_t launch_v_tiles_bf16(const KeySrc& v, void* vt, int nseq, int len, int H, hipStream_t stream);
// fp32 rows of a key source gathered into a contiguous [nseq*len][H][64] copy.
hipError_t launch_gather_keys_f32(const KeySrc& src, float* dst, int nseq, int len, int H, hipStream_t stream);
// Append n keys (K and V [n][H][64] bf16) to single-sequence tile buffers that own
// dst_ntile tiles per head, at key offset key0; keys of the last tile past key0 + n are
// zeroed, keys below key0 are kept.
hipError_t launch_tiles_append_bf16(const void* k, const void* v, void* kt, void* vt, int dst_ntile, int key0, int n,
                                    int H, hipStream_t stream);
hipError_t launch_pool(const void* k, const void* v, void* kd, void* vd, bool bf16, int S, int T, int H, int gh,
                       int gw, int patch_begin, int ph, int pw, int Dn, hipStream_t stream);

// Query tile of the bf16 kernel and key tile of both kernels (the split size
// must be a multiple of the key tile).
constexpr int kAttnKeyTile = 64;
int attn_bf16_query_tile();
int attn_bf16_workgroups_per_cu();
int attn_f32_query_tile();

}  // namespace vggt
