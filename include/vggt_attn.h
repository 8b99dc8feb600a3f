/*
 * vggt_attn.h -- C ABI of the MI355X (gfx950) alternating-attention library
 * for VGGT-style feed-forward reconstruction models.
 *
 * The aggregator of these models alternates two softmax attentions over the
 * tokens of S frames (the "VGGT 論文報告" slide deck, Section XI "架構",
 * slide 3/7, "Global + Frame Attention"; the VGGT-JAX README's attention
 * kernel-trial table shows them as [S, T, 16, 64] frame and [1, S*T, 16, 64]
 * global attention):
 *   - frame attention: each frame's T tokens attend to that frame only;
 *   - global attention: all S*T tokens attend to all S*T tokens.
 * The FlashVGGT variant (FlashVGGT README, "Overview") replaces global
 * attention by cross-attention from every token to a compact per-frame set of
 * spatially pooled descriptor keys/values.
 *
 * Tensor layout (every call): contiguous row-major [S, T, H, 64], i.e. token
 * t of frame s, head h, channel c lives at ((s*T + t)*H + h)*64 + c.  The
 * frame view and the global view are the same memory.  Head dim is 64
 * (embed 1024 = 16 heads x 64, VGGT-Omega config article, field table).
 *
 * Element types: VGGT_BF16 (bf16 in/out, fp32 accumulation and softmax) or
 * VGGT_F32 (fp32 in/out, fp32 arithmetic throughout; a debug mode for tight
 * numerical comparison).
 *
 * Conventions for every call:
 *   - Ownership: the caller owns all device buffers, including the workspace
 *     sized by the matching *_workspace() query.  The compute calls never
 *     allocate, free or synchronise.  The diagnostic kernel timer is the one
 *     exception: vggt_timer_start creates HIP events (2 per armed launch) and
 *     vggt_timer_stop waits for them and destroys them.
 *   - Streams: `stream` is a hipStream_t passed as void*; NULL means the null
 *     stream.  Work is enqueued asynchronously on it.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a failed check returns a status, enqueues nothing and leaves
 *     outputs untouched.  A failed launch returns VGGT_ERR_DEVICE; the detail
 *     is in vggt_last_error() (thread-local).  No C++ exception crosses the ABI.
 *   - Pointers: device pointers, 16-byte aligned.  Outputs must not overlap
 *     inputs (VGGT_ERR_ALIAS), except that vggt_attn_rope works in place.
 *   - Device: the current HIP device must be gfx950 (VGGT_ERR_UNSUPPORTED).
 *   - Reentrancy: calls are reentrant; calls that share a workspace must be
 *     ordered on one stream by the caller.
 *   - Empty calls: S = 0 (n = 0 for vggt_descriptor_cache_append, nq = 0 for
 *     vggt_descriptor_cache_attn) is valid once the dtype and the other sizes
 *     pass their checks: the call returns VGGT_OK without reading any pointer
 *     or touching the device, and the workspace queries return 0.  The one
 *     exception is vggt_global_attn_ex with n_extra > 0 and S = 0, which is
 *     VGGT_ERR_SHAPE.
 *   - Running time (bf16 forward calls): the kernel first computes every
 *     row's softmax against a fixed reference and checks, at the end, each
 *     row's sum and that its un-normalised output stayed finite.  A workgroup
 *     with a row outside the range recomputes its 256 rows exactly, taking up
 *     to about 2.4x the usual time.  Such a row has a largest logit above
 *     about 50 or all logits below about -40 (natural units, scale included),
 *     or large values: weights up to 2^100 times |V| overflow float32 once
 *     |V| exceeds about 2^28.  Results are the same softmax either way, up to
 *     rounding.
 *   - Value range: the exact recomputation keeps every weight in (0, 1], so
 *     its float32 accumulators hold at most (keys) * max|V|; outputs are
 *     finite and exact up to rounding for max|V| * keys below 2^127.
 */
#ifndef VGGT_ATTN_H
#define VGGT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VGGT_ATTN_ABI_VERSION 6
#define VGGT_HEAD_DIM 64

typedef enum {
  VGGT_OK = 0,
  VGGT_ERR_NULL = 1,        /* a required pointer is NULL */
  VGGT_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  VGGT_ERR_UNSUPPORTED = 3, /* unsupported dtype or device (not gfx950) */
  VGGT_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  VGGT_ERR_ALIAS = 5,       /* an output overlaps an input */
  VGGT_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
  VGGT_ERR_DEVICE = 7       /* a HIP call failed; see vggt_last_error() */
} vggt_status;

typedef enum { VGGT_BF16 = 0, VGGT_F32 = 1 } vggt_dtype;

/* Returns VGGT_ATTN_ABI_VERSION of the built library. */
int vggt_abi_version(void);
/* Static string naming a status code. */
const char* vggt_status_str(int status);
/* Thread-local detail of the last failure on this thread ("" if none). */
const char* vggt_last_error(void);

/*
 * 2D rotary position embedding, in place.
 * Source: VGGT-Omega-1B-512-bf16 config article, input-parameter section
 * (rope_base 100; the RoPE frequency buffers are fp32); frequency schedule of
 * the "VGGT 論文報告" slide deck, Section IV, slide 4/6 (pair i of a width-d
 * axis turns at pos / base^(2i/d)).
 *   x       [S, T, H, 64] device, dtype dt; rotated in place.
 *   pos_yx  [T, 2] int32 device: (row, col) of token t in every frame.
 *   base    rope base (> 0).
 * Channels 0..31 rotate by the row, 32..63 by the column; pair (2k, 2k+1) of
 * a half turns by p * base^(-2k/32), k = 0..15.  Position (0, 0) is the
 * identity, bit for bit.  Angles are formed in fp64, cos/sin rounded to fp32,
 * the rotation done in fp32 and stored with round-to-nearest-even.
 */
vggt_status vggt_attn_rope(void* x, vggt_dtype dt, int S, int T, int H, const int32_t* pos_yx, float base,
                           void* stream);

/* Flags of the workspace queries' `rope_on` argument: bit 0 = positions are
 * passed (RoPE), bit 1 = a vggt_qk_norm is passed (Q/K LayerNorm).  Any other
 * nonzero value than these bits reads as RoPE only, as before. */
#define VGGT_PRE_ROPE 1
#define VGGT_PRE_QKNORM 2

/*
 * Per-head LayerNorm of Q and K applied before RoPE (VGGT-JAX README,
 * kernel-trial table: LayerNorm over the Q/K shapes, centred fp32 LayerNorm
 * kept; VGGT-Omega-1B-512-bf16 config article: layer_norm_eps 1e-05).  For
 * each token and head, over its 64 channels:
 *   u' = (u - mean(u)) / sqrt(var(u) + eps) * gamma + beta   (biased variance)
 * gamma/beta: [64] float32 device arrays shared by all heads; eps > 0.
 * Computed in fp32 inside the K tile pre-pass and the attention kernel's Q
 * prologue (fp32 debug mode: a separate pass into the rotated copies); the
 * normalised and rotated values are rounded to bf16 once.
 */
typedef struct {
  const float* q_gamma;
  const float* q_beta;
  const float* k_gamma;
  const float* k_beta;
  float eps;
} vggt_qk_norm;

/*
 * Frame-wise attention: S independent sequences of T tokens (slide deck
 * Section XI, slide 3/7; Section V, slide 5/10 for softmax(Q K^T / sqrt(d)) V,
 * slide 9/10 for independent heads).  No mask.
 *   q, k, v [S, T, H, 64] device, dtype dt (read only).
 *   o       [S, T, H, 64] device, dtype dt (written).
 *   pos_yx  [T, 2] int32 device or NULL (NULL: no RoPE); with positions, q
 *           and k are rotated as in vggt_attn_rope before the product.
 *   scale   softmax scale; <= 0 selects 1/sqrt(64) = 0.125.
 *   workspace: device scratch of at least vggt_frame_attn_workspace(...) bytes
 *           (may be NULL when that is 0).
 */
size_t vggt_frame_attn_workspace(int S, int T, int H, int rope_on, vggt_dtype dt);
vggt_status vggt_frame_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T,
                            int H, const int32_t* pos_yx, float rope_base, float scale, void* workspace,
                            size_t ws_bytes, void* stream);

/*
 * vggt_frame_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * vggt_frame_attn; the workspace is a library-owned device array of
 * VGGT_NOALLOC_SCRATCH_BYTES on each device that calls it, held until the
 * process ends.  The call itself allocates, frees and synchronises nothing.
 *   Limit: vggt_frame_attn_workspace(S, T, H, pos_yx != NULL, dt) must not
 *   exceed VGGT_NOALLOC_SCRATCH_BYTES, else VGGT_ERR_WORKSPACE before anything
 *   is enqueued (bf16 with RoPE: S * H * ceil(T / 64) <= about 8000 for
 *   frames under 8192 tokens, e.g. 22 frames of 1374 tokens x 16 heads; about
 *   4000 for longer frames, whose V also goes through a tile pre-pass).
 *   Every call on one device uses the same array: calls that may overlap on
 *   one device (different streams without ordering) race; order them.
 */
#define VGGT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
vggt_status vggt_frame_attn_noalloc(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                    int T, int H, const int32_t* pos_yx, float rope_base, float scale, void* stream);
/* The same with the Q/K LayerNorm prologue (norm: host pointer, NULL = none;
 * the workspace is sized with rope_on = VGGT_PRE_QKNORM | (RoPE ? VGGT_PRE_ROPE : 0)).
 * VGGT_ERR_NULL if a parameter array is NULL, VGGT_ERR_SHAPE if eps <= 0,
 * VGGT_ERR_ALIAS if a parameter array overlaps o or the workspace. */
vggt_status vggt_frame_attn_qknorm(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T,
                                   int H, const int32_t* pos_yx, float rope_base, float scale,
                                   const vggt_qk_norm* norm, void* workspace, size_t ws_bytes, void* stream);

/*
 * Global attention over all N = S*T tokens (slide deck Section XI, slide 3/7;
 * Section V, slides 5/10 and 9/10).  Each token keeps its within-frame
 * position for RoPE (frames carry no index of their own).
 *   Arguments as for vggt_frame_attn, plus
 *   kv_splits  number of key ranges computed by separate workgroups and merged
 *              exactly by log-sum-exp; 0 lets the library choose (1..64) from
 *              the shape and the current device's CU count, so a workspace
 *              query and its call must see the same current device.
 */
size_t vggt_global_attn_workspace(int S, int T, int H, int kv_splits, int rope_on, vggt_dtype dt);
vggt_status vggt_global_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T,
                             int H, const int32_t* pos_yx, float rope_base, float scale, int kv_splits,
                             void* workspace, size_t ws_bytes, void* stream);
/* The same with the Q/K LayerNorm prologue, as for vggt_frame_attn_qknorm. */
vggt_status vggt_global_attn_qknorm(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T,
                                    int H, const int32_t* pos_yx, float rope_base, float scale, int kv_splits,
                                    const vggt_qk_norm* norm, void* workspace, size_t ws_bytes, void* stream);

/*
 * VGGT-Omega block variants (VGGT-Omega-1B-512-bf16 config article, field
 * table and special-token notes: 16 register tokens follow each frame's
 * patches and join attention only in blocks 2, 6, 9, 14 and 20; 4 storage
 * tokens are shared by all frames as global memory; one camera token gathers
 * the camera information of every frame).
 *
 * Tokens keep the [S, T, H, 64] layout; only the first T_active tokens of each
 * frame take part (1 <= T_active <= T; T_active = T - 16 in the blocks without
 * registers).  Rows T_active..T-1 of every frame of o are left untouched.
 *
 * vggt_frame_attn_ex: each frame's active tokens attend to that frame's
 * active tokens.
 *
 * vggt_global_attn_ex: the token set is every frame's active tokens, in frame
 * order, followed by n_extra sequence-level tokens (xq, xk, xv, xo
 * [n_extra, H, 64], dtype dt; NULL allowed when n_extra == 0).  Every token of
 * the set is a query and a key.  Extra tokens carry no position (identity
 * rotation); the LayerNorm, if given, applies to them too.  kv_splits applies
 * to the frame tokens' queries; the extra tokens' queries (a separate launch
 * over the same prepared keys) always use the library's split choice.
 * n_extra in [0, 4096], and 0 when S = 0.  No output may overlap an input
 * (VGGT_ERR_ALIAS).
 *
 * Positions, scale, norm (NULL = none) and the workspace are as for
 * vggt_frame_attn_qknorm; `flags` of the workspace queries are
 * VGGT_PRE_ROPE | VGGT_PRE_QKNORM as used by the call.
 */
size_t vggt_frame_attn_ex_workspace(int S, int T, int T_active, int H, int flags, vggt_dtype dt);
vggt_status vggt_frame_attn_ex(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T,
                               int T_active, int H, const int32_t* pos_yx, float rope_base, float scale,
                               const vggt_qk_norm* norm, void* workspace, size_t ws_bytes, void* stream);
size_t vggt_global_attn_ex_workspace(int S, int T, int T_active, int n_extra, int H, int kv_splits, int flags,
                                     vggt_dtype dt);
vggt_status vggt_global_attn_ex(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T,
                                int T_active, int H, const void* xq, const void* xk, const void* xv, void* xo,
                                int n_extra, const int32_t* pos_yx, float rope_base, float scale, int kv_splits,
                                const vggt_qk_norm* norm, void* workspace, size_t ws_bytes, void* stream);

/*
 * Training support: the forward pass that also saves each query row's
 * log-normaliser, and the gradients of frame and global attention (the chain
 * rule through softmax(Q K^T * scale) V of the slide deck, Section V, slide
 * 5/10, with RoPE as in vggt_attn_rope; the VGGT-JAX README trains and checks
 * gradients of this attention).
 *
 * vggt_frame_attn_train / vggt_global_attn_train: as vggt_frame_attn /
 * vggt_global_attn, and lse [S*T, H] float32 (device, written) receives
 * log(sum_j exp(scale * <q'_i, k'_j>)) of every query row (natural log; q', k'
 * rotated).  lse must not overlap another buffer (VGGT_ERR_ALIAS).
 *
 * vggt_frame_attn_backward / vggt_global_attn_backward: given q, k, v, the
 * forward output o, its upstream gradient dout (all [S, T, H, 64], dtype dt)
 * and lse from the training forward, write dq, dk, dv [S, T, H, 64] (dtype
 * dt): the gradients with respect to the unrotated q and k and to v.  bf16:
 * products in bf16 on the matrix cores with fp32 accumulation (probabilities
 * and score gradients rounded to bf16 before their products); fp32: fp32
 * throughout (debug).  Workspace of vggt_attn_backward_workspace(S, T, H,
 * global, rope_on, dt) bytes.  The gradients must not overlap any input, lse,
 * the workspace or each other.  No LayerNorm prologue in the backward.
 */
vggt_status vggt_frame_attn_train(const void* q, const void* k, const void* v, void* o, float* lse, vggt_dtype dt,
                                  int S, int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                  void* workspace, size_t ws_bytes, void* stream);
vggt_status vggt_global_attn_train(const void* q, const void* k, const void* v, void* o, float* lse, vggt_dtype dt,
                                   int S, int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                   int kv_splits, void* workspace, size_t ws_bytes, void* stream);
size_t vggt_attn_backward_workspace(int S, int T, int H, int global, int rope_on, vggt_dtype dt);
vggt_status vggt_frame_attn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                     const float* lse, void* dq, void* dk, void* dv, vggt_dtype dt, int S, int T,
                                     int H, const int32_t* pos_yx, float rope_base, float scale, void* workspace,
                                     size_t ws_bytes, void* stream);
vggt_status vggt_global_attn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                      const float* lse, void* dq, void* dk, void* dv, vggt_dtype dt, int S, int T,
                                      int H, const int32_t* pos_yx, float rope_base, float scale, void* workspace,
                                      size_t ws_bytes, void* stream);

/*
 * FlashVGGT descriptor pooling (FlashVGGT README, "Overview": each frame's
 * spatial information is compressed into a compact descriptor set; "Key
 * Arguments": --kv_downfactor, default 4, taken here as a ph x pw = 2 x 2
 * token-count factor).
 *   k, v    [S, T, H, 64] device, dtype dt; the patch grid is tokens
 *           [patch_begin, patch_begin + gh*gw) of each frame, row-major.
 *   kd, vd  [S, Dn, H, 64] device, Dn = vggt_descriptor_count(T, gh, gw, ph, pw):
 *           first the T - gh*gw special tokens copied in order, then one
 *           descriptor per ph x pw window (row-major over ceil(gh/ph) x
 *           ceil(gw/pw) windows) holding the mean of the window's cells that
 *           lie inside the grid.  Sums in fp32, stored with round-to-nearest-even.
 */
int vggt_descriptor_count(int T, int gh, int gw, int ph, int pw);
vggt_status vggt_descriptor_pool(const void* k, const void* v, void* kd, void* vd, vggt_dtype dt, int S, int T,
                                 int H, int gh, int gw, int patch_begin, int ph, int pw, void* stream);

/*
 * FlashVGGT descriptor cross-attention (FlashVGGT README, "Overview": global
 * attention becomes cross-attention between all image tokens and the smaller
 * descriptor set).  All S*T query tokens attend to all S*Dn descriptors; no
 * RoPE inside (rotate q and k with vggt_attn_rope before pooling if wanted).
 *   q   [S, T, H, 64]; kd, vd [S, Dn, H, 64]; o [S, T, H, 64]; dtype dt.
 *   scale, kv_splits, workspace as for vggt_global_attn.
 */
size_t vggt_descriptor_xattn_workspace(int S, int T, int Dn, int H, int kv_splits, vggt_dtype dt);
vggt_status vggt_descriptor_xattn(const void* q, const void* kd, const void* vd, void* o, vggt_dtype dt, int S,
                                  int T, int Dn, int H, float scale, int kv_splits, void* workspace,
                                  size_t ws_bytes, void* stream);

/*
 * FlashVGGT chunk-recursive (streaming) descriptor attention (FlashVGGT README,
 * "Overview": online inference over long sequences reuses the cached
 * descriptors of earlier chunks; "Key Arguments": --chunksize, frames per
 * chunk, default 10).  Frames arrive in chunks; after chunk c has been pooled
 * and appended, the queries of chunk c attend to every descriptor cached so
 * far (chunks 0..c, own chunk included), in frame order.
 *
 * A descriptor cache is caller-owned device memory of
 * vggt_descriptor_cache_bytes(capacity, H, dt) bytes (256-byte aligned) for up
 * to `capacity` descriptors of H heads, kept in the layout the attention
 * kernels read, so that attending to it needs no per-call preparation:
 *   VGGT_BF16: K and V in 64-descriptor tiles (K rows, V transposed), the
 *              slots past the last appended descriptor of a tile zeroed;
 *   VGGT_F32 : K [capacity][H][64] followed by V [capacity][H][64], float32.
 * Its contents are defined only for the descriptors appended so far; the
 * caller keeps that count (`used`).  Appends and attention calls on one cache
 * must be ordered on one stream.
 */
size_t vggt_descriptor_cache_bytes(int capacity, int H, vggt_dtype dt);

/*
 * Append n descriptors (kd, vd [n, H, 64] device, dtype dt: e.g. the output of
 * vggt_descriptor_pool for a chunk of frames, [S_chunk, Dn, H, 64]) at
 * positions used .. used+n-1 of the cache.  Requires 0 <= used and
 * used + n <= capacity (VGGT_ERR_SHAPE otherwise).  Descriptors below `used`
 * are left as they are; kd/vd must not overlap the cache (VGGT_ERR_ALIAS).
 */
vggt_status vggt_descriptor_cache_append(void* cache, vggt_dtype dt, int capacity, int H, int used, const void* kd,
                                         const void* vd, int n, void* stream);

/*
 * nq query tokens (q [nq, H, 64]) attend to the first `used` cached
 * descriptors (1 <= used <= capacity); o [nq, H, 64].  No RoPE inside.
 * scale and kv_splits as for vggt_global_attn; workspace of at least
 * vggt_descriptor_cache_attn_workspace(nq, used, H, kv_splits, dt) bytes.
 * o must not overlap q, the cache or the workspace.
 */
size_t vggt_descriptor_cache_attn_workspace(int nq, int used, int H, int kv_splits, vggt_dtype dt);
vggt_status vggt_descriptor_cache_attn(const void* q, const void* cache, void* o, vggt_dtype dt, int capacity, int H,
                                       int used, int nq, float scale, int kv_splits, void* workspace,
                                       size_t ws_bytes, void* stream);

/*
 * Every chunk at once, in one launch: the cache holds the descriptors of all S
 * frames (S*Dn <= capacity, appended in frame order from position 0); the
 * query tokens of frames [c*F, min(S, (c+1)*F)) attend to the descriptors of
 * frames [0, min(S, (c+1)*F)), F = chunk_frames >= 1.  The result equals S/F
 * streaming steps.  q, o [S, T, H, 64]; no workspace.
 */
vggt_status vggt_descriptor_chunked_xattn(const void* q, const void* cache, void* o, vggt_dtype dt, int capacity,
                                          int H, int S, int T, int Dn, int chunk_frames, float scale, void* stream);

/*
 * Diagnostics: device-side timing of the attention kernel of each call, for
 * measuring the kernel on its own (its key-tile preparation, RoPE table and
 * split-merge passes are not included).  Nothing here is needed to compute.
 *
 * vggt_timer_start(capacity) creates 2*capacity HIP events on the current
 * device and arms the timer: each later attention kernel launch on that
 * device (by vggt_frame_attn, vggt_global_attn, vggt_descriptor_xattn,
 * vggt_descriptor_cache_attn or vggt_descriptor_chunked_xattn, their _qknorm,
 * _ex and _train forms, and the two kernels of the bf16 backward), up to
 * `capacity` of them, is bracketed by two events recorded on the call's
 * stream.  capacity in [1, 2^20]; VGGT_ERR_SHAPE if the timer is already
 * running.
 *
 * vggt_timer_stop(ms, kinds, n_max, n_recorded) waits for the recorded
 * events, writes the first min(n_max, recorded) durations in milliseconds and
 * call kinds (vggt_timer_kind) in launch order, stores the number recorded in
 * *n_recorded (if not NULL), then disarms the timer and destroys its events.
 * VGGT_ERR_SHAPE if the timer is not running.  One timer per process; calls
 * made from several threads while it is armed are recorded in the order they
 * claim a slot.
 */
typedef enum {
  VGGT_TIMER_FRAME = 1,
  VGGT_TIMER_GLOBAL = 2,
  VGGT_TIMER_XATTN = 3,
  VGGT_TIMER_CACHE = 4,
  VGGT_TIMER_CHUNKED = 5,
  VGGT_TIMER_BWD_DQ = 6,   /* bf16 backward: the dQ kernel */
  VGGT_TIMER_BWD_DKDV = 7  /* bf16 backward: the dK/dV kernel */
} vggt_timer_kind;
vggt_status vggt_timer_start(int capacity);
vggt_status vggt_timer_stop(float* ms, int* kinds, int n_max, int* n_recorded);

#ifdef __cplusplus
}
#endif

#endif /* VGGT_ATTN_H */
