// C ABI of libvggt_attn: host-side validation, workspace layout and launch
// sequencing.  Every check runs before anything is enqueued; a failed check
// enqueues nothing.  See include/vggt_attn.h for the contract of each call.
#include "vggt_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

#define VGGT_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

vggt_status fail(vggt_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

constexpr int kMaxHeads = 128;
constexpr int64_t kMaxTokens = int64_t(1) << 28;
constexpr int kMaxSplits = 64;
constexpr int kDefaultCUs = 256;  // MI355X; the split plan's CU count if the device cannot be queried

// ---- device check, cached per device (read-only after first use)
struct DevInfo {
  bool checked = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

vggt_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VGGT_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(VGGT_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(VGGT_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = true;
  }
  if (!d.gfx950) return fail(VGGT_ERR_UNSUPPORTED, "current device is not gfx950");
  return VGGT_OK;
}

// CU count of the current device (cached with the device check); sizes the key split
int current_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return kDefaultCUs;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = true;
  }
  return d.cus > 0 ? d.cus : kDefaultCUs;
}

size_t elem_size(vggt_dtype dt) { return dt == VGGT_F32 ? 4 : 2; }
bool dtype_ok(vggt_dtype dt) { return dt == VGGT_BF16 || dt == VGGT_F32; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

bool tokens_ok(int S, int T, int H) {
  if (S < 0 || T < 1 || H < 1 || H > kMaxHeads) return false;
  return (int64_t)S * T < kMaxTokens;
}

// ---- key-split plan (a function of the shape and the current device's CU
//      count, shared by the workspace queries and the calls)
struct SplitPlan {
  int splits;
  int keys_per_split;
};

int query_tile(vggt_dtype dt) { return dt == VGGT_F32 ? vggt::attn_f32_query_tile() : vggt::attn_bf16_query_tile(); }

SplitPlan plan_splits(int64_t nq, int64_t nk, int H, int requested, vggt_dtype dt) {
  const int kt = vggt::kAttnKeyTile;
  const int64_t ktiles = (nk + kt - 1) / kt;
  int splits = 1;
  if (requested > 0) {
    splits = requested;
  } else if (nk > 0 && nq > 0) {
    // Balance the last round of workgroups against the merge pass.  Time is
    // modelled in units of one key tile processed by one resident workgroup.
    // Workgroups run in rounds of `slots`; a last round at most half full runs
    // one workgroup per CU, which finishes in about half a round, while a
    // fuller one still pairs workgroups on some CUs and takes a whole round
    // (measured over global attention at 6 to 40 frames of 1374 tokens):
    //   attention(s) = ceil(ktiles / s) * (full rounds + tail)
    //   merge(s)     = partial bytes / (bytes one slot-tile-time moves), s > 1
    const int64_t wg = ((nq + query_tile(dt) - 1) / query_tile(dt)) * H;
    // resident workgroups per CU: the bf16 kernel's declared occupancy; the untuned fp32
    // debug kernel is planned with the same two
    const int per_cu = dt == VGGT_F32 ? 2 : vggt::attn_bf16_workgroups_per_cu();
    const int64_t slots = (int64_t)current_cus() * per_cu;
    double best = 1e300;
    for (int s = 1; s <= kMaxSplits && s <= ktiles; ++s) {
      const double rounds = (double)(wg * s) / (double)slots;
      const double full = std::floor(rounds), part = rounds - full;
      const double tail = part <= 0.0 ? 0.0 : (part <= 0.5 ? 0.5 : 1.0);
      const double att = (double)((ktiles + s - 1) / s) * (full + tail);
      // one tile-time ~ 1.8 us; merge moves s*nq*H*(64+2)*4 bytes twice plus
      // the output, at ~5 TB/s -> bytes / (5e6 B/us) / 1.8 us
      const double bytes = s > 1 ? (double)nq * H * (2.0 * s * 66 * 4 + 64 * 2) : 0.0;
      const double cost = att + bytes / 5.0e6 / 1.8;
      if (cost < best - 1e-9) {
        best = cost;
        splits = s;
      }
    }
  }
  if (splits > ktiles) splits = (int)std::max<int64_t>(1, ktiles);
  const int64_t tiles_per = (ktiles + splits - 1) / splits;
  SplitPlan p;
  p.keys_per_split = (int)(tiles_per * kt);
  p.splits = (int)((nk + p.keys_per_split - 1) / p.keys_per_split);
  if (p.splits < 1) p.splits = 1;
  return p;
}

// ---- diagnostics: device-side timing of attention kernel launches (armed by
//      vggt_timer_start; one timer per process)
struct KernelTimer {
  std::mutex mu;
  bool armed = false;
  int device = -1;
  int next = 0;
  std::vector<hipEvent_t> ev;  // two per slot
  std::vector<int> kind;
};
KernelTimer g_timer;

// Claims the next slot for a launch of `kind` on the current device, or -1.
int timer_claim(int kind) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.armed || g_timer.next >= (int)g_timer.kind.size()) return -1;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != g_timer.device) return -1;
  g_timer.kind[g_timer.next] = kind;
  return g_timer.next++;
}

hipError_t run_attention(const vggt::AttnProblem& p, vggt_dtype dt, hipStream_t st, int kind) {
  const int slot = timer_claim(kind);
  hipError_t e = hipSuccess;
  if (slot >= 0) e = hipEventRecord(g_timer.ev[2 * slot], st);
  if (e != hipSuccess) return e;
  e = dt == VGGT_F32 ? vggt::launch_attn_f32(p, st) : vggt::launch_attn_bf16(p, st);
  if (e != hipSuccess) return e;
  if (slot >= 0) e = hipEventRecord(g_timer.ev[2 * slot + 1], st);
  if (e != hipSuccess) return e;
  if (p.splits > 1) e = vggt::launch_attn_merge(p, dt == VGGT_BF16, st);
  return e;
}

float scale_log2(float scale) {
  const double s = scale > 0.0f ? (double)scale : 0.125;
  return (float)(s * 1.4426950408889634074);  // log2(e)
}

vggt_status device_error(const char* what, hipError_t e) {
  return fail(VGGT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

VGGT_API int vggt_abi_version(void) { return VGGT_ATTN_ABI_VERSION; }

VGGT_API const char* vggt_status_str(int s) {
  switch (s) {
    case VGGT_OK: return "VGGT_OK";
    case VGGT_ERR_NULL: return "VGGT_ERR_NULL";
    case VGGT_ERR_SHAPE: return "VGGT_ERR_SHAPE";
    case VGGT_ERR_UNSUPPORTED: return "VGGT_ERR_UNSUPPORTED";
    case VGGT_ERR_ALIGN: return "VGGT_ERR_ALIGN";
    case VGGT_ERR_ALIAS: return "VGGT_ERR_ALIAS";
    case VGGT_ERR_WORKSPACE: return "VGGT_ERR_WORKSPACE";
    case VGGT_ERR_DEVICE: return "VGGT_ERR_DEVICE";
    default: return "VGGT_ERR_UNKNOWN";
  }
}

VGGT_API const char* vggt_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------------------
// RoPE
// ---------------------------------------------------------------------------

VGGT_API vggt_status vggt_attn_rope(void* x, vggt_dtype dt, int S, int T, int H, const int32_t* pos_yx, float base,
                                    void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (!(base > 0.0f) || !std::isfinite(base)) return fail(VGGT_ERR_SHAPE, "rope base must be finite and > 0");
  if (S == 0) return VGGT_OK;
  if (!x || !pos_yx) return fail(VGGT_ERR_NULL, "x and pos_yx are required");
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(pos_yx) & 3u)) return fail(VGGT_ERR_ALIGN, "misaligned pointer");
  const size_t bytes = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  if (overlap(x, bytes, pos_yx, (size_t)T * 8)) return fail(VGGT_ERR_ALIAS, "pos_yx overlaps x");
  if (vggt_status s = check_device()) return s;
  hipError_t e = vggt::launch_rope(x, x, dt == VGGT_BF16, (int64_t)S * T, T, H, pos_yx, (double)base,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return device_error("rope launch", e);
  return VGGT_OK;
}

// ---------------------------------------------------------------------------
// Frame and global attention
// ---------------------------------------------------------------------------

namespace {

struct QKVO {
  const void *q, *k, *v;
  void* o;
};

vggt_status validate_attn(const QKVO& t, const int32_t* pos, float base, size_t need_ws, const void* ws,
                          size_t ws_bytes, size_t q_bytes, size_t kv_bytes) {
  if (!t.q || !t.k || !t.v || !t.o) return fail(VGGT_ERR_NULL, "q, k, v and o are required");
  if (!aligned16(t.q) || !aligned16(t.k) || !aligned16(t.v) || !aligned16(t.o))
    return fail(VGGT_ERR_ALIGN, "q/k/v/o must be 16-byte aligned");
  if (pos && (reinterpret_cast<uintptr_t>(pos) & 3u)) return fail(VGGT_ERR_ALIGN, "pos_yx must be 4-byte aligned");
  if (pos && (!(base > 0.0f) || !std::isfinite(base))) return fail(VGGT_ERR_SHAPE, "rope base must be finite and > 0");
  if (overlap(t.o, q_bytes, t.q, q_bytes) || overlap(t.o, q_bytes, t.k, kv_bytes) ||
      overlap(t.o, q_bytes, t.v, kv_bytes))
    return fail(VGGT_ERR_ALIAS, "o overlaps q, k or v");
  if (need_ws > 0) {
    if (!ws) return fail(VGGT_ERR_WORKSPACE, "workspace of %zu bytes required", need_ws);
    if (ws_bytes < need_ws) return fail(VGGT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need_ws);
    if (!aligned16(ws)) return fail(VGGT_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (overlap(ws, need_ws, t.q, q_bytes) || overlap(ws, need_ws, t.k, kv_bytes) ||
        overlap(ws, need_ws, t.v, kv_bytes) || overlap(ws, need_ws, t.o, q_bytes))
      return fail(VGGT_ERR_ALIAS, "workspace overlaps a tensor");
  }
  return VGGT_OK;
}

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

// The bf16 kernel reads V rows in place (no V^T pre-pass) when fewer than this many query
// tiles share a key set.  The pre-pass costs one read and one write of V; reading in place
// costs twice the LDS reads of the V operand in every query tile, about 2% of the kernel's
// time (measured at 6 query tiles per key set, frame attention at T = 1374, where reading in
// place saves 4% of the call, and at 172, global attention at N = 43968, where it costs 1.5%).
constexpr int kVInPlaceMaxQueryTiles = 32;
bool v_in_place(int64_t nq) {
  const int bq = vggt::attn_bf16_query_tile();
  return (nq + bq - 1) / bq < kVInPlaceMaxQueryTiles;
}

// Workspace layout of one attention call.  bf16: RoPE table, rotated K and,
// unless V is read in place, transposed V for the matrix-core kernel; fp32:
// rotated copies of Q and K.  Both: split partials.  Offsets are 256-byte
// aligned.
struct Layout {
  size_t table = 0, qr = 0, kr = 0, kt = 0, vt = 0, part_o = 0, part_ml = 0, total = 0;
  bool use_table = false, use_qr = false, use_kr = false, use_vt = false;
  int ktiles = 0;  // bf16: key tiles of 64 per sequence
  SplitPlan sp{1, 0};
};

void add(Layout& L, size_t& off, size_t bytes) {
  off = L.total;
  L.total += align256(bytes);
}

// nseq sequences of nq queries and nk keys; q tensor has nseq*nq tokens,
// k/v tensors nseq*nk tokens; positions repeat every rope_T tokens.
// bf16: RoPE table plus K and (unless V is read in place) V^T in 64-key tile
// layout; fp32: rotated copies of Q and K.  Both: split partials.  Offsets are
// 256-byte aligned.
Layout plan(int nseq, int64_t nq, int64_t nk, int H, int rope_T, bool rope_on, bool allow_split, int kv_splits,
            vggt_dtype dt, bool norm_on = false) {
  Layout L;
  const size_t es = elem_size(dt);
  if (dt == VGGT_BF16) {
    if (rope_on) {
      L.use_table = true;
      add(L, L.table, (size_t)rope_T * 32 * 8);
    }
    L.ktiles = (int)((nk + 63) / 64);
    const size_t tiles_bytes = (size_t)nseq * H * L.ktiles * 64 * vggt::kHeadDim * 2;
    add(L, L.kt, tiles_bytes);
    L.use_vt = !v_in_place(nq);
    if (L.use_vt) add(L, L.vt, tiles_bytes);
  } else if (rope_on || norm_on) {
    L.use_qr = true;
    add(L, L.qr, (size_t)nseq * nq * H * vggt::kHeadDim * es);
    L.use_kr = true;
    add(L, L.kr, (size_t)nseq * nk * H * vggt::kHeadDim * es);
  }
  L.sp = allow_split ? plan_splits(nq, nk, H, kv_splits, dt) : SplitPlan{1, (int)pad64(nk)};
  if (L.sp.splits > 1) {
    add(L, L.part_o, (size_t)L.sp.splits * nseq * nq * H * vggt::kHeadDim * 4);
    add(L, L.part_ml, (size_t)L.sp.splits * nseq * nq * H * 2 * 4);
  }
  return L;
}

vggt::AttnProblem base_problem(const void* q, const void* k, const void* v, void* o, int H, float scale) {
  vggt::AttnProblem p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.tok_stride = (int64_t)H * vggt::kHeadDim;
  p.H = H;
  p.scale_log2 = scale_log2(scale);
  return p;
}

// Enqueue the preparation passes and the attention for one call.
hipError_t run_call(const Layout& L, vggt::AttnProblem p, vggt_dtype dt, int nseq, int64_t nq, int64_t nk,
                    const int32_t* pos, float base, int rope_T, char* ws, hipStream_t st, int kind,
                    const vggt_qk_norm* norm = nullptr) {
  const int H = p.H;
  hipError_t e = hipSuccess;
  if (dt == VGGT_BF16) {
    if (norm) {
      p.q_ln_g = norm->q_gamma;
      p.q_ln_b = norm->q_beta;
      p.ln_eps = norm->eps;
    }
    const void* table = nullptr;
    if (L.use_table) {
      e = vggt::launch_rope_table(pos, rope_T, (double)base, ws + L.table, st);
      if (e != hipSuccess) return e;
      table = ws + L.table;
      p.rope_tab = (const vggt::f32x2*)table;
      p.rope_T = rope_T;
    }
    e = vggt::launch_k_tiles_bf16(vggt::contiguous_keys(p.k, (int)nk), ws + L.kt, nseq, (int)nk, H,
                                  table, rope_T,
                                  norm ? norm->k_gamma : nullptr, norm ? norm->k_beta : nullptr,
                                  norm ? norm->eps : 0.0f, st);
    if (e == hipSuccess && L.use_vt)
      e = vggt::launch_v_tiles_bf16(vggt::contiguous_keys(p.v, (int)nk), ws + L.vt, nseq, (int)nk, H,
                                    st);
    if (e != hipSuccess) return e;
    p.k = ws + L.kt;
    p.vt = L.use_vt ? ws + L.vt : nullptr;
    p.ktiles_seq = L.ktiles;
  } else if (L.use_qr) {
    // fp32: LayerNorm and/or RoPE into the rotated copies
    const int64_t nqt = (int64_t)nseq * nq, nkt = (int64_t)nseq * nk;
    const void* qs = p.q;
    const void* ks = p.k;
    if (norm) {
      e = vggt::launch_layer_norm_f32((const float*)p.q, (float*)(ws + L.qr), nqt, H, norm->q_gamma, norm->q_beta,
                                      norm->eps, st);
      if (e == hipSuccess)
        e = vggt::launch_layer_norm_f32((const float*)p.k, (float*)(ws + L.kr), nkt, H, norm->k_gamma, norm->k_beta,
                                        norm->eps, st);
      if (e != hipSuccess) return e;
      qs = ws + L.qr;
      ks = ws + L.kr;
    }
    if (pos) {
      e = vggt::launch_rope(qs, ws + L.qr, false, nqt, rope_T, H, pos, (double)base, st);
      if (e == hipSuccess) e = vggt::launch_rope(ks, ws + L.kr, false, nkt, rope_T, H, pos, (double)base, st);
      if (e != hipSuccess) return e;
    }
    p.q = ws + L.qr;
    p.k = ws + L.kr;
  }
  p.nq = (int)nq;
  p.nk = (int)nk;
  p.nseq = nseq;
  p.nq_total = (int64_t)nseq * nq;
  p.q_seq_stride = nseq > 1 ? nq : 0;
  p.k_seq_stride = nseq > 1 ? nk : 0;
  p.splits = L.sp.splits;
  p.keys_per_split = L.sp.keys_per_split;
  if (L.sp.splits > 1) {
    p.part_o = (float*)(ws + L.part_o);
    p.part_ml = (float*)(ws + L.part_ml);
  }
  return run_attention(p, dt, st, kind);
}

}  // namespace

VGGT_API size_t vggt_frame_attn_workspace(int S, int T, int H, int rope_on, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H)) return 0;
  if (S == 0) return 0;
  return plan(S, T, T, H, T, (rope_on & VGGT_PRE_ROPE) != 0, false, 1, dt, (rope_on & VGGT_PRE_QKNORM) != 0).total;
}

namespace {

vggt_status check_norm(const vggt_qk_norm* n) {
  if (!n) return VGGT_OK;
  if (!n->q_gamma || !n->q_beta || !n->k_gamma || !n->k_beta)
    return fail(VGGT_ERR_NULL, "q/k LayerNorm gamma and beta are required");
  if (((reinterpret_cast<uintptr_t>(n->q_gamma) | reinterpret_cast<uintptr_t>(n->q_beta) |
        reinterpret_cast<uintptr_t>(n->k_gamma) | reinterpret_cast<uintptr_t>(n->k_beta)) & 3u) != 0)
    return fail(VGGT_ERR_ALIGN, "LayerNorm parameters must be 4-byte aligned");
  if (!(n->eps > 0.0f) || !std::isfinite(n->eps)) return fail(VGGT_ERR_SHAPE, "LayerNorm eps must be finite and > 0");
  return VGGT_OK;
}

// The LayerNorm parameters are read while o and the workspace are written.
vggt_status check_norm_alias(const vggt_qk_norm* n, const void* o, size_t o_bytes, const void* ws, size_t ws_need) {
  if (!n) return VGGT_OK;
  const size_t pb = vggt::kHeadDim * sizeof(float);
  for (const float* a : {n->q_gamma, n->q_beta, n->k_gamma, n->k_beta})
    if (overlap(a, pb, o, o_bytes) || overlap(a, pb, ws, ws_need))
      return fail(VGGT_ERR_ALIAS, "LayerNorm parameters overlap the output or the workspace");
  return VGGT_OK;
}

vggt_status check_lse(float* lse, size_t lse_bytes, const void* const* others, const size_t* sizes, int n) {
  if (!lse) return fail(VGGT_ERR_NULL, "lse is required");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(VGGT_ERR_ALIGN, "lse must be 4-byte aligned");
  for (int i = 0; i < n; ++i)
    if (overlap(lse, lse_bytes, others[i], sizes[i])) return fail(VGGT_ERR_ALIAS, "lse overlaps another buffer");
  return VGGT_OK;
}

vggt_status frame_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T, int H,
                       const int32_t* pos_yx, float rope_base, float scale, const vggt_qk_norm* norm, void* workspace,
                       size_t ws_bytes, void* stream, float* lse = nullptr, bool want_lse = false) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (vggt_status s = check_norm(norm)) return s;
  if (S == 0) return VGGT_OK;
  const size_t bytes = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  const Layout L = plan(S, T, T, H, T, pos_yx != nullptr, false, 1, dt, norm != nullptr);
  if (vggt_status s = validate_attn({q, k, v, o}, pos_yx, rope_base, L.total, workspace, ws_bytes, bytes, bytes))
    return s;
  if (vggt_status s = check_norm_alias(norm, o, bytes, workspace, L.total)) return s;
  if (want_lse) {
    const void* others[] = {q, k, v, o, workspace};
    const size_t sizes[] = {bytes, bytes, bytes, bytes, L.total};
    if (vggt_status s = check_lse(lse, (size_t)S * T * H * 4, others, sizes, 5)) return s;
  }
  if (vggt_status s = check_device()) return s;
  vggt::AttnProblem p = base_problem(q, k, v, o, H, scale);
  p.lse = lse;
  hipError_t e = run_call(L, p, dt, S, T, T, pos_yx, rope_base, T, (char*)workspace, (hipStream_t)stream,
                          VGGT_TIMER_FRAME, norm);
  if (e != hipSuccess) return device_error("frame attention launch", e);
  return VGGT_OK;
}

vggt_status global_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S, int T, int H,
                        const int32_t* pos_yx, float rope_base, float scale, int kv_splits, const vggt_qk_norm* norm,
                        void* workspace, size_t ws_bytes, void* stream, float* lse = nullptr, bool want_lse = false) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (kv_splits < 0 || kv_splits > kMaxSplits) return fail(VGGT_ERR_SHAPE, "kv_splits must be in [0, %d]", kMaxSplits);
  if (vggt_status s = check_norm(norm)) return s;
  if (S == 0) return VGGT_OK;
  const int64_t N = (int64_t)S * T;
  const size_t bytes = (size_t)N * H * vggt::kHeadDim * elem_size(dt);
  const Layout L = plan(1, N, N, H, T, pos_yx != nullptr, true, kv_splits, dt, norm != nullptr);
  if (vggt_status s = validate_attn({q, k, v, o}, pos_yx, rope_base, L.total, workspace, ws_bytes, bytes, bytes))
    return s;
  if (vggt_status s = check_norm_alias(norm, o, bytes, workspace, L.total)) return s;
  if (want_lse) {
    const void* others[] = {q, k, v, o, workspace};
    const size_t sizes[] = {bytes, bytes, bytes, bytes, L.total};
    if (vggt_status s = check_lse(lse, (size_t)N * H * 4, others, sizes, 5)) return s;
  }
  if (vggt_status s = check_device()) return s;
  vggt::AttnProblem p = base_problem(q, k, v, o, H, scale);
  p.lse = lse;
  hipError_t e = run_call(L, p, dt, 1, N, N, pos_yx, rope_base, T, (char*)workspace, (hipStream_t)stream,
                          VGGT_TIMER_GLOBAL, norm);
  if (e != hipSuccess) return device_error("global attention launch", e);
  return VGGT_OK;
}

}  // namespace

VGGT_API vggt_status vggt_frame_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                     int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                     void* workspace, size_t ws_bytes, void* stream) {
  return frame_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, nullptr, workspace, ws_bytes, stream);
}

// ---- allocation-free frame attention: the workspace lives in a file-scope device
//      array of kNoallocScratchBytes, shared by every call on a device.  In host code
//      `scratch` is only a stand-in for the symbol: its device address is looked up
//      once per device with hipGetSymbolAddress and only that address is used.
namespace {

constexpr size_t kNoallocScratchBytes = VGGT_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoallocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch[64];  // device address of `scratch` per device index, null until looked up

vggt_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VGGT_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(VGGT_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return device_error("hipGetSymbolAddress(scratch)", e != hipSuccess ? e : hipErrorUnknown);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return VGGT_OK;
}

}  // namespace

VGGT_API vggt_status vggt_frame_attn_noalloc(const void* q, const void* k, const void* v, void* o, vggt_dtype dt,
                                             int S, int T, int H, const int32_t* pos_yx, float rope_base,
                                             float scale, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (S == 0) return VGGT_OK;
  const size_t need = vggt_frame_attn_workspace(S, T, H, pos_yx != nullptr, dt);
  if (need > kNoallocScratchBytes)
    return fail(VGGT_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the allocation-free call has %zu", need,
                kNoallocScratchBytes);
  const size_t bytes = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  if (vggt_status s = validate_attn({q, k, v, o}, pos_yx, rope_base, 0, nullptr, 0, bytes, bytes)) return s;
  if (vggt_status s = check_device()) return s;
  void* ws = nullptr;
  if (vggt_status s = scratch_address(&ws)) return s;
  return frame_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, nullptr, ws, kNoallocScratchBytes, stream);
}

VGGT_API vggt_status vggt_frame_attn_qknorm(const void* q, const void* k, const void* v, void* o, vggt_dtype dt,
                                            int S, int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                            const vggt_qk_norm* norm, void* workspace, size_t ws_bytes,
                                            void* stream) {
  return frame_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, norm, workspace, ws_bytes, stream);
}

VGGT_API size_t vggt_global_attn_workspace(int S, int T, int H, int kv_splits, int rope_on, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H) || kv_splits < 0 || kv_splits > kMaxSplits) return 0;
  if (S == 0) return 0;
  const int64_t N = (int64_t)S * T;
  return plan(1, N, N, H, T, (rope_on & VGGT_PRE_ROPE) != 0, true, kv_splits, dt, (rope_on & VGGT_PRE_QKNORM) != 0)
      .total;
}

VGGT_API vggt_status vggt_global_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                      int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                      int kv_splits, void* workspace, size_t ws_bytes, void* stream) {
  return global_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, kv_splits, nullptr, workspace, ws_bytes,
                     stream);
}

VGGT_API vggt_status vggt_global_attn_qknorm(const void* q, const void* k, const void* v, void* o, vggt_dtype dt,
                                             int S, int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                             int kv_splits, const vggt_qk_norm* norm, void* workspace,
                                             size_t ws_bytes, void* stream) {
  return global_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, kv_splits, norm, workspace, ws_bytes,
                     stream);
}

// ---------------------------------------------------------------------------
// FlashVGGT descriptors
// ---------------------------------------------------------------------------

VGGT_API int vggt_descriptor_count(int T, int gh, int gw, int ph, int pw) {
  if (T < 1 || gh < 1 || gw < 1 || ph < 1 || pw < 1 || (int64_t)gh * gw > T) return -1;
  return (T - gh * gw) + ((gh + ph - 1) / ph) * ((gw + pw - 1) / pw);
}

VGGT_API vggt_status vggt_descriptor_pool(const void* k, const void* v, void* kd, void* vd, vggt_dtype dt, int S,
                                          int T, int H, int gh, int gw, int patch_begin, int ph, int pw,
                                          void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  const int Dn = vggt_descriptor_count(T, gh, gw, ph, pw);
  if (Dn < 1 || patch_begin < 0 || (int64_t)patch_begin + (int64_t)gh * gw > T)
    return fail(VGGT_ERR_SHAPE, "bad grid: T=%d gh=%d gw=%d patch_begin=%d ph=%d pw=%d", T, gh, gw, patch_begin, ph, pw);
  if (S == 0) return VGGT_OK;
  if (!k || !v || !kd || !vd) return fail(VGGT_ERR_NULL, "k, v, kd and vd are required");
  if (!aligned16(k) || !aligned16(v) || !aligned16(kd) || !aligned16(vd))
    return fail(VGGT_ERR_ALIGN, "pointers must be 16-byte aligned");
  const size_t in_b = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  const size_t out_b = (size_t)S * Dn * H * vggt::kHeadDim * elem_size(dt);
  if (overlap(kd, out_b, k, in_b) || overlap(kd, out_b, v, in_b) || overlap(vd, out_b, k, in_b) ||
      overlap(vd, out_b, v, in_b) || overlap(kd, out_b, vd, out_b))
    return fail(VGGT_ERR_ALIAS, "outputs overlap inputs or each other");
  if (vggt_status s = check_device()) return s;
  hipError_t e = vggt::launch_pool(k, v, kd, vd, dt == VGGT_BF16, S, T, H, gh, gw, patch_begin, ph, pw, Dn,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return device_error("pool launch", e);
  return VGGT_OK;
}

VGGT_API size_t vggt_descriptor_xattn_workspace(int S, int T, int Dn, int H, int kv_splits, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H) || Dn < 1 || !tokens_ok(S, Dn, H) || kv_splits < 0 ||
      kv_splits > kMaxSplits)
    return 0;
  if (S == 0) return 0;
  return plan(1, (int64_t)S * T, (int64_t)S * Dn, H, 1, false, true, kv_splits, dt).total;
}

VGGT_API vggt_status vggt_descriptor_xattn(const void* q, const void* kd, const void* vd, void* o, vggt_dtype dt,
                                           int S, int T, int Dn, int H, float scale, int kv_splits, void* workspace,
                                           size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H) || Dn < 1 || !tokens_ok(S, Dn, H))
    return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d Dn=%d H=%d", S, T, Dn, H);
  if (kv_splits < 0 || kv_splits > kMaxSplits) return fail(VGGT_ERR_SHAPE, "kv_splits must be in [0, %d]", kMaxSplits);
  if (S == 0) return VGGT_OK;
  const int64_t nq = (int64_t)S * T, nk = (int64_t)S * Dn;
  const size_t q_b = (size_t)nq * H * vggt::kHeadDim * elem_size(dt);
  const size_t kv_b = (size_t)nk * H * vggt::kHeadDim * elem_size(dt);
  const Layout L = plan(1, nq, nk, H, 1, false, true, kv_splits, dt);
  if (vggt_status s = validate_attn({q, kd, vd, o}, nullptr, 0.0f, L.total, workspace, ws_bytes, q_b, kv_b))
    return s;
  if (vggt_status s = check_device()) return s;
  hipError_t e = run_call(L, base_problem(q, kd, vd, o, H, scale), dt, 1, nq, nk, nullptr, 0.0f, 1,
                          (char*)workspace, (hipStream_t)stream, VGGT_TIMER_XATTN);
  if (e != hipSuccess) return device_error("descriptor attention launch", e);
  return VGGT_OK;
}

// ---------------------------------------------------------------------------
// FlashVGGT chunk-recursive attention over a descriptor cache
// ---------------------------------------------------------------------------

namespace {

// Where K and V live inside a cache buffer.
struct CacheView {
  int cap_tiles = 0;  // bf16: 64-descriptor tiles per head
  size_t k_bytes = 0;
  size_t total = 0;
};

bool cache_dims_ok(int capacity, int H) { return capacity >= 1 && capacity < kMaxTokens && H >= 1 && H <= kMaxHeads; }

CacheView cache_view(int capacity, int H, vggt_dtype dt) {
  CacheView c;
  if (dt == VGGT_BF16) {
    c.cap_tiles = (capacity + 63) / 64;
    c.k_bytes = (size_t)H * c.cap_tiles * 64 * vggt::kHeadDim * 2;
  } else {
    c.k_bytes = (size_t)capacity * H * vggt::kHeadDim * 4;
  }
  c.total = 2 * c.k_bytes;
  return c;
}

vggt::AttnProblem cache_problem(const void* q, const void* cache, const CacheView& c, void* o, int H, float scale,
                                vggt_dtype dt) {
  const char* base = (const char*)cache;
  vggt::AttnProblem p = base_problem(q, base, nullptr, o, H, scale);
  if (dt == VGGT_BF16) {
    p.vt = base + c.k_bytes;
    p.ktiles_seq = c.cap_tiles;
  } else {
    p.v = base + c.k_bytes;
  }
  p.k_seq_stride = 0;  // every query sequence reads the one cache
  return p;
}

Layout partials_layout(int64_t nq, int64_t nk, int H, int kv_splits, vggt_dtype dt) {
  Layout L;
  L.sp = plan_splits(nq, nk, H, kv_splits, dt);
  if (L.sp.splits > 1) {
    add(L, L.part_o, (size_t)L.sp.splits * nq * H * vggt::kHeadDim * 4);
    add(L, L.part_ml, (size_t)L.sp.splits * nq * H * 2 * 4);
  }
  return L;
}

}  // namespace

VGGT_API size_t vggt_descriptor_cache_bytes(int capacity, int H, vggt_dtype dt) {
  if (!dtype_ok(dt) || !cache_dims_ok(capacity, H)) return 0;
  return cache_view(capacity, H, dt).total;
}

VGGT_API vggt_status vggt_descriptor_cache_append(void* cache, vggt_dtype dt, int capacity, int H, int used,
                                                  const void* kd, const void* vd, int n, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!cache_dims_ok(capacity, H)) return fail(VGGT_ERR_SHAPE, "bad cache shape capacity=%d H=%d", capacity, H);
  if (used < 0 || n < 0 || (int64_t)used + n > capacity)
    return fail(VGGT_ERR_SHAPE, "append of %d descriptors at %d exceeds capacity %d", n, used, capacity);
  if (n == 0) return VGGT_OK;
  if (!cache || !kd || !vd) return fail(VGGT_ERR_NULL, "cache, kd and vd are required");
  if (!aligned16(cache) || !aligned16(kd) || !aligned16(vd)) return fail(VGGT_ERR_ALIGN, "misaligned pointer");
  const CacheView c = cache_view(capacity, H, dt);
  const size_t in_b = (size_t)n * H * vggt::kHeadDim * elem_size(dt);
  if (overlap(cache, c.total, kd, in_b) || overlap(cache, c.total, vd, in_b))
    return fail(VGGT_ERR_ALIAS, "kd/vd overlap the cache");
  if (vggt_status s = check_device()) return s;
  char* base = (char*)cache;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dt == VGGT_BF16) {
    e = vggt::launch_tiles_append_bf16(kd, vd, base, base + c.k_bytes, c.cap_tiles, used, n, H, st);
  } else {
    const size_t off = (size_t)used * H * vggt::kHeadDim * 4;
    e = hipMemcpyAsync(base + off, kd, in_b, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(base + c.k_bytes + off, vd, in_b, hipMemcpyDeviceToDevice, st);
  }
  if (e != hipSuccess) return device_error("descriptor cache append", e);
  return VGGT_OK;
}

VGGT_API size_t vggt_descriptor_cache_attn_workspace(int nq, int used, int H, int kv_splits, vggt_dtype dt) {
  if (!dtype_ok(dt) || nq < 0 || nq >= kMaxTokens || !cache_dims_ok(used, H) || kv_splits < 0 ||
      kv_splits > kMaxSplits)
    return 0;
  if (nq == 0) return 0;
  return partials_layout(nq, used, H, kv_splits, dt).total;
}

VGGT_API vggt_status vggt_descriptor_cache_attn(const void* q, const void* cache, void* o, vggt_dtype dt, int capacity,
                                                int H, int used, int nq, float scale, int kv_splits, void* workspace,
                                                size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!cache_dims_ok(capacity, H) || used < 1 || used > capacity || nq < 0 || nq >= kMaxTokens)
    return fail(VGGT_ERR_SHAPE, "bad shape capacity=%d H=%d used=%d nq=%d", capacity, H, used, nq);
  if (kv_splits < 0 || kv_splits > kMaxSplits) return fail(VGGT_ERR_SHAPE, "kv_splits must be in [0, %d]", kMaxSplits);
  if (nq == 0) return VGGT_OK;
  const CacheView c = cache_view(capacity, H, dt);
  const size_t q_b = (size_t)nq * H * vggt::kHeadDim * elem_size(dt);
  const Layout L = partials_layout(nq, used, H, kv_splits, dt);
  // the cache plays the role of both k and v in the overlap checks
  if (vggt_status s = validate_attn({q, cache, cache, o}, nullptr, 0.0f, L.total, workspace, ws_bytes, q_b, c.total))
    return s;
  if (vggt_status s = check_device()) return s;
  vggt::AttnProblem p = cache_problem(q, cache, c, o, H, scale, dt);
  p.nq = nq;
  p.nk = used;
  p.nseq = 1;
  p.nq_total = nq;
  p.splits = L.sp.splits;
  p.keys_per_split = L.sp.keys_per_split;
  if (L.sp.splits > 1) {
    p.part_o = (float*)((char*)workspace + L.part_o);
    p.part_ml = (float*)((char*)workspace + L.part_ml);
  }
  hipError_t e = run_attention(p, dt, (hipStream_t)stream, VGGT_TIMER_CACHE);
  if (e != hipSuccess) return device_error("descriptor cache attention launch", e);
  return VGGT_OK;
}

VGGT_API vggt_status vggt_descriptor_chunked_xattn(const void* q, const void* cache, void* o, vggt_dtype dt,
                                                   int capacity, int H, int S, int T, int Dn, int chunk_frames,
                                                   float scale, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!cache_dims_ok(capacity, H) || !tokens_ok(S, T, H) || Dn < 1 || chunk_frames < 1 ||
      (int64_t)S * Dn > capacity)
    return fail(VGGT_ERR_SHAPE, "bad shape capacity=%d H=%d S=%d T=%d Dn=%d chunk_frames=%d", capacity, H, S, T, Dn,
                chunk_frames);
  if (S == 0) return VGGT_OK;
  const CacheView c = cache_view(capacity, H, dt);
  const size_t q_b = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  if (vggt_status s = validate_attn({q, cache, cache, o}, nullptr, 0.0f, 0, nullptr, 0, q_b, c.total)) return s;
  if (vggt_status s = check_device()) return s;
  const int F = std::min(chunk_frames, S);
  vggt::AttnProblem p = cache_problem(q, cache, c, o, H, scale, dt);
  p.nseq = (S + F - 1) / F;
  p.nq = F * T;
  p.q_seq_stride = (int64_t)F * T;
  p.nq_total = (int64_t)S * T;
  p.nk = S * Dn;
  p.nk_step = F * Dn;
  p.splits = 1;
  p.keys_per_split = (int)pad64(p.nk);
  hipError_t e = run_attention(p, dt, (hipStream_t)stream, VGGT_TIMER_CHUNKED);
  if (e != hipSuccess) return device_error("chunked descriptor attention launch", e);
  return VGGT_OK;
}

// ---------------------------------------------------------------------------
// Diagnostics: attention kernel timer
// ---------------------------------------------------------------------------

namespace {
void timer_release_locked() {
  for (hipEvent_t e : g_timer.ev)
    if (e) (void)hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.kind.clear();
  g_timer.armed = false;
  g_timer.next = 0;
  g_timer.device = -1;
}
}  // namespace

VGGT_API vggt_status vggt_timer_start(int capacity) {
  g_last_error[0] = 0;
  if (capacity < 1 || capacity > (1 << 20)) return fail(VGGT_ERR_SHAPE, "timer capacity must be in [1, 2^20]");
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (g_timer.armed) return fail(VGGT_ERR_SHAPE, "timer already running");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error("hipGetDevice", e);
  g_timer.ev.assign(2 * (size_t)capacity, nullptr);
  for (hipEvent_t& ev : g_timer.ev) {
    e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      ev = nullptr;
      timer_release_locked();
      return device_error("hipEventCreate", e);
    }
  }
  g_timer.kind.assign((size_t)capacity, 0);
  g_timer.device = dev;
  g_timer.next = 0;
  g_timer.armed = true;
  return VGGT_OK;
}

VGGT_API vggt_status vggt_timer_stop(float* ms, int* kinds, int n_max, int* n_recorded) {
  g_last_error[0] = 0;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.armed) return fail(VGGT_ERR_SHAPE, "timer not running");
  if (n_max < 0 || (n_max > 0 && (!ms || !kinds))) {
    timer_release_locked();
    return fail(VGGT_ERR_NULL, "ms and kinds are required when n_max > 0");
  }
  vggt_status st = VGGT_OK;
  const int n = g_timer.next;
  for (int i = 0; i < n && i < n_max; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[2 * i + 1]);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) {
      st = device_error("timer event", e);
      break;
    }
    ms[i] = t;
    kinds[i] = g_timer.kind[i];
  }
  if (n_recorded) *n_recorded = n;
  timer_release_locked();
  return st;
}

// ---------------------------------------------------------------------------
// VGGT-Omega block variants: a subset of each frame's tokens, and global-only
// extra tokens
// ---------------------------------------------------------------------------

namespace {

constexpr int kMaxExtra = 4096;

// Workspace of one frame/global "ex" call.  bf16: RoPE table and the key
// tiles of the compacted key set (V^T tiles unless a frame's V rows are read
// in place); fp32: normalised/rotated copies and the gathered key set.  Global
// calls also hold the split partials of the frame tokens' queries and of the
// extra tokens' queries.
struct ExLayout {
  size_t table = 0, kt = 0, vt = 0, qr = 0, kc = 0, vc = 0, xqr = 0;
  size_t part_o = 0, part_ml = 0, xpart_o = 0, xpart_ml = 0, total = 0;
  bool use_qr = false, use_kc = false, use_vc = false, use_xqr = false, use_vt = false;
  int nseq_k = 1;
  int64_t nk = 0;
  int ktiles = 0;
  SplitPlan sp{1, 0}, spx{1, 0};
};

void add_ex(ExLayout& L, size_t& off, size_t bytes) {
  off = L.total;
  L.total += align256(bytes);
}

ExLayout plan_ex(bool global, int S, int T, int Ta, int E, int H, int kv_splits, bool rope, bool norm,
                 vggt_dtype dt) {
  ExLayout L;
  const size_t row = (size_t)H * vggt::kHeadDim * elem_size(dt);
  L.nseq_k = global ? 1 : S;
  L.nk = global ? (int64_t)S * Ta + E : Ta;
  if (dt == VGGT_BF16) {
    if (rope) add_ex(L, L.table, (size_t)T * 32 * 8);
    L.ktiles = (int)((L.nk + 63) / 64);
    const size_t tiles = (size_t)L.nseq_k * H * L.ktiles * 64 * vggt::kHeadDim * 2;
    add_ex(L, L.kt, tiles);
    // a frame's active tokens are a contiguous run of V rows; the global key set (active
    // tokens of every frame, then the extras) is not, and always goes through V^T tiles
    L.use_vt = global || !v_in_place(Ta);
    if (L.use_vt) add_ex(L, L.vt, tiles);
  } else {
    if (rope || norm) {
      L.use_qr = true;
      add_ex(L, L.qr, (size_t)S * T * row);
    }
    if (global) {
      L.use_kc = L.use_vc = true;
      add_ex(L, L.kc, (size_t)L.nk * row);
      add_ex(L, L.vc, (size_t)L.nk * row);
    } else if (rope || norm) {
      L.use_kc = true;
      add_ex(L, L.kc, (size_t)S * T * row);
    }
    if (global && norm && E > 0) {
      L.use_xqr = true;
      add_ex(L, L.xqr, (size_t)E * row);
    }
  }
  if (global) {
    const int bq = query_tile(dt);
    // workgroups see S sequences of ceil(Ta / bq) query tiles
    L.sp = plan_splits((int64_t)S * ((Ta + bq - 1) / bq) * bq, L.nk, H, kv_splits, dt);
    if (L.sp.splits > 1) {
      add_ex(L, L.part_o, (size_t)L.sp.splits * S * Ta * H * vggt::kHeadDim * 4);
      add_ex(L, L.part_ml, (size_t)L.sp.splits * S * Ta * H * 2 * 4);
    }
    if (E > 0) {
      L.spx = plan_splits(E, L.nk, H, 0, dt);
      if (L.spx.splits > 1) {
        add_ex(L, L.xpart_o, (size_t)L.spx.splits * E * H * vggt::kHeadDim * 4);
        add_ex(L, L.xpart_ml, (size_t)L.spx.splits * E * H * 2 * 4);
      }
    }
  } else {
    L.sp = SplitPlan{1, (int)pad64(Ta)};
  }
  return L;
}

struct ExArgs {
  bool global;
  const void *q, *k, *v;
  void* o;
  const void *xq, *xk, *xv;
  void* xo;
  int S, T, Ta, E, H;
  const int32_t* pos;
  float base, scale;
  const vggt_qk_norm* norm;
};

hipError_t run_ex(const ExLayout& L, const ExArgs& a, vggt_dtype dt, char* ws, hipStream_t st) {
  hipError_t e = hipSuccess;
  const int H = a.H;
  vggt::AttnProblem p = base_problem(a.q, a.k, a.v, a.o, H, a.scale);
  vggt::KeySrc ks, vs;
  ks.main = a.k;
  vs.main = a.v;
  if (a.global) {
    ks.extra = a.xk;
    vs.extra = a.xv;
    ks.frame_len = vs.frame_len = a.Ta;
    ks.frame_stride = vs.frame_stride = a.T;
    ks.n_main = vs.n_main = (int64_t)a.S * a.Ta;
  } else {
    ks.seq_rows = vs.seq_rows = a.T;
    ks.n_main = vs.n_main = a.Ta;
  }
  if (dt == VGGT_BF16) {
    const void* table = nullptr;
    if (a.pos) {
      e = vggt::launch_rope_table(a.pos, a.T, (double)a.base, ws + L.table, st);
      if (e != hipSuccess) return e;
      table = ws + L.table;
      p.rope_tab = (const vggt::f32x2*)table;
      p.rope_T = a.T;
    }
    if (a.norm) {
      p.q_ln_g = a.norm->q_gamma;
      p.q_ln_b = a.norm->q_beta;
      p.ln_eps = a.norm->eps;
    }
    e = vggt::launch_k_tiles_bf16(ks, ws + L.kt, L.nseq_k, (int)L.nk, H, table, a.T,
                                  a.norm ? a.norm->k_gamma : nullptr, a.norm ? a.norm->k_beta : nullptr,
                                  a.norm ? a.norm->eps : 0.0f, st);
    if (e == hipSuccess && L.use_vt) e = vggt::launch_v_tiles_bf16(vs, ws + L.vt, L.nseq_k, (int)L.nk, H, st);
    if (e != hipSuccess) return e;
    p.k = ws + L.kt;
    p.vt = L.use_vt ? ws + L.vt : nullptr;
    p.ktiles_seq = L.ktiles;
  } else {
    const int64_t full = (int64_t)a.S * a.T;
    if (L.use_qr) {
      const void* src = a.q;
      if (a.norm) {
        e = vggt::launch_layer_norm_f32((const float*)a.q, (float*)(ws + L.qr), full, H, a.norm->q_gamma,
                                        a.norm->q_beta, a.norm->eps, st);
        src = ws + L.qr;
      }
      if (e == hipSuccess && a.pos) e = vggt::launch_rope(src, ws + L.qr, false, full, a.T, H, a.pos, (double)a.base, st);
      if (e != hipSuccess) return e;
      p.q = ws + L.qr;
    }
    if (a.global) {
      // the compacted key set: active frame tokens in frame order, then the extras
      e = vggt::launch_gather_keys_f32(ks, (float*)(ws + L.kc), 1, (int)L.nk, H, st);
      if (e == hipSuccess) e = vggt::launch_gather_keys_f32(vs, (float*)(ws + L.vc), 1, (int)L.nk, H, st);
      if (e == hipSuccess && a.norm)
        e = vggt::launch_layer_norm_f32((const float*)(ws + L.kc), (float*)(ws + L.kc), L.nk, H, a.norm->k_gamma,
                                        a.norm->k_beta, a.norm->eps, st);
      if (e == hipSuccess && a.pos)
        e = vggt::launch_rope(ws + L.kc, ws + L.kc, false, (int64_t)a.S * a.Ta, a.Ta, H, a.pos, (double)a.base, st);
      if (e != hipSuccess) return e;
      p.k = ws + L.kc;
      p.v = ws + L.vc;
    } else if (L.use_kc) {
      const void* src = a.k;
      if (a.norm) {
        e = vggt::launch_layer_norm_f32((const float*)a.k, (float*)(ws + L.kc), full, H, a.norm->k_gamma,
                                        a.norm->k_beta, a.norm->eps, st);
        src = ws + L.kc;
      }
      if (e == hipSuccess && a.pos) e = vggt::launch_rope(src, ws + L.kc, false, full, a.T, H, a.pos, (double)a.base, st);
      if (e != hipSuccess) return e;
      p.k = ws + L.kc;
    }
  }
  // the frame tokens' queries: S sequences of Ta rows, T rows apart
  p.nseq = a.S;
  p.nq = a.Ta;
  p.q_seq_stride = a.T;
  p.nq_total = (int64_t)a.S * a.Ta;
  p.nk = (int)L.nk;
  p.k_seq_stride = a.global ? 0 : a.T;  // tokens between frames (bf16: nonzero = per-frame tiles)
  p.splits = L.sp.splits;
  p.keys_per_split = L.sp.keys_per_split;
  if (L.sp.splits > 1) {
    p.part_o = (float*)(ws + L.part_o);
    p.part_ml = (float*)(ws + L.part_ml);
  }
  e = run_attention(p, dt, st, a.global ? VGGT_TIMER_GLOBAL : VGGT_TIMER_FRAME);
  if (e != hipSuccess || !a.global || a.E == 0) return e;
  // the extra tokens' queries: one sequence of E rows against the same keys, no rotation
  vggt::AttnProblem x = p;
  x.q = (dt == VGGT_F32 && L.use_xqr) ? (const void*)(ws + L.xqr) : a.xq;
  if (dt == VGGT_F32 && L.use_xqr) {
    e = vggt::launch_layer_norm_f32((const float*)a.xq, (float*)(ws + L.xqr), a.E, H, a.norm->q_gamma,
                                    a.norm->q_beta, a.norm->eps, st);
    if (e != hipSuccess) return e;
  }
  x.o = a.xo;
  x.rope_tab = nullptr;
  x.nseq = 1;
  x.nq = a.E;
  x.q_seq_stride = 0;
  x.nq_total = a.E;
  x.splits = L.spx.splits;
  x.keys_per_split = L.spx.keys_per_split;
  x.part_o = L.spx.splits > 1 ? (float*)(ws + L.xpart_o) : nullptr;
  x.part_ml = L.spx.splits > 1 ? (float*)(ws + L.xpart_ml) : nullptr;
  return run_attention(x, dt, st, VGGT_TIMER_GLOBAL);
}

vggt_status ex_call(const ExArgs& a, vggt_dtype dt, int kv_splits, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(a.S, a.T, a.H) || a.Ta < 1 || a.Ta > a.T || a.E < 0 || a.E > kMaxExtra ||
      (!a.global && a.E != 0) || (a.S == 0 && a.E != 0))
    return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d T_active=%d n_extra=%d H=%d", a.S, a.T, a.Ta, a.E, a.H);
  if (kv_splits < 0 || kv_splits > kMaxSplits) return fail(VGGT_ERR_SHAPE, "kv_splits must be in [0, %d]", kMaxSplits);
  if (vggt_status s = check_norm(a.norm)) return s;
  if (a.S == 0) return VGGT_OK;
  const size_t bytes = (size_t)a.S * a.T * a.H * vggt::kHeadDim * elem_size(dt);
  const size_t xbytes = (size_t)a.E * a.H * vggt::kHeadDim * elem_size(dt);
  const ExLayout L = plan_ex(a.global, a.S, a.T, a.Ta, a.E, a.H, kv_splits, a.pos != nullptr, a.norm != nullptr, dt);
  if (vggt_status s = validate_attn({a.q, a.k, a.v, a.o}, a.pos, a.base, L.total, workspace, ws_bytes, bytes, bytes))
    return s;
  if (vggt_status s = check_norm_alias(a.norm, a.o, bytes, workspace, L.total)) return s;
  if (a.E > 0) {
    if (!a.xq || !a.xk || !a.xv || !a.xo) return fail(VGGT_ERR_NULL, "xq, xk, xv and xo are required");
    if (!aligned16(a.xq) || !aligned16(a.xk) || !aligned16(a.xv) || !aligned16(a.xo))
      return fail(VGGT_ERR_ALIGN, "extra-token tensors must be 16-byte aligned");
    for (const void* in : {a.q, a.k, a.v})
      if (overlap(a.xo, xbytes, in, bytes)) return fail(VGGT_ERR_ALIAS, "xo overlaps q, k or v");
    for (const void* in : {a.xq, a.xk, a.xv})
      if (overlap(a.xo, xbytes, in, xbytes) || overlap(a.o, bytes, in, xbytes))
        return fail(VGGT_ERR_ALIAS, "an output overlaps an extra-token input");
    if (overlap(a.xo, xbytes, a.o, bytes) || overlap(a.xo, xbytes, workspace, L.total))
      return fail(VGGT_ERR_ALIAS, "xo overlaps o or the workspace");
    if (vggt_status s = check_norm_alias(a.norm, a.xo, xbytes, nullptr, 0)) return s;
  }
  if (vggt_status s = check_device()) return s;
  hipError_t e = run_ex(L, a, dt, (char*)workspace, (hipStream_t)stream);
  if (e != hipSuccess) return device_error(a.global ? "global attention (ex) launch" : "frame attention (ex) launch", e);
  return VGGT_OK;
}

}  // namespace

VGGT_API size_t vggt_frame_attn_ex_workspace(int S, int T, int T_active, int H, int flags, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H) || T_active < 1 || T_active > T) return 0;
  if (S == 0) return 0;
  return plan_ex(false, S, T, T_active, 0, H, 1, (flags & VGGT_PRE_ROPE) != 0, (flags & VGGT_PRE_QKNORM) != 0, dt)
      .total;
}

VGGT_API vggt_status vggt_frame_attn_ex(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                        int T, int T_active, int H, const int32_t* pos_yx, float rope_base,
                                        float scale, const vggt_qk_norm* norm, void* workspace, size_t ws_bytes,
                                        void* stream) {
  const ExArgs a{false, q, k, v, o, nullptr, nullptr, nullptr, nullptr, S, T, T_active, 0, H, pos_yx, rope_base,
                 scale, norm};
  return ex_call(a, dt, 1, workspace, ws_bytes, stream);
}

VGGT_API size_t vggt_global_attn_ex_workspace(int S, int T, int T_active, int n_extra, int H, int kv_splits,
                                              int flags, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H) || T_active < 1 || T_active > T || n_extra < 0 ||
      n_extra > kMaxExtra || kv_splits < 0 || kv_splits > kMaxSplits)
    return 0;
  if (S == 0) return 0;
  return plan_ex(true, S, T, T_active, n_extra, H, kv_splits, (flags & VGGT_PRE_ROPE) != 0,
                 (flags & VGGT_PRE_QKNORM) != 0, dt)
      .total;
}

VGGT_API vggt_status vggt_global_attn_ex(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                         int T, int T_active, int H, const void* xq, const void* xk, const void* xv,
                                         void* xo, int n_extra, const int32_t* pos_yx, float rope_base, float scale,
                                         int kv_splits, const vggt_qk_norm* norm, void* workspace, size_t ws_bytes,
                                         void* stream) {
  const ExArgs a{true, q, k, v, o, xq, xk, xv, xo, S, T, T_active, n_extra, H, pos_yx, rope_base, scale, norm};
  return ex_call(a, dt, kv_splits, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Training: forward with the log-normaliser, and the gradients
// ---------------------------------------------------------------------------

VGGT_API vggt_status vggt_frame_attn_train(const void* q, const void* k, const void* v, void* o, float* lse,
                                           vggt_dtype dt, int S, int T, int H, const int32_t* pos_yx,
                                           float rope_base, float scale, void* workspace, size_t ws_bytes,
                                           void* stream) {
  return frame_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, nullptr, workspace, ws_bytes, stream, lse,
                    true);
}

VGGT_API vggt_status vggt_global_attn_train(const void* q, const void* k, const void* v, void* o, float* lse,
                                            vggt_dtype dt, int S, int T, int H, const int32_t* pos_yx,
                                            float rope_base, float scale, int kv_splits, void* workspace,
                                            size_t ws_bytes, void* stream) {
  return global_attn(q, k, v, o, dt, S, T, H, pos_yx, rope_base, scale, kv_splits, nullptr, workspace, ws_bytes,
                     stream, lse, true);
}

namespace {

// Workspace of one backward call.  bf16: RoPE table, a rotated copy of K, four
// row-tile sets (K, V, scaled Q, dO) and the per-row statistics; fp32: rotated
// copies and rotated-frame gradients.
struct BwdLayout {
  size_t table = 0, qr = 0, kr = 0, tiles[4] = {0, 0, 0, 0}, lse2 = 0, dsum = 0, dqr = 0, dkr = 0;
  size_t total = 0;
  int nseq = 1, n = 0, ntile = 0;
};

void add_b(BwdLayout& L, size_t& off, size_t bytes) {
  off = L.total;
  L.total += align256(bytes);
}

BwdLayout plan_bwd(bool global, int S, int T, int H, bool rope, vggt_dtype dt) {
  BwdLayout L;
  L.nseq = global ? 1 : S;
  L.n = global ? S * T : T;
  L.ntile = (L.n + 63) / 64;
  const size_t tensor = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  if (dt == VGGT_BF16) {
    // the kernels read the transposes they need from these tiles in LDS
    if (rope) {
      add_b(L, L.table, (size_t)T * 32 * 8);
      add_b(L, L.kr, tensor);
    }
    const size_t tiles = (size_t)L.nseq * H * L.ntile * 64 * vggt::kHeadDim * 2;
    for (size_t& t : L.tiles) add_b(L, t, tiles);
  } else if (rope) {
    add_b(L, L.qr, tensor);
    add_b(L, L.kr, tensor);
    add_b(L, L.dqr, tensor);
    add_b(L, L.dkr, tensor);
  }
  const size_t stats = (size_t)L.nseq * H * L.ntile * 64 * 4;
  add_b(L, L.lse2, stats);
  add_b(L, L.dsum, stats);
  return L;
}

vggt_status attn_backward(bool global, const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, vggt_dtype dt, int S, int T, int H,
                          const int32_t* pos, float base, float scale, void* workspace, size_t ws_bytes,
                          void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (pos && (!(base > 0.0f) || !std::isfinite(base))) return fail(VGGT_ERR_SHAPE, "rope base must be finite and > 0");
  if (S == 0) return VGGT_OK;
  const void* in[] = {q, k, v, o, dout};
  void* out[] = {dq, dk, dv};
  for (const void* t : in)
    if (!t) return fail(VGGT_ERR_NULL, "q, k, v, o and dout are required");
  for (const void* t : out)
    if (!t) return fail(VGGT_ERR_NULL, "dq, dk and dv are required");
  if (!lse) return fail(VGGT_ERR_NULL, "lse is required");
  for (const void* t : in)
    if (!aligned16(t)) return fail(VGGT_ERR_ALIGN, "tensors must be 16-byte aligned");
  for (const void* t : out)
    if (!aligned16(t)) return fail(VGGT_ERR_ALIGN, "tensors must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (pos && (reinterpret_cast<uintptr_t>(pos) & 3u)))
    return fail(VGGT_ERR_ALIGN, "lse and pos_yx must be 4-byte aligned");
  const size_t bytes = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  const size_t lse_b = (size_t)S * T * H * 4;
  const BwdLayout L = plan_bwd(global, S, T, H, pos != nullptr, dt);
  if (!workspace) return fail(VGGT_ERR_WORKSPACE, "workspace of %zu bytes required", L.total);
  if (ws_bytes < L.total) return fail(VGGT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, L.total);
  if (!aligned16(workspace)) return fail(VGGT_ERR_ALIGN, "workspace must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    for (const void* t : in)
      if (overlap(out[i], bytes, t, bytes)) return fail(VGGT_ERR_ALIAS, "a gradient overlaps an input");
    if (overlap(out[i], bytes, lse, lse_b) || overlap(out[i], bytes, workspace, L.total))
      return fail(VGGT_ERR_ALIAS, "a gradient overlaps lse or the workspace");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], bytes, out[j], bytes)) return fail(VGGT_ERR_ALIAS, "gradients overlap each other");
  }
  for (const void* t : in)
    if (overlap(workspace, L.total, t, bytes)) return fail(VGGT_ERR_ALIAS, "workspace overlaps an input");
  if (overlap(workspace, L.total, lse, lse_b)) return fail(VGGT_ERR_ALIAS, "workspace overlaps lse");
  if (vggt_status s = check_device()) return s;

  char* ws = (char*)workspace;
  const hipStream_t st = (hipStream_t)stream;
  const int64_t N = (int64_t)S * T;
  const float c = scale_log2(scale);
  const float sc = scale > 0.0f ? scale : 0.125f;
  hipError_t e = hipSuccess;
  float* lse2 = (float*)(ws + L.lse2);
  float* dsum = (float*)(ws + L.dsum);
  const int64_t seq_stride = global ? 0 : T;
  e = vggt::launch_attn_bwd_pre(o, dout, dt == VGGT_BF16, lse, lse2, dsum, L.nseq, L.n, seq_stride, H, L.ntile, st);
  if (e != hipSuccess) return device_error("backward pre-pass", e);
  if (dt == VGGT_BF16) {
    const void* table = nullptr;
    const void* kr = k;
    if (pos) {
      e = vggt::launch_rope_table(pos, T, (double)base, ws + L.table, st);
      if (e == hipSuccess) e = vggt::launch_rope(k, ws + L.kr, true, N, T, H, pos, (double)base, st);
      if (e != hipSuccess) return device_error("backward rotation", e);
      table = ws + L.table;
      kr = ws + L.kr;
    }
    char* tk = ws + L.tiles[0];
    char* tv = ws + L.tiles[1];
    char* tq = ws + L.tiles[2];
    char* tdo = ws + L.tiles[3];
    const int n = L.n, ns = L.nseq;
    e = vggt::launch_k_tiles_bf16(vggt::contiguous_keys(k, n), tk, ns, n, H, table, T, nullptr,
                                  nullptr, 0.0f, st);
    if (e == hipSuccess)
      e = vggt::launch_k_tiles_bf16(vggt::contiguous_keys(v, n), tv, ns, n, H, nullptr, 1, nullptr,
                                    nullptr, 0.0f, st);
    if (e == hipSuccess)
      e = vggt::launch_k_tiles_bf16(vggt::contiguous_keys(q, n), tq, ns, n, H, table, T, nullptr, nullptr, 0.0f, st,
                                    c);
    if (e == hipSuccess)
      e = vggt::launch_k_tiles_bf16(vggt::contiguous_keys(dout, n), tdo, ns, n, H, nullptr, 1, nullptr, nullptr, 0.0f,
                                    st);
    if (e != hipSuccess) return device_error("backward tile pre-pass", e);
    vggt::AttnBwdProblem p;
    std::memset(&p, 0, sizeof(p));
    p.q = q;
    p.dout = dout;
    p.kr = kr;
    p.v = v;
    p.rope_tab = (const vggt::f32x2*)table;
    p.rope_T = T;
    p.k_rows = tk;
    p.v_rows = tv;
    p.q_rows = tq;
    p.do_rows = tdo;
    p.lse2 = lse2;
    p.dsum = dsum;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.tok_stride = (int64_t)H * vggt::kHeadDim;
    p.seq_stride = seq_stride;
    p.nseq = ns;
    p.n = n;
    p.H = H;
    p.ntile = L.ntile;
    p.scale_log2 = c;
    p.scale = sc;
    for (int pass = 0; pass < 2; ++pass) {
      const int slot = timer_claim(pass == 0 ? VGGT_TIMER_BWD_DQ : VGGT_TIMER_BWD_DKDV);
      if (slot >= 0) e = hipEventRecord(g_timer.ev[2 * slot], st);
      if (e == hipSuccess) e = vggt::launch_attn_bwd_bf16(p, pass == 0, st);
      if (e == hipSuccess && slot >= 0) e = hipEventRecord(g_timer.ev[2 * slot + 1], st);
      if (e != hipSuccess) return device_error("backward launch", e);
    }
    return VGGT_OK;
  }
  // fp32 debug path
  const float* qr = (const float*)q;
  const float* kr = (const float*)k;
  float* dqr = (float*)dq;
  float* dkr = (float*)dk;
  if (pos) {
    e = vggt::launch_rope(q, ws + L.qr, false, N, T, H, pos, (double)base, st);
    if (e == hipSuccess) e = vggt::launch_rope(k, ws + L.kr, false, N, T, H, pos, (double)base, st);
    if (e != hipSuccess) return device_error("backward rotation", e);
    qr = (const float*)(ws + L.qr);
    kr = (const float*)(ws + L.kr);
    dqr = (float*)(ws + L.dqr);
    dkr = (float*)(ws + L.dkr);
  }
  e = vggt::launch_attn_bwd_f32(qr, kr, (const float*)v, (const float*)dout, lse2, dsum, dqr, dkr, (float*)dv, L.nseq,
                                L.n, seq_stride, H, L.ntile, c, sc, st);
  if (e == hipSuccess && pos) e = vggt::launch_rope(dqr, dq, false, N, T, H, pos, (double)base, st, true);
  if (e == hipSuccess && pos) e = vggt::launch_rope(dkr, dk, false, N, T, H, pos, (double)base, st, true);
  if (e != hipSuccess) return device_error("backward launch", e);
  return VGGT_OK;
}

}  // namespace

VGGT_API size_t vggt_attn_backward_workspace(int S, int T, int H, int global, int rope_on, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H)) return 0;
  if (S == 0) return 0;
  return plan_bwd(global != 0, S, T, H, rope_on != 0, dt).total;
}

VGGT_API vggt_status vggt_frame_attn_backward(const void* q, const void* k, const void* v, const void* o,
                                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                              vggt_dtype dt, int S, int T, int H, const int32_t* pos_yx,
                                              float rope_base, float scale, void* workspace, size_t ws_bytes,
                                              void* stream) {
  return attn_backward(false, q, k, v, o, dout, lse, dq, dk, dv, dt, S, T, H, pos_yx, rope_base, scale, workspace,
                       ws_bytes, stream);
}

VGGT_API vggt_status vggt_global_attn_backward(const void* q, const void* k, const void* v, const void* o,
                                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                               vggt_dtype dt, int S, int T, int H, const int32_t* pos_yx,
                                               float rope_base, float scale, void* workspace, size_t ws_bytes,
                                               void* stream) {
  return attn_backward(true, q, k, v, o, dout, lse, dq, dk, dv, dt, S, T, H, pos_yx, rope_base, scale, workspace,
                       ws_bytes, stream);
}
