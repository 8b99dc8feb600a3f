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

#include "common.h"

#define VGGT_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

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
constexpr int kAssumedCUs = 256;       // MI355X; used only to size the key split
constexpr int kWorkgroupsPerCU = 2;

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

// ---- key-split plan (a pure function of the shape, shared by the workspace
//      queries and the calls)
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
    // Balance the last wave of workgroups against the merge pass.  Time is
    // modelled in units of one key tile processed by one resident workgroup:
    //   attention(s) = ceil(wg * s / slots) * ceil(ktiles / s)
    //   merge(s)     = partial bytes / (bytes one slot-tile-time moves), s > 1
    const int64_t wg = ((nq + query_tile(dt) - 1) / query_tile(dt)) * H;
    const int64_t slots = (int64_t)kAssumedCUs * kWorkgroupsPerCU;
    double best = 1e300;
    for (int s = 1; s <= kMaxSplits && s <= ktiles; ++s) {
      const double att = (double)((wg * s + slots - 1) / slots) * (double)((ktiles + s - 1) / s);
      // one tile-time ~ 0.7 us; merge moves s*nq*H*(64+2)*4 bytes twice plus
      // the output, at ~4 TB/s -> bytes / (4e6 B/us) / 0.7 us
      const double bytes = s > 1 ? (double)nq * H * (2.0 * s * 66 * 4 + 64 * 2) : 0.0;
      const double cost = att + bytes / 4.0e6 / 0.7;
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

size_t partial_bytes(int64_t nq, int H, int splits) {
  if (splits <= 1) return 0;
  return align256((size_t)splits * nq * H * vggt::kHeadDim * 4) + align256((size_t)splits * nq * H * 2 * 4);
}

hipError_t run_attention(const vggt::AttnProblem& p, vggt_dtype dt, hipStream_t st) {
  hipError_t e = dt == VGGT_F32 ? vggt::launch_attn_f32(p, st) : vggt::launch_attn_bf16(p, st);
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

vggt_status validate_attn(const QKVO& t, vggt_dtype dt, int S, int T, int H, const int32_t* pos, float base,
                          size_t need_ws, const void* ws, size_t ws_bytes, size_t q_bytes, size_t kv_bytes) {
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
  (void)S; (void)T; (void)H; (void)dt;
  return VGGT_OK;
}

size_t rope_copy_bytes(int S, int T, int H, vggt_dtype dt) {
  return align256((size_t)S * T * H * vggt::kHeadDim * elem_size(dt));
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

}  // namespace

VGGT_API size_t vggt_frame_attn_workspace(int S, int T, int H, int rope_on, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H)) return 0;
  return rope_on ? 2 * rope_copy_bytes(S, T, H, dt) : 0;
}

VGGT_API vggt_status vggt_frame_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                     int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                     void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (S == 0) return VGGT_OK;
  const size_t bytes = (size_t)S * T * H * vggt::kHeadDim * elem_size(dt);
  const size_t need = vggt_frame_attn_workspace(S, T, H, pos_yx != nullptr, dt);
  if (vggt_status s = validate_attn({q, k, v, o}, dt, S, T, H, pos_yx, rope_base, need, workspace, ws_bytes, bytes,
                                    bytes))
    return s;
  if (vggt_status s = check_device()) return s;
  hipStream_t st = (hipStream_t)stream;
  const void *qa = q, *ka = k;
  if (pos_yx) {
    char* ws = (char*)workspace;
    void* qr = ws;
    void* kr = ws + rope_copy_bytes(S, T, H, dt);
    hipError_t e = vggt::launch_rope(q, qr, dt == VGGT_BF16, (int64_t)S * T, T, H, pos_yx, rope_base, st);
    if (e == hipSuccess) e = vggt::launch_rope(k, kr, dt == VGGT_BF16, (int64_t)S * T, T, H, pos_yx, rope_base, st);
    if (e != hipSuccess) return device_error("rope launch", e);
    qa = qr;
    ka = kr;
  }
  vggt::AttnProblem p = base_problem(qa, ka, v, o, H, scale);
  p.q_seq_stride = T;
  p.k_seq_stride = T;
  p.nq = T;
  p.nk = T;
  p.nseq = S;
  p.nq_total = (int64_t)S * T;
  p.splits = 1;
  p.keys_per_split = ((T + vggt::kAttnKeyTile - 1) / vggt::kAttnKeyTile) * vggt::kAttnKeyTile;
  hipError_t e = run_attention(p, dt, st);
  if (e != hipSuccess) return device_error("attention launch", e);
  return VGGT_OK;
}

VGGT_API size_t vggt_global_attn_workspace(int S, int T, int H, int kv_splits, int rope_on, vggt_dtype dt) {
  if (!dtype_ok(dt) || !tokens_ok(S, T, H) || kv_splits < 0 || kv_splits > kMaxSplits) return 0;
  const int64_t N = (int64_t)S * T;
  const SplitPlan sp = plan_splits(N, N, H, kv_splits, dt);
  return (rope_on ? 2 * rope_copy_bytes(S, T, H, dt) : 0) + partial_bytes(N, H, sp.splits);
}

VGGT_API vggt_status vggt_global_attn(const void* q, const void* k, const void* v, void* o, vggt_dtype dt, int S,
                                      int T, int H, const int32_t* pos_yx, float rope_base, float scale,
                                      int kv_splits, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!dtype_ok(dt)) return fail(VGGT_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (!tokens_ok(S, T, H)) return fail(VGGT_ERR_SHAPE, "bad shape S=%d T=%d H=%d", S, T, H);
  if (kv_splits < 0 || kv_splits > kMaxSplits) return fail(VGGT_ERR_SHAPE, "kv_splits must be in [0, %d]", kMaxSplits);
  if (S == 0) return VGGT_OK;
  const int64_t N = (int64_t)S * T;
  const size_t bytes = (size_t)N * H * vggt::kHeadDim * elem_size(dt);
  const size_t need = vggt_global_attn_workspace(S, T, H, kv_splits, pos_yx != nullptr, dt);
  if (vggt_status s = validate_attn({q, k, v, o}, dt, S, T, H, pos_yx, rope_base, need, workspace, ws_bytes, bytes,
                                    bytes))
    return s;
  if (vggt_status s = check_device()) return s;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const void *qa = q, *ka = k;
  if (pos_yx) {
    void* qr = ws;
    void* kr = ws + rope_copy_bytes(S, T, H, dt);
    hipError_t e = vggt::launch_rope(q, qr, dt == VGGT_BF16, N, T, H, pos_yx, rope_base, st);
    if (e == hipSuccess) e = vggt::launch_rope(k, kr, dt == VGGT_BF16, N, T, H, pos_yx, rope_base, st);
    if (e != hipSuccess) return device_error("rope launch", e);
    qa = qr;
    ka = kr;
    ws += 2 * rope_copy_bytes(S, T, H, dt);
  }
  const SplitPlan sp = plan_splits(N, N, H, kv_splits, dt);
  vggt::AttnProblem p = base_problem(qa, ka, v, o, H, scale);
  p.q_seq_stride = 0;
  p.k_seq_stride = 0;
  p.nq = (int)N;
  p.nk = (int)N;
  p.nseq = 1;
  p.nq_total = N;
  p.splits = sp.splits;
  p.keys_per_split = sp.keys_per_split;
  if (sp.splits > 1) {
    p.part_o = (float*)ws;
    p.part_ml = (float*)(ws + align256((size_t)sp.splits * N * H * vggt::kHeadDim * 4));
  }
  hipError_t e = run_attention(p, dt, st);
  if (e != hipSuccess) return device_error("attention launch", e);
  return VGGT_OK;
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
  const int64_t nq = (int64_t)S * T, nk = (int64_t)S * Dn;
  const SplitPlan sp = plan_splits(nq, nk, H, kv_splits, dt);
  return partial_bytes(nq, H, sp.splits);
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
  const size_t need = vggt_descriptor_xattn_workspace(S, T, Dn, H, kv_splits, dt);
  if (vggt_status s = validate_attn({q, kd, vd, o}, dt, S, T, H, nullptr, 0.0f, need, workspace, ws_bytes, q_b, kv_b))
    return s;
  if (vggt_status s = check_device()) return s;
  const SplitPlan sp = plan_splits(nq, nk, H, kv_splits, dt);
  vggt::AttnProblem p = base_problem(q, kd, vd, o, H, scale);
  p.nq = (int)nq;
  p.nk = (int)nk;
  p.nseq = 1;
  p.nq_total = nq;
  p.splits = sp.splits;
  p.keys_per_split = sp.keys_per_split;
  if (sp.splits > 1) {
    char* ws = (char*)workspace;
    p.part_o = (float*)ws;
    p.part_ml = (float*)(ws + align256((size_t)sp.splits * nq * H * vggt::kHeadDim * 4));
  }
  hipError_t e = run_attention(p, dt, (hipStream_t)stream);
  if (e != hipSuccess) return device_error("attention launch", e);
  return VGGT_OK;
}
