/*
 * Reference oracle for the alternating-attention hot path of VGGT-style
 * aggregators (frame-wise attention, global attention, FlashVGGT descriptor
 * pooling and descriptor cross-attention, 2D rotary position embedding).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Everything is float64.  Inputs arrive as float64 arrays that the caller
 * converted exactly from the bf16 (or fp32) bit patterns the GPU consumes.
 * Memory layout of every token tensor: [token][head][dim], row-major, i.e. the
 * [S, T, H, D] layout flattened over (S, T).
 *
 * No tiling, no online rescaling, no fusion: each function is the textbook
 * definition, with threads only splitting independent (row, head) items.
 *
 * Sources (web pages):
 *  - "VGGT 論文報告" slide deck (computer-vision-3uw.pages.dev):
 *      Section V "Attention", slides 4/10 (softmax), 5/10 (scaled
 *      dot-product attention softmax(Q K^T / sqrt(d_k)) V), 9/10 (multi-head);
 *      Section IV "Positional Encoding", slide 4/6 (frequency schedule
 *      pos / 10000^(2i/d), even/odd dimension pairs);
 *      Section XI "架構" slide 3/7 (Global + Frame Attention).
 *  - "VGGT-Omega-1B-512-bf16" config article (lpnh.cn): the input-parameter
 *      section (rope_base 100.0; the RoPE "periods" buffers are fp32).
 *  - "FlashVGGT: Efficient and Scalable Visual Geometry Transformers with
 *      Compressed Descriptor Attention" README: Overview (per-frame compact
 *      descriptor set, cross-attention from all tokens to it) and Key
 *      Arguments (--kv_downfactor, default 4).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - RoPE: the head vector splits into two halves; the first half rotates by
 *    the token's row, the second by its column.  Inside a half of width
 *    d_axis, pair (2k, 2k+1) rotates by angle p * base^(-2k/d_axis).
 *  - No attention mask.  Scale defaults to 1/sqrt(D).
 *  - Pooling windows that overhang the grid average only their valid cells.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* 2D rotary position embedding                                             */
/* ------------------------------------------------------------------------ */

/*
 * Angular frequency of rotation pair k inside one axis of width d_axis.
 * The slide deck's sinusoidal encoding (Section IV, slide 4/6) divides the
 * position by base^(2i/d) for pair i; written as a frequency that is
 * base^(-2k/d_axis).
 */
double oracle_rope_freq(double base, int d_axis, int k) {
  return pow(base, -2.0 * (double)k / (double)d_axis);
}

/*
 * Rotate every head vector of n_tok tokens in place.
 *   x      [n_tok][H][D] float64, D divisible by 4
 *   pos_yx [n_tok][2] int32 (row, col) of each token
 * For axis a (0 = row, 1 = col), the half x[a*D/2 .. a*D/2 + D/2) is split
 * into D/4 pairs (2k, 2k+1), each rotated by theta = p_a * freq(base, D/2, k):
 *   x'[i]   = x[i] cos(theta) - x[i+1] sin(theta)
 *   x'[i+1] = x[i] sin(theta) + x[i+1] cos(theta)
 * Position (0, 0) gives theta = 0 for every pair, the identity.
 */
void oracle_rope(double* x, int64_t n_tok, int H, int D, const int32_t* pos_yx, double base) {
  const int half = D / 2;
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int h = 0; h < H; ++h) {
      double* u = x + (t * H + h) * (int64_t)D;
      for (int a = 0; a < 2; ++a) {
        const double p = (double)pos_yx[2 * t + a];
        for (int k = 0; k < half / 2; ++k) {
          const double theta = p * oracle_rope_freq(base, half, k);
          const double c = cos(theta), s = sin(theta);
          const int i = a * half + 2 * k;
          const double u0 = u[i], u1 = u[i + 1];
          u[i] = u0 * c - u1 * s;
          u[i + 1] = u0 * s + u1 * c;
        }
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Per-head LayerNorm of Q and K                                            */
/* ------------------------------------------------------------------------ */

/*
 * Centered LayerNorm over the D channels of every head vector, in place
 * (VGGT-JAX README, kernel-trial table: LayerNorm on the Q/K shapes, the
 * existing centered LayerNorm kept; VGGT-Omega-1B-512-bf16 config article,
 * model-structure section: layer_norm_eps 1e-05):
 *   mu     = mean_c u_c
 *   var    = mean_c (u_c - mu)^2              (biased)
 *   u'_c   = (u_c - mu) / sqrt(var + eps) * gamma_c + beta_c
 *   x      [n_tok][H][D] float64; gamma, beta [D] float64, shared by the heads.
 */
void oracle_layer_norm(double* x, int64_t n_tok, int H, int D, const double* gamma, const double* beta,
                       double eps) {
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int h = 0; h < H; ++h) {
      double* u = x + (t * H + h) * (int64_t)D;
      double mu = 0.0;
      for (int c = 0; c < D; ++c) mu += u[c];
      mu /= D;
      double var = 0.0;
      for (int c = 0; c < D; ++c) var += (u[c] - mu) * (u[c] - mu);
      var /= D;
      const double inv = 1.0 / sqrt(var + eps);
      for (int c = 0; c < D; ++c) u[c] = (u[c] - mu) * inv * gamma[c] + beta[c];
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Scaled dot-product attention, multi-head                                 */
/* ------------------------------------------------------------------------ */

/*
 * One query row of one head against a key set of nk tokens
 * (slide deck Section V, slides 4/10 and 5/10):
 *   s_j = scale * <q, k_j>
 *   p_j = exp(s_j - max_j s_j)            (softmax numerator; the max shift
 *                                          leaves the quotient unchanged)
 *   o   = sum_j p_j v_j / sum_j p_j
 * k and v point at head h of key token 0; consecutive key tokens are
 * `stride` doubles apart.  `scores` is caller scratch of nk doubles.
 */
static void attend_row(const double* q, const double* k, const double* v, int64_t nk, int64_t stride,
                       int D, double scale, double* scores, double* o) {
  double m = -INFINITY;
  for (int64_t j = 0; j < nk; ++j) {
    const double* kj = k + j * stride;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * kj[d];
    scores[j] = scale * dot;
    if (scores[j] > m) m = scores[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    scores[j] = exp(scores[j] - m);
    l += scores[j];
  }
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    const double* vj = v + j * stride;
    for (int d = 0; d < D; ++d) o[d] += scores[j] * vj[d];
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
}

/*
 * The key set of query token r:
 *   group_q == 0 : every key token (global attention, descriptor
 *                  cross-attention);
 *   group_q  > 0 : query tokens are grouped in consecutive runs of group_q
 *                  (one frame each); query r sees the keys of its own frame,
 *                  the run [ (r / group_q) * group_k, ... + group_k ).
 * (Frame vs global attention: slide deck Section XI, slide 3/7.)
 */
typedef struct {
  const double *q, *k, *v;
  double* o;
  int64_t nq, nk;
  int H, D;
  int64_t group_q, group_k;
  double scale;
  const int64_t* rows;  /* query tokens to evaluate, or NULL = all */
  int64_t nrows;
  int64_t next;         /* shared work counter over (row, head) items */
  pthread_mutex_t lock;
} attn_job;

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  const int64_t stride = (int64_t)J->H * J->D;
  const int64_t kmax = J->group_q > 0 ? J->group_k : J->nk;
  double* scores = (double*)malloc(sizeof(double) * (size_t)(kmax > 0 ? kmax : 1));
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const int64_t item = J->next;
    J->next += 1;
    pthread_mutex_unlock(&J->lock);
    if (item >= J->nrows * J->H) break;
    const int64_t ri = item / J->H;
    const int h = (int)(item % J->H);
    const int64_t r = J->rows ? J->rows[ri] : ri;
    int64_t k0 = 0, nk = J->nk;
    if (J->group_q > 0) {
      k0 = (r / J->group_q) * J->group_k;
      nk = J->group_k;
    }
    const double* q = J->q + r * stride + (int64_t)h * J->D;
    const double* k = J->k + k0 * stride + (int64_t)h * J->D;
    const double* v = J->v + k0 * stride + (int64_t)h * J->D;
    double* o = J->o + ri * stride + (int64_t)h * J->D;
    attend_row(q, k, v, nk, stride, J->D, J->scale, scores, o);
  }
  free(scores);
  return NULL;
}

/*
 * Multi-head attention (slide deck Section V, slide 9/10: heads are
 * independent and their outputs are concatenated along the feature axis).
 *   q [nq][H][D], k/v [nk][H][D] float64; o [nrows][H][D] (row ri of o holds
 *   query token rows[ri], or token ri when rows == NULL).
 * group_q/group_k select frame-wise grouping as described above.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attention(const double* q, const double* k, const double* v, double* o, int64_t nq, int64_t nk,
                     int H, int D, int64_t group_q, int64_t group_k, double scale, const int64_t* rows,
                     int64_t nrows, int nthreads) {
  if (H <= 0 || D <= 0 || nq < 0 || nk <= 0) return -1;
  if (group_q > 0 && (group_k <= 0 || nq % group_q != 0 || (nq / group_q) * group_k != nk)) return -1;
  if (rows) {
    for (int64_t i = 0; i < nrows; ++i)
      if (rows[i] < 0 || rows[i] >= nq) return -1;
  } else {
    nrows = nq;
  }
  attn_job J;
  J.q = q; J.k = k; J.v = v; J.o = o;
  J.nq = nq; J.nk = nk; J.H = H; J.D = D;
  J.group_q = group_q; J.group_k = group_k; J.scale = scale;
  J.rows = rows; J.nrows = nrows; J.next = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, attn_worker, &J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J.lock);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention gradients                                                      */
/* ------------------------------------------------------------------------ */

/*
 * The chain rule through one head of o_i = sum_j p_ij v_j,
 * p_ij = exp(s_ij) / sum_l exp(s_il), s_ij = scale <q_i, k_j>, given the
 * upstream gradient do_i of every output row:
 *   dv_j  = sum_i p_ij do_i
 *   dp_ij = <do_i, v_j>
 *   ds_ij = p_ij (dp_ij - sum_l p_il dp_il)      (Jacobian of the softmax row)
 *   dq_i  = scale sum_j ds_ij k_j
 *   dk_j  = scale sum_i ds_ij q_i
 * lse_i = log sum_l exp(s_il) is the row's log-normaliser, so that
 * p_ij = exp(s_ij - lse_i).  Key sets (group_q/group_k) as for
 * oracle_attention.  The work is done in three plain passes per head:
 *   1. every query row: lse_i and c_i = sum_l p_il dp_il (two-pass softmax);
 *   2. the requested query rows: dq_i;
 *   3. the requested key rows: dk_j and dv_j, summing over the queries whose
 *      key set holds j.
 * rows/cols select query/key tokens (NULL = all); dq is [nrows][H][D], dk and
 * dv are [ncols][H][D].  Threads split (head, row) items of each pass.
 */
typedef struct {
  const double *q, *k, *v, *dout;
  double *dq, *dk, *dv, *lse, *csum;
  const char* need;  /* pass 1 runs for the query rows that passes 2 and 3 read */
  int64_t nq, nk;
  int H, D;
  int64_t group_q, group_k;
  double scale;
  const int64_t *rows, *cols;
  int64_t nrows, ncols;
  int phase;
  int64_t next;
  pthread_mutex_t lock;
} bwd_job;

static void key_range(const bwd_job* J, int64_t i, int64_t* k0, int64_t* nk) {
  *k0 = 0;
  *nk = J->nk;
  if (J->group_q > 0) {
    *k0 = (i / J->group_q) * J->group_k;
    *nk = J->group_k;
  }
}

static double dot(const double* a, const double* b, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += a[d] * b[d];
  return s;
}

static void* bwd_worker(void* arg) {
  bwd_job* J = (bwd_job*)arg;
  const int64_t stride = (int64_t)J->H * J->D;
  const int D = J->D;
  const int64_t kmax = J->group_q > 0 ? J->group_k : J->nk;
  double* sc = (double*)malloc(sizeof(double) * (size_t)(kmax > 0 ? kmax : 1));
  const int64_t items = J->phase == 1 ? J->nq : (J->phase == 2 ? J->nrows : J->ncols);
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const int64_t item = J->next;
    J->next += 1;
    pthread_mutex_unlock(&J->lock);
    if (item >= items * J->H) break;
    const int64_t it = item / J->H;
    const int h = (int)(item % J->H);
    if (J->phase == 1 || J->phase == 2) {
      const int64_t i = J->phase == 1 ? it : (J->rows ? J->rows[it] : it);
      int64_t k0, nk;
      key_range(J, i, &k0, &nk);
      const double* qi = J->q + i * stride + (int64_t)h * D;
      const double* doi = J->dout + i * stride + (int64_t)h * D;
      if (J->phase == 1) {
        if (!J->need[i]) continue;
        double m = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
          sc[j] = J->scale * dot(qi, J->k + (k0 + j) * stride + (int64_t)h * D, D);
          if (sc[j] > m) m = sc[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nk; ++j) l += exp(sc[j] - m);
        const double lse = m + log(l);
        double c = 0.0;
        for (int64_t j = 0; j < nk; ++j)
          c += exp(sc[j] - lse) * dot(doi, J->v + (k0 + j) * stride + (int64_t)h * D, D);
        J->lse[i * J->H + h] = lse;
        J->csum[i * J->H + h] = c;
      } else {
        double* dqi = J->dq + it * stride + (int64_t)h * D;
        for (int d = 0; d < D; ++d) dqi[d] = 0.0;
        const double lse = J->lse[i * J->H + h], c = J->csum[i * J->H + h];
        for (int64_t j = 0; j < nk; ++j) {
          const double* kj = J->k + (k0 + j) * stride + (int64_t)h * D;
          const double p = exp(J->scale * dot(qi, kj, D) - lse);
          const double ds = p * (dot(doi, J->v + (k0 + j) * stride + (int64_t)h * D, D) - c);
          for (int d = 0; d < D; ++d) dqi[d] += J->scale * ds * kj[d];
        }
      }
    } else {
      const int64_t j = J->cols ? J->cols[it] : it;
      const double* kj = J->k + j * stride + (int64_t)h * D;
      const double* vj = J->v + j * stride + (int64_t)h * D;
      double* dkj = J->dk + it * stride + (int64_t)h * D;
      double* dvj = J->dv + it * stride + (int64_t)h * D;
      for (int d = 0; d < D; ++d) dkj[d] = dvj[d] = 0.0;
      int64_t i0 = 0, i1 = J->nq;  /* queries whose key set holds key j */
      if (J->group_q > 0) {
        i0 = (j / J->group_k) * J->group_q;
        i1 = i0 + J->group_q;
      }
      for (int64_t i = i0; i < i1; ++i) {
        const double* qi = J->q + i * stride + (int64_t)h * D;
        const double* doi = J->dout + i * stride + (int64_t)h * D;
        const double p = exp(J->scale * dot(qi, kj, D) - J->lse[i * J->H + h]);
        const double ds = p * (dot(doi, vj, D) - J->csum[i * J->H + h]);
        for (int d = 0; d < D; ++d) {
          dvj[d] += p * doi[d];
          dkj[d] += J->scale * ds * qi[d];
        }
      }
    }
  }
  free(sc);
  return NULL;
}

int oracle_attention_backward(const double* q, const double* k, const double* v, const double* dout, double* dq,
                              double* dk, double* dv, double* lse, int64_t nq, int64_t nk, int H, int D,
                              int64_t group_q, int64_t group_k, double scale, const int64_t* rows, int64_t nrows,
                              const int64_t* cols, int64_t ncols, int nthreads) {
  if (H <= 0 || D <= 0 || nq <= 0 || nk <= 0) return -1;
  if (group_q > 0 && (group_k <= 0 || nq % group_q != 0 || (nq / group_q) * group_k != nk)) return -1;
  if (rows) {
    for (int64_t i = 0; i < nrows; ++i)
      if (rows[i] < 0 || rows[i] >= nq) return -1;
  } else {
    nrows = nq;
  }
  if (cols) {
    for (int64_t i = 0; i < ncols; ++i)
      if (cols[i] < 0 || cols[i] >= nk) return -1;
  } else {
    ncols = nk;
  }
  /* rows whose log-normaliser is read: the requested query rows, and every query
     whose key set holds a requested key */
  char* need = (char*)calloc((size_t)nq, 1);
  for (int64_t i = 0; i < nrows; ++i) need[rows ? rows[i] : i] = 1;
  for (int64_t c = 0; c < ncols; ++c) {
    const int64_t j = cols ? cols[c] : c;
    const int64_t i0 = group_q > 0 ? (j / group_k) * group_q : 0;
    const int64_t i1 = group_q > 0 ? i0 + group_q : nq;
    for (int64_t i = i0; i < i1; ++i) need[i] = 1;
  }
  bwd_job J;
  J.need = need;
  J.q = q; J.k = k; J.v = v; J.dout = dout;
  J.dq = dq; J.dk = dk; J.dv = dv;
  J.lse = lse;  /* [nq][H], filled by pass 1 */
  J.csum = (double*)malloc(sizeof(double) * (size_t)(nq * H));
  J.nq = nq; J.nk = nk; J.H = H; J.D = D;
  J.group_q = group_q; J.group_k = group_k; J.scale = scale;
  J.rows = rows; J.cols = cols; J.nrows = nrows; J.ncols = ncols;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int phase = 1; phase <= 3; ++phase) {
    J.phase = phase;
    J.next = 0;
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  }
  pthread_mutex_destroy(&J.lock);
  free(J.csum);
  free(need);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* FlashVGGT descriptor pooling                                             */
/* ------------------------------------------------------------------------ */

/*
 * Number of descriptor tokens per frame: the special tokens (those outside
 * the gh x gw patch grid) plus one cell per ph x pw window of the grid, with
 * windows that overhang the last row/column kept (ceil division).
 */
int oracle_descriptor_count(int T, int gh, int gw, int ph, int pw) {
  const int cells_h = (gh + ph - 1) / ph, cells_w = (gw + pw - 1) / pw;
  return (T - gh * gw) + cells_h * cells_w;
}

/*
 * Per-frame spatial compression of keys or values into descriptor tokens
 * (FlashVGGT README, Overview; the window size is the --kv_downfactor of the
 * Key Arguments read as a token-count factor, 4 = 2 x 2).
 *   in  [S][T][H][D]; the patch grid occupies tokens
 *       [patch_begin, patch_begin + gh*gw) of each frame, row-major.
 *   out [S][Dn][H][D], Dn = oracle_descriptor_count(...):
 *       first the special tokens in their original order, copied;
 *       then cell (a, b) for a < ceil(gh/ph), b < ceil(gw/pw), row-major,
 *       holding the mean over the valid grid cells
 *       r in [a*ph, min((a+1)*ph, gh)), c in [b*pw, min((b+1)*pw, gw)).
 */
int oracle_descriptor_pool(const double* in, double* out, int S, int T, int H, int D, int gh, int gw,
                           int patch_begin, int ph, int pw) {
  if (S < 0 || T <= 0 || H <= 0 || D <= 0 || gh <= 0 || gw <= 0 || ph <= 0 || pw <= 0) return -1;
  if (patch_begin < 0 || patch_begin + gh * gw > T) return -1;
  const int Dn = oracle_descriptor_count(T, gh, gw, ph, pw);
  const int cells_h = (gh + ph - 1) / ph, cells_w = (gw + pw - 1) / pw;
  const int64_t tok = (int64_t)H * D;
  for (int s = 0; s < S; ++s) {
    const double* fin = in + (int64_t)s * T * tok;
    double* fout = out + (int64_t)s * Dn * tok;
    int w = 0;
    for (int t = 0; t < T; ++t) {
      if (t >= patch_begin && t < patch_begin + gh * gw) continue;
      memcpy(fout + (int64_t)w * tok, fin + (int64_t)t * tok, sizeof(double) * (size_t)tok);
      ++w;
    }
    for (int a = 0; a < cells_h; ++a) {
      for (int b = 0; b < cells_w; ++b) {
        double* cell = fout + (int64_t)w * tok;
        for (int64_t e = 0; e < tok; ++e) cell[e] = 0.0;
        int count = 0;
        for (int r = a * ph; r < (a + 1) * ph && r < gh; ++r) {
          for (int c = b * pw; c < (b + 1) * pw && c < gw; ++c) {
            const double* src = fin + (int64_t)(patch_begin + r * gw + c) * tok;
            for (int64_t e = 0; e < tok; ++e) cell[e] += src[e];
            ++count;
          }
        }
        for (int64_t e = 0; e < tok; ++e) cell[e] /= (double)count;
        ++w;
      }
    }
  }
  return 0;
}
