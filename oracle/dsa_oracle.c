/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DeepSeek Sparse Attention (DSA) path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this file;
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header, table or helper with the HIP path.
 *
 * Source of the arithmetic (web pages on DeepSeek-V3.2):
 *   - "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models" (velog summary),
 *     section 1.1 "Lightning Indexer", equation I_{t,s} = sum_j w^I_{t,j} * ReLU(q^I_{t,j} . k^I_s),
 *     scored between a query token and the tokens before it; the indexer is FP8 with few heads.
 *   - same page, section 1.2 "Fine-grained Token Selection & Attention": only the key/value
 *     entries whose index score is in Top-k(I_{t,:}) are retrieved, u_t = Attn(h_t, {c_s}).
 *   - same page, section 1.3: MLA in MQA mode, every latent KV entry shared by all query heads.
 *   - same page, "Continued Pre-Training", Stage 2: 2048 key/value tokens selected per query.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - causal domain is s <= pos_t (the query's own token is a candidate);
 *   - fp8 is OCP e4m3fn; dequantisation is one fp32 rounding of code * scale, per the stated
 *     "indexer in fp32 from fp8-dequantised inputs"; dot products and the head sum are
 *     accumulated in double and the score is rounded once to fp32;
 *   - top-k ties go to the lower index, -0 equals +0, rows with fewer than k candidates keep
 *     all of them, selections are emitted in ascending index order, padded with -1;
 *   - attention: K is the whole latent row (d_qk columns), V is its first d_v columns,
 *     softmax scale is an explicit argument; everything in double;
 *   - sparse training stage: the main model's gradient is the chain rule through that attention
 *     (the key and value gradients add on the shared latent row); the indexer's target there is the
 *     head mean of the sparse attention probabilities (zero outside the selection), and its loss keeps
 *     the warm-up form, KL to the softmax of the index scores over every causal key.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC dsa_oracle.c -o liboracle.so -lm
 * OpenMP only distributes independent rows over threads; it changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- number formats */

/* OCP 8-bit float E4M3 ("fn" flavour): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
 * Exponent field 0 encodes subnormals m/8 * 2^-6.  S.1111.111 is NaN; there is no infinity,
 * so the largest finite magnitude is 1.75 * 2^8 = 448. */
float oracle_e4m3_to_f32(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return (float)(sign ? -mag : mag);
}

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void oracle_decode_e4m3(const uint8_t* codes, int64_t n, float* out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_to_f32(codes[i]);
}

void oracle_decode_bf16(const uint16_t* bits, int64_t n, float* out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_to_f32(bits[i]);
}

/* Dequantise row-scaled fp8: out[r][c] = fp32( e4m3(codes[r][c]) * scale[r] ), one fp32 rounding. */
void oracle_dequant_e4m3(const uint8_t* codes, const float* scales, int64_t rows, int64_t cols,
                         float* out) {
  for (int64_t r = 0; r < rows; r++) {
    float s = scales[r];
    for (int64_t c = 0; c < cols; c++) {
      float v = oracle_e4m3_to_f32(codes[r * cols + c]);
      out[r * cols + c] = v * s; /* product of two floats, rounded to float */
    }
  }
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- lightning indexer */

/* Index scores of n_rows query tokens against the key tokens 0..pos[r].
 *   q      [n_rows][H][d]   indexer queries q^I_{t,j} (already dequantised, fp32)
 *   w      [n_rows][H]      indexer head weights w^I_{t,j}
 *   k      [n_kv][d]        indexer keys k^I_s, one per token, shared by all indexer heads
 *   pos    [n_rows]         position of each query token; keys s = 0..pos[r] are scored
 *   scores [n_rows][ld]     out: I[r][s] for s <= pos[r] (fp32); other entries untouched
 *   mag    [n_rows][ld]     out (nullable): sum_j |w| * ReLU(q.k), the magnitude the sum is made of
 *   absmag [n_rows][ld]     out (nullable): sum_j |w| * sum_i |q_i k_i|, the magnitude of every product
 *                           (bounds the rounding of the dot products, which can cancel)
 * I = sum_j w_j * max(q_j . k, 0), with the dot and the head sum in double, one final fp32 rounding.
 */
void oracle_indexer(const float* q, const float* w, const float* k, int64_t n_rows, const int64_t* pos,
                    int H, int d, float* scores, int64_t ld, float* mag, float* absmag) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; r++) {
    const float* qr = q + r * (int64_t)H * d;
    const float* wr = w + r * (int64_t)H;
    for (int64_t s = 0; s <= pos[r]; s++) {
      const float* ks = k + s * (int64_t)d;
      double acc = 0.0, amag = 0.0, pmag = 0.0;
      for (int j = 0; j < H; j++) {
        double dot = 0.0, dabs = 0.0;
        for (int i = 0; i < d; i++) {
          double prod = (double)qr[j * d + i] * (double)ks[i];
          dot += prod;
          dabs += fabs(prod);
        }
        double relu = dot > 0.0 ? dot : 0.0;
        acc += (double)wr[j] * relu;
        amag += fabs((double)wr[j]) * relu;
        pmag += fabs((double)wr[j]) * dabs;
      }
      scores[r * ld + s] = (float)acc + 0.0f; /* + 0.0f maps -0 to +0 */
      if (mag) mag[r * ld + s] = (float)amag;
      if (absmag) absmag[r * ld + s] = (float)pmag;
    }
  }
}

/* ---------------------------------------------------------------- top-k selection */

typedef struct {
  float v;
  int32_t s;
} cand_t;

/* Order: higher score first; equal scores (including -0 == +0) by lower index first. */
static int cand_cmp(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->s < y->s) ? -1 : (x->s > y->s) ? 1 : 0;
}

static int int_cmp(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x < y) ? -1 : (x > y) ? 1 : 0;
}

/* Per row: the k candidates s in 0..pos[r] with the largest scores, emitted in ascending s,
 * padded with -1.  kth[r] receives the k-th largest score, or -INFINITY when the row has at
 * most k candidates (then every candidate is kept). */
void oracle_topk(const float* scores, int64_t ld, int64_t n_rows, const int64_t* pos, int k,
                 int32_t* idx, float* kth) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; r++) {
    int64_t n = pos[r] + 1;
    int32_t* out = idx + r * (int64_t)k;
    if (n <= k) {
      for (int64_t i = 0; i < k; i++) out[i] = (i < n) ? (int32_t)i : -1;
      if (kth) kth[r] = -INFINITY;
      continue;
    }
    cand_t* c = (cand_t*)malloc((size_t)n * sizeof(cand_t));
    for (int64_t s = 0; s < n; s++) {
      c[s].v = scores[r * ld + s];
      c[s].s = (int32_t)s;
    }
    qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
    for (int i = 0; i < k; i++) out[i] = c[i].s;
    if (kth) kth[r] = c[k - 1].v;
    qsort(out, (size_t)k, sizeof(int32_t), int_cmp);
    free(c);
  }
}

/* ---------------------------------------------------------------- sparse MLA attention (MQA mode) */

/* For every query row r and head h, attention over the selected latent rows only:
 *   z_s   = sm_scale * sum_{i<d_qk} q[r][h][i] * kv[s][i]       for s in idx[r][:], s != -1
 *   out   = sum_s softmax(z)_s * kv[s][0:d_v]
 *   lse   = log sum_s exp(z_s)
 * kv rows are shared by all heads (MQA mode).  Entries equal to -1 are skipped.  All in double.
 *   q   [n_rows][H][d_qk], kv [n_kv][d_qk], idx [n_rows][k], out [n_rows][H][d_v], lse [n_rows][H]
 */
void oracle_sparse_attn(const float* q, const float* kv, const int32_t* idx, int64_t n_rows, int H,
                        int d_qk, int d_v, int k, double sm_scale, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t r = 0; r < n_rows; r++) {
    for (int h = 0; h < H; h++) {
      const float* qh = q + (r * H + h) * (int64_t)d_qk;
      const int32_t* sel = idx + r * (int64_t)k;
      double* o = out + (r * H + h) * (int64_t)d_v;
      double* z = (double*)malloc((size_t)k * sizeof(double));
      double m = -INFINITY;
      for (int i = 0; i < k; i++) {
        if (sel[i] < 0) continue;
        const float* c = kv + (int64_t)sel[i] * d_qk;
        double dot = 0.0;
        for (int e = 0; e < d_qk; e++) dot += (double)qh[e] * (double)c[e];
        z[i] = sm_scale * dot;
        if (z[i] > m) m = z[i];
      }
      for (int e = 0; e < d_v; e++) o[e] = 0.0;
      double l = 0.0;
      for (int i = 0; i < k; i++) {
        if (sel[i] < 0) continue;
        const float* c = kv + (int64_t)sel[i] * d_qk;
        double p = exp(z[i] - m);
        l += p;
        for (int e = 0; e < d_v; e++) o[e] += p * (double)c[e];
      }
      if (l > 0.0) {
        for (int e = 0; e < d_v; e++) o[e] /= l;
        lse[r * H + h] = m + log(l);
      } else {
        lse[r * H + h] = -INFINITY;
      }
      free(z);
    }
  }
}

/* Masked MHA mode (velog summary, section 3.3 Inference Cost; notes.yuuk.io, section on inference
 * cost): short prefills run attention in MHA form, each head with its own key and value rows, and
 * simulate DSA by masking every key outside the query's top-k selection.  Masking the other keys out
 * of the softmax leaves exactly the attention over the selected entries, so this is the same
 * definition as oracle_sparse_attn with per-head rows:
 *   z_s   = sm_scale * sum_e q[r][h][e] * k[s][h][e]            for s in idx[r] (entries -1 skipped)
 *   out   = sum_s softmax(z)_s * v[s][h][0:d_v],  lse = log sum_s exp(z_s)
 *   q [n_rows][H][d_qk], k [n_kv][H][d_qk], v [n_kv][H][d_v], idx [n_rows][k_sel],
 *   out [n_rows][H][d_v], lse [n_rows][H].  All in double.
 */
void oracle_sparse_attn_mha(const float* q, const float* kk, const float* v, const int32_t* idx, int64_t n_rows,
                            int H, int d_qk, int d_v, int k_sel, double sm_scale, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t r = 0; r < n_rows; r++) {
    for (int h = 0; h < H; h++) {
      const float* qh = q + (r * H + h) * (int64_t)d_qk;
      const int32_t* sel = idx + r * (int64_t)k_sel;
      double* o = out + (r * H + h) * (int64_t)d_v;
      double* z = (double*)malloc((size_t)k_sel * sizeof(double));
      double m = -INFINITY;
      for (int i = 0; i < k_sel; i++) {
        if (sel[i] < 0) continue;
        const float* ks = kk + ((int64_t)sel[i] * H + h) * d_qk;
        double dot = 0.0;
        for (int e = 0; e < d_qk; e++) dot += (double)qh[e] * (double)ks[e];
        z[i] = sm_scale * dot;
        if (z[i] > m) m = z[i];
      }
      for (int e = 0; e < d_v; e++) o[e] = 0.0;
      double l = 0.0;
      for (int i = 0; i < k_sel; i++) {
        if (sel[i] < 0) continue;
        const float* vs = v + ((int64_t)sel[i] * H + h) * d_v;
        const double p = exp(z[i] - m);
        l += p;
        for (int e = 0; e < d_v; e++) o[e] += p * (double)vs[e];
      }
      if (l > 0.0) {
        for (int e = 0; e < d_v; e++) o[e] /= l;
        lse[r * H + h] = m + log(l);
      } else {
        lse[r * H + h] = -INFINITY;
      }
      free(z);
    }
  }
}

/* ---------------------------------------------------------------- indexer warm-up loss
 * Dense warm-up stage (velog summary, Continued Pre-Training, Stage 1): the main model is frozen and
 * only the indexer learns.  Its target for query t is the main attention summed over heads and
 * L1-normalised; its loss is the KL divergence from that target to the softmax of the index scores:
 *   A_h[t][s] = softmax_s(sm_scale * q[t][h] . kv[s])              over s <= pos_t (dense, causal)
 *   p[t][s]   = sum_h A_h[t][s] / sum_s' sum_h A_h[t][s']  =  (1/H) sum_h A_h[t][s]
 *   L_t       = KL(p[t] || softmax(I[t]))  = sum_s p (log p - log softmax(I)_s)   (0 log 0 = 0)
 * and the gradient of L = sum_t L_t with respect to the index scores is g = softmax(I[t]) - p[t].
 */

/* p [n_rows][ld] (double) from q [n_rows][H][d_qk], kv [n_kv][d_qk]; entries past pos untouched. */
void oracle_warmup_target(const float* q, const float* kv, int64_t n_rows, const int64_t* pos, int H, int d_qk,
                          double sm_scale, double* p, int64_t ld) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; r++) {
    const int64_t n = pos[r] + 1;
    double* z = (double*)malloc((size_t)n * sizeof(double));
    double* pr = p + r * ld;
    for (int64_t s = 0; s < n; s++) pr[s] = 0.0;
    for (int h = 0; h < H; h++) {
      const float* qh = q + (r * H + h) * (int64_t)d_qk;
      double m = -INFINITY;
      for (int64_t s = 0; s < n; s++) {
        const float* c = kv + s * (int64_t)d_qk;
        double dot = 0.0;
        for (int e = 0; e < d_qk; e++) dot += (double)qh[e] * (double)c[e];
        z[s] = sm_scale * dot;
        if (z[s] > m) m = z[s];
      }
      double l = 0.0;
      for (int64_t s = 0; s < n; s++) l += exp(z[s] - m);
      for (int64_t s = 0; s < n; s++) pr[s] += exp(z[s] - m) / l;  /* A_h[t][s] */
    }
    double tot = 0.0;
    for (int64_t s = 0; s < n; s++) tot += pr[s];
    for (int64_t s = 0; s < n; s++) pr[s] /= tot;  /* L1 normalisation */
    free(z);
  }
}

/* loss [n_rows] and g [n_rows][ld] from the target p and the index scores I (both over s <= pos). */
void oracle_warmup_loss(const double* p, const float* scores, int64_t n_rows, const int64_t* pos, int64_t ld_p,
                        int64_t ld_s, double* loss, double* g, int64_t ld_g) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; r++) {
    const int64_t n = pos[r] + 1;
    const double* pr = p + r * ld_p;
    const float* ir = scores + r * ld_s;
    double m = -INFINITY;
    for (int64_t s = 0; s < n; s++)
      if ((double)ir[s] > m) m = (double)ir[s];
    double l = 0.0;
    for (int64_t s = 0; s < n; s++) l += exp((double)ir[s] - m);
    const double lse = m + log(l);
    double kl = 0.0;
    for (int64_t s = 0; s < n; s++) {
      const double logq = (double)ir[s] - lse;
      if (pr[s] > 0.0) kl += pr[s] * (log(pr[s]) - logq);
      g[r * ld_g + s] = exp(logq) - pr[s];
    }
    loss[r] = kl;
  }
}

/* Gradients of L through I[t][s] = sum_j w[t][j] * ReLU(q[t][j] . k[s]) (s <= pos_t), given g = dL/dI:
 *   dw[t][j]    = sum_s g[t][s] * ReLU(q[t][j] . k[s])
 *   dq[t][j][:] = sum_s g[t][s] * w[t][j] * [q[t][j] . k[s] > 0] * k[s][:]
 *   dk[s][:]    = sum_t sum_j g[t][s] * w[t][j] * [q[t][j] . k[s] > 0] * q[t][j][:]
 * q [n_rows][H][d], k [n_kv][d] dequantised fp32 (the gradient is with respect to these values); all sums
 * in double.  The dot products decide the indicator in double.
 */
void oracle_warmup_backward(const float* q, const float* w, const float* k, const double* g, int64_t n_rows,
                            const int64_t* pos, int H, int d, int64_t n_kv, int64_t ld_g, double* dq, double* dw,
                            double* dk) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; r++) {
    for (int j = 0; j < H; j++) {
      const float* qj = q + (r * H + j) * (int64_t)d;
      double* dqj = dq + (r * H + j) * (int64_t)d;
      for (int i = 0; i < d; i++) dqj[i] = 0.0;
      double dwj = 0.0;
      for (int64_t s = 0; s <= pos[r]; s++) {
        const float* ks = k + s * (int64_t)d;
        double dot = 0.0;
        for (int i = 0; i < d; i++) dot += (double)qj[i] * (double)ks[i];
        if (dot > 0.0) {
          const double gs = g[r * ld_g + s];
          dwj += gs * dot;
          for (int i = 0; i < d; i++) dqj[i] += gs * (double)w[r * H + j] * (double)ks[i];
        }
      }
      dw[r * H + j] = dwj;
    }
  }
  /* dk: one key at a time, summing over every (query, head) that sees it */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t s = 0; s < n_kv; s++) {
    double* dks = dk + s * (int64_t)d;
    const float* ks = k + s * (int64_t)d;
    for (int i = 0; i < d; i++) dks[i] = 0.0;
    for (int64_t r = 0; r < n_rows; r++) {
      if (s > pos[r]) continue;
      const double gs = g[r * ld_g + s];
      for (int j = 0; j < H; j++) {
        const float* qj = q + (r * H + j) * (int64_t)d;
        double dot = 0.0;
        for (int i = 0; i < d; i++) dot += (double)qj[i] * (double)ks[i];
        if (dot > 0.0) {
          const double c = gs * (double)w[r * H + j];
          for (int i = 0; i < d; i++) dks[i] += c * (double)qj[i];
        }
      }
    }
  }
}


/* ---------------------------------------------------------------- sparse training backward
 * Sparse training stage (velog summary, Continued Pre-Training, Stage 2): the whole main model trains
 * through the top-k selection, so its gradient passes through the attention of oracle_sparse_attn only.
 * Given dout = dL/dout for every (row, head), the chain rule through the softmax over the selected
 * entries i (s_i = idx[r][i] != -1):
 *   z_i   = sm_scale q . kv[s_i],   P_i = exp(z_i) / sum_j exp(z_j)
 *   dP_i  = dout . kv[s_i][0:d_v]
 *   dz_i  = P_i (dP_i - sum_j P_j dP_j)                      (softmax Jacobian)
 *   dq    = sm_scale sum_i dz_i kv[s_i]
 *   dkv[s_i][0:d_qk] += sm_scale dz_i q,   dkv[s_i][0:d_v] += P_i dout    (K and V share the row)
 * The same stage trains the indexer alone, on its own loss; its target for row r is the head mean of
 * the attention probabilities, pbar[r][i] = (1/H) sum_h P_i (0 for skipped entries).
 * q [n_rows][H][d_qk], kv [n_kv][d_qk], idx [n_rows][k], dout [n_rows][H][d_v]; dq [n_rows][H][d_qk],
 * dkv [n_kv][d_qk] (overwritten), pbar [n_rows][k]; all in double.  OpenMP threads each sum their rows'
 * dkv terms apart and the partial sums are added at the end (only the order of the double sums differs).
 */
void oracle_sparse_attn_backward(const float* q, const float* kv, const int32_t* idx, int64_t n_rows, int H,
                                 int d_qk, int d_v, int k, double sm_scale, const float* dout, int64_t n_kv,
                                 double* dq, double* dkv, double* pbar) {
  for (int64_t e = 0; e < n_kv * (int64_t)d_qk; e++) dkv[e] = 0.0;
  for (int64_t e = 0; e < n_rows * (int64_t)k; e++) pbar[e] = 0.0;
#pragma omp parallel
  {
    double* part = (double*)calloc((size_t)(n_kv * (int64_t)d_qk), sizeof(double));
    double* z = (double*)malloc((size_t)k * sizeof(double));
    double* dp = (double*)malloc((size_t)k * sizeof(double));
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < n_rows; r++) {
      for (int h = 0; h < H; h++) {
        const float* qh = q + (r * H + h) * (int64_t)d_qk;
        const float* doh = dout + (r * H + h) * (int64_t)d_v;
        const int32_t* sel = idx + r * (int64_t)k;
        double* dqh = dq + (r * H + h) * (int64_t)d_qk;
        for (int e = 0; e < d_qk; e++) dqh[e] = 0.0;
        double m = -INFINITY;
        for (int i = 0; i < k; i++) {
          if (sel[i] < 0) continue;
          const float* c = kv + (int64_t)sel[i] * d_qk;
          double dot = 0.0, dv = 0.0;
          for (int e = 0; e < d_qk; e++) dot += (double)qh[e] * (double)c[e];
          for (int e = 0; e < d_v; e++) dv += (double)doh[e] * (double)c[e];
          z[i] = sm_scale * dot;
          dp[i] = dv;
          if (z[i] > m) m = z[i];
        }
        if (m == -INFINITY) continue;  /* nothing selected: no gradient */
        double l = 0.0;
        for (int i = 0; i < k; i++)
          if (sel[i] >= 0) l += exp(z[i] - m);
        double pdp = 0.0;  /* sum_j P_j dP_j */
        for (int i = 0; i < k; i++)
          if (sel[i] >= 0) pdp += exp(z[i] - m) / l * dp[i];
        for (int i = 0; i < k; i++) {
          if (sel[i] < 0) continue;
          const double p = exp(z[i] - m) / l;
          const double dz = p * (dp[i] - pdp);
          const float* c = kv + (int64_t)sel[i] * d_qk;
          double* acc = part + (int64_t)sel[i] * d_qk;
          for (int e = 0; e < d_qk; e++) {
            dqh[e] += sm_scale * dz * (double)c[e];
            acc[e] += sm_scale * dz * (double)qh[e];
          }
          for (int e = 0; e < d_v; e++) acc[e] += p * (double)doh[e];
#pragma omp atomic
          pbar[r * k + i] += p / H;
        }
      }
    }
#pragma omp critical
    for (int64_t e = 0; e < n_kv * (int64_t)d_qk; e++) dkv[e] += part[e];
    free(part);
    free(z);
    free(dp);
  }
}
