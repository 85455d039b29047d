/*
 * rola_oracle.c -- plain, slow CPU definition of RoLA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or table with the HIP library.
 *
 * What is computed (pages: "SparkDiffusion: 265x Faster Video Generation on
 * Consumer GPUs via Sparse Attention & Distillation", section "RoLA:
 * Preserving Global Context at Extreme Sparsity"; "SparkDiffusion/SparkWan"
 * news article, section "What's New"):  RoLA attention keeps the high-energy
 * query-key blocks in a block-sparse softmax branch, and adds a low-rank
 * linear-attention branch with rotary positions that restores the global
 * context the sparse branch drops.  The output is the sum of both branches.
 * The keep ratio ``topk`` (README "AlibabaResearch/SparkDiffusion",
 * inference section) is the fraction of key blocks each query block keeps.
 *
 * Readings taken where the pages are silent:
 *  - 64-token blocks in raster (t,h,w) order; block energy is the mean of the
 *    block's valid tokens (the tail block's padding is excluded);
 *  - pooling sums in a fixed binary tree (pairs at distance 32,16,...,1) in
 *    fp32, then multiplies by fp32(1/count); scores are a sequential fp32 fma
 *    chain over d = 0..D-1 from +0.0, with no 1/sqrt(D) and no softmax (both
 *    are monotone per row and would only add roundings);
 *  - per query block, the kb = max(1, floor(topk*nb)) key blocks with the
 *    largest score are kept, ties going to the lower block index; the map is
 *    stored in ascending block order;
 *  - sparse branch: softmax(q k^T * scale) v over the tokens of the kept key
 *    blocks that lie below N, scale = D^-1/2;
 *  - 3-D rotary embedding on the head_dim vector before the low-rank
 *    projection: dims split (d_t, d_h, d_w) over the axes, pairs interleaved
 *    (x[o+2p], x[o+2p+1]) rotated by pos * theta^(-2p/d_axis);
 *  - features phi(x) = elu(x) + 1; the linear branch is normalised,
 *    O_lr = (a^T S)/(a^T z), S = sum_n b_n v_n^T, z = sum_n b_n over all N
 *    valid keys; one state per (batch, head) (the global scope; the
 *    complement scope, where each query block's state covers only the key
 *    blocks it does not keep, is the alternative reading, selected per call);
 *  - output = sparse + low-rank for rows < N, zero for padded rows;
 *  - optional learned output gate on the low-rank term (README
 *    "AlibabaResearch/SparkDiffusion", sparse-finetune section, names the
 *    trainable gate_proj and gate_bias without giving their form): read here
 *    as g = sigmoid(q . w + b) per token and head, from the raw (unrotated)
 *    query, with one gate vector [w_0 .. w_{D-1}, b] shared by all heads like
 *    the two projections; the output is then sparse + g * low-rank;
 *  - fp8 mode: per (batch, head, 64-token block) absmax scale, codes are
 *    OCP e4m3 (max 448) rounded to nearest even from x * fl32(448/absmax),
 *    values dequantise as code * fl32(absmax/448).
 *
 * Arrays are contiguous: tokens [BH, n_pad, D] (BH = batch*heads), bf16 held
 * as uint16 bit patterns; pooled [BH, nb, D]; scores [BH, nb, nb]; map
 * [BH, nb, kb] int32; projections [D, r] fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define RO_BLOCK 64

int ro_version(void) { return 1; }

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Token index -> (t, h, w) for a raster-ordered T x Hg x W grid. */
void ro_position(int64_t n, int grid_h, int grid_w, int32_t *pos3) {
  pos3[0] = (int32_t)(n / ((int64_t)grid_h * grid_w));
  pos3[1] = (int32_t)((n / grid_w) % grid_h);
  pos3[2] = (int32_t)(n % grid_w);
}

/* ---------------------------------------------------------------- pooling */
/* out[bh][c][d] = (pinned fp32 tree sum of the block's valid tokens) * fl32(1/count). */
void ro_pool(const uint16_t *x, int64_t bh_count, int64_t n_pad, int64_t n_valid, int d_model,
             float *out) {
  const int64_t nb = n_pad / RO_BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    for (int64_t c = 0; c < nb; ++c) {
      int64_t count = n_valid - c * RO_BLOCK;
      if (count > RO_BLOCK) count = RO_BLOCK;
      if (count < 0) count = 0;
      const float inv = count > 0 ? 1.0f / (float)count : 0.0f;
      for (int d = 0; d < d_model; ++d) {
        float v[RO_BLOCK];
        for (int s = 0; s < RO_BLOCK; ++s) {
          const int64_t n = c * RO_BLOCK + s;
          v[s] = n < n_valid ? bf16_to_f32(x[(bh * n_pad + n) * d_model + d]) : 0.0f;
        }
        for (int stride = RO_BLOCK / 2; stride >= 1; stride /= 2)
          for (int i = 0; i < stride; ++i) v[i] = v[i] + v[i + stride];
        out[(bh * nb + c) * d_model + d] = v[0] * inv;
      }
    }
  }
}

/* ----------------------------------------------------------------- scores */
/* s[bh][i][j] = fma chain over d of qp[i][d] * kp[j][d], starting at +0.0. */
void ro_scores(const float *qp, const float *kp, int64_t bh_count, int nb, int d_model, float *s) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    for (int i = 0; i < nb; ++i) {
      const float *qi = qp + (bh * nb + i) * d_model;
      for (int j = 0; j < nb; ++j) {
        const float *kj = kp + (bh * nb + j) * d_model;
        float acc = 0.0f;
        for (int d = 0; d < d_model; ++d) acc = fmaf(qi[d], kj[d], acc);
        s[(bh * nb + i) * (int64_t)nb + j] = acc;
      }
    }
  }
}

/* -------------------------------------------------------------- selection */
/*
 * Key blocks kept per query block for the keep ratio topk (README
 * "AlibabaResearch/SparkDiffusion", inference section: 0.1, 0.05 and 0.03
 * keep 10%, 5% and 3% of the blocks): floor(topk * nb), at least 1 and at
 * most nb.  topk arrives as a float32, so a decimal ratio is off by up to
 * 2^-24 of itself; the product is taken with a relative allowance of 2^-22
 * so that, e.g., 0.7 of 4000 blocks keeps 2800, as the decimal ratio does.
 */
int ro_keep_blocks(float topk, int nb) {
  const double prod = (double)topk * (double)nb;
  double k = floor(prod + prod * ldexp(1.0, -22));
  if (k < 1.0) k = 1.0;
  if (k > (double)nb) k = (double)nb;
  return (int)k;
}

typedef struct {
  float s;
  int32_t j;
} ro_cand;

/* Order: larger score first; equal scores (including -0.0 == +0.0) by lower index. */
static int cand_cmp(const void *a, const void *b) {
  const ro_cand *x = (const ro_cand *)a, *y = (const ro_cand *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int int_cmp(const void *a, const void *b) {
  const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* s [BH, nq, nb] -> map [BH, nq, kb] (nq = nb for a full score matrix). */
void ro_select(const float *s, int64_t bh_count, int nq, int nb, int kb, int32_t *map) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    ro_cand *row = (ro_cand *)malloc(sizeof(ro_cand) * (size_t)nb);
    for (int i = 0; i < nq; ++i) {
      const float *si = s + (bh * nq + i) * (int64_t)nb;
      for (int j = 0; j < nb; ++j) {
        row[j].s = si[j];
        row[j].j = j;
      }
      qsort(row, (size_t)nb, sizeof(ro_cand), cand_cmp);
      int32_t *mi = map + (bh * nq + i) * (int64_t)kb;
      for (int t = 0; t < kb; ++t) mi[t] = row[t].j;
      qsort(mi, (size_t)kb, sizeof(int32_t), int_cmp);
    }
    free(row);
  }
}

/* ---------------------------------------------------------- sparse branch */
/* One query row: softmax over the valid tokens of the kept key blocks. */
static void sparse_row(const double *q, const double *k, const double *v, const int32_t *blocks,
                       int kb, int64_t n_valid, int d_model, double scale, double *out,
                       double *buf) {
  int64_t cnt = 0;
  double m = -INFINITY;
  for (int t = 0; t < kb; ++t) {
    for (int s = 0; s < RO_BLOCK; ++s) {
      const int64_t n = (int64_t)blocks[t] * RO_BLOCK + s;
      if (n >= n_valid) continue;
      double dot = 0.0;
      for (int d = 0; d < d_model; ++d) dot += q[d] * k[n * d_model + d];
      dot *= scale;
      buf[cnt++] = dot;
      if (dot > m) m = dot;
    }
  }
  for (int d = 0; d < d_model; ++d) out[d] = 0.0;
  double l = 0.0;
  cnt = 0;
  for (int t = 0; t < kb; ++t) {
    for (int s = 0; s < RO_BLOCK; ++s) {
      const int64_t n = (int64_t)blocks[t] * RO_BLOCK + s;
      if (n >= n_valid) continue;
      const double p = exp(buf[cnt++] - m);
      l += p;
      for (int d = 0; d < d_model; ++d) out[d] += p * v[n * d_model + d];
    }
  }
  for (int d = 0; d < d_model; ++d) out[d] /= l;
}

/*
 * Sparse branch on selected rows.  q, k, v: fp64 [BH, n_pad, D]; rows[r] =
 * bh * n_pad + n with n < n_valid; out: [nrows, D].
 */
void ro_sparse_rows(const double *q, const double *k, const double *v, const int32_t *map,
                    int64_t n_pad, int64_t n_valid, int d_model, int kb, double scale,
                    int64_t nrows, const int64_t *rows, double *out) {
  const int64_t nb = n_pad / RO_BLOCK;
#pragma omp parallel
  {
    double *buf = (double *)malloc(sizeof(double) * (size_t)kb * RO_BLOCK);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t bh = rows[r] / n_pad, n = rows[r] % n_pad;
      const int64_t base = bh * n_pad * d_model;
      sparse_row(q + rows[r] * d_model, k + base, v + base, map + (bh * nb + n / RO_BLOCK) * kb, kb,
                 n_valid, d_model, scale, out + r * d_model, buf);
    }
    free(buf);
  }
}

/* ----------------------------------------------------------- 3-D rotary */
/*
 * y = R(t,h,w) x.  Axis a owns dims [o_a, o_a + d_a) with o = (0, d_t, d_t+d_h);
 * pair p of axis a, (x[o_a+2p], x[o_a+2p+1]), turns by pos_a * theta^(-2p/d_a).
 */
void ro_rope3d(const double *x, const int32_t *pos3, const int32_t *split, double theta,
               int d_model, double *y) {
  int off = 0;
  for (int d = 0; d < d_model; ++d) y[d] = x[d];
  for (int a = 0; a < 3; ++a) {
    const int da = split[a];
    for (int p = 0; p < da / 2; ++p) {
      const double ang = (double)pos3[a] * pow(theta, -2.0 * p / (double)da);
      const double c = cos(ang), s = sin(ang);
      const double x0 = x[off + 2 * p], x1 = x[off + 2 * p + 1];
      y[off + 2 * p] = x0 * c - x1 * s;
      y[off + 2 * p + 1] = x0 * s + x1 * c;
    }
    off += da;
  }
}

/* feature map phi(u) = elu(u) + 1 */
static double phi(double u) { return u > 0.0 ? u + 1.0 : exp(u); }

/* f[r] = phi(sum_d RoPE(x)[d] * w[d][r]) for token n of the grid. */
static void lowrank_feature(const double *x, int64_t n, const int32_t *grid, const int32_t *split,
                            double theta, const float *w, int d_model, int rank, double *rot,
                            double *f) {
  int32_t pos3[3];
  ro_position(n, grid[1], grid[2], pos3);
  ro_rope3d(x, pos3, split, theta, d_model, rot);
  for (int r = 0; r < rank; ++r) {
    double u = 0.0;
    for (int d = 0; d < d_model; ++d) u += rot[d] * (double)w[d * rank + r];
    f[r] = phi(u);
  }
}

/* Public for tests: the feature vector of one token. */
void ro_lowrank_feature(const double *x, int64_t n, const int32_t *grid, const int32_t *split,
                        double theta, const float *w, int d_model, int rank, double *f) {
  double rot[512];
  lowrank_feature(x, n, grid, split, theta, w, d_model, rank, rot, f);
}

/* S[bh][r][d] = sum_{n<N} b_n[r] v_n[d],  z[bh][r] = sum_{n<N} b_n[r],  b_n = phi(Wk^T RoPE(k_n)). */
void ro_lowrank_state(const double *k, const double *v, const float *wk, int64_t bh_count,
                      int64_t n_pad, int64_t n_valid, int d_model, int rank, const int32_t *grid,
                      const int32_t *split, double theta, double *S, double *z) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    double rot[512], f[64];
    double *Sb = S + bh * rank * d_model, *zb = z + bh * rank;
    for (int64_t i = 0; i < (int64_t)rank * d_model; ++i) Sb[i] = 0.0;
    for (int r = 0; r < rank; ++r) zb[r] = 0.0;
    for (int64_t n = 0; n < n_valid; ++n) {
      const double *kn = k + (bh * n_pad + n) * d_model, *vn = v + (bh * n_pad + n) * d_model;
      lowrank_feature(kn, n, grid, split, theta, wk, d_model, rank, rot, f);
      for (int r = 0; r < rank; ++r) {
        zb[r] += f[r];
        for (int d = 0; d < d_model; ++d) Sb[r * d_model + d] += f[r] * vn[d];
      }
    }
  }
}

/* O_lr for selected rows: (a^T S) / (a^T z), a = phi(Wq^T RoPE(q)). */
void ro_lowrank_rows(const double *q, const float *wq, const double *S, const double *z,
                     int64_t n_pad, int d_model, int rank, const int32_t *grid,
                     const int32_t *split, double theta, int64_t nrows, const int64_t *rows,
                     double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    double rot[512], a[64];
    const int64_t bh = rows[r] / n_pad, n = rows[r] % n_pad;
    lowrank_feature(q + rows[r] * d_model, n, grid, split, theta, wq, d_model, rank, rot, a);
    const double *Sb = S + bh * rank * d_model, *zb = z + bh * rank;
    double den = 0.0;
    for (int i = 0; i < rank; ++i) den += a[i] * zb[i];
    for (int d = 0; d < d_model; ++d) {
      double num = 0.0;
      for (int i = 0; i < rank; ++i) num += a[i] * Sb[i * d_model + d];
      out[r * d_model + d] = num / den;
    }
  }
}

/*
 * Complement scope of the low-rank branch (an alternative reading of the
 * article's statement that the linear branch restores the context that
 * sparsification drops): the state a query block sees covers only the key
 * blocks it does NOT keep.  Per-block states of one (batch, head):
 * Sb[j][r][d] = sum over the valid tokens n of block j of b_n[r] v_n[d],
 * zb[j][r] = sum of b_n[r] over the same tokens.
 */
void ro_lowrank_block_states(const double *k, const double *v, const float *wk, int64_t n_pad,
                             int64_t n_valid, int d_model, int rank, const int32_t *grid,
                             const int32_t *split, double theta, double *Sb, double *zb) {
  const int64_t nb = n_pad / RO_BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nb; ++j) {
    double rot[512], f[64];
    double *S = Sb + j * rank * d_model, *z = zb + j * rank;
    for (int64_t i = 0; i < (int64_t)rank * d_model; ++i) S[i] = 0.0;
    for (int r = 0; r < rank; ++r) z[r] = 0.0;
    for (int64_t n = j * RO_BLOCK; n < (j + 1) * RO_BLOCK && n < n_valid; ++n) {
      lowrank_feature(k + n * d_model, n, grid, split, theta, wk, d_model, rank, rot, f);
      for (int r = 0; r < rank; ++r) {
        z[r] += f[r];
        for (int d = 0; d < d_model; ++d) S[r * d_model + d] += f[r] * v[n * d_model + d];
      }
    }
  }
}

/* Complement-scope low-rank rows of one (batch, head): a row of query block i
 * uses S_i = sum of Sb[j] over the blocks j not in map[i] (z_i likewise), and
 * O_lr = (a^T S_i) / (a^T z_i); when i keeps every block the branch is 0. */
void ro_lowrank_rows_complement(const double *q, const float *wq, const double *Sb,
                                const double *zb, const int32_t *map, int kb, int64_t n_pad,
                                int d_model, int rank, const int32_t *grid, const int32_t *split,
                                double theta, int64_t nrows, const int64_t *rows, double *out) {
  const int64_t nb = n_pad / RO_BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    double rot[512], a[64], z[64];
    double *S = (double *)malloc(sizeof(double) * rank * d_model);
    const int64_t n = rows[r], i = n / RO_BLOCK;
    const int32_t *kept = map + i * kb;
    for (int64_t e = 0; e < (int64_t)rank * d_model; ++e) S[e] = 0.0;
    for (int c = 0; c < rank; ++c) z[c] = 0.0;
    int64_t left = 0;
    for (int64_t j = 0; j < nb; ++j) {
      int is_kept = 0;
      for (int t = 0; t < kb; ++t) is_kept |= kept[t] == j;
      if (is_kept) continue;
      ++left;
      for (int64_t e = 0; e < (int64_t)rank * d_model; ++e) S[e] += Sb[j * rank * d_model + e];
      for (int c = 0; c < rank; ++c) z[c] += zb[j * rank + c];
    }
    double *o = out + r * d_model;
    if (left == 0) {
      for (int d = 0; d < d_model; ++d) o[d] = 0.0;
      free(S);
      continue;
    }
    lowrank_feature(q + n * d_model, n, grid, split, theta, wq, d_model, rank, rot, a);
    double den = 0.0;
    for (int c = 0; c < rank; ++c) den += a[c] * z[c];
    for (int d = 0; d < d_model; ++d) {
      double num = 0.0;
      for (int c = 0; c < rank; ++c) num += a[c] * S[c * d_model + d];
      o[d] = num / den;
    }
    free(S);
  }
}

/* Output gate of one token: sigmoid(b + sum_d q[d] w[d]), gate = [w_0 .. w_{D-1}, b]. */
double ro_gate(const double *q, const float *gate, int d_model) {
  double u = (double)gate[d_model];
  for (int d = 0; d < d_model; ++d) u += q[d] * (double)gate[d];
  return 1.0 / (1.0 + exp(-u));
}

/* --------------------------------------------------------------- fp8 e4m3 */
/* OCP e4m3 value of a code (no infinities; 0x7f/0xff are NaN). */
double ro_e4m3_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Nearest e4m3 code to y (ties to the even code), saturating at +-448. */
uint8_t ro_e4m3_encode(float y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0;
  double a = fabs((double)y);
  if (a >= 448.0) return sign | 0x7e;
  /* candidates are the non-negative codes 0..0x7e in increasing value */
  int lo = 0, hi = 0x7e;
  while (hi - lo > 1) { /* largest code with value <= a */
    const int mid = (lo + hi) / 2;
    if (ro_e4m3_value((uint8_t)mid) <= a) lo = mid; else hi = mid;
  }
  const double vlo = ro_e4m3_value((uint8_t)lo), vhi = ro_e4m3_value((uint8_t)hi);
  int pick;
  if (a - vlo < vhi - a) pick = lo;
  else if (a - vlo > vhi - a) pick = hi;
  else pick = (lo & 1) ? hi : lo;
  if (vlo == a) pick = lo;
  return sign | (uint8_t)pick;
}

/*
 * Per-(bh, block) quantisation of bf16 tokens.  codes [BH, n_pad, D];
 * scale [BH, nb] = fl32(absmax/448); deq [BH, n_pad, D] fp64 = value(code) * scale.
 * Padded rows are excluded from absmax and quantise to 0.
 */
void ro_quant_e4m3(const uint16_t *x, int64_t bh_count, int64_t n_pad, int64_t n_valid,
                   int d_model, uint8_t *codes, float *scale, double *deq) {
  const int64_t nb = n_pad / RO_BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    for (int64_t c = 0; c < nb; ++c) {
      float amax = 0.0f;
      for (int s = 0; s < RO_BLOCK; ++s) {
        const int64_t n = c * RO_BLOCK + s;
        if (n >= n_valid) break;
        for (int d = 0; d < d_model; ++d) {
          const float a = fabsf(bf16_to_f32(x[(bh * n_pad + n) * d_model + d]));
          if (a > amax) amax = a;
        }
      }
      const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
      const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      scale[bh * nb + c] = sc;
      for (int s = 0; s < RO_BLOCK; ++s) {
        const int64_t n = c * RO_BLOCK + s;
        for (int d = 0; d < d_model; ++d) {
          const int64_t idx = (bh * n_pad + n) * d_model + d;
          uint8_t code = 0;
          if (n < n_valid) code = ro_e4m3_encode(bf16_to_f32(x[idx]) * inv);
          codes[idx] = code;
          deq[idx] = ro_e4m3_value(code) * (double)sc;
        }
      }
    }
  }
}

/* ------------------------------------------- w8a8 linear layers (fp8 GEMM) */
/*
 * The projections either side of attention in the fp8 pipeline (README
 * "AlibabaResearch/SparkDiffusion", highlights: optional weight-activation
 * quantisation, w8a8; project page, section "FP8 Quantization & Fused
 * Kernels").  Reading taken: activations are quantised per token (row of
 * x [M, K]) and weights per output channel (row of W [N, K]), both with the
 * e4m3 absmax rule used for attention inputs, and the layer computes
 *   y[m, n] = sa[m] * sw[n] * sum_k value(a[m, k]) * value(w[n, k]) + bias[n].
 */

/* Per-row quantisation of a bf16 matrix x [rows, cols] with row stride ld.
 * codes [rows, cols]; scale [rows] = fl32(absmax/448) (1 for a zero row);
 * deq [rows, cols] fp64 = value(code) * scale. */
void ro_quant_rows_e4m3(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                        uint8_t *codes, float *scale, double *deq) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < rows; ++m) {
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      const float a = fabsf(bf16_to_f32(x[m * ld + c]));
      if (a > amax) amax = a;
    }
    const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    scale[m] = sc;
    for (int64_t c = 0; c < cols; ++c) {
      const uint8_t code = ro_e4m3_encode(bf16_to_f32(x[m * ld + c]) * inv);
      codes[m * cols + c] = code;
      deq[m * cols + c] = ro_e4m3_value(code) * (double)sc;
    }
  }
}

/* y [M, N] fp64 from codes a [M, K], w [N, K], scales sa [M], sw [N] and an
 * optional fp32 bias [N] (NULL: none).  Each product of two e4m3 values is
 * a multiple of 2^-18 below 2^18, so for K <= 65536 every partial sum is a
 * multiple of 2^-18 below 2^34, held exactly in fp64: the dot product is
 * exact in any order.  It is then scaled and the bias added.
 * yabs [M, N] (optional) receives sa*sw*sum_k |value*value| + |bias|, the
 * magnitude that bounds the rounding of any fp32 evaluation. */
void ro_gemm_w8a8(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                  const float *bias, int64_t M, int64_t N, int64_t K, double *y, double *yabs) {
  double *wv = (double *)malloc(sizeof(double) * (size_t)(N * K));
  for (int64_t i = 0; i < N * K; ++i) wv[i] = ro_e4m3_value(w[i]);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double *av = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t k = 0; k < K; ++k) av[k] = ro_e4m3_value(a[m * K + k]);
    for (int64_t n = 0; n < N; ++n) {
      double dot = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        dot += av[k] * wv[n * K + k];
        mag += fabs(av[k] * wv[n * K + k]);
      }
      const double s = (double)sa[m] * (double)sw[n];
      const double b = bias ? (double)bias[n] : 0.0;
      y[m * N + n] = s * dot + b;
      if (yabs) yabs[m * N + n] = s * mag + fabs(b);
    }
    free(av);
  }
  free(wv);
}

/* ------------------------------------------------------------ full forward */
static void widen(const uint16_t *x, int64_t count, double *y) {
  for (int64_t i = 0; i < count; ++i) y[i] = (double)bf16_to_f32(x[i]);
}

/*
 * The whole RoLA forward for `bh_count` (batch, head) slices of bf16 tokens.
 * map_out [BH, nb, kb]; out [BH, n_pad, D] fp64.  Threads run over slices.
 * fp8 != 0 runs the sparse branch on the e4m3-dequantised Q, K, V; selection
 * and the low-rank branch always use the bf16 values.  gate (fp32 [D+1], may
 * be NULL for no gate) scales the low-rank term by ro_gate of the bf16 query.
 * complement != 0 takes the low-rank state over the unkept blocks of each
 * query block (ro_lowrank_rows_complement) instead of all blocks.
 */
void ro_forward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *wq,
                const float *wk, const float *gate, int64_t bh_count, int64_t n_pad,
                int64_t n_valid, int d_model, int rank, int kb, const int32_t *grid,
                const int32_t *split, double theta, double scale, int fp8, int complement,
                int32_t *map_out, double *out) {
  const int64_t nb = n_pad / RO_BLOCK;
  const int64_t per = n_pad * d_model;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    float *qp = (float *)malloc(sizeof(float) * nb * d_model);
    float *kp = (float *)malloc(sizeof(float) * nb * d_model);
    float *sc = (float *)malloc(sizeof(float) * nb * nb);
    double *qd = (double *)malloc(sizeof(double) * per);
    double *kd = (double *)malloc(sizeof(double) * per);
    double *vd = (double *)malloc(sizeof(double) * per);
    double *S = (double *)malloc(sizeof(double) * rank * d_model);
    double *z = (double *)malloc(sizeof(double) * rank);
    double *lr = (double *)malloc(sizeof(double) * d_model);
    double *buf = (double *)malloc(sizeof(double) * kb * RO_BLOCK);
    int32_t *map = map_out + bh * nb * kb;
    const uint16_t *qb = q + bh * per, *kbf = k + bh * per, *vb = v + bh * per;

    ro_pool(qb, 1, n_pad, n_valid, d_model, qp);
    ro_pool(kbf, 1, n_pad, n_valid, d_model, kp);
    ro_scores(qp, kp, 1, (int)nb, d_model, sc);
    ro_select(sc, 1, (int)nb, (int)nb, kb, map);

    widen(qb, per, qd);
    widen(kbf, per, kd);
    widen(vb, per, vd);
    ro_lowrank_state(kd, vd, wk, 1, n_pad, n_valid, d_model, rank, grid, split, theta, S, z);
    double *Sb = NULL, *zb = NULL;
    if (complement) {
      Sb = (double *)malloc(sizeof(double) * nb * rank * d_model);
      zb = (double *)malloc(sizeof(double) * nb * rank);
      ro_lowrank_block_states(kd, vd, wk, n_pad, n_valid, d_model, rank, grid, split, theta, Sb, zb);
    }

    double *qs = qd, *ks = kd, *vs = vd;
    uint8_t *codes = NULL;
    float *scl = NULL;
    if (fp8) {
      codes = (uint8_t *)malloc((size_t)per);
      scl = (float *)malloc(sizeof(float) * nb);
      qs = (double *)malloc(sizeof(double) * per);
      ks = (double *)malloc(sizeof(double) * per);
      vs = (double *)malloc(sizeof(double) * per);
      ro_quant_e4m3(qb, 1, n_pad, n_valid, d_model, codes, scl, qs);
      ro_quant_e4m3(kbf, 1, n_pad, n_valid, d_model, codes, scl, ks);
      ro_quant_e4m3(vb, 1, n_pad, n_valid, d_model, codes, scl, vs);
    }
    double *ob = out + bh * per;
    for (int64_t n = 0; n < n_pad; ++n) {
      double *on = ob + n * d_model;
      if (n >= n_valid) {
        for (int d = 0; d < d_model; ++d) on[d] = 0.0;
        continue;
      }
      sparse_row(qs + n * d_model, ks, vs, map + (n / RO_BLOCK) * kb, kb, n_valid, d_model, scale,
                 on, buf);
      const int64_t row = n; /* rows are relative to this slice */
      if (complement)
        ro_lowrank_rows_complement(qd, wq, Sb, zb, map, kb, n_pad, d_model, rank, grid, split,
                                   theta, 1, &row, lr);
      else
        ro_lowrank_rows(qd, wq, S, z, n_pad, d_model, rank, grid, split, theta, 1, &row, lr);
      const double g = gate ? ro_gate(qd + n * d_model, gate, d_model) : 1.0;
      for (int d = 0; d < d_model; ++d) on[d] += g * lr[d];
    }
    if (fp8) {
      free(codes); free(scl); free(qs); free(ks); free(vs);
    }
    free(qp); free(kp); free(sc); free(qd); free(kd); free(vd);
    free(S); free(z); free(lr); free(buf); free(Sb); free(zb);
  }
}
