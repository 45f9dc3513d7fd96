/*
 * oracle.c — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU implementation of what the
 * library computes: 3-D rotary position embedding on the video tokens of Q/K,
 * the RMS QK-norm that precedes it, the joint concat + sequence->head
 * re-layout, full non-causal softmax
 * attention, a separately written chunked form with a log-sum-exp merge, and
 * the n-way log-sum-exp merge of partial attention outputs.
 *
 * Only the tests, the package smoke check and the benchmark's CPU-baseline
 * leg may load this file's library.  It shares no code, header, table or
 * helper with the HIP path, and the HIP path never calls it.
 *
 * Sources of the operations (the pages only name them; the readings taken
 * where they are silent are listed per function):
 *  - "Context Parallelism in vLLM Omni Neuron", §Self-Attention with Context
 *    Parallelism: Q/K are rotated by apply_rotary_emb_wan before the
 *    transpose to [B,N,S,D]; V is not rotated; _nf_attend(q,k,v,scale) is full
 *    attention (§Overview: "maintaining full attention computation").
 *  - same page, §Ring attention / §Memory and Compute Benefits: K/V chunks are
 *    visited one at a time and partial results are combined so that the full
 *    attention result is kept.
 *  - xDiT PR "Adds support for KV-cache and joint tensors to USP method":
 *    joint (text) tensors are concatenated to the sharded sequence inside
 *    attention; the Ulysses input all-to-all moves Q/K/V from sequence- to
 *    head-partitioned layout.
 *  - Problem statement of the benchmark workloads: RoPE theta 10000, the D
 *    split over (t,h,w), scale, kv_chunk.
 *
 * Numerics: every floating-point step is IEEE double with the default
 * round-to-nearest mode.  Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Rounding to the storage formats.                                          */
/* ------------------------------------------------------------------------ */

/*
 * Round a double to the nearest bfloat16 value, ties to even, returned as a
 * double.  bfloat16 = 1 sign bit, 8 exponent bits (bias 127, like binary32),
 * 7 stored fraction bits.  Normal numbers carry 8 significant bits, so the
 * spacing of representable values in [2^e, 2^(e+1)) is 2^(e-7); below 2^-126
 * the spacing stays 2^-133 (subnormals).  Values whose rounded magnitude
 * exceeds the largest finite bfloat16, (2 - 2^-7) * 2^127, become infinities.
 * rint() rounds to nearest-even in the default rounding mode and x/q, y*q
 * are exact (powers of two), so the result is the correctly rounded value.
 */
double oracle_round_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  frexp(fabs(x), &e);           /* |x| = f * 2^e, f in [0.5, 1) => exponent e-1 */
  int exp2_floor = e - 1;
  if (exp2_floor < -126) exp2_floor = -126;
  double q = ldexp(1.0, exp2_floor - 7);
  double y = rint(x / q) * q;
  const double max_bf16 = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 = 255 * 2^120 */
  if (fabs(y) > max_bf16) y = copysign(INFINITY, x);
  return y;
}

void oracle_round_bf16_array(const double* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_bf16(x[i]);
}

/* Round to binary32 (the C conversion rounds to nearest-even). */
void oracle_round_f32_array(const double* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = (double)(float)x[i];
}

/* ------------------------------------------------------------------------ */
/* 3-D rotary position embedding.                                            */
/* ------------------------------------------------------------------------ */

/*
 * Rotate one head vector x[0..D) of a token at grid position (pt, ph, pw).
 *
 * Reading (the pages name apply_rotary_emb_wan(query, freqs_cos, freqs_sin)
 * and say the rotary tables are indexed by sequence position, "Context
 * Parallelism in vLLM Omni Neuron", §WanTransformer3DModel and §Positional
 * Embedding Handling, but never give the formula):
 *  - D is split into three contiguous segments [d_t | d_h | d_w], one per
 *    grid axis, in that order; each is an independent 1-D rotary embedding.
 *  - Inside the segment of axis a (length d_a, offset off_a), element pair
 *    (off_a + 2j, off_a + 2j + 1), j = 0 .. d_a/2 - 1, is rotated
 *    counter-clockwise by the angle  p_a * theta^(-2j / d_a):
 *        (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
 *  - Positions are 0-based integers; d_a = 0 leaves that axis out.
 */
void oracle_rope_vec(const double* x, double* y, int64_t D, int64_t pt, int64_t ph,
                     int64_t pw, int d_t, int d_h, int d_w, double theta) {
  const int seg_len[3] = {d_t, d_h, d_w};
  const int64_t pos[3] = {pt, ph, pw};
  int off = 0;
  for (int64_t i = 0; i < D; ++i) y[i] = x[i];
  for (int a = 0; a < 3; ++a) {
    const int da = seg_len[a];
    for (int j = 0; j < da / 2; ++j) {
      const double omega = pow(theta, -2.0 * (double)j / (double)da);
      const double phi = (double)pos[a] * omega;
      const double c = cos(phi), s = sin(phi);
      const double x0 = x[off + 2 * j], x1 = x[off + 2 * j + 1];
      y[off + 2 * j] = x0 * c - x1 * s;
      y[off + 2 * j + 1] = x0 * s + x1 * c;
    }
    off += da;
  }
}

/*
 * x, y: [B, Nv, H, D] (video tokens only).  Token n sits at grid position
 * (t, h, w) with n = (t * grid_h + h) * grid_w + w, the row-major flattening
 * of the latent grid latent_frames x post_patch_h x post_patch_w ("Context
 * Parallelism in vLLM Omni Neuron", §Sequence Length Constraints / §Problem).
 * Returns -1 if Nv != grid_t*grid_h*grid_w or d_t+d_h+d_w != D or any d odd.
 */
int oracle_rope3d(const double* x, double* y, int64_t B, int64_t Nv, int64_t H, int64_t D,
                  int64_t grid_t, int64_t grid_h, int64_t grid_w, int d_t, int d_h, int d_w,
                  double theta) {
  if (grid_t * grid_h * grid_w != Nv) return -1;
  if ((int64_t)d_t + d_h + d_w != D || (d_t | d_h | d_w) & 1) return -1;
  int64_t rows = B * Nv;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t n = r % Nv;
    const int64_t t = n / (grid_h * grid_w);
    const int64_t h = (n / grid_w) % grid_h;
    const int64_t w = n % grid_w;
    for (int64_t hd = 0; hd < H; ++hd) {
      const int64_t o = (r * H + hd) * D;
      oracle_rope_vec(x + o, y + o, D, t, h, w, d_t, d_h, d_w, theta);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* QK-norm: RMS normalisation of a token's whole hidden vector.              */
/* ------------------------------------------------------------------------ */

/*
 * x, y: [rows, n], n = H*D: a token's projected q (or k) before it is split
 * into heads; w: [n].
 *     y[r, i] = x[r, i] / sqrt(mean_j x[r, j]^2 + eps) * w[i].
 * "Context Parallelism in vLLM Omni Neuron", §Self-Attention with Context
 * Parallelism: norm_q / norm_k act on the projected q, k of shape [B, S, H]
 * (hidden size H = heads x head_dim) before .unflatten(2, (num_heads,
 * head_dim)) and before the rotary embedding; §Distributed Normalization:
 * the norm's statistic is a sum of squares over the hidden dimension.
 * Reading (the pages print neither the formula nor eps): root-mean-square
 * normalisation with a learned per-channel weight, the mean square taken
 * over the whole hidden vector, eps added to the mean square.
 * Returns -1 if n <= 0 or eps < 0.
 */
int oracle_rms_norm(const double* x, double* y, int64_t rows, int64_t n, const double* w,
                    double eps) {
  if (n <= 0 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* xr = x + r * n;
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += xr[i] * xr[i];
    const double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) y[r * n + i] = xr[i] * inv * w[i];
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Joint concat + sequence->head re-layout.                                  */
/* ------------------------------------------------------------------------ */

/*
 * segs[i]: [B, S_i, H, D] elements of elt_bytes bytes each (any type: this is
 * a byte copy).  out: [B, H, S, D] with S = sum S_i, segments placed in the
 * given order (video, audio, text).  out[b,h,s,:] = segs[i][b, s - off_i, h, :]
 * where off_i = S_0 + ... + S_(i-1).  This is the single-device form of the
 * Ulysses input all-to-all followed by .transpose(1, 2) ("Context
 * Parallelism in vLLM Omni Neuron", §Self-Attention with Context
 * Parallelism; xDiT PR #586, joint tensors).
 */
int oracle_joint_concat_permute(const void* const* segs, const int64_t* seg_len, int n_segs,
                                void* out, int64_t elt_bytes, int64_t B, int64_t H, int64_t D) {
  int64_t S = 0;
  for (int i = 0; i < n_segs; ++i) {
    if (seg_len[i] < 0) return -1;
    S += seg_len[i];
  }
  const int64_t row = D * elt_bytes;
  unsigned char* o = (unsigned char*)out;
  int64_t off = 0;
  for (int i = 0; i < n_segs; ++i) {
    const unsigned char* src = (const unsigned char*)segs[i];
    const int64_t Si = seg_len[i];
    for (int64_t b = 0; b < B; ++b)
      for (int64_t s = 0; s < Si; ++s)
        for (int64_t h = 0; h < H; ++h)
          memcpy(o + (((b * H + h) * S) + off + s) * row, src + ((b * Si + s) * H + h) * row,
                 (size_t)row);
    off += Si;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention.                                                                */
/* ------------------------------------------------------------------------ */

/*
 * One query row against all keys, the plain two-pass definition of softmax
 * attention ("Context Parallelism in vLLM Omni Neuron", §Self-Attention:
 * _nf_attend(query, key, value, scale); non-causal, no dropout):
 *   s_j = scale * <q, k_j>;  m = max_j s_j;  l = sum_j exp(s_j - m);
 *   out = sum_j exp(s_j - m) v_j / l;  lse = m + ln l  (natural log).
 * k, v point at the [Skv, D] slab of this (b, h); s is Skv doubles of scratch.
 */
static void attend_row(const double* q, const double* k, const double* v, int64_t Skv,
                       int64_t D, double scale, double* s, double* out, double* lse) {
  double m = -INFINITY;
  for (int64_t j = 0; j < Skv; ++j) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * k[j * D + d];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t j = 0; j < Skv; ++j) {
    const double p = exp(s[j] - m);
    l += p;
    for (int64_t d = 0; d < D; ++d) out[d] += p * v[j * D + d];
  }
  for (int64_t d = 0; d < D; ++d) out[d] /= l;
  *lse = m + log(l);
}

/*
 * q: [B,H,Sq,D], k, v: [B,H,Skv,D], out: [B,H,Sq,D], lse: [B,H,Sq] (may be
 * NULL).  Full attention over all Skv keys for every query row.
 */
int oracle_attention(const double* q, const double* k, const double* v, double* out,
                     double* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                     double scale) {
  if (Skv <= 0) return -1;
  const int64_t rows = B * H * Sq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t bh = r / Sq;
      double l_r;
      attend_row(q + r * D, k + bh * Skv * D, v + bh * Skv * D, Skv, D, scale, s, out + r * D,
                 &l_r);
      if (lse) lse[r] = l_r;
    }
    free(s);
  }
  return 0;
}

/*
 * The same definition evaluated only for the listed rows.  rows[i] is the
 * flat index (b*H + h)*Sq + i_q of a query row; out_rows: [n_rows, D],
 * lse_rows: [n_rows].  Each output row depends only on its own query row, so
 * this equals the corresponding rows of oracle_attention.
 */
int oracle_attention_rows(const double* q, const double* k, const double* v,
                          const int64_t* rows, int64_t n_rows, double* out_rows,
                          double* lse_rows, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                          int64_t D, double scale) {
  if (Skv <= 0) return -1;
  for (int64_t i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= B * H * Sq) return -1;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      const int64_t r = rows[i];
      const int64_t bh = r / Sq;
      attend_row(q + r * D, k + bh * Skv * D, v + bh * Skv * D, Skv, D, scale, s,
                 out_rows + i * D, &lse_rows[i]);
    }
    free(s);
  }
  return 0;
}

/*
 * Chunked form, written separately from the above.  Keys are visited in
 * chunks [c*kv_chunk, min((c+1)*kv_chunk, Skv)) (kv_chunk <= 0 or >= Skv:
 * one chunk).  Each chunk gets its own two-pass softmax (O_c, lse_c); the
 * running result (O, L), started at (0, -inf), is merged with it by
 *   L' = ln(e^L + e^lse_c),  O <- O e^(L - L') + O_c e^(lse_c - L'),  L <- L'.
 * This is the combine step that lets ring attention visit one K/V shard per
 * round and still produce full attention ("Context Parallelism in vLLM Omni
 * Neuron", §Ring attention, §Memory and Compute Benefits).
 */
int oracle_attention_chunked(const double* q, const double* k, const double* v, double* out,
                             double* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                             int64_t D, double scale, int64_t kv_chunk) {
  if (Skv <= 0) return -1;
  if (kv_chunk <= 0 || kv_chunk > Skv) kv_chunk = Skv;
  const int64_t rows = B * H * Sq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)kv_chunk);
    double* oc = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t bh = r / Sq;
      const double* kb = k + bh * Skv * D;
      const double* vb = v + bh * Skv * D;
      double* o = out + r * D;
      double L = -INFINITY;
      for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
      for (int64_t c0 = 0; c0 < Skv; c0 += kv_chunk) {
        const int64_t n = (Skv - c0 < kv_chunk) ? (Skv - c0) : kv_chunk;
        double lse_c;
        attend_row(q + r * D, kb + c0 * D, vb + c0 * D, n, D, scale, s, oc, &lse_c);
        const double hi = (L > lse_c) ? L : lse_c;
        const double Lnew = hi + log(exp(L - hi) + exp(lse_c - hi));
        const double wa = exp(L - Lnew), wb = exp(lse_c - Lnew);
        for (int64_t d = 0; d < D; ++d) o[d] = o[d] * wa + oc[d] * wb;
        L = Lnew;
      }
      if (lse) lse[r] = L;
    }
    free(oc);
    free(s);
  }
  return 0;
}

/*
 * n-way log-sum-exp merge of partial attention results (the ring combine,
 * "Context Parallelism in vLLM Omni Neuron", §Ring attention).
 * parts: [n, rows, D], lse_parts: [n, rows] -> out: [rows, D], lse_out: [rows]
 * (may be NULL).  L = ln sum_i e^(lse_i); out = sum_i e^(lse_i - L) parts_i.
 * Reading for the degenerate case: when every lse_i is -inf the row has no
 * keys; out = 0 and L = -inf.
 */
int oracle_lse_merge(const double* parts, const double* lse_parts, int64_t n, int64_t rows,
                     int64_t D, double* out, double* lse_out) {
  if (n <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double hi = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
      if (lse_parts[i * rows + r] > hi) hi = lse_parts[i * rows + r];
    double* o = out + r * D;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (hi == -INFINITY) {
      if (lse_out) lse_out[r] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) sum += exp(lse_parts[i * rows + r] - hi);
    const double L = hi + log(sum);
    for (int64_t i = 0; i < n; ++i) {
      const double w = exp(lse_parts[i * rows + r] - L);
      const double* p = parts + (i * rows + r) * D;
      for (int64_t d = 0; d < D; ++d) o[d] += w * p[d];
    }
    if (lse_out) lse_out[r] = L;
  }
  return 0;
}
