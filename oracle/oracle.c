/*
 * oracle.c -- plain, slow CPU oracle (fp64) for the int4 q4_0 decode step.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py; never by the product path.  It shares no code
 * with the HIP library.  OpenMP is used only across independent outputs
 * (matrix rows, attention heads); every sum runs in its natural index order.
 *
 * Sources (the five pages this project follows):
 *   [zoo]   coreai-model-zoo "gemma4-12b" card: q4_0 = per-block-32 absmax
 *           symmetric int4 (intro); architecture notes (attention_k_eq_v,
 *           dual RoPE, layer_scalar, tied embeddings, softcap); "The fix"
 *           (mask-free GQA-16:1 flash decode, scale 1.0, fp32 online softmax).
 *   [12b]   "Gemma-4-12B-CoreAI" card: "v5/ -- ring extent R = 2W" (slot ->
 *           implied position rule and window test); tiered-v3 (fp16 vocab path).
 *   [e4b]   "gemma-4-E4B-CoreAI" card: Provenance (q4_0 grid, symmetric with
 *           clipping); ring/ (written, causal, in-window slots; GQA fold).
 *   [128k]  "gemma-4-12b-it-coreml-128k" card: Key numbers (ring of 1024 for
 *           sliding layers; full [1,131072,512] state); greedy argmax head.
 * Readings of points the pages leave open are listed beside each function.
 */
#include "oracle.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* fp16 (IEEE binary16) conversion, round to nearest, ties to even.          */
/* ------------------------------------------------------------------------ */
uint16_t orc_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sign | 0x7E00);
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | 0x7C00);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);            /* a = m * 2^ex, m in [0.5, 1) */
  int e = ex - 1;           /* a in [2^e, 2^(e+1)) */
  if (e < -14) {            /* fp16 subnormal range: quantum 2^-24 */
    double r = nearbyint(ldexp(a, 24));   /* exact scaling, RNE */
    /* r in [0, 1024]; r == 1024 encodes the smallest normal 2^-14 */
    return (uint16_t)(sign | (uint16_t)r);
  }
  double r = nearbyint(ldexp(a, 10 - e)); /* r in [1024, 2048] */
  int biased = e + 15;
  if (r >= 2048.0) { r = 1024.0; biased += 1; }
  if (biased >= 31) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)r - 1024));
}

uint16_t orc_f32_to_f16(float x) { return orc_f64_to_f16((double)x); }

double orc_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1, ex = (h >> 10) & 31, m = h & 1023;
  double v;
  if (ex == 0) v = ldexp((double)m, -24);
  else if (ex == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), ex - 25);
  return s ? -v : v;
}

void orc_f64_to_f16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_f64_to_f16(x[i]);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* q4_0 packing and the int4 matrix-vector product                           */
/* ------------------------------------------------------------------------ */
/* [zoo] intro + [e4b] Provenance: per block of 32 weights, scale from the
 * absolute maximum, codes on the grid [-8, 7].  Readings: d = fp16(absmax/8)
 * (a positive scale); the codes are taken against the stored fp16 scale;
 * q = clamp(round_half_away(w / d), -8, 7) with w / d an IEEE fp32 quotient,
 * so +absmax maps to 8 and is clipped to 7; a zero (or underflowing) scale
 * gives all-zero codes.  A block with a non-finite weight, or whose scale
 * absmax/8 overflows fp16 (above 65504 after rounding), has no q4_0 encoding:
 * it is stored as the zero block (scale 0, every code 0), the same rule as
 * the int8 format below. */
void orc_q4_pack(const float* w, int64_t N, int64_t K, uint8_t* blocks) {
  const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t b = 0; b < nb; b++) {
      const float* src = w + n * K + b * 32;
      uint8_t* blk = blocks + (n * nb + b) * 18;
      float amax = 0.0f;
      int finite = 1;
      for (int i = 0; i < 32; i++) {
        if (!isfinite(src[i])) finite = 0;
        float a = fabsf(src[i]);
        if (a > amax) amax = a;
      }
      uint16_t d16 = finite ? orc_f32_to_f16(amax / 8.0f) : 0;
      float d = (float)orc_f16_to_f64(d16);
      if (!isfinite(d)) { d16 = 0; d = 0.0f; }
      int q[32];
      for (int i = 0; i < 32; i++) {
        if (d == 0.0f) { q[i] = 0; continue; }
        float rr = roundf(src[i] / d);      /* IEEE fp32 quotient, half away from zero */
        q[i] = (rr > 7.0f) ? 7 : (rr < -8.0f ? -8 : (int)rr);
      }
      blk[0] = (uint8_t)(d16 & 0xFF);
      blk[1] = (uint8_t)(d16 >> 8);
      for (int j = 0; j < 16; j++)
        blk[2 + j] = (uint8_t)((q[j] + 8) | ((q[j + 16] + 8) << 4));
    }
  }
}

static inline int blk_code(const uint8_t* blk, int i) {
  int byte = blk[2 + (i & 15)];
  int nib = (i < 16) ? (byte & 15) : (byte >> 4);
  return nib - 8;
}
static inline double blk_scale(const uint8_t* blk) {
  return orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
}

void orc_q4_dequant(const uint8_t* blocks, int64_t N, int64_t K, double* w_hat) {
  const int64_t nb = K / 32;
  for (int64_t n = 0; n < N; n++)
    for (int64_t b = 0; b < nb; b++) {
      const uint8_t* blk = blocks + (n * nb + b) * 18;
      double d = blk_scale(blk);
      for (int i = 0; i < 32; i++) w_hat[n * K + b * 32 + i] = d * (double)blk_code(blk, i);
    }
}

/* y[b][n] = sum_k (d * q)[n][k] * x[b][k]; the matrix-vector product the
 * weight stream feeds ([zoo] "Decode is otherwise weight-bandwidth-bound"). */
void orc_q4_gemv(const uint8_t* blocks, int64_t N, int64_t K,
                 const uint16_t* x, int B, double* y) {
  const int64_t nb = K / 32;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(B * K));
  for (int64_t i = 0; i < (int64_t)B * K; i++) xd[i] = orc_f16_to_f64(x[i]);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    for (int b = 0; b < B; b++) {
      const double* xb = xd + (int64_t)b * K;
      double acc = 0.0;
      for (int64_t blkI = 0; blkI < nb; blkI++) {
        const uint8_t* blk = blocks + (n * nb + blkI) * 18;
        double d = blk_scale(blk);
        for (int i = 0; i < 32; i++)
          acc += d * (double)blk_code(blk, i) * xb[blkI * 32 + i];
      }
      y[(int64_t)b * N + n] = acc;
    }
  }
  free(xd);
}

/* ------------------------------------------------------------------------ */
/* q8 ("int8lin") packing and the int8 matrix-vector product                 */
/* ------------------------------------------------------------------------ */
/* [zoo] intro and Throughput table: the int8lin ship is the verified-clean
 * variant beside the faster int4linsym.  Reading (the pages give no block
 * size for it): the int4 rule with the int8 grid, per block of 32 weights
 * d = fp16(absmax/127) and q = clamp(round_half_away(w / d), -127, 127) with
 * w / d an IEEE fp32 quotient against the stored fp16 scale; a zero or
 * underflowing scale gives zero codes; a block holding a non-finite weight,
 * or whose scale overflows fp16, is stored as a zero block. */
void orc_q8_pack(const float* w, int64_t N, int64_t K, uint8_t* blocks) {
  const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t b = 0; b < nb; b++) {
      const float* src = w + n * K + b * 32;
      uint8_t* blk = blocks + (n * nb + b) * 34;
      float amax = 0.0f;
      int finite = 1;
      for (int i = 0; i < 32; i++) {
        if (!isfinite(src[i])) finite = 0;
        float a = fabsf(src[i]);
        if (a > amax) amax = a;
      }
      uint16_t d16 = finite ? orc_f32_to_f16(amax / 127.0f) : 0;
      float d = (float)orc_f16_to_f64(d16);
      if (!isfinite(d)) { d16 = 0; d = 0.0f; }
      blk[0] = (uint8_t)(d16 & 0xFF);
      blk[1] = (uint8_t)(d16 >> 8);
      for (int i = 0; i < 32; i++) {
        int qi = 0;
        if (d != 0.0f) {
          float rr = roundf(src[i] / d);      /* fp32 quotient, half away from zero */
          qi = (rr > 127.0f) ? 127 : (rr < -127.0f ? -127 : (int)rr);
        }
        blk[2 + i] = (uint8_t)(int8_t)qi;
      }
    }
  }
}

static inline double q8_scale(const uint8_t* blk) {
  return orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
}

void orc_q8_dequant(const uint8_t* blocks, int64_t N, int64_t K, double* w_hat) {
  const int64_t nb = K / 32;
  for (int64_t n = 0; n < N; n++)
    for (int64_t b = 0; b < nb; b++) {
      const uint8_t* blk = blocks + (n * nb + b) * 34;
      double d = q8_scale(blk);
      for (int i = 0; i < 32; i++) w_hat[n * K + b * 32 + i] = d * (double)(int8_t)blk[2 + i];
    }
}

void orc_q8_gemv(const uint8_t* blocks, int64_t N, int64_t K,
                 const uint16_t* x, int B, double* y) {
  const int64_t nb = K / 32;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(B * K));
  for (int64_t i = 0; i < (int64_t)B * K; i++) xd[i] = orc_f16_to_f64(x[i]);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    for (int b = 0; b < B; b++) {
      const double* xb = xd + (int64_t)b * K;
      double acc = 0.0;
      for (int64_t blkI = 0; blkI < nb; blkI++) {
        const uint8_t* blk = blocks + (n * nb + blkI) * 34;
        double d = q8_scale(blk);
        for (int i = 0; i < 32; i++) acc += d * (double)(int8_t)blk[2 + i] * xb[blkI * 32 + i];
      }
      y[(int64_t)b * N + n] = acc;
    }
  }
  free(xd);
}

void orc_f16_gemv(const uint16_t* W, int64_t N, int64_t K,
                  const uint16_t* x, int B, double* y) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)(B * K));
  for (int64_t i = 0; i < (int64_t)B * K; i++) xd[i] = orc_f16_to_f64(x[i]);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    for (int b = 0; b < B; b++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++) acc += orc_f16_to_f64(W[n * K + k]) * xd[(int64_t)b * K + k];
      y[(int64_t)b * N + n] = acc;
    }
  }
  free(xd);
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */
/* [12b] v5/: slot j of an R-slot ring holds implied position
 * p = q - ((q - j) mod R); it is admitted iff it is in the window, q - p < W.
 * Reading: it must also have been written, p >= 0 ([e4b] ring/: "written,
 * causal, in-window"). */
void orc_ring_admit(int64_t q, int64_t R, int64_t W, uint8_t* admit) {
  for (int64_t j = 0; j < R; j++) {
    int64_t m = (q - j) % R;
    if (m < 0) m += R;
    int64_t p = q - m;
    admit[j] = (uint8_t)(p >= 0 && q - p < W);
  }
}

/* softmax(scale * q.k) v over the admitted slots, per query head; head h
 * reads KV head h / (Hq / Hkv) (grouped-query attention). */
void orc_attend(const uint16_t* q, int Hq, int Hkv, int D,
                const uint16_t* k, const uint16_t* v, int64_t head_stride,
                const uint8_t* admit, int64_t n_slots, double scale, double* out) {
  const int group = Hq / Hkv;
  if (D > 1024 || group < 1) return;
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hq; h++) {
    const int g = h / group;
    const uint16_t* kg = k + (int64_t)g * head_stride;
    const uint16_t* vg = v + (int64_t)g * head_stride;
    double* s = (double*)malloc(sizeof(double) * (size_t)(n_slots > 0 ? n_slots : 1));
    double qd[1024];
    for (int d = 0; d < D; d++) qd[d] = orc_f16_to_f64(q[(int64_t)h * D + d]);
    double m = -INFINITY;
    for (int64_t t = 0; t < n_slots; t++) {
      if (!admit[t]) continue;
      double dot = 0.0;
      for (int d = 0; d < D; d++) dot += qd[d] * orc_f16_to_f64(kg[t * D + d]);
      s[t] = scale * dot;
      if (s[t] > m) m = s[t];
    }
    double den = 0.0;
    double* o = out + (int64_t)h * D;
    for (int d = 0; d < D; d++) o[d] = 0.0;
    for (int64_t t = 0; t < n_slots; t++) {
      if (!admit[t]) continue;
      double e = exp(s[t] - m);
      den += e;
      for (int d = 0; d < D; d++) o[d] += e * orc_f16_to_f64(vg[t * D + d]);
    }
    for (int d = 0; d < D; d++) o[d] = (den > 0.0) ? o[d] / den : 0.0;
    free(s);
  }
}

/* [zoo] "The fix": the full layers hold one global KV head and a decode
 * query attends every written key; row i of a verify block sits at
 * position pos0+i and attends positions [0, pos0+i] (causal). */
void orc_flash_full(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int64_t cap, int Hq, int D, int64_t pos0, int n_rows,
                    double scale, double* out) {
  uint8_t* admit = (uint8_t*)malloc((size_t)cap);
  for (int i = 0; i < n_rows; i++) {
    int64_t P = pos0 + i;
    for (int64_t t = 0; t < cap; t++) admit[t] = (uint8_t)(t <= P);
    orc_attend(q + (int64_t)i * Hq * D, Hq, 1, D, k, v, 0, admit, cap, scale,
               out + (int64_t)i * Hq * D);
  }
  free(admit);
}

void orc_flash_ring(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int Hq, int Hkv, int D, int64_t R, int64_t W,
                    int64_t pos0, int n_rows, double scale, double* out) {
  uint8_t* admit = (uint8_t*)malloc((size_t)R);
  for (int i = 0; i < n_rows; i++) {
    orc_ring_admit(pos0 + i, R, W, admit);
    orc_attend(q + (int64_t)i * Hq * D, Hq, Hkv, D, k, v, R * D, admit, R, scale,
               out + (int64_t)i * Hq * D);
  }
  free(admit);
}

/* Full layer whose cache keeps ONE fp16 row per position ("vrow").  [12b]
 * "The per-tier cost": the full-layer pair costs 2 x 512 fp16 per position and
 * layer, the one KV term that grows with the context, and cutting it is named
 * as an open lever.  [zoo] architecture notes: on a full layer V is the
 * scale-free RMSNorm of the raw k projection and K is the k_norm-weighted
 * RMSNorm of the same row, rotated.  With one eps for both norms, K = RoPE(w .*
 * V) exactly, so the row v_t alone determines both.  Reading: the stored row is
 * fp16(v_t); the key is formed from that stored row at full precision,
 * k_t = RoPE_t(w .* v_t) (never rounded), and v_t is used as stored.
 * kw: the layer's k_norm multiplier [D]; the rotation is orc_rope's. */
void orc_flash_full_vrow(const uint16_t* q, const uint16_t* vrow, int64_t cap, int Hq, int D,
                         int64_t pos0, int n_rows, const float* kw, double theta, int rot_pairs,
                         double scale, double* out) {
  const int64_t npos = pos0 + n_rows;
  if (npos > cap || D > 1024) return;
  double* kd = (double*)malloc(sizeof(double) * (size_t)(npos > 0 ? npos : 1) * (size_t)D);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < npos; t++) {
    double* kt = kd + t * D;
    for (int d = 0; d < D; d++) kt[d] = (double)kw[d] * orc_f16_to_f64(vrow[t * D + d]);
    orc_rope(kt, D, t, theta, rot_pairs);
  }
  for (int i = 0; i < n_rows; i++) {
    const int64_t P = pos0 + i;
    const uint16_t* qi = q + (int64_t)i * Hq * D;
    double* oi = out + (int64_t)i * Hq * D;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hq; h++) {
      double* s = (double*)malloc(sizeof(double) * (size_t)(P + 1));
      double qd[1024];
      for (int d = 0; d < D; d++) qd[d] = orc_f16_to_f64(qi[(int64_t)h * D + d]);
      double m = -INFINITY;
      for (int64_t t = 0; t <= P; t++) {
        double dot = 0.0;
        for (int d = 0; d < D; d++) dot += qd[d] * kd[t * D + d];
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
      }
      double den = 0.0;
      double* o = oi + (int64_t)h * D;
      for (int d = 0; d < D; d++) o[d] = 0.0;
      for (int64_t t = 0; t <= P; t++) {
        double e = exp(s[t] - m);
        den += e;
        for (int d = 0; d < D; d++) o[d] += e * orc_f16_to_f64(vrow[t * D + d]);
      }
      for (int d = 0; d < D; d++) o[d] /= den;
      free(s);
    }
  }
  free(kd);
}

/* ------------------------------------------------------------------------ */
/* elementwise pieces                                                        */
/* ------------------------------------------------------------------------ */
/* Reading: RMSNorm(x) = x * w / sqrt(mean(x^2) + eps), w the effective
 * multiplier; w == NULL is the scale-free form ([zoo] architecture notes:
 * "a scale-free V RMSNorm"). */
void orc_rmsnorm(const double* x, const float* w, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; i++) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; i++) out[i] = x[i] * inv * (w ? (double)w[i] : 1.0);
}

/* [zoo] architecture notes: dual RoPE, sliding theta 1e4 rotating every pair,
 * full theta 1e6 "proportional" with the first 64 of 256 frequency pairs
 * rotating and the rest position-free.  Reading: half-split pairs
 * (i, i + D/2); frequency theta^(-2i/D) over the full head dim; angle in fp64. */
void orc_rope(double* x, int D, int64_t pos, double theta, int rot_pairs) {
  const int half = D / 2;
  for (int i = 0; i < rot_pairs && i < half; i++) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
    double ang = (double)pos * inv_freq;
    double c = cos(ang), s = sin(ang);
    double a = x[i], b = x[i + half];
    x[i] = a * c - b * s;
    x[i + half] = b * c + a * s;
  }
}

/* Reading: the gated MLP's activation is GELU with the tanh approximation. */
double orc_gelu_tanh(double g) {
  const double k0 = 0.7978845608028654; /* sqrt(2/pi) */
  return 0.5 * g * (1.0 + tanh(k0 * (g + 0.044715 * g * g * g)));
}

/* [zoo] architecture notes: final logit softcap in the graph; c * tanh(z / c). */
double orc_softcap(double z, double c) { return c * tanh(z / c); }

/* ------------------------------------------------------------------------ */
/* decode step                                                               */
/* ------------------------------------------------------------------------ */
static void to_f16(const double* x, int64_t n, uint16_t* out) { orc_f64_to_f16_array(x, n, out); }

static int check_rows(const orc_model* m, int l, int n, int64_t pos0) {
  if (!m || n < 1 || pos0 < 0 || l < 0 || l >= m->n_layers) return -1;
  if (m->window > m->ring || m->ring < m->window + n - 1) return -1;
  if (m->layers[l].is_full && pos0 + n - 1 >= m->full_cap) return -1;
  if (m->kv_format != 0 && m->kv_format != 1) return -1;
  if (m->kv_format == 1 && m->layers[l].is_full && !m->layers[l].v_norm) return -1;
  return 0;
}

/* embedding: fp16 row of the tied table times sqrt(hidden) (reading) */
int orc_embed(const orc_model* m, const int32_t* tokens, int n, double* h) {
  if (!m || !tokens || n < 1) return -1;
  const int H = m->hidden;
  for (int i = 0; i < n; i++) if (tokens[i] < 0 || tokens[i] >= m->vocab) return -1;
  const double emb_scale = sqrt((double)H);
  for (int i = 0; i < n; i++)
    for (int c = 0; c < H; c++)
      h[(int64_t)i * H + c] = orc_f16_to_f64(m->embed[(int64_t)tokens[i] * H + c]) * emb_scale;
  return 0;
}

/* the product of a layer matrix in the model's weight format */
static void wgemv(const orc_model* m, const uint8_t* blocks, int64_t N, int64_t K,
                  const uint16_t* x, int B, double* y) {
  if (m->weight_format == 1) orc_q8_gemv(blocks, N, K, x, B, y);
  else orc_q4_gemv(blocks, N, K, x, B, y);
}

static int layer_ok(const orc_model* m, int l, int n) {
  return m && n >= 1 && l >= 0 && l < m->n_layers;
}

/* One decoder layer ([zoo] architecture notes: gemma3_text-like pre/post
 * norms, attention_k_eq_v on full layers, dual RoPE, layer_scalar), as the
 * stages that orc_run_layer composes; each stage starts from the storage
 * values of the previous one (the fp16 rounding points), so a stage can also
 * be run on another implementation's values.  Row i sits at position pos0+i.
 */

/* Stage 1a: x16 = fp16(RMSNorm(h, attn_norm)), the projections' input. */
int orc_stage_attn_in(const orc_model* m, int l, const double* h, int n, uint16_t* x16) {
  if (!layer_ok(m, l, n)) return -1;
  const int H = m->hidden;
  double* t0 = (double*)malloc(sizeof(double) * (size_t)H);
  for (int i = 0; i < n; i++) {
    orc_rmsnorm(h + (int64_t)i * H, m->layers[l].attn_norm, H, m->eps, t0);
    to_f16(t0, H, x16 + (int64_t)i * H);
  }
  free(t0);
  return 0;
}

/* Stage 1b: raw projections q = Wq x16, k = Wk x16, and v = Wv x16 on
 * sliding layers or the raw k itself on full layers (attention_k_eq_v).
 * q [n][Hq*D], k and v [n][Hkv*D]. */
int orc_stage_qkv(const orc_model* m, int l, const uint16_t* x16, int n, double* q, double* k, double* v) {
  if (!layer_ok(m, l, n)) return -1;
  const int H = m->hidden, Hq = m->n_heads;
  const orc_layer* L = &m->layers[l];
  const int full = L->is_full;
  const int D = full ? m->full_head_dim : m->sl_head_dim;
  const int Hkv = full ? 1 : m->sl_kv_heads;
  wgemv(m, L->wq, (int64_t)Hq * D, H, x16, n, q);
  wgemv(m, L->wk, (int64_t)Hkv * D, H, x16, n, k);
  if (full) memcpy(v, k, sizeof(double) * (size_t)n * Hkv * D);
  else wgemv(m, L->wv, (int64_t)Hkv * D, H, x16, n, v);
  return 0;
}

/* Stage 2: per head, q16 = fp16(RoPE(RMSNorm(q, q_norm))); the key
 * RoPE(RMSNorm(k, k_norm)) and the value (scale-free RMSNorm of v when the
 * layer normalises V, else v) are rounded to fp16 and written into the
 * layer's cache at position pos0 + i (ring slot p mod R, full row p; a
 * kv_format 1 model keeps only the V row of a full layer). */
int orc_stage_finish(const orc_model* m, int l, const double* q, const double* k, const double* v,
                     int n, int64_t pos0, uint16_t* q16) {
  if (check_rows(m, l, n, pos0)) return -1;
  const int Hq = m->n_heads;
  const orc_layer* L = &m->layers[l];
  const int full = L->is_full;
  const int D = full ? m->full_head_dim : m->sl_head_dim;
  const int Hkv = full ? 1 : m->sl_kv_heads;
  const int64_t R = m->ring;
  const double theta = full ? m->full_theta : m->sl_theta;
  const int rot = full ? m->full_rot_pairs : m->sl_rot_pairs;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  for (int i = 0; i < n; i++) {
    const int64_t P = pos0 + i;
    for (int hh = 0; hh < Hq; hh++) {
      orc_rmsnorm(q + (int64_t)i * Hq * D + (int64_t)hh * D, L->q_norm, D, m->eps, tmp);
      orc_rope(tmp, D, P, theta, rot);
      to_f16(tmp, D, q16 + (int64_t)i * Hq * D + (int64_t)hh * D);
    }
    for (int gg = 0; gg < Hkv; gg++) {
      const double* kh = k + (int64_t)i * Hkv * D + (int64_t)gg * D;
      const double* vh = v + (int64_t)i * Hkv * D + (int64_t)gg * D;
      orc_rmsnorm(kh, L->k_norm, D, m->eps, tmp);
      orc_rope(tmp, D, P, theta, rot);
      uint16_t* kdst; uint16_t* vdst;
      if (full && m->kv_format == 1) { kdst = NULL; vdst = L->v_cache + P * D; }   /* vrow: V only */
      else if (full) { kdst = L->k_cache + P * D; vdst = L->v_cache + P * D; }
      else {
        int64_t slot = P % R;
        kdst = L->k_cache + ((int64_t)gg * R + slot) * D;
        vdst = L->v_cache + ((int64_t)gg * R + slot) * D;
      }
      if (kdst) to_f16(tmp, D, kdst);
      if (L->v_norm) { orc_rmsnorm(vh, NULL, D, m->eps, tmp); to_f16(tmp, D, vdst); }
      else to_f16(vh, D, vdst);
    }
  }
  free(tmp);
  return 0;
}

/* Stage 3: attention of the rows' fp16 queries q16 [n][Hq][D] over the
 * layer's cache (every row of the block already written), att [n][Hq][D]. */
int orc_stage_attend(const orc_model* m, int l, const uint16_t* q16, int n, int64_t pos0, double* att) {
  if (check_rows(m, l, n, pos0)) return -1;
  const orc_layer* L = &m->layers[l];
  const int full = L->is_full;
  const int D = full ? m->full_head_dim : m->sl_head_dim;
  const int Hkv = full ? 1 : m->sl_kv_heads;
  const double theta = full ? m->full_theta : m->sl_theta;
  const int rot = full ? m->full_rot_pairs : m->sl_rot_pairs;
  const double scale = full ? m->full_scale : m->sl_scale;
  if (full && m->kv_format == 1)
    orc_flash_full_vrow(q16, L->v_cache, m->full_cap, m->n_heads, D, pos0, n, L->k_norm, theta, rot, scale, att);
  else if (full) orc_flash_full(q16, L->k_cache, L->v_cache, m->full_cap, m->n_heads, D, pos0, n, scale, att);
  else orc_flash_ring(q16, L->k_cache, L->v_cache, m->n_heads, Hkv, D, m->ring, m->window, pos0, n, scale, att);
  return 0;
}

/* Stage 4: output projection of the fp16 attention output o16 [n][Hq*D],
 * post-attention RMSNorm, residual: h += RMSNorm(Wo o16, post_attn_norm). */
int orc_stage_oproj(const orc_model* m, int l, const uint16_t* o16, int n, double* h) {
  if (!layer_ok(m, l, n)) return -1;
  const int H = m->hidden;
  const orc_layer* L = &m->layers[l];
  const int D = L->is_full ? m->full_head_dim : m->sl_head_dim;
  double* y = (double*)malloc(sizeof(double) * (size_t)n * H);
  double* t0 = (double*)malloc(sizeof(double) * (size_t)H);
  wgemv(m, L->wo, H, (int64_t)m->n_heads * D, o16, n, y);
  for (int i = 0; i < n; i++) {
    orc_rmsnorm(y + (int64_t)i * H, L->post_attn_norm, H, m->eps, t0);
    for (int c = 0; c < H; c++) h[(int64_t)i * H + c] += t0[c];
  }
  free(y); free(t0);
  return 0;
}

/* Stage 5a: x16 = fp16(RMSNorm(h, pre_ff_norm)), the gated MLP's input. */
int orc_stage_mlp_in(const orc_model* m, int l, const double* h, int n, uint16_t* x16) {
  if (!layer_ok(m, l, n)) return -1;
  const int H = m->hidden;
  double* t0 = (double*)malloc(sizeof(double) * (size_t)H);
  for (int i = 0; i < n; i++) {
    orc_rmsnorm(h + (int64_t)i * H, m->layers[l].pre_ff_norm, H, m->eps, t0);
    to_f16(t0, H, x16 + (int64_t)i * H);
  }
  free(t0);
  return 0;
}

/* Stage 5b: a16 = fp16(gelu_tanh(Wg x16) * (Wu x16)), a16 [n][inter]. */
int orc_stage_gateup(const orc_model* m, int l, const uint16_t* x16, int n, uint16_t* a16) {
  if (!layer_ok(m, l, n)) return -1;
  const int H = m->hidden, I = m->inter;
  const orc_layer* L = &m->layers[l];
  double* g = (double*)malloc(sizeof(double) * (size_t)n * I);
  double* u = (double*)malloc(sizeof(double) * (size_t)n * I);
  wgemv(m, L->wg, I, H, x16, n, g);
  wgemv(m, L->wu, I, H, x16, n, u);
  for (int64_t e = 0; e < (int64_t)n * I; e++) g[e] = orc_gelu_tanh(g[e]) * u[e];
  to_f16(g, (int64_t)n * I, a16);
  free(g); free(u);
  return 0;
}

/* Stage 6: down projection, post-FF RMSNorm, residual, layer scalar:
 * h = (h + RMSNorm(Wd a16, post_ff_norm)) * layer_scalar. */
int orc_stage_down(const orc_model* m, int l, const uint16_t* a16, int n, double* h) {
  if (!layer_ok(m, l, n)) return -1;
  const int H = m->hidden;
  const orc_layer* L = &m->layers[l];
  double* y = (double*)malloc(sizeof(double) * (size_t)n * H);
  double* t0 = (double*)malloc(sizeof(double) * (size_t)H);
  wgemv(m, L->wd, H, m->inter, a16, n, y);
  for (int i = 0; i < n; i++) {
    orc_rmsnorm(y + (int64_t)i * H, L->post_ff_norm, H, m->eps, t0);
    for (int c = 0; c < H; c++) {
      double* hc = &h[(int64_t)i * H + c];
      *hc = (*hc + t0[c]) * (double)L->layer_scalar;
    }
  }
  free(y); free(t0);
  return 0;
}

/* One decoder layer on the residual stream h [n][hidden] (updated in place):
 * the stages in order; the layer's cache receives every row's K/V before
 * any row attends. */
int orc_run_layer(const orc_model* m, int l, double* h, int n, int64_t pos0) {
  if (check_rows(m, l, n, pos0)) return -1;
  const int H = m->hidden, Hq = m->n_heads, I = m->inter;
  const int Hs = m->sl_kv_heads, Ds = m->sl_head_dim, Df = m->full_head_dim;
  const int Dmax = Ds > Df ? Ds : Df;
  const int64_t qdim = (int64_t)Hq * Dmax;
  const int64_t kvdim = (int64_t)(Hs > 1 ? Hs : 1) * Dmax;
  uint16_t* x16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * H);
  uint16_t* a16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * I);
  double* qv = (double*)malloc(sizeof(double) * (size_t)n * qdim);
  double* kv = (double*)malloc(sizeof(double) * (size_t)n * kvdim);
  double* vv = (double*)malloc(sizeof(double) * (size_t)n * kvdim);
  uint16_t* q16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * qdim);
  double* att = (double*)malloc(sizeof(double) * (size_t)n * qdim);
  const int D = m->layers[l].is_full ? Df : Ds;
  int rc = orc_stage_attn_in(m, l, h, n, x16);
  if (rc == 0) rc = orc_stage_qkv(m, l, x16, n, qv, kv, vv);
  if (rc == 0) rc = orc_stage_finish(m, l, qv, kv, vv, n, pos0, q16);
  if (rc == 0) rc = orc_stage_attend(m, l, q16, n, pos0, att);
  if (rc == 0) {
    to_f16(att, (int64_t)n * Hq * D, q16);             /* o16: the output projection's input */
    rc = orc_stage_oproj(m, l, q16, n, h);
  }
  if (rc == 0) rc = orc_stage_mlp_in(m, l, h, n, x16);
  if (rc == 0) rc = orc_stage_gateup(m, l, x16, n, a16);
  if (rc == 0) rc = orc_stage_down(m, l, a16, n, h);
  free(x16); free(a16); free(qv); free(kv); free(vv); free(q16); free(att);
  return rc;
}

/* final norm, tied fp16 head, softcap, greedy argmax (lowest index on ties)
 * ([zoo] architecture notes: tied embeddings, final softcap; [128k]: the head
 * emits the greedy id).  orc_head_input: x16 = fp16(RMSNorm(h, final_norm));
 * orc_head_logits: logits = c * tanh(E x16 / c) and the argmax. */
int orc_head_input(const orc_model* m, const double* h, int n, uint16_t* x16) {
  if (!m || n < 1) return -1;
  const int H = m->hidden;
  double* t0 = (double*)malloc(sizeof(double) * (size_t)H);
  for (int i = 0; i < n; i++) {
    orc_rmsnorm(h + (int64_t)i * H, m->final_norm, H, m->eps, t0);
    to_f16(t0, H, x16 + (int64_t)i * H);
  }
  free(t0);
  return 0;
}

int orc_head_logits(const orc_model* m, const uint16_t* x16, int n, double* logits, int32_t* argmax) {
  if (!m || n < 1) return -1;
  const int H = m->hidden, V = m->vocab;
  double* z = (double*)malloc(sizeof(double) * (size_t)n * V);
  orc_f16_gemv(m->embed, V, H, x16, n, z);
  for (int i = 0; i < n; i++) {
    int32_t best = 0;
    for (int64_t j = 0; j < V; j++) {
      double zz = orc_softcap(z[(int64_t)i * V + j], m->softcap);
      z[(int64_t)i * V + j] = zz;
      if (zz > z[(int64_t)i * V + best]) best = (int32_t)j;
    }
    if (argmax) argmax[i] = best;
  }
  if (logits) memcpy(logits, z, sizeof(double) * (size_t)n * V);
  free(z);
  return 0;
}

int orc_head(const orc_model* m, const double* h, int n, double* logits, int32_t* argmax) {
  if (!m || n < 1) return -1;
  uint16_t* x16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * m->hidden);
  int rc = orc_head_input(m, h, n, x16);
  if (rc == 0) rc = orc_head_logits(m, x16, n, logits, argmax);
  free(x16);
  return rc;
}

int orc_decode_step(const orc_model* m, const int32_t* tokens, int n, int64_t pos0,
                    double* logits, int32_t* argmax) {
  if (!m || !tokens || n < 1 || pos0 < 0) return -1;
  for (int l = 0; l < m->n_layers; l++) if (check_rows(m, l, n, pos0)) return -1;
  double* h = (double*)calloc((size_t)n * m->hidden, sizeof(double));
  int rc = orc_embed(m, tokens, n, h);
  for (int l = 0; l < m->n_layers && rc == 0; l++) rc = orc_run_layer(m, l, h, n, pos0);
  if (rc == 0) rc = orc_head(m, h, n, logits, argmax);
  free(h);
  return rc;
}
