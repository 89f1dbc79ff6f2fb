/*
 * oracle.h -- plain, slow CPU oracle for the batch-1 / width-4 int4 (q4_0 grid)
 * decode step of a Gemma-4-12B-style dense interleaved-attention decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code, header, table or constant with
 * the HIP library; the two meet only through the seeded inputs.
 *
 * Arithmetic: fp64 everywhere, except
 *   - the storage formats the pages fix (fp16 weights scales, fp16 KV cache,
 *     fp16 query, fp16 vocab table) and the fp16 activations fed to every
 *     matrix-vector product; each of these is an explicit RNE rounding point;
 *   - the q4_0 quantisation decision, which is taken in IEEE fp32 (the same
 *     precision as the GPU packer) so that both sides pick the same code.
 *
 * Parity unpinned (oracle <-> pages): the model readings that the pages leave
 * open (norm placement, eps, GELU form, softcap value, embedding scale, V-norm
 * on sliding layers, layer_scalar placement).  They are pinned only by
 * invariants and special cases in tests/, not against a real checkpoint.
 */
#ifndef Q4_ORACLE_H
#define Q4_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- fp16 storage helpers (IEEE binary16, round to nearest even) ---- */
uint16_t orc_f64_to_f16(double x);
uint16_t orc_f32_to_f16(float x);
double   orc_f16_to_f64(uint16_t h);
void     orc_f64_to_f16_array(const double* x, int64_t n, uint16_t* out);

/* ---- q4_0 grid (gemma4-12b card: per-block-32 absmax symmetric int4;
 *      E4B card, Provenance: "symmetric-with-clipping", grid [-8,7]) ----
 * Canonical block = 18 bytes: bytes 0..1 fp16 scale d (little endian), bytes
 * 2..17 codes; code byte j holds element j in its low nibble and element j+16
 * in its high nibble; a nibble stores q+8.  Blocks are row-major [N][K/32]. */
void orc_q4_pack(const float* w, int64_t N, int64_t K, uint8_t* blocks);
/* dequantised weight w_hat = d*q (exact in fp64), row-major [N][K] */
void orc_q4_dequant(const uint8_t* blocks, int64_t N, int64_t K, double* w_hat);
/* y[b][n] = sum_k w_hat[n][k] * x[b][k], x given as fp16 bits [B][K] */
void orc_q4_gemv(const uint8_t* blocks, int64_t N, int64_t K,
                 const uint16_t* x, int B, double* y);
/* ---- q8 "int8lin" weights (gemma4-12b card: the int8lin ship beside int4linsym;
 *      reading: per-block-32 absmax symmetric int8, grid [-127, 127]) ----
 * Canonical block = 34 bytes: bytes 0..1 fp16 scale d = fp16(absmax/127)
 * (little endian), bytes 2..33 the codes q as int8 (two's complement), element
 * i in byte 2+i.  Blocks are row-major [N][K/32]. */
void orc_q8_pack(const float* w, int64_t N, int64_t K, uint8_t* blocks);
void orc_q8_dequant(const uint8_t* blocks, int64_t N, int64_t K, double* w_hat);
void orc_q8_gemv(const uint8_t* blocks, int64_t N, int64_t K,
                 const uint16_t* x, int B, double* y);
/* same for an fp16 matrix W [N][K] (the tied vocab table) */
void orc_f16_gemv(const uint16_t* W, int64_t N, int64_t K,
                  const uint16_t* x, int B, double* y);

/* ---- ring admission (Gemma-4-12B-CoreAI card, "v5/ -- ring extent R = 2W"):
 * slot j holds implied position p = q - ((q - j) mod R) (non-negative mod) and
 * is admitted iff p >= 0 and q - p < W.  admit[j] = 1/0 for j in [0,R). */
void orc_ring_admit(int64_t q, int64_t R, int64_t W, uint8_t* admit);

/* ---- attention for one query row over an explicit admitted slot set ----
 * q: fp16 [Hq][D]; k, v: fp16, slot s of KV head g at k + g*head_stride + s*D;
 * head h reads KV head h / (Hq/Hkv).  out[h][d] = sum_t softmax_t(scale*q.k_t) v_t
 * over the admitted slots, in fp64. */
void orc_attend(const uint16_t* q, int Hq, int Hkv, int D,
                const uint16_t* k, const uint16_t* v, int64_t head_stride,
                const uint8_t* admit, int64_t n_slots, double scale, double* out);

/* full-attention layer cache [cap][D] (one KV head shared by all Hq heads,
 * gemma4-12b card architecture notes); row i of the block attends positions
 * [0, pos0+i].  q [n_rows][Hq][D] fp16, out [n_rows][Hq][D]. */
void orc_flash_full(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int64_t cap, int Hq, int D, int64_t pos0, int n_rows,
                    double scale, double* out);
/* full layer caching one fp16 row per position ("vrow": the scale-free normed
 * raw k, which is V): the key of position t is RoPE_t(kw .* v_t), formed at
 * full precision from the stored row; q, v and the row rule as orc_flash_full.
 * vrow [cap][D]; kw [D] the layer's k_norm multiplier. */
void orc_flash_full_vrow(const uint16_t* q, const uint16_t* vrow, int64_t cap, int Hq, int D,
                         int64_t pos0, int n_rows, const float* kw, double theta, int rot_pairs,
                         double scale, double* out);
/* sliding-window layer ring [Hkv][R][D]; row i sits at position pos0+i. */
void orc_flash_ring(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int Hq, int Hkv, int D, int64_t R, int64_t W,
                    int64_t pos0, int n_rows, double scale, double* out);

/* ---- elementwise pieces of the decoder layer ---- */
/* RMSNorm: x * w / sqrt(mean(x^2) + eps); w may be NULL (scale-free). */
void   orc_rmsnorm(const double* x, const float* w, int64_t n, double eps, double* out);
/* rotary embedding on half-split pairs (i, i + D/2), i < rot_pairs, angle
 * pos * theta^(-2i/D); pairs at or beyond rot_pairs are left as they are. */
void   orc_rope(double* x, int D, int64_t pos, double theta, int rot_pairs);
double orc_gelu_tanh(double g);
double orc_softcap(double z, double c);

/* ---- the decode step ---- */
typedef struct {
  int is_full;            /* 1: full attention layer, 0: sliding ring layer  */
  int v_norm;             /* apply the scale-free RMSNorm to V               */
  const uint8_t *wq, *wk, *wv, *wo, *wg, *wu, *wd; /* canonical blocks (q4_0 or int8, per the model's
                                                      weight_format); wv unused on full layers */
  const float *attn_norm, *q_norm, *k_norm, *post_attn_norm, *pre_ff_norm, *post_ff_norm;
  float layer_scalar;
  uint16_t *k_cache, *v_cache; /* sliding: [Hkv][R][D]; full: [cap][D] (k_cache unused
                                  when the model's kv_format is 1) */
} orc_layer;

typedef struct {
  int hidden, n_heads, inter, vocab, n_layers;
  int sl_kv_heads, sl_head_dim, full_head_dim;
  int64_t window, ring, full_cap;
  double sl_theta, full_theta;
  int sl_rot_pairs, full_rot_pairs;
  double sl_scale, full_scale, eps, softcap;
  const uint16_t* embed;      /* fp16 [vocab][hidden], tied with the head */
  const float* final_norm;    /* [hidden] */
  orc_layer* layers;          /* [n_layers] */
  int weight_format;          /* 0: the layers' matrices are canonical q4_0 blocks; 1: int8 (q8) blocks */
  int kv_format;              /* 0: full layers cache K and V rows; 1: they cache only the V row
                                 (orc_flash_full_vrow; needs v_norm on full layers) */
} orc_model;

/* The step in three parts (used alone for teacher-forced checks):
 * orc_embed: h[i] = fp16 table row of tokens[i] times sqrt(hidden);
 * orc_run_layer: layer l on h [n][hidden] in place, rows at pos0 + i;
 * orc_head: final RMSNorm, fp16 tied head, softcap, argmax. */
int orc_embed(const orc_model* m, const int32_t* tokens, int n, double* h);
int orc_run_layer(const orc_model* m, int l, double* h, int n, int64_t pos0);
int orc_head(const orc_model* m, const double* h, int n, double* logits, int32_t* argmax);

/* The layer as the stages orc_run_layer composes (each from the storage
 * values of the previous one; q, k, v raw fp64 projections, x16 / q16 / o16 /
 * a16 fp16 bits; h is updated in place by stages 4 and 6), and the head as
 * its input norm and its product:
 *   1a orc_stage_attn_in: x16 = fp16(RMSNorm(h, attn_norm))
 *   1b orc_stage_qkv:     q, k, v projections of x16 (v = k on full layers)
 *   2  orc_stage_finish:  q16 = fp16(RoPE(RMSNorm(q))); K/V rows into the cache
 *   3  orc_stage_attend:  att = attention of q16 over the cache
 *   4  orc_stage_oproj:   h += RMSNorm(Wo o16, post_attn_norm)
 *   5a orc_stage_mlp_in:  x16 = fp16(RMSNorm(h, pre_ff_norm))
 *   5b orc_stage_gateup:  a16 = fp16(gelu_tanh(Wg x16) * Wu x16)
 *   6  orc_stage_down:    h = (h + RMSNorm(Wd a16, post_ff_norm)) * layer_scalar */
int orc_stage_attn_in(const orc_model* m, int l, const double* h, int n, uint16_t* x16);
int orc_stage_qkv(const orc_model* m, int l, const uint16_t* x16, int n, double* q, double* k, double* v);
int orc_stage_finish(const orc_model* m, int l, const double* q, const double* k, const double* v,
                     int n, int64_t pos0, uint16_t* q16);
int orc_stage_attend(const orc_model* m, int l, const uint16_t* q16, int n, int64_t pos0, double* att);
int orc_stage_oproj(const orc_model* m, int l, const uint16_t* o16, int n, double* h);
int orc_stage_mlp_in(const orc_model* m, int l, const double* h, int n, uint16_t* x16);
int orc_stage_gateup(const orc_model* m, int l, const uint16_t* x16, int n, uint16_t* a16);
int orc_stage_down(const orc_model* m, int l, const uint16_t* a16, int n, double* h);
int orc_head_input(const orc_model* m, const double* h, int n, uint16_t* x16);
int orc_head_logits(const orc_model* m, const uint16_t* x16, int n, double* logits, int32_t* argmax);

/* Runs n rows (tokens[i] at position pos0+i) through the model, writing K/V
 * of every row into the caches first and then attending with per-row
 * causality.  logits [n][vocab] (softcapped), argmax [n] (lowest index on
 * ties); either may be NULL.  Returns 0, or -1 on a bad argument. */
int orc_decode_step(const orc_model* m, const int32_t* tokens, int n, int64_t pos0,
                    double* logits, int32_t* argmax);

int orc_num_threads(void);
void orc_set_num_threads(int n);   /* OpenMP threads of the later calls (n > 0) */

#ifdef __cplusplus
}
#endif
#endif
