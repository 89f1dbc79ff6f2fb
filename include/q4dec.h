/*
 * q4dec.h -- C ABI of the MI355X (gfx950) int4 q4_0 decode-step library.
 *
 * The library computes the batch-1 (or width-4 speculative verify) decode step
 * of a Gemma-4-12B-style dense decoder that interleaves sliding-window and full
 * attention layers:
 *   - a weight-streaming matrix-vector product over per-block-32 absmax
 *     symmetric int4 weights on the q4_0 grid [-8, 7] with one fp16 scale per
 *     block (gemma4-12b card, intro: q4_0 = per-block-32 absmax symmetric int4;
 *     gemma-4-E4B-CoreAI card, Provenance: symmetric with clipping);
 *   - flash-decode attention over a sliding-window ring of R slots, where slot
 *     j holds implied position p = q - ((q - j) mod R) and is admitted only if
 *     q - p < W (Gemma-4-12B-CoreAI card, "v5/ -- ring extent R = 2W"), and
 *     over a full-attention cache with one KV head whose value is the raw key
 *     projection after a scale-free RMSNorm (gemma4-12b card, architecture
 *     notes: attention_k_eq_v; "The fix": mask-free GQA flash decode, scale 1).
 *
 * Conventions (every entry point):
 *   - Pointers marked "device" are HIP device pointers; "host" pointers are
 *     read during the call only.  The library keeps no pointer after a call
 *     returns, except the captured decode-step graphs (see q4dec_release).
 *   - The library never allocates device memory; workspaces come from the
 *     caller.  All work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream) and calls never synchronise the device.
 *   - Argument checks are synchronous and host-only: on a non-zero status no
 *     kernel has been launched.  A failed launch returns Q4_EHIP.
 *   - fp16 values are IEEE binary16 bit patterns in uint16_t.
 *   - Device pointers must be 16-byte aligned (Q4_EALIGN otherwise).
 */
#ifndef Q4DEC_H
#define Q4DEC_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int q4_status;
#define Q4_OK        0
#define Q4_EINVAL   -1   /* null pointer where one is required, bad enum      */
#define Q4_ESHAPE   -2   /* unsupported or inconsistent sizes                  */
#define Q4_EALIGN   -3   /* device pointer not 16-byte aligned                 */
#define Q4_ERANGE   -4   /* position / capacity / window out of range          */
#define Q4_ENOSPACE -5   /* buffer or workspace smaller than required          */
#define Q4_EHIP     -6   /* a HIP runtime call or kernel launch failed         */

/* Human-readable name of a status code (static string). */
const char* q4dec_status_str(q4_status s);
/* Library version string (static): "q4dec <version> gfx950 src <hash>", where
 * <hash> is the first 16 hex digits of the SHA-256 of the library's sources
 * (the binding refuses a library whose hash differs from its tree's). */
const char* q4dec_version(void);

/* ------------------------------------------------------------------------ */
/* q4_0 packing                                                              */
/* ------------------------------------------------------------------------ */
enum { Q4_F32 = 0, Q4_BF16 = 1 };

/* Bytes of the packed form of an [N, K] matrix:
 * ceil(N/16)*16 rows * ceil(K/128)*4 blocks * 18 bytes (= N*K/32*18 when N is a
 * multiple of 16 and K of 128).  Returns 0 when K is not a positive multiple
 * of 32 or N < 1. */
size_t q4_packed_bytes(int N, int K);

/* Quantises W (device, row-major [N, K], fp32 or bf16) onto the q4_0 grid
 * (gemma4-12b card, intro; gemma-4-E4B-CoreAI card, Provenance): for each row
 * and block of 32 weights, d = fp16_rne(absmax / 8) and
 * q = clamp(round_half_away(w / d), -8, 7) with w / d an IEEE fp32 quotient
 * taken against the stored fp16 scale (d == 0 gives q = 0).
 * `packed` (device, packed_bytes >= q4_packed_bytes(N, K)) receives the
 * device layout: "quads" of 16 rows x 4 blocks, one 1 KB wave-wide load each;
 * codes [N/16][K/128][64 lanes][16 B] (lane l: row l % 16, block l / 16 of
 * the quad) followed by scales [N/16][K/128][64 lanes] fp16; padding rows and
 * blocks have zero scale.
 * `nonfinite` (device int32, may be NULL) is incremented once per block that
 * holds a non-finite weight or whose scale overflows fp16 (such blocks get
 * d = 0 and q = 0); it is data-dependent, so it is read after a sync.
 * Errors: Q4_EINVAL (null w/packed, bad dtype), Q4_ESHAPE (N < 1, K % 32),
 * Q4_ENOSPACE (packed_bytes too small), Q4_EALIGN, Q4_EHIP. */
q4_status q4_pack(const void* w, int w_dtype, int N, int K, void* packed,
                  size_t packed_bytes, int32_t* nonfinite, void* stream);

/* Exports the packed matrix in the canonical q4_0 block format (test and
 * interchange use): `blocks` (device) receives N*K/32 blocks of 18 bytes,
 * row-major [N][K/32]; each block is the fp16 scale (little endian) followed
 * by 16 code bytes, byte j holding element j (low nibble) and element j+16
 * (high nibble) as q + 8. */
q4_status q4_unpack(const void* packed, int N, int K, uint8_t* blocks, void* stream);

/* ------------------------------------------------------------------------ */
/* int4 matrix-vector product                                                */
/* ------------------------------------------------------------------------ */
/* y[b][n] = sum_k (d * q)[n][k] * x[b][k] for b < B, fp32 accumulation
 * (the weight stream of the decode step; gemma4-12b card, Throughput:
 * "decode is otherwise weight-bandwidth-bound").
 * packed: device, from q4_pack(N, K).  x: device fp16 [B][K].  y: device fp32
 * [B][N].  B in 1..4 (4 = the width-4 verify block; B > 1 runs on MFMA).
 * K <= 16384 (B == 1) or 15360 (B > 1).  No workspace; each 16-row tile is
 * finished by one workgroup, so results are deterministic.
 * Errors: Q4_EINVAL, Q4_ESHAPE (K % 32, K too large, B outside 1..4),
 * Q4_EALIGN, Q4_EHIP. */
q4_status q4_gemv(const void* packed, int N, int K, const uint16_t* x, int B,
                  float* y, void* stream);

/* ------------------------------------------------------------------------ */
/* int8 ("int8lin") weights                                                  */
/* ------------------------------------------------------------------------ */
/* The verified-clean weight variant (gemma4-12b card, intro and Throughput
 * table: the int8lin ship beside int4linsym).  The pages give no block format
 * for it; the reading is the q4_0 rule on the int8 grid: for each row and
 * block of 32 weights, d = fp16_rne(absmax / 127) and
 * q = clamp(round_half_away(w / d), -127, 127), w / d an IEEE fp32 quotient
 * against the stored fp16 scale (d == 0 gives q = 0); 1.0625 B per weight.
 *
 * Bytes of the packed form of an [N, K] matrix:
 * ceil(N/16) * ceil(K/64) * 1088 (= N*K/32*34 when N is a multiple of 16 and K
 * of 64).  Returns 0 when K is not a positive multiple of 32 or N < 1. */
size_t q8_packed_bytes(int N, int K);

/* Quantises W (device, row-major [N, K], fp32 or bf16) onto the int8 grid.
 * `packed` (device, packed_bytes >= q8_packed_bytes(N, K)) receives the
 * device layout: "pairs" of 16 rows x 2 blocks (64 columns), one 1 KB
 * wave-wide load each; codes [N/16][K/64][64 lanes][16 B] (lane l: row l % 16,
 * columns 16 (l / 16) .. +15 of the pair, byte j = q + 128 of column j of
 * those 16) followed by scales [N/16][K/64][2 blocks][16 rows] fp16; padding
 * rows and blocks have zero scale.  `nonfinite` as for q4_pack.
 * Errors: Q4_EINVAL, Q4_ESHAPE (N < 1, K % 32), Q4_ENOSPACE, Q4_EALIGN, Q4_EHIP. */
q4_status q8_pack(const void* w, int w_dtype, int N, int K, void* packed,
                  size_t packed_bytes, int32_t* nonfinite, void* stream);

/* Exports the packed matrix as canonical 34-byte blocks (device `blocks`,
 * row-major [N][K/32]): the fp16 scale (little endian) followed by the 32
 * codes as int8, element i in byte 2 + i. */
q4_status q8_unpack(const void* packed, int N, int K, uint8_t* blocks, void* stream);

/* y[b][n] = sum_k (d * q)[n][k] * x[b][k] for b < B, fp32 accumulation.
 * packed: device, from q8_pack(N, K).  x: device fp16 [B][K].  y: device fp32
 * [B][N].  B in 1..4 (B > 1 runs on MFMA).  K <= 16384.  No workspace;
 * each 16-row tile is finished by one workgroup, so results are deterministic.
 * Errors: Q4_EINVAL, Q4_ESHAPE (K % 32, K too large, B outside 1..4),
 * Q4_EALIGN, Q4_EHIP. */
q4_status q8_gemv(const void* packed, int N, int K, const uint16_t* x, int B,
                  float* y, void* stream);

/* ------------------------------------------------------------------------ */
/* flash-decode attention                                                    */
/* ------------------------------------------------------------------------ */
/* Workspace bytes for flash_decode_full / flash_decode_ring. */
size_t flash_decode_workspace_size(int n_seq, int n_rows, int Hq, int D);

/* Full-attention flash decode (gemma4-12b card, "The fix": one global KV head,
 * every written key attended, fp32 online softmax; split-K over positions with
 * a log-sum-exp combine).  For sequence s and row i (position pos0[s] + i):
 *   out[s][i][h] = sum_t softmax_t(scale * q[s][i][h] . k[s][t]) v[s][t],
 *   t in [0, pos0[s] + i]   (row i of a verify block is causal).
 * q: device fp16 [n_seq][n_rows][Hq][D].  k, v: device fp16, sequence s at
 * k + s*seq_stride, rows [cap][D] (one KV head).  pos0: host int32 [n_seq].
 * out: device fp32 [n_seq][n_rows][Hq][D].  Hq in 1..16, D in {64,128,256,512},
 * n_rows in 1..4, n_seq in 1..64.
 * Errors: Q4_ERANGE if pos0[s] < 0 or pos0[s] + n_rows - 1 >= cap;
 * Q4_ESHAPE, Q4_EINVAL, Q4_ENOSPACE, Q4_EALIGN, Q4_EHIP. */
q4_status flash_decode_full(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int64_t seq_stride, int cap, int Hq, int D,
                            const int32_t* pos0, int n_seq, int n_rows, float scale,
                            float* out, void* ws, size_t ws_bytes, void* stream);

/* flash_decode_full for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, with the split records in the library's own static device
 * array of flash_decode_noalloc_max_bytes() = 8,454,144 bytes per GPU
 * (enough for every call with n_seq * n_rows <= 32 and Hq <= 16, D <= 512)
 * instead of a workspace argument.  It calls no allocating routine.  Every
 * call on one GPU shares that array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be ordered
 * by the caller.  Nothing in the array needs clearing (every record is
 * written before it is read).  Arguments and results as flash_decode_full;
 * Q4_ENOSPACE when flash_decode_workspace_size(n_seq, n_rows, Hq, D) exceeds
 * the array; Q4_EHIP if the array's device address cannot be obtained. */
size_t flash_decode_noalloc_max_bytes(void);
q4_status flash_decode_full_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride,
                                    int cap, int Hq, int D, const int32_t* pos0, int n_seq, int n_rows,
                                    float scale, float* out, void* stream);

/* Full-attention flash decode over a cache that keeps ONE fp16 row per
 * position (Gemma-4-12B-CoreAI card, "The per-tier cost": the full-layer K/V
 * pair is the KV term that grows with the context; gemma4-12b card,
 * architecture notes: a full layer's V is the scale-free RMSNorm of the raw k
 * projection and its K the k_norm-weighted norm of the same row, rotated, so
 * K = RoPE(kw * V)).  The row is V; the key of row t is formed from it at full
 * precision in the kernel:
 *   k_t = RoPE_t(kw * v_t), pair (i, i + D/2) turned by t * theta^(-2i/D) for
 *   i < rot_pairs, never rounded to fp16;
 *   out[s][i][h] = sum_t softmax_t(scale * q[s][i][h] . k_t) v_t, t in [0, pos0[s] + i].
 * Half the bytes per position of flash_decode_full.  vrow: device fp16,
 * sequence s at vrow + s*seq_stride, rows [cap][D].  kw: device fp32 [D],
 * 16-byte aligned.  D in {128, 512}; rot_pairs in 0..64; theta > 0; the rest
 * as flash_decode_full (same workspace size).
 * Errors: Q4_ESHAPE (D, rot_pairs, theta), Q4_ERANGE, Q4_EINVAL, Q4_ENOSPACE,
 * Q4_EALIGN, Q4_EHIP. */
q4_status flash_decode_full_vrow(const uint16_t* q, const uint16_t* vrow, int64_t seq_stride, int cap,
                                 int Hq, int D, const float* kw, double theta, int rot_pairs,
                                 const int32_t* pos0, int n_seq, int n_rows, float scale,
                                 float* out, void* ws, size_t ws_bytes, void* stream);

/* Sliding-window flash decode over a ring (Gemma-4-12B-CoreAI card, "v5/ --
 * ring extent R = 2W"; gemma-4-E4B-CoreAI card, ring/: written, causal,
 * in-window slots).  Row i of sequence s sits at position P = pos0[s] + i and
 * attends the slots j whose implied position p = P - ((P - j) mod R) satisfies
 * p >= 0 and P - p < W, i.e. positions max(0, P-W+1) .. P at slots p mod R.
 * Query head h reads KV head h / (Hq / Hkv).
 * q: device fp16 [n_seq][n_rows][Hq][D].  k_ring, v_ring: device fp16,
 * sequence s at +s*seq_stride, [Hkv][R][D].  pos0: host int32 [n_seq].
 * out: device fp32 [n_seq][n_rows][Hq][D].  Hq % Hkv == 0, Hq/Hkv <= 16.
 * Errors: Q4_ERANGE if W < 1, W > R, R < W + n_rows - 1 (the rows of a
 * verify block written after row i must stay outside row i's window) or
 * pos0[s] < 0; Q4_ESHAPE if R < 32 (a ring holds at least one 32-position
 * tile), and Q4_ESHAPE, Q4_EINVAL, Q4_ENOSPACE, Q4_EALIGN, Q4_EHIP as above. */
q4_status flash_decode_ring(const uint16_t* q, const uint16_t* k_ring, const uint16_t* v_ring,
                            int64_t seq_stride, int Hq, int Hkv, int D, int R, int W,
                            const int32_t* pos0, int n_seq, int n_rows, float scale,
                            float* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* decode step                                                               */
/* ------------------------------------------------------------------------ */
/* One decoder layer.  Weight pointers are device buffers produced by q4_pack
 * with the shapes given in q4dec_model; norm vectors are device fp32. */
typedef struct q4dec_layer {
  int32_t is_full;              /* 1: full attention layer; 0: sliding ring layer   */
  int32_t v_norm;               /* 1: scale-free RMSNorm on the V rows              */
  const void* wq;               /* [Hq*D, hidden]                                    */
  const void* wk;               /* [Hkv*D, hidden]; full layers: Hkv = 1             */
  const void* wv;               /* [Hkv*D, hidden]; NULL on full layers (V = raw k)  */
  const void* wo;               /* [hidden, Hq*D]                                    */
  const void* wg;               /* [inter, hidden]                                   */
  const void* wu;               /* [inter, hidden]                                   */
  const void* wd;               /* [hidden, inter]                                   */
  const float* attn_norm;       /* [hidden] */
  const float* q_norm;          /* [D]      */
  const float* k_norm;          /* [D]      */
  const float* post_attn_norm;  /* [hidden] */
  const float* pre_ff_norm;     /* [hidden] */
  const float* post_ff_norm;    /* [hidden] */
  float layer_scalar;           /* h <- h * layer_scalar at the end of the layer    */
  uint16_t* k_cache;            /* fp16; sliding [Hkv][R][D]; full [full_cap][D]     */
  uint16_t* v_cache;            /* same shape as k_cache                             */
} q4dec_layer;

typedef struct q4dec_model {
  int32_t hidden, n_heads, inter, vocab, n_layers;
  int32_t sl_kv_heads, sl_head_dim, full_head_dim;
  int32_t window, ring, full_cap;
  int32_t sl_rot_pairs, full_rot_pairs;  /* pairs (i, i+D/2), i < rot_pairs, rotate */
  double sl_theta, full_theta;           /* RoPE bases (1e4 sliding, 1e6 full)         */
  float sl_scale, full_scale;            /* softmax scales (1.0 on the pages)          */
  float eps;                             /* RMSNorm epsilon                            */
  float softcap;                         /* final logit softcap c: c * tanh(z / c)     */
  const uint16_t* embed;                 /* device fp16 [vocab][hidden], tied head      */
  const float* final_norm;               /* device fp32 [hidden]                        */
  const q4dec_layer* layers;             /* host array [n_layers]                       */
  int32_t weight_format;                 /* 0: wq..wd packed by q4_pack; 1: by q8_pack   */
  int32_t kv_format;                     /* 0: full layers cache K and V rows; 1: only the V
                                            row (see flash_decode_full_vrow): k_cache of a
                                            full layer is then unused and may be NULL;
                                            needs v_norm on full layers, full_head_dim 128
                                            or 512 and full_rot_pairs <= 64               */
} q4dec_model;

/* Workspace bytes decode_step needs for `m` and n rows. */
size_t decode_step_workspace_size(const q4dec_model* m, int n);

/* Runs n rows (tokens[i] at position pos0 + i) through the model: embedding
 * times sqrt(hidden); per layer RMSNorm, q/k/v projections, per-head q/k
 * RMSNorm and dual RoPE (gemma4-12b card, architecture notes), fp16 K/V
 * written at ring slot P mod R or full row P, flash-decode attention, output
 * projection with post-norm residual, gated-GELU MLP with post-norm
 * residual, h *= layer_scalar; then final RMSNorm, the tied fp16 head and the
 * softcap.  All n rows' K/V are written before any row attends; row i sees
 * positions <= pos0 + i only.
 * tokens: host int32 [n].  logits: device fp32 [n][vocab] or NULL.
 * argmax: device int32 [n] or NULL (greedy id, lowest index on ties).
 * ws: device workspace of decode_step_workspace_size(m, n) bytes.
 * The first call for a given (model descriptor and layer table, n, ws)
 * captures a HIP graph of the step; later calls replay it on any stream.
 * Positions, tokens and the logits/argmax pointers are written to the
 * workspace by a kernel launched before the graph and read on the device,
 * so one graph serves every position and every pair of output buffers.  At
 * most 16 graphs are kept: capturing a 17th first destroys the least
 * recently used one, after synchronising the stream it last ran on.
 * A width-4 block finishes all rows first, then its rows share every K/V
 * tile they read (one pass over each layer's cache per block).
 * Errors: Q4_ERANGE (pos0 < 0; pos0 + n - 1 >= full_cap; R < W + n - 1;
 * token outside [0, vocab)); Q4_ESHAPE (n outside 1..4, ring < 32 or
 * unsupported dimensions); Q4_EINVAL; Q4_ENOSPACE; Q4_EALIGN; Q4_EHIP. */
q4_status decode_step(const q4dec_model* m, const int32_t* tokens, int n, int pos0,
                      float* logits, int32_t* argmax, void* ws, size_t ws_bytes,
                      void* stream);

/* Copies the residual stream after the last layer (before the final norm)
 * of the most recent step run with workspace `ws`: device fp32 [n][hidden].
 * This is the hidden state a drafter reads; the tests use it to check every
 * layer of the step.  Errors: Q4_EINVAL, Q4_ESHAPE, Q4_ENOSPACE, Q4_EHIP. */
q4_status decode_step_hidden(const q4dec_model* m, const void* ws, size_t ws_bytes, int n,
                             float* h_out, void* stream);

/* Stages of the last layer of the most recent step run with workspace `ws`
 * (rows 0 .. n-1; the tests compare each with the oracle fed the same inputs;
 * gemma4-12b card, architecture notes, for the layer they belong to):
 *   Q4_STAGE_H_OUT   fp32 [n][hidden]  residual stream after the layer
 *   Q4_STAGE_H_MID   fp32 [n][hidden]  residual after attention (+ post-attn norm)
 *   Q4_STAGE_X_ATTN  fp16 [n][hidden]  attention input (RMSNorm, attn_norm)
 *   Q4_STAGE_QKV     fp32 [n][ld]      raw q | k | v projections (v on sliding
 *                                      layers only); ld = the widest layer's row
 *   Q4_STAGE_Q16     fp16 [n][Hq][D]   queries after q_norm and RoPE
 *   Q4_STAGE_O16     fp16 [n][Hq][D]   attention output, input of the o-proj
 *   Q4_STAGE_X_MLP   fp16 [n][hidden]  MLP input (RMSNorm, pre_ff_norm)
 *   Q4_STAGE_A16     fp16 [n][inter]   gelu_tanh(gate) * up
 *   Q4_STAGE_X_HEAD  fp16 [n][hidden]  head input (final RMSNorm)
 * decode_step_stage_bytes gives the size (0 for a bad argument); D is the
 * last layer's head size.  decode_step_stage copies that many bytes to dst
 * (device).  Errors: Q4_EINVAL (null pointer, unknown stage), Q4_ESHAPE,
 * Q4_ENOSPACE (ws or dst too small), Q4_EHIP. */
enum {
  Q4_STAGE_H_OUT = 0, Q4_STAGE_H_MID = 1, Q4_STAGE_X_ATTN = 2, Q4_STAGE_QKV = 3, Q4_STAGE_Q16 = 4,
  Q4_STAGE_O16 = 5, Q4_STAGE_X_MLP = 6, Q4_STAGE_A16 = 7, Q4_STAGE_X_HEAD = 8
};
size_t decode_step_stage_bytes(const q4dec_model* m, int n, int stage);
q4_status decode_step_stage(const q4dec_model* m, const void* ws, size_t ws_bytes, int n, int stage,
                            void* dst, size_t dst_bytes, void* stream);

/* Measurement: enqueues only the q/k/v, output-projection and down products
 * of every layer of a step of width n (3 launches per layer of the step's
 * most launched kernel, with exactly the step's launch configuration),
 * reading the activations the workspace holds and writing its partial
 * products; no other kernel of the step.  Used to time that kernel in its
 * step configuration (gemma4-12b card, Throughput: decode is bound by the
 * weight stream).  Errors: Q4_EINVAL, Q4_ESHAPE, Q4_ENOSPACE, Q4_EALIGN,
 * Q4_EHIP. */
q4_status decode_step_gemvs(const q4dec_model* m, int n, void* ws, size_t ws_bytes, void* stream);

/* Number of captured decode-step graphs the library holds (at most 16). */
int q4dec_graph_count(void);

/* Same step without graph capture (every kernel launched directly). */
q4_status decode_step_eager(const q4dec_model* m, const int32_t* tokens, int n, int pos0,
                            float* logits, int32_t* argmax, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* prefill chunk                                                             */
/* ------------------------------------------------------------------------ */
/* Y[b][n] = sum_k (d * q)[n][k] * x[b][k] for the n <= 64 rows of a chunk, the
 * product of the prefill path, on MFMA (the q4 layout as q4_gemv takes it;
 * the scale enters the operand as an exact fp16 hi + lo split, sums are fp32).
 * packed: device, from q4_pack(N, K).  x: device fp16 [n][K].  y: device fp32
 * [n][N].  Requires |d * q| < 65504 (block absmax below 65504).
 * Errors: Q4_EINVAL, Q4_ESHAPE (K % 32, n outside 1..64), Q4_EALIGN (pointers,
 * K % 8), Q4_EHIP. */
q4_status q4_gemm(const void* packed, int N, int K, const uint16_t* x, int n, float* y,
                  void* stream);

/* Workspace bytes for prefill_chunk (any n <= 64); 0 for an unsupported model. */
size_t prefill_chunk_workspace_size(const q4dec_model* m);

/* One prefill chunk: n <= 64 tokens at positions pos0 .. pos0 + n - 1 through
 * the whole model in one pass (gemma-4-E4B-CoreAI card, Provenance and ring/:
 * a second entry point beside the S = 1 decode takes 64-token prefill chunks,
 * and the sliding ring holds the window plus one chunk; Gemma-4-12B-CoreAI
 * card, "v5/ -- ring extent R = 2W": the slot rule stays causal for a block of
 * rows while R >= W + rows - 1).  Every layer writes the K/V rows of all n
 * rows into the caller's caches, then each row attends its causal, in-window
 * positions as a decode row would; the products run on q4_gemm's kernel.
 * Same model descriptor as decode_step (weight_format 0; kv_format 0 or 1).
 * tokens: host int32 [n].  logits: device fp32 [vocab] of the LAST row, or
 * NULL.  argmax: device int32 [1] (greedy id of the last row), or NULL.
 * h_out: device fp32 [n][hidden], the residual stream of every row after the
 * last layer, or NULL.  No alignment of pos0 is needed (every row's ring slot
 * is written on its own).
 * Errors: as decode_step with n in 1..64; Q4_ESHAPE for weight_format != 0. */
q4_status prefill_chunk(const q4dec_model* m, const int32_t* tokens, int n, int pos0,
                        float* logits, int32_t* argmax, float* h_out, void* ws,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* speculative verify: greedy acceptance                                     */
/* ------------------------------------------------------------------------ */
/* The host half of one speculative verify block (host only, no device work).
 * block (host int32 [n]): the tokens fed to decode_step(n) at pos0 -- block[0]
 * is the last emitted token, block[1..n-1] are draft tokens for positions
 * pos0+1 .. pos0+n-1.  argmax (host int32 [n]): that step's argmax rows, row i
 * being the target's greedy token after block[0..i].
 * The accepted prefix is the longest a <= n-1 with block[i+1] == argmax[i]
 * for every i < a.  emitted (host int32 [n]) receives block[1..a] followed by
 * argmax[a], the target's own token after the prefix (a correction, or one more
 * token when every draft is accepted); *n_emitted = a + 1.  Every emitted
 * token is therefore one the target chose, so the emitted stream equals plain
 * greedy decoding by the same target (gemma-4-12b-coreml-iphone-practical-chat
 * card, speculative assets: the verifier, not the drafter, picks every token;
 * gemma-4-12b-it-coreml-128k card, Key numbers: identical output with
 * speculation on and off).
 * The caller continues with block[0] = emitted[a] at position pos0 + a + 1.
 * decode_step writes all n rows of the block; with R >= W + n - 1 the rows of
 * rejected drafts are never admitted by a later query and are overwritten when
 * their positions are decoded again, so one pass per block suffices
 * (Gemma-4-12B-CoreAI card, "v5/ -- ring extent R = 2W": single-pass
 * speculative verify).
 * Errors: Q4_EINVAL (null pointer), Q4_ESHAPE (n outside 1..4). */
q4_status q4_spec_accept(const int32_t* block, const int32_t* argmax, int n, int32_t* emitted,
                         int* n_emitted);

/* ------------------------------------------------------------------------ */
/* measurement                                                               */
/* ------------------------------------------------------------------------ */
/* A plain streaming read, the achievable-bandwidth reference for the
 * weight-streaming kernels: reads `bytes` (a multiple of 16) from src (device,
 * 16-byte aligned) with 16-byte loads and writes q4_stream_read_sink_words()
 * uint32 words to sink (device): word b is the XOR of the 32-bit words that
 * workgroup b read, so the XOR of all sink words is the XOR of every 32-bit
 * word of src.  Errors: Q4_EINVAL, Q4_ESHAPE, Q4_EALIGN, Q4_EHIP. */
int q4_stream_read_sink_words(void);
q4_status q4_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Destroys every captured decode-step graph.  Call before freeing buffers a
 * graph refers to if the same addresses may be reused for a different model. */
q4_status q4dec_release(void);

#ifdef __cplusplus
}
#endif
#endif /* Q4DEC_H */
