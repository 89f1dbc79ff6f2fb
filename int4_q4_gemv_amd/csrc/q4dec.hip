// q4dec.hip -- C ABI of the gfx950 int4 q4_0 decode-step library: argument
// checks, launch configuration, the decode-step launch sequence and its HIP
// graph cache.  Declarations and contracts: include/q4dec.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/q4dec.h"
#include "attn_kernels.h"
#include "gemv_kernels.h"
#include "pack_kernels.h"
#include "step_kernels.h"

using namespace q4k;

namespace {

constexpr int kMaxRows = 4;
constexpr int kFullSplits = 256;     // decode-step splits of a full layer's positions
constexpr int kTilePos = 128;        // positions per workgroup pass (4 waves x 32)

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

q4_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? Q4_OK : Q4_EHIP;
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

// ------------------------------------------------------------- GEMV plan ----
struct GemvPlan {
  int T = 0, NB = 0, CB = 0, G = 0;
  size_t partial_floats(int B) const { return (G > 1) ? (size_t)T * G * B * 64 : 0; }
};

GemvPlan gemv_plan(int T, int K) {
  GemvPlan p;
  p.T = T;
  p.NB = K / 32;
  const long want = (long)p.NB * T / 1024;     // aim for >= ~1024 waves per launch
  p.CB = want >= 16 ? 16 : (want >= 8 ? 8 : 4);
  const int C = (int)ceil_div(p.NB, p.CB);
  p.G = (int)ceil_div(C, 4);
  return p;
}

template <int B, int EPI>
void launch_gemv(const GemvArgs& a, int T, hipStream_t st) {
  const dim3 grid(T * a.G), block(256);
  if (a.CB == 16) hipLaunchKernelGGL((k_q4_gemv<B, EPI, 16>), grid, block, 0, st, a);
  else if (a.CB == 8) hipLaunchKernelGGL((k_q4_gemv<B, EPI, 8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_q4_gemv<B, EPI, 4>), grid, block, 0, st, a);
}

void fill_seg(GemvSeg& s, const void* packed, int N, int K, int tile0, int out_off) {
  const int T = (int)ceil_div(N, 64);
  const size_t code_bytes = (size_t)T * (K / 32) * 64 * 16;
  s.codes = reinterpret_cast<const u4v*>(packed);
  s.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + code_bytes);
  s.N = N;
  s.T = T;
  s.tile0 = tile0;
  s.out_off = out_off;
}

// ---------------------------------------------------------- attention plan ----
int fd_split_cap(int n_seq, int n_rows) { return std::max(8, 256 / std::max(1, n_seq * n_rows)); }

bool attn_attr_set = false;
std::mutex g_mu;

q4_status set_attn_attrs() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (attn_attr_set) return Q4_OK;
  const int sizes[4] = {64, 128, 256, 512};
  const void* fns[4] = {reinterpret_cast<const void*>(&k_fd_partial<64>),
                        reinterpret_cast<const void*>(&k_fd_partial<128>),
                        reinterpret_cast<const void*>(&k_fd_partial<256>),
                        reinterpret_cast<const void*>(&k_fd_partial<512>)};
  for (int i = 0; i < 4; i++) {
    const int bytes = 4 * 32 * (sizes[i] + 2) * 2;
    if (hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return Q4_EHIP;
  }
  attn_attr_set = true;
  return Q4_OK;
}

size_t attn_lds_bytes(int D) { return (size_t)4 * 32 * (D + 2) * 2; }

void launch_fd(const AttnArgs& a, int D, int n_seq, float* out32, uint16_t* out16, hipStream_t st) {
  const dim3 grid(a.S, a.Hkv, n_seq * a.n_rows);
  const dim3 cgrid(n_seq * a.n_rows, a.Hq);
  const size_t lds = attn_lds_bytes(D);
  switch (D) {
    case 64:
      hipLaunchKernelGGL(k_fd_partial<64>, grid, dim3(256), lds, st, a);
      hipLaunchKernelGGL(k_fd_combine<64>, cgrid, dim3(256), 0, st, a, out32, out16);
      break;
    case 128:
      hipLaunchKernelGGL(k_fd_partial<128>, grid, dim3(256), lds, st, a);
      hipLaunchKernelGGL(k_fd_combine<128>, cgrid, dim3(256), 0, st, a, out32, out16);
      break;
    case 256:
      hipLaunchKernelGGL(k_fd_partial<256>, grid, dim3(256), lds, st, a);
      hipLaunchKernelGGL(k_fd_combine<256>, cgrid, dim3(256), 0, st, a, out32, out16);
      break;
    default:
      hipLaunchKernelGGL(k_fd_partial<512>, grid, dim3(256), lds, st, a);
      hipLaunchKernelGGL(k_fd_combine<512>, cgrid, dim3(256), 0, st, a, out32, out16);
      break;
  }
}

bool valid_d(int D) { return D == 64 || D == 128 || D == 256 || D == 512; }

// ------------------------------------------------------ decode-step layout ----
struct StepLayout {
  size_t sp, cnt, best, h, x, qkv, qh, o, y, gu, a, gpart, apart, total;
  int ncnt;
  int qkv_ld, o_ld;
  int Dmax;
  GemvPlan plan_qkv_s, plan_qkv_f, plan_o_s, plan_o_f, plan_gu, plan_d;
  int S_full, S_ring;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool model_dims_ok(const q4dec_model* m) {
  if (m->hidden < 32 || m->hidden % 32 || m->hidden % 8 || m->hidden > 4096) return false;
  if (m->inter < 32 || m->inter % 32) return false;
  if (m->n_heads < 1 || m->n_heads > 16 || m->n_layers < 1 || m->vocab < 1) return false;
  if (!valid_d(m->sl_head_dim) || !valid_d(m->full_head_dim)) return false;
  if (m->sl_kv_heads < 1 || m->n_heads % m->sl_kv_heads) return false;
  if (m->n_heads / m->sl_kv_heads > 16) return false;
  if (m->sl_rot_pairs < 0 || m->sl_rot_pairs > m->sl_head_dim / 2) return false;
  if (m->full_rot_pairs < 0 || m->full_rot_pairs > m->full_head_dim / 2) return false;
  return true;
}

StepLayout step_layout(const q4dec_model* m, int n) {
  (void)n;
  StepLayout L{};
  const int H = m->hidden, I = m->inter, Hq = m->n_heads;
  const int Ds = m->sl_head_dim, Df = m->full_head_dim, Hs = m->sl_kv_heads;
  L.Dmax = std::max(Ds, Df);
  L.qkv_ld = std::max(Hq * Ds + 2 * Hs * Ds, Hq * Df + Df);
  L.o_ld = Hq * L.Dmax;
  L.plan_qkv_s = gemv_plan((int)(ceil_div(Hq * Ds, 64) + 2 * ceil_div(Hs * Ds, 64)), H);
  L.plan_qkv_f = gemv_plan((int)(ceil_div(Hq * Df, 64) + ceil_div(Df, 64)), H);
  L.plan_o_s = gemv_plan((int)ceil_div(H, 64), Hq * Ds);
  L.plan_o_f = gemv_plan((int)ceil_div(H, 64), Hq * Df);
  L.plan_gu = gemv_plan((int)(2 * ceil_div(I, 64)), H);
  L.plan_d = gemv_plan((int)ceil_div(H, 64), I);
  L.S_full = kFullSplits;
  L.S_ring = (int)std::min<long>(16, std::max<long>(1, ceil_div(m->window, kTilePos)));
  size_t gpart = 0;
  for (const GemvPlan* p : {&L.plan_qkv_s, &L.plan_qkv_f, &L.plan_o_s, &L.plan_o_f, &L.plan_gu, &L.plan_d})
    gpart = std::max(gpart, p->partial_floats(kMaxRows));
  int maxT = 0;
  for (const GemvPlan* p : {&L.plan_qkv_s, &L.plan_qkv_f, &L.plan_o_s, &L.plan_o_f, &L.plan_gu, &L.plan_d})
    maxT = std::max(maxT, p->T);
  // counters: tile counters, group counters, head counter
  L.ncnt = maxT + maxT + 8;
  const size_t apart_full = (size_t)kMaxRows * 1 * L.S_full * Hq * (Df + 4);
  const size_t apart_ring = (size_t)kMaxRows * Hs * L.S_ring * (Hq / Hs) * (Ds + 4);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.sp = take(sizeof(StepParams));
  L.cnt = take(sizeof(unsigned) * L.ncnt);
  L.best = take(sizeof(unsigned long long) * 4);
  L.h = take(sizeof(float) * kMaxRows * H);
  L.x = take(sizeof(uint16_t) * kMaxRows * std::max(H, I));
  L.qkv = take(sizeof(float) * kMaxRows * L.qkv_ld);
  L.qh = take(sizeof(uint16_t) * kMaxRows * Hq * L.Dmax);
  L.o = take(sizeof(uint16_t) * kMaxRows * L.o_ld);
  L.y = take(sizeof(float) * kMaxRows * H);
  L.gu = take(sizeof(float) * kMaxRows * 2 * I);
  L.a = take(sizeof(uint16_t) * kMaxRows * I);
  L.gpart = take(sizeof(float) * std::max<size_t>(gpart, 64));
  L.apart = take(sizeof(float) * std::max(apart_full, apart_ring));
  L.total = off;
  return L;
}

struct StepPtrs {
  StepParams* sp;
  unsigned* cnt;
  unsigned long long* best;
  float *h, *qkv, *y, *gu, *gpart, *apart;
  uint16_t *x, *qh, *o, *a;
};

StepPtrs step_ptrs(const StepLayout& L, void* ws) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  StepPtrs p;
  p.sp = reinterpret_cast<StepParams*>(b + L.sp);
  p.cnt = reinterpret_cast<unsigned*>(b + L.cnt);
  p.best = reinterpret_cast<unsigned long long*>(b + L.best);
  p.h = reinterpret_cast<float*>(b + L.h);
  p.x = reinterpret_cast<uint16_t*>(b + L.x);
  p.qkv = reinterpret_cast<float*>(b + L.qkv);
  p.qh = reinterpret_cast<uint16_t*>(b + L.qh);
  p.o = reinterpret_cast<uint16_t*>(b + L.o);
  p.y = reinterpret_cast<float*>(b + L.y);
  p.gu = reinterpret_cast<float*>(b + L.gu);
  p.a = reinterpret_cast<uint16_t*>(b + L.a);
  p.gpart = reinterpret_cast<float*>(b + L.gpart);
  p.apart = reinterpret_cast<float*>(b + L.apart);
  return p;
}

template <int B>
q4_status enqueue_layers(const q4dec_model* m, const StepLayout& L, const StepPtrs& P, int n,
                         float* logits, int32_t* argmax, hipStream_t st) {
  const int H = m->hidden, I = m->inter, Hq = m->n_heads;
  unsigned* tile_cnt = P.cnt;
  unsigned* grp_cnt = P.cnt + (L.ncnt - 8) / 2;
  unsigned* head_cnt = P.cnt + L.ncnt - 1;
  for (int l = 0; l < m->n_layers; l++) {
    const q4dec_layer& ly = m->layers[l];
    const bool full = ly.is_full != 0;
    const int D = full ? m->full_head_dim : m->sl_head_dim;
    const int Hkv = full ? 1 : m->sl_kv_heads;
    // ---- q/k/v projections; last arrival per head finishes norm, RoPE, cache write
    {
      GemvArgs a{};
      const GemvPlan& pl = full ? L.plan_qkv_f : L.plan_qkv_s;
      int t0 = 0;
      fill_seg(a.seg[0], ly.wq, Hq * D, H, t0, 0);
      t0 += a.seg[0].T;
      fill_seg(a.seg[1], ly.wk, Hkv * D, H, t0, Hq * D);
      t0 += a.seg[1].T;
      a.nseg = 2;
      if (!full) {
        fill_seg(a.seg[2], ly.wv, Hkv * D, H, t0, (Hq + Hkv) * D);
        t0 += a.seg[2].T;
        a.nseg = 3;
      }
      a.K = H; a.NB = pl.NB; a.CB = pl.CB; a.G = pl.G;
      a.x = P.x; a.ldx = H; a.y = P.qkv; a.ldy = L.qkv_ld;
      a.partial = P.gpart; a.tile_cnt = tile_cnt; a.n_rows = n;
      EpiArgs& e = a.e;
      e.sp = P.sp; e.grp_cnt = grp_cnt; e.grp_tiles = D / 64;
      e.Hq = Hq; e.Hkv = Hkv; e.D = D; e.is_full = full; e.v_norm = ly.v_norm;
      e.rot_pairs = full ? m->full_rot_pairs : m->sl_rot_pairs;
      e.R = m->ring; e.theta = full ? m->full_theta : m->sl_theta; e.eps = m->eps;
      e.q_norm = ly.q_norm; e.k_norm = ly.k_norm; e.q_out = P.qh;
      e.k_cache = ly.k_cache; e.v_cache = ly.v_cache;
      launch_gemv<B, EPI_QKV>(a, t0, st);
    }
    // ---- attention
    {
      AttnArgs a{};
      a.q = P.qh; a.k = ly.k_cache; a.v = ly.v_cache; a.seq_stride = 0;
      a.Hq = Hq; a.Hkv = Hkv; a.GQ = Hq / Hkv;
      a.ring = full ? 0 : 1; a.R = m->ring; a.W = m->window;
      a.n_rows = n; a.S = full ? L.S_full : L.S_ring;
      a.scale_log2 = (full ? m->full_scale : m->sl_scale) * 1.4426950408889634f;
      a.sp = P.sp; a.part = P.apart;
      launch_fd(a, D, 1, nullptr, P.o, st);
    }
    // ---- output projection + post-attention norm residual + pre-FF norm
    {
      GemvArgs a{};
      const GemvPlan& pl = full ? L.plan_o_f : L.plan_o_s;
      fill_seg(a.seg[0], ly.wo, H, Hq * D, 0, 0);
      a.nseg = 1;
      a.K = Hq * D; a.NB = pl.NB; a.CB = pl.CB; a.G = pl.G;
      a.x = P.o; a.ldx = Hq * D; a.y = P.y; a.ldy = H;
      a.partial = P.gpart; a.tile_cnt = tile_cnt; a.n_rows = n;
      EpiArgs& e = a.e;
      e.sp = P.sp; e.grp_cnt = grp_cnt; e.H = H; e.h = P.h; e.eps = m->eps;
      e.w_post = ly.post_attn_norm; e.w_next = ly.pre_ff_norm; e.scalar = 1.0f; e.x_out = P.x;
      launch_gemv<B, EPI_RESID>(a, a.seg[0].T, st);
    }
    // ---- gate/up with GELU(gate) * up
    {
      GemvArgs a{};
      const GemvPlan& pl = L.plan_gu;
      fill_seg(a.seg[0], ly.wg, I, H, 0, 0);
      fill_seg(a.seg[1], ly.wu, I, H, a.seg[0].T, I);
      a.nseg = 2;
      a.K = H; a.NB = pl.NB; a.CB = pl.CB; a.G = pl.G;
      a.x = P.x; a.ldx = H; a.y = P.gu; a.ldy = 2 * I;
      a.partial = P.gpart; a.tile_cnt = tile_cnt; a.n_rows = n;
      EpiArgs& e = a.e;
      e.sp = P.sp; e.grp_cnt = grp_cnt; e.inter = I; e.a_out = P.a;
      launch_gemv<B, EPI_GATEUP>(a, 2 * a.seg[0].T, st);
    }
    // ---- down projection + post-FF norm residual, layer scalar, next norm
    {
      GemvArgs a{};
      const GemvPlan& pl = L.plan_d;
      fill_seg(a.seg[0], ly.wd, H, I, 0, 0);
      a.nseg = 1;
      a.K = I; a.NB = pl.NB; a.CB = pl.CB; a.G = pl.G;
      a.x = P.a; a.ldx = I; a.y = P.y; a.ldy = H;
      a.partial = P.gpart; a.tile_cnt = tile_cnt; a.n_rows = n;
      EpiArgs& e = a.e;
      e.sp = P.sp; e.grp_cnt = grp_cnt; e.H = H; e.h = P.h; e.eps = m->eps;
      e.w_post = ly.post_ff_norm; e.scalar = ly.layer_scalar; e.x_out = P.x;
      e.w_next = (l + 1 < m->n_layers) ? m->layers[l + 1].attn_norm : m->final_norm;
      launch_gemv<B, EPI_RESID>(a, a.seg[0].T, st);
    }
  }
  // ---- tied fp16 head, softcap, argmax
  {
    HeadArgs a{};
    a.E = m->embed; a.x = P.x; a.V = m->vocab; a.H = H; a.softcap = m->softcap;
    a.logits = logits; a.best = P.best; a.cnt = head_cnt; a.argmax = argmax;
    a.sp = P.sp; a.n_rows = n;
    const int waves = 8192;
    a.rows_per_wave = (int)std::max<long>(2, ceil_div(m->vocab, waves));
    if (a.rows_per_wave & 1) a.rows_per_wave++;
    const int grid = (int)ceil_div(ceil_div(m->vocab, a.rows_per_wave), 4);
    hipLaunchKernelGGL((k_head<B>), dim3(grid), dim3(256), 0, st, a);
  }
  return launch_status();
}

q4_status check_model(const q4dec_model* m, int n, int pos0, const int32_t* tokens) {
  if (!m || !m->layers || !m->embed || !m->final_norm || !tokens) return Q4_EINVAL;
  if (n < 1 || n > kMaxRows) return Q4_ESHAPE;
  if (!model_dims_ok(m)) return Q4_ESHAPE;
  if (!al16(m->embed) || !al16(m->final_norm)) return Q4_EALIGN;
  if (pos0 < 0) return Q4_ERANGE;
  if (m->window < 1 || m->window > m->ring || m->ring < m->window + n - 1) return Q4_ERANGE;
  bool any_full = false;
  for (int l = 0; l < m->n_layers; l++) {
    const q4dec_layer& ly = m->layers[l];
    const bool full = ly.is_full != 0;
    any_full |= full;
    if (!ly.wq || !ly.wk || !ly.wo || !ly.wg || !ly.wu || !ly.wd || (!full && !ly.wv)) return Q4_EINVAL;
    if (!ly.attn_norm || !ly.q_norm || !ly.k_norm || !ly.post_attn_norm || !ly.pre_ff_norm ||
        !ly.post_ff_norm || !ly.k_cache || !ly.v_cache)
      return Q4_EINVAL;
    const void* ps[] = {ly.wq, ly.wk, ly.wo, ly.wg, ly.wu, ly.wd, ly.attn_norm, ly.q_norm, ly.k_norm,
                        ly.post_attn_norm, ly.pre_ff_norm, ly.post_ff_norm, ly.k_cache, ly.v_cache};
    for (const void* p : ps)
      if (!al16(p)) return Q4_EALIGN;
    if (!full && !al16(ly.wv)) return Q4_EALIGN;
  }
  if (any_full && (long)pos0 + n - 1 >= (long)m->full_cap) return Q4_ERANGE;
  for (int i = 0; i < n; i++)
    if (tokens[i] < 0 || tokens[i] >= m->vocab) return Q4_ERANGE;
  return Q4_OK;
}

// ----------------------------------------------------------- graph cache ----
std::map<std::string, hipGraphExec_t> g_graphs;

std::string graph_key(const q4dec_model* m, int n, const void* ws, size_t ws_bytes, const float* logits,
                      const int32_t* argmax, hipStream_t st) {
  std::string k;
  k.append(reinterpret_cast<const char*>(m), sizeof(q4dec_model));
  k.append(reinterpret_cast<const char*>(m->layers), sizeof(q4dec_layer) * m->n_layers);
  const void* extra[] = {ws, logits, argmax, st};
  k.append(reinterpret_cast<const char*>(extra), sizeof(extra));
  k.append(reinterpret_cast<const char*>(&n), sizeof(n));
  k.append(reinterpret_cast<const char*>(&ws_bytes), sizeof(ws_bytes));
  return k;
}

q4_status begin_step(const q4dec_model* m, const StepLayout& L, const StepPtrs& P, const int32_t* tokens,
                     int n, int pos0, hipStream_t st) {
  BeginArgs b{};
  b.sp = P.sp; b.pos0 = pos0; b.n = n;
  for (int i = 0; i < 4; i++) b.tokens[i] = i < n ? tokens[i] : 0;
  b.cnt = P.cnt; b.ncnt = L.ncnt; b.best = P.best;
  b.E = m->embed; b.H = m->hidden; b.emb_scale = (float)std::sqrt((double)m->hidden);
  b.h = P.h; b.w_norm = m->layers[0].attn_norm; b.eps = m->eps; b.x = P.x;
  hipLaunchKernelGGL(k_step_begin, dim3(n), dim3(256), 0, st, b);
  return launch_status();
}

q4_status decode_step_impl(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                           int32_t* argmax, void* ws, size_t ws_bytes, void* stream, bool use_graph) {
  q4_status rc = check_model(m, n, pos0, tokens);
  if (rc != Q4_OK) return rc;
  if (!ws) return Q4_EINVAL;
  if (!al16(ws) || (logits && !al16(logits))) return Q4_EALIGN;
  const StepLayout L = step_layout(m, n);
  if (ws_bytes < L.total) return Q4_ENOSPACE;
  rc = set_attn_attrs();
  if (rc != Q4_OK) return rc;
  const StepPtrs P = step_ptrs(L, ws);
  hipStream_t st = S(stream);
  rc = begin_step(m, L, P, tokens, n, pos0, st);
  if (rc != Q4_OK) return rc;
  if (!use_graph || st == nullptr) {
    return n == 1 ? enqueue_layers<1>(m, L, P, n, logits, argmax, st)
                  : enqueue_layers<4>(m, L, P, n, logits, argmax, st);
  }
  const std::string key = graph_key(m, n, ws, ws_bytes, logits, argmax, st);
  hipGraphExec_t exec = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_graphs.find(key);
    if (it != g_graphs.end()) exec = it->second;
  }
  if (!exec) {
    if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) return Q4_EHIP;
    q4_status r2 = n == 1 ? enqueue_layers<1>(m, L, P, n, logits, argmax, st)
                          : enqueue_layers<4>(m, L, P, n, logits, argmax, st);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(st, &graph);
    if (r2 != Q4_OK || e != hipSuccess || !graph) {
      if (graph) hipGraphDestroy(graph);
      return Q4_EHIP;
    }
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess) return Q4_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    g_graphs[key] = exec;
  }
  if (hipGraphLaunch(exec, st) != hipSuccess) return Q4_EHIP;
  return Q4_OK;
}

}  // namespace

// =================================================================== C ABI ==
extern "C" {

const char* q4dec_status_str(q4_status s) {
  switch (s) {
    case Q4_OK: return "Q4_OK";
    case Q4_EINVAL: return "Q4_EINVAL: null pointer or invalid enum";
    case Q4_ESHAPE: return "Q4_ESHAPE: unsupported or inconsistent sizes";
    case Q4_EALIGN: return "Q4_EALIGN: device pointer not 16-byte aligned";
    case Q4_ERANGE: return "Q4_ERANGE: position, capacity or window out of range";
    case Q4_ENOSPACE: return "Q4_ENOSPACE: buffer or workspace too small";
    case Q4_EHIP: return "Q4_EHIP: HIP runtime call or kernel launch failed";
    default: return "unknown q4dec status";
  }
}

const char* q4dec_version(void) { return "q4dec 0.1 gfx950"; }

size_t q4_packed_bytes(int N, int K) {
  if (N < 1 || K < 32 || K % 32) return 0;
  return (size_t)ceil_div(N, 64) * 64 * (K / 32) * 18;
}

q4_status q4_pack(const void* w, int w_dtype, int N, int K, void* packed, size_t packed_bytes,
                  int32_t* nonfinite, void* stream) {
  if (!w || !packed) return Q4_EINVAL;
  if (w_dtype != Q4_F32 && w_dtype != Q4_BF16) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32) return Q4_ESHAPE;
  if (packed_bytes < q4_packed_bytes(N, K)) return Q4_ENOSPACE;
  if (!al16(w) || !al16(packed)) return Q4_EALIGN;
  const int T = (int)ceil_div(N, 64);
  const long total = (long)T * (K / 32) * 64;
  const size_t code_bytes = (size_t)total * 16;
  u4v* codes = static_cast<u4v*>(packed);
  uint16_t* scales = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(packed) + code_bytes);
  const dim3 grid((unsigned)ceil_div(total, 256));
  if (w_dtype == Q4_F32)
    hipLaunchKernelGGL(k_q4_pack<0>, grid, dim3(256), 0, S(stream), w, N, K, codes, scales, T, nonfinite);
  else
    hipLaunchKernelGGL(k_q4_pack<1>, grid, dim3(256), 0, S(stream), w, N, K, codes, scales, T, nonfinite);
  return launch_status();
}

q4_status q4_unpack(const void* packed, int N, int K, uint8_t* blocks, void* stream) {
  if (!packed || !blocks) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32) return Q4_ESHAPE;
  if (!al16(packed)) return Q4_EALIGN;
  const int T = (int)ceil_div(N, 64);
  const size_t code_bytes = (size_t)T * (K / 32) * 64 * 16;
  const u4v* codes = static_cast<const u4v*>(packed);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + code_bytes);
  const long total = (long)N * (K / 32);
  hipLaunchKernelGGL(k_q4_unpack, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, S(stream), codes,
                     scales, N, K, blocks);
  return launch_status();
}

size_t q4_gemv_workspace_size(int N, int K, int B) {
  if (N < 1 || K < 32 || K % 32 || B < 1 || B > kMaxRows) return 0;
  const GemvPlan p = gemv_plan((int)ceil_div(N, 64), K);
  const size_t cnt = align256(sizeof(unsigned) * p.T);
  return cnt + align256(sizeof(float) * std::max<size_t>(64, p.partial_floats(B == 1 ? 1 : 4)));
}

q4_status q4_gemv(const void* packed, int N, int K, const uint16_t* x, int B, float* y, void* ws,
                  size_t ws_bytes, void* stream) {
  if (!packed || !x || !y || !ws) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32 || B < 1 || B > kMaxRows) return Q4_ESHAPE;
  if (ws_bytes < q4_gemv_workspace_size(N, K, B)) return Q4_ENOSPACE;
  if (!al16(packed) || !al16(x) || !al16(y) || !al16(ws)) return Q4_EALIGN;
  const GemvPlan p = gemv_plan((int)ceil_div(N, 64), K);
  GemvArgs a{};
  fill_seg(a.seg[0], packed, N, K, 0, 0);
  a.nseg = 1;
  a.K = K; a.NB = p.NB; a.CB = p.CB; a.G = p.G;
  a.x = x; a.ldx = K; a.y = y; a.ldy = N; a.n_rows = B;
  a.tile_cnt = static_cast<unsigned*>(ws);
  a.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256(sizeof(unsigned) * p.T));
  if (B == 1) launch_gemv<1, EPI_STORE>(a, p.T, S(stream));
  else launch_gemv<4, EPI_STORE>(a, p.T, S(stream));
  return launch_status();
}

size_t flash_decode_workspace_size(int n_seq, int n_rows, int Hq, int D) {
  if (n_seq < 1 || n_seq > 64 || n_rows < 1 || n_rows > kMaxRows || Hq < 1 || !valid_d(D)) return 0;
  return (size_t)n_seq * n_rows * Hq * fd_split_cap(n_seq, n_rows) * (D + 4) * sizeof(float);
}

static q4_status fd_common(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride,
                           int Hq, int Hkv, int D, const int32_t* pos0, int n_seq, int n_rows,
                           float* out, void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !pos0 || !out || !ws) return Q4_EINVAL;
  if (n_seq < 1 || n_seq > 64 || n_rows < 1 || n_rows > kMaxRows) return Q4_ESHAPE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || Hq / Hkv > 16 || !valid_d(D) || seq_stride < 0) return Q4_ESHAPE;
  if (n_seq > 1 && seq_stride == 0) return Q4_ESHAPE;
  if (ws_bytes < flash_decode_workspace_size(n_seq, n_rows, Hq, D)) return Q4_ENOSPACE;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(out) || !al16(ws) || (seq_stride * 2) % 16) return Q4_EALIGN;
  return Q4_OK;
}

q4_status flash_decode_full(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride,
                            int cap, int Hq, int D, const int32_t* pos0, int n_seq, int n_rows, float scale,
                            float* out, void* ws, size_t ws_bytes, void* stream) {
  q4_status rc = fd_common(q, k, v, seq_stride, Hq, 1, D, pos0, n_seq, n_rows, out, ws, ws_bytes);
  if (rc != Q4_OK) return rc;
  if (cap < 1) return Q4_ESHAPE;
  if (n_seq > 1 && seq_stride < (int64_t)cap * D) return Q4_ESHAPE;
  long maxlen = 1;
  for (int s = 0; s < n_seq; s++) {
    if (pos0[s] < 0 || (long)pos0[s] + n_rows - 1 >= cap) return Q4_ERANGE;
    maxlen = std::max(maxlen, (long)pos0[s] + n_rows);
  }
  rc = set_attn_attrs();
  if (rc != Q4_OK) return rc;
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.seq_stride = seq_stride;
  a.Hq = Hq; a.Hkv = 1; a.GQ = Hq; a.ring = 0; a.R = cap; a.W = cap;
  a.n_rows = n_rows;
  a.S = (int)std::min<long>(fd_split_cap(n_seq, n_rows), std::max<long>(1, ceil_div(maxlen, kTilePos)));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sp = nullptr; a.part = static_cast<float*>(ws);
  for (int s = 0; s < n_seq; s++) a.pos0[s] = pos0[s];
  launch_fd(a, D, n_seq, out, nullptr, S(stream));
  return launch_status();
}

q4_status flash_decode_ring(const uint16_t* q, const uint16_t* k_ring, const uint16_t* v_ring,
                            int64_t seq_stride, int Hq, int Hkv, int D, int R, int W, const int32_t* pos0,
                            int n_seq, int n_rows, float scale, float* out, void* ws, size_t ws_bytes,
                            void* stream) {
  q4_status rc = fd_common(q, k_ring, v_ring, seq_stride, Hq, Hkv, D, pos0, n_seq, n_rows, out, ws, ws_bytes);
  if (rc != Q4_OK) return rc;
  if (W < 1 || R < 1 || W > R || (long)R < (long)W + n_rows - 1) return Q4_ERANGE;
  if (n_seq > 1 && seq_stride < (int64_t)Hkv * R * D) return Q4_ESHAPE;
  for (int s = 0; s < n_seq; s++)
    if (pos0[s] < 0 || (long)pos0[s] + n_rows - 1 > 0x7FFFFFFFL) return Q4_ERANGE;
  rc = set_attn_attrs();
  if (rc != Q4_OK) return rc;
  AttnArgs a{};
  a.q = q; a.k = k_ring; a.v = v_ring; a.seq_stride = seq_stride;
  a.Hq = Hq; a.Hkv = Hkv; a.GQ = Hq / Hkv; a.ring = 1; a.R = R; a.W = W;
  a.n_rows = n_rows;
  a.S = (int)std::min<long>(fd_split_cap(n_seq, n_rows), std::max<long>(1, ceil_div(W, kTilePos)));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sp = nullptr; a.part = static_cast<float*>(ws);
  for (int s = 0; s < n_seq; s++) a.pos0[s] = pos0[s];
  launch_fd(a, D, n_seq, out, nullptr, S(stream));
  return launch_status();
}

size_t decode_step_workspace_size(const q4dec_model* m, int n) {
  if (!m || n < 1 || n > kMaxRows || !model_dims_ok(m)) return 0;
  return step_layout(m, n).total;
}

q4_status decode_step(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                      int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(m, tokens, n, pos0, logits, argmax, ws, ws_bytes, stream, true);
}

q4_status decode_step_eager(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                            int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(m, tokens, n, pos0, logits, argmax, ws, ws_bytes, stream, false);
}

q4_status q4dec_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  q4_status rc = Q4_OK;
  for (auto& kv : g_graphs)
    if (hipGraphExecDestroy(kv.second) != hipSuccess) rc = Q4_EHIP;
  g_graphs.clear();
  return rc;
}

}  // extern "C"
