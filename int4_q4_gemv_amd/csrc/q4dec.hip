// q4dec.hip -- C ABI of the gfx950 int4 q4_0 decode-step library: argument
// checks, launch configuration, the decode-step launch sequence and its HIP
// graph cache.  Declarations and contracts: include/q4dec.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/q4dec.h"
#include "attn_kernels.h"
#include "chunk_kernels.h"
#include "gemv_kernels.h"
#include "pack_kernels.h"
#include "q8_kernels.h"
#include "step_kernels.h"

using namespace q4k;

namespace {

constexpr int kMaxRows = 4;
constexpr int kFullSplits = 256;     // decode-step splits of a full layer's positions
constexpr int kTilePos = 128;        // positions per workgroup pass (4 waves x 32)
constexpr int kMaxLds = 160 * 1024;
constexpr int kSplitCols = 4096;     // decode step: longest run of K columns per workgroup (down)
constexpr int kSplitColsO = 2048;    // decode step: the same for the output projection

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

q4_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? Q4_OK : Q4_EHIP;
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

// ------------------------------------------------------------- GEMV plan ----
// Weight formats: 0 = q4 (units of 16 rows x 128 columns), 1 = int8 (units of
// 16 rows x 64 columns); one unit is one 1 KB wave-wide load of codes.
constexpr int unit_cols(int fmt) { return fmt == 0 ? 128 : 64; }

struct GemvPlan {
  int T = 0, NQ = 0, CQ = 0, W = 0, S = 1, NQs = 0, fmt = 0;
};

// [N x K] product: S runs of K (NQs units each; S = 1 unless split_cols > 0
// caps a run), W waves per tile streaming CQ units each.  CQ is the smallest
// of 4, 8, 16 that keeps W within max_waves; W = -1 when none does.
GemvPlan gemv_plan(int N, int K, int max_waves, int split_cols = 0, int fmt = 0) {
  GemvPlan p;
  p.fmt = fmt;
  p.T = (int)ceil_div(N, 16);
  p.NQ = (int)ceil_div(K, unit_cols(fmt));
  p.S = split_cols > 0 ? (int)ceil_div(p.NQ, split_cols / unit_cols(fmt)) : 1;
  p.NQs = (int)ceil_div(p.NQ, p.S);
  p.W = -1;
  for (int cq : {4, 8, 16}) {
    const int w = (int)ceil_div(p.NQs, cq);
    if (w <= max_waves) {
      p.CQ = cq;
      p.W = w;
      break;
    }
  }
  return p;
}

size_t gemv_lds(int B, const GemvPlan& p) { return (size_t)B * (p.NQs * unit_cols(p.fmt) + (B > 1 ? 8 : 0)) * 2; }

// grid: (tiles, splits); block: a.W waves (2 a.W for EPI_GATEUP, both
// halves), as the kernel assumes
template <int B, int EPI, int FMT>
void launch_gemv_f(const GemvArgs& a, const GemvPlan& p, int tiles, size_t lds, hipStream_t st) {
  const dim3 g(tiles, p.S), blk(64 * (EPI == EPI_GATEUP ? 2 * a.W : a.W));
  if (p.CQ == 16) hipLaunchKernelGGL((k_q4_gemv<B, EPI, 16, FMT>), g, blk, lds, st, a);
  else if (p.CQ == 8) hipLaunchKernelGGL((k_q4_gemv<B, EPI, 8, FMT>), g, blk, lds, st, a);
  else hipLaunchKernelGGL((k_q4_gemv<B, EPI, 4, FMT>), g, blk, lds, st, a);
}

template <int B, int EPI>
void launch_gemv(const GemvArgs& a, const GemvPlan& p, int tiles, size_t lds, hipStream_t st) {
  if (p.fmt == 0) launch_gemv_f<B, EPI, 0>(a, p, tiles, lds, st);
  else launch_gemv_f<B, EPI, 1>(a, p, tiles, lds, st);
}

void fill_seg(GemvSeg& s, const void* packed, int N, int K, int tile0, int out_off, int fmt = 0) {
  const int T = (int)ceil_div(N, 16);
  const size_t code_bytes = (size_t)T * ceil_div(K, unit_cols(fmt)) * 64 * 16;
  s.codes = reinterpret_cast<const u4v*>(packed);
  s.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + code_bytes);
  s.N = N;
  s.T = T;
  s.tile0 = tile0;
  s.out_off = out_off;
}

// ---------------------------------------------------------- attention plan ----
int fd_split_cap(int n_seq, int n_rows) { return std::max(8, 256 / std::max(1, n_seq * n_rows)); }

bool attrs_set = false;
std::mutex g_mu;

template <typename F>
hipError_t max_lds(F* fn, int bytes = kMaxLds - 8 * 1024) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int B, int FMT>
hipError_t gemv_attrs() {
  hipError_t e = hipSuccess;
  e = e != hipSuccess ? e : max_lds(&k_q4_gemv<B, EPI_STORE, 4, FMT>);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemv<B, EPI_STORE, 8, FMT>);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemv<B, EPI_STORE, 16, FMT>);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemv<B, EPI_GATEUP, 4, FMT>);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemv<B, EPI_GATEUP, 8, FMT>);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemv<B, EPI_GATEUP, 16, FMT>);
  return e;
}

q4_status set_attrs() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (attrs_set) return Q4_OK;
  hipError_t e = hipSuccess;
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<64>, (int)fd_lds_bytes<64>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<128>, (int)fd_lds_bytes<128>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<256>, (int)fd_lds_bytes<256>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<512>, (int)fd_lds_bytes<512>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<128, true>, (int)fd_lds_bytes<128>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<512, true>, (int)fd_lds_bytes<512>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<64, false, true>, (int)fd_lds_bytes<64>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<128, false, true>, (int)fd_lds_bytes<128>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<256, false, true>, (int)fd_lds_bytes<256>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<512, false, true>, (int)fd_lds_bytes<512>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<128, true, true>, (int)fd_lds_bytes<128>());
  e = e != hipSuccess ? e : max_lds(&k_fd_partial<512, true, true>, (int)fd_lds_bytes<512>());
  e = e != hipSuccess ? e : max_lds(&k_q4_gemm<EPI_STORE, 1, kChunkRunQ>, (int)kGemmLds);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemm<EPI_STORE, 2, kChunkRunQ>, (int)kGemmLds);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemm<EPI_GATEUP, 1, kChunkRunQ>, (int)kGemmLds);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemm<EPI_STORE, 1, kGemmRunQ>, (int)kGemmLds);
  e = e != hipSuccess ? e : max_lds(&k_q4_gemm<EPI_STORE, 2, kGemmRunQ>, (int)kGemmLds);
  e = e != hipSuccess ? e : gemv_attrs<1, 0>();
  e = e != hipSuccess ? e : gemv_attrs<4, 0>();
  e = e != hipSuccess ? e : gemv_attrs<1, 1>();
  e = e != hipSuccess ? e : gemv_attrs<4, 1>();
  if (e != hipSuccess) return Q4_EHIP;
  attrs_set = true;
  return Q4_OK;
}

// tail: rows of a block past each group's first (ring splits of several rows
// per workgroup, S <= 32); h16: records holding O / l in fp16 (the full
// layers' kernels)
template <int D>
void launch_combine(const AttnArgs& a, int n_seq, float* out32, uint16_t* out16, hipStream_t st, bool tail = false,
                    bool h16 = false) {
  const dim3 cgrid(a.Hkv, a.GQ, n_seq * a.n_rows * (D / 64));  // 256 threads each
  if (h16 && a.S <= 32) hipLaunchKernelGGL((k_fd_combine<D, 32, false, true>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (h16 && a.S <= 64) hipLaunchKernelGGL((k_fd_combine<D, 64, false, true>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (h16) hipLaunchKernelGGL((k_fd_combine<D, kMaxSplits, false, true>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (tail && a.S <= 16) hipLaunchKernelGGL((k_fd_combine<D, 16, true>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (tail) hipLaunchKernelGGL((k_fd_combine<D, 32, true>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (a.S <= 16) hipLaunchKernelGGL((k_fd_combine<D, 16>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (a.S <= 32) hipLaunchKernelGGL((k_fd_combine<D, 32>), cgrid, dim3(256), 0, st, out32, out16, a);
  else if (a.S <= 64) hipLaunchKernelGGL((k_fd_combine<D, 64>), cgrid, dim3(256), 0, st, out32, out16, a);
  else hipLaunchKernelGGL((k_fd_combine<D, kMaxSplits>), cgrid, dim3(256), 0, st, out32, out16, a);
}

template <int D>
void launch_fd_d(const AttnArgs& a, int n_seq, float* out32, uint16_t* out16, hipStream_t st) {
  const int rpw = a.rpw > 1 ? a.rpw : 1;
  const dim3 grid(a.kvh_major ? a.Hkv : a.S, a.kvh_major ? a.S : a.Hkv, n_seq * (int)ceil_div(a.n_rows, rpw));
  // without the finishing prologue only the V rows (which also hold the
  // merge buffer) are used: a smaller allocation lets more workgroups share a CU
  const size_t lds = (a.fin_on || a.vrow) ? fd_lds_bytes<D>() : fd_lds_vbytes<D>();   // VR parks q lo parts
  const bool mr = rpw > 1;
  if constexpr (D == 128 || D == 512) {
    if (a.vrow && mr) hipLaunchKernelGGL((k_fd_partial<D, true, true>), grid, dim3(256), lds, st, a);
    else if (a.vrow) hipLaunchKernelGGL((k_fd_partial<D, true>), grid, dim3(256), lds, st, a);
    else if (mr) hipLaunchKernelGGL((k_fd_partial<D, false, true>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((k_fd_partial<D, false>), grid, dim3(256), lds, st, a);
  } else {
    if (mr) hipLaunchKernelGGL((k_fd_partial<D, false, true>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((k_fd_partial<D, false>), grid, dim3(256), lds, st, a);
  }
  launch_combine<D>(a, n_seq, out32, out16, st);
}

// Compute units of the current device (queried once per device).
int num_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// k_head's grid: as many workgroups of 4 waves as are resident at once
// (per_cu of them per CU: 4 at batch 1, 2 at batch 4, by the kernel's
// registers), so that none starts after the first have finished; each wave
// takes two rows per iteration
int head_grid(long vocab, int per_cu) {
  return (int)std::min<long>(std::min<long>((long)num_cus() * per_cu, ceil_div(vocab, 8)), kHeadSlots);
}

// The chunk's full layers: 4 rows per workgroup over shared K/V tiles, then
// the combine.
template <int D>
void launch_rows4_d(const AttnArgs& a, int n_seq, uint16_t* out16, hipStream_t st) {
  const dim3 grid(a.S, a.Hkv, n_seq * (int)ceil_div(a.n_rows, 4));
  // two tile buffers while the grid fits one workgroup per CU, else one (two
  // workgroups per CU); static LDS only
  if ((long)grid.x * grid.y * grid.z <= num_cus()) hipLaunchKernelGGL((k_fd_rows4<D, 2>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_fd_rows4<D, 1>), grid, dim3(256), 0, st, a);
  launch_combine<D>(a, n_seq, nullptr, out16, st, false, true);
}

void launch_rows4(const AttnArgs& a, int D, int n_seq, uint16_t* out16, hipStream_t st) {
  switch (D) {
    case 128: launch_rows4_d<128>(a, n_seq, out16, st); break;
    case 256: launch_rows4_d<256>(a, n_seq, out16, st); break;
    default: launch_rows4_d<512>(a, n_seq, out16, st); break;
  }
}

// Ring layers whose splits hold at most one tile, one row per workgroup:
// the head dimension dealt to the 4 waves of a workgroup.
// With several rows per workgroup (a.rpw > 1) their columns share the tile.
template <int D>
void launch_ring_ds_d(const AttnArgs& a, int n_seq, float* out32, uint16_t* out16, hipStream_t st) {
  const int rpw = a.rpw > 1 ? a.rpw : 1;
  const dim3 grid(a.kvh_major ? a.Hkv : a.S, a.kvh_major ? a.S : a.Hkv, n_seq * (int)ceil_div(a.n_rows, rpw));
  const size_t lds = 0;                       // static LDS only
  if (rpw > 1) hipLaunchKernelGGL((k_fd_ring_ds<D, true, true>), grid, dim3(256), lds, st, a);
  else if (a.fin_on) hipLaunchKernelGGL((k_fd_ring_ds<D, false, true>), grid, dim3(256), lds, st, a);
  else hipLaunchKernelGGL((k_fd_ring_ds<D, false, false>), grid, dim3(256), lds, st, a);
  launch_combine<D>(a, n_seq, out32, out16, st, rpw > 1);
}

// every split holds at most one tile of the first row's window.  Several
// rows per workgroup: with the finishing prologue and its query export (the
// combine adds each row's positions past the first row's from the cache),
// one sequence, at most 32 splits and kMaxTail rows past a group's first.
bool ring_ds_ok(const AttnArgs& a, int D) {
  return a.ring && D >= 128 && (long)a.S * 32 >= a.W && !a.vrow &&
         (a.rpw <= 1 || (a.fin_on && a.fin.q_out && a.GQ * a.rpw <= 16 && a.S <= 32 &&
                         std::min(a.rpw, a.n_rows) - 1 <= kMaxTail));
}

// Full layers, one row per workgroup: 8 waves, the head dimension dealt
// to the waves of each 4-wave group.
template <int D>
void launch_full_ds_d(const AttnArgs& a, int n_seq, float* out32, uint16_t* out16, hipStream_t st) {
  const dim3 grid(a.S, a.Hkv, n_seq * a.n_rows);
  if (a.vrow) hipLaunchKernelGGL((k_fd_full_ds<D, true>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((k_fd_full_ds<D, false>), grid, dim3(512), 0, st, a);
  launch_combine<D>(a, n_seq, out32, out16, st, false, true);
}

bool full_ds_ok(const AttnArgs& a, int D) { return !a.ring && (D == 256 || D == 512) && a.rpw <= 1; }

// Split-K partials then the combine (S <= kMaxSplits).
void launch_fd(const AttnArgs& a, int D, int n_seq, float* out32, uint16_t* out16, hipStream_t st) {
  if (full_ds_ok(a, D)) {
    if (D == 256) launch_full_ds_d<256>(a, n_seq, out32, out16, st);
    else launch_full_ds_d<512>(a, n_seq, out32, out16, st);
    return;
  }
  if (ring_ds_ok(a, D)) {
    switch (D) {
      case 128: launch_ring_ds_d<128>(a, n_seq, out32, out16, st); break;
      case 256: launch_ring_ds_d<256>(a, n_seq, out32, out16, st); break;
      default: launch_ring_ds_d<512>(a, n_seq, out32, out16, st); break;
    }
    return;
  }
  switch (D) {
    case 64: launch_fd_d<64>(a, n_seq, out32, out16, st); break;
    case 128: launch_fd_d<128>(a, n_seq, out32, out16, st); break;
    case 256: launch_fd_d<256>(a, n_seq, out32, out16, st); break;
    default: launch_fd_d<512>(a, n_seq, out32, out16, st); break;
  }
}

bool valid_d(int D) { return D == 64 || D == 128 || D == 256 || D == 512; }

// ------------------------------------------------------ decode-step layout ----
struct StepLayout {
  size_t sp, best, rope, hA, hB, qkv, q16, o, y, a, xf, xf2, xh, apart, total;
  int qkv_ld, o_ld;
  int Dmax;
  GemvPlan p_qkv_s, p_qkv_f, p_o_s, p_o_f, p_gu, p_d;
  int ymax;       // largest split count of a product that writes y
  int S_full, S_ring;
  int S_ring4;    // ring splits of a 4-row verify block (one 32-position tile each)
  bool ok;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// head sizes and rotations a one-row-per-position full layer supports
bool vrow_dims_ok(int D, int rot_pairs) {
  if (D == 128) return rot_pairs >= 0 && rot_pairs <= vr_max_rot<128>();
  if (D == 512) return rot_pairs >= 0 && rot_pairs <= vr_max_rot<512>();
  return false;
}

bool model_dims_ok(const q4dec_model* m) {
  if (m->hidden < 32 || m->hidden % 32 || m->hidden > 4096) return false;
  if (m->inter < 32 || m->inter % 32) return false;
  if (m->n_heads < 1 || m->n_heads > 16 || m->n_layers < 1 || m->vocab < 1) return false;
  if (!valid_d(m->sl_head_dim) || !valid_d(m->full_head_dim)) return false;
  if (m->sl_kv_heads < 1 || m->n_heads % m->sl_kv_heads) return false;
  if (m->n_heads / m->sl_kv_heads > 16) return false;
  if (m->sl_rot_pairs < 0 || m->sl_rot_pairs > m->sl_head_dim / 2) return false;
  if (m->full_rot_pairs < 0 || m->full_rot_pairs > m->full_head_dim / 2) return false;
  if (m->ring < 32) return false;   // a tile's 32 positions wrap the ring at most once
  if (m->weight_format != 0 && m->weight_format != 1) return false;
  if (m->kv_format != 0 && m->kv_format != 1) return false;
  if (m->kv_format == 1 && !vrow_dims_ok(m->full_head_dim, m->full_rot_pairs)) return false;
  return true;
}

StepLayout step_layout(const q4dec_model* m) {
  StepLayout L{};
  const int H = m->hidden, I = m->inter, Hq = m->n_heads;
  const int Ds = m->sl_head_dim, Df = m->full_head_dim, Hs = m->sl_kv_heads;
  L.Dmax = std::max(Ds, Df);
  L.qkv_ld = std::max(Hq * Ds + 2 * Hs * Ds, Hq * Df + Df);
  L.o_ld = Hq * L.Dmax;
  // Products whose K is long are split so that each has enough workgroups;
  // gate/up keeps K whole (its epilogue needs both full sums).
  const int fmt = m->weight_format;
  L.p_qkv_s = gemv_plan(Hq * Ds + 2 * Hs * Ds, H, 8, 0, fmt);
  L.p_qkv_f = gemv_plan(Hq * Df + Df, H, 8, 0, fmt);
  L.p_o_s = gemv_plan(H, Hq * Ds, 8, kSplitColsO, fmt);
  L.p_o_f = gemv_plan(H, Hq * Df, 8, kSplitColsO, fmt);
  L.p_gu = gemv_plan(I, H, 4, 0, fmt);
  L.p_d = gemv_plan(H, I, 8, kSplitCols, fmt);
  L.ymax = std::max(std::max(L.p_o_s.S, L.p_o_f.S), L.p_d.S);
  L.ok = true;
  for (const GemvPlan* p : {&L.p_qkv_s, &L.p_qkv_f, &L.p_o_s, &L.p_o_f, &L.p_gu, &L.p_d})
    if (p->W < 1 || gemv_lds(kMaxRows, *p) > (size_t)kMaxLds - 8 * 1024) L.ok = false;
  if (L.p_gu.S != 1 || L.ymax > 4) L.ok = false;
  L.S_full = kFullSplits;
  L.S_ring = (int)std::min<long>(32, std::max<long>(1, ceil_div(m->window, 32)));
  L.S_ring4 = (int)std::min<long>(64, std::max<long>(1, ceil_div(m->window + kMaxRows - 1, 32)));
  const size_t apart_full = (size_t)kMaxRows * 1 * L.S_full * Hq * (Df + 4);
  const size_t apart_ring = (size_t)kMaxRows * Hs * std::max(L.S_ring, L.S_ring4) * (Hq / Hs) * (Ds + 4);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.sp = take(sizeof(StepParams));
  L.best = take(sizeof(unsigned long long) * 4 * kHeadSlots);   // the head's per-workgroup slots
  L.rope = take(sizeof(float2) * kMaxRows * (Ds / 2 + Df / 2));
  L.hA = take(sizeof(float) * kMaxRows * H);
  L.hB = take(sizeof(float) * kMaxRows * H);
  L.qkv = take(sizeof(float) * kMaxRows * L.qkv_ld);
  L.q16 = take(sizeof(uint16_t) * kMaxRows * L.o_ld);
  L.o = take(sizeof(uint16_t) * kMaxRows * L.o_ld);
  L.y = take(sizeof(float) * L.ymax * kMaxRows * H);
  L.a = take(sizeof(uint16_t) * kMaxRows * I);
  L.xf = take(sizeof(uint16_t) * kMaxRows * H);
  L.xf2 = take(sizeof(uint16_t) * kMaxRows * H);
  L.xh = take(sizeof(uint16_t) * kMaxRows * H);
  L.apart = take(sizeof(float) * std::max(apart_full, apart_ring));
  L.total = off;
  return L;
}

struct StepPtrs {
  StepParams* sp;
  unsigned long long* best;
  float2* rope;
  float *hA, *hB, *qkv, *y, *apart;
  uint16_t *q16, *o, *a, *xf, *xf2, *xh;
};

StepPtrs step_ptrs(const StepLayout& L, void* ws) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  StepPtrs p;
  p.sp = reinterpret_cast<StepParams*>(b + L.sp);
  p.best = reinterpret_cast<unsigned long long*>(b + L.best);
  p.rope = reinterpret_cast<float2*>(b + L.rope);
  p.hA = reinterpret_cast<float*>(b + L.hA);
  p.hB = reinterpret_cast<float*>(b + L.hB);
  p.qkv = reinterpret_cast<float*>(b + L.qkv);
  p.q16 = reinterpret_cast<uint16_t*>(b + L.q16);
  p.o = reinterpret_cast<uint16_t*>(b + L.o);
  p.y = reinterpret_cast<float*>(b + L.y);
  p.a = reinterpret_cast<uint16_t*>(b + L.a);
  p.xf = reinterpret_cast<uint16_t*>(b + L.xf);
  p.xf2 = reinterpret_cast<uint16_t*>(b + L.xf2);
  p.xh = reinterpret_cast<uint16_t*>(b + L.xh);
  p.apart = reinterpret_cast<float*>(b + L.apart);
  return p;
}

// Attention of a block of rows that the one-launch path does not take: every
// row finished first (queries to q16, K/V rows into the caches), then the
// rows' attention over the caches, sharing K/V tiles.
void enqueue_chunk_attn(const q4dec_model* m, const StepLayout& L, const StepPtrs& P, const q4dec_layer& ly, int n,
                        bool full, int D, int Hkv, bool vrow, const float2* rope_l, int cs_ld, hipStream_t st) {
  const int Hq = m->n_heads;
  {
    ChunkFinArgs f{};
    f.qkv = P.qkv; f.ldq = L.qkv_ld; f.ny = 1; f.y_split = 0;
    f.Hq = Hq; f.Hkv = Hkv; f.ring = full ? 0 : 1; f.R = m->ring;
    f.v_norm = ly.v_norm; f.vrow = vrow ? 1 : 0;
    f.q_norm = ly.q_norm; f.k_norm = ly.k_norm;
    f.theta = full ? m->full_theta : m->sl_theta;
    f.rot_pairs = full ? m->full_rot_pairs : m->sl_rot_pairs;
    f.eps = m->eps; f.pos0 = 0; f.sp = P.sp; f.rope_cs = rope_l; f.cs_ld = cs_ld;
    f.q16 = P.q16; f.kc = ly.k_cache; f.vc = ly.v_cache;
    const dim3 grid(n, Hq + 2 * Hkv);
    switch (D) {
      case 64: hipLaunchKernelGGL(k_chunk_finish<64>, grid, dim3(64), 0, st, f); break;
      case 128: hipLaunchKernelGGL(k_chunk_finish<128>, grid, dim3(64), 0, st, f); break;
      case 256: hipLaunchKernelGGL(k_chunk_finish<256>, grid, dim3(64), 0, st, f); break;
      default: hipLaunchKernelGGL(k_chunk_finish<512>, grid, dim3(64), 0, st, f); break;
    }
  }
  // then the rows' attention over the caches, sharing K/V tiles
  AttnArgs a{};
  a.q = P.q16; a.k = ly.k_cache; a.v = ly.v_cache; a.seq_stride = 0;
  a.Hq = Hq; a.Hkv = Hkv; a.GQ = Hq / Hkv;
  a.ring = full ? 0 : 1; a.R = m->ring; a.W = m->window;
  a.n_rows = n; a.S = full ? L.S_full : L.S_ring4;
  a.scale_log2 = (full ? m->full_scale : m->sl_scale) * 1.4426950408889634f;
  a.sp = P.sp; a.part = P.apart;
  a.fin_on = 0;
  a.kvh_major = full ? 0 : 1;
  if (vrow) {
    a.vrow = 1; a.k = ly.v_cache; a.kw = ly.k_norm; a.theta = m->full_theta; a.krot = m->full_rot_pairs;
  }
  a.rpw = 16 % a.GQ == 0 ? 16 / a.GQ : 1;
  if (a.rpw <= 1 && !vrow && full && D >= 128) launch_rows4(a, D, 1, P.o, st);
  else launch_fd(a, D, 1, nullptr, P.o, st);
}

// Launch sequence of one step (every kernel reads positions, the row count
// and the output pointers from the device-side StepParams, so the sequence is
// position- and output-free):
// per layer: input RMSNorm of the residual stream (with the previous layer's
// post-FF residual), q/k/v projections, attention, combine, output
// projection, post-attention residual and pre-FF norm, gate/up with GELU *
// up, down projection; then the final norm, the tied head and the argmax
// read-out.  Attention of one row finishes q/k/v in the partial kernel's
// prologue.  The rows of a width-4 verify block share each K/V tile, so the
// block reads each cached position once (Gemma-4-12B-CoreAI card, "v5/ --
// ring extent R = 2W": one pass per block; gemma-4-E4B-CoreAI card, ring3/:
// the GQA fold): on a ring layer as MFMA columns of one workgroup ((row,
// query head) pairs) of the head-dimension-split kernel, which also finishes
// the rows, the combine adding each row's positions past the first row's;
// on a full layer every row is finished first in its own launch (queries to
// q16, K/V rows into the cache), then the 4-row kernel (one wave per row
// over tiles staged once in LDS) reads them.
// Buffers: x of attention (xf), of the MLP (xf2) and of the head (xh) are
// kept apart, so after a step the workspace holds the last layer's stages.
// gemvs_only: only the q/k/v, output and down products (the step's most
// launched kernel in its step launch configuration, for measurement).
template <int B>
q4_status enqueue_layers(const q4dec_model* m, const StepLayout& L, const StepPtrs& P, int n, hipStream_t st,
                         bool gemvs_only = false) {
  const int H = m->hidden, I = m->inter, Hq = m->n_heads;
  const int fmt = m->weight_format;
  for (int l = 0; l < m->n_layers; l++) {
    const q4dec_layer& ly = m->layers[l];
    const bool full = ly.is_full != 0;
    const int D = full ? m->full_head_dim : m->sl_head_dim;
    const int Hkv = full ? 1 : m->sl_kv_heads;
    // ---- q/k/v projections
    {
      GemvArgs a{};
      const GemvPlan& pl = full ? L.p_qkv_f : L.p_qkv_s;
      int t0 = 0;
      fill_seg(a.seg[0], ly.wq, Hq * D, H, t0, 0, fmt);
      t0 += a.seg[0].T;
      fill_seg(a.seg[1], ly.wk, Hkv * D, H, t0, Hq * D, fmt);
      t0 += a.seg[1].T;
      a.nseg = 2;
      if (!full) {
        fill_seg(a.seg[2], ly.wv, Hkv * D, H, t0, (Hq + Hkv) * D, fmt);
        t0 += a.seg[2].T;
        a.nseg = 3;
      }
      NormIn ni{};
      if (l == 0) { ni.h_src = P.hA; ni.y = nullptr; ni.w_post = nullptr; ni.scalar = 1.0f; ni.h_dst = nullptr; }
      else {
        const q4dec_layer& prev = m->layers[l - 1];
        ni.h_src = P.hB; ni.y = P.y; ni.w_post = prev.post_ff_norm; ni.scalar = prev.layer_scalar; ni.h_dst = P.hA;
        ni.ny = L.p_d.S; ni.y_split = (long)n * H;
      }
      ni.w_in = ly.attn_norm; ni.H = H; ni.eps = m->eps;
      if (!gemvs_only) hipLaunchKernelGGL(k_norm_rows<4>, dim3(n), dim3(512), 0, st, ni, P.xf);
      a.K = H; a.NQ = pl.NQ; a.W = pl.W; a.NQs = pl.NQs;
      a.x = P.xf; a.ldx = H;
      a.y = P.qkv; a.ldy = L.qkv_ld; a.n_rows = n;
      launch_gemv<B, EPI_STORE>(a, pl, t0, gemv_lds(B, pl), st);
    }
    // ---- attention: q/k/v finishing, split-K partials, combine
    const bool vrow = full && m->kv_format == 1;
    const float2* rope_l = full ? P.rope + m->sl_head_dim / 2 : P.rope;
    const int cs_ld = m->sl_head_dim / 2 + m->full_head_dim / 2;
    if (gemvs_only) {
      // attention skipped
    } else {
      // rows finished inside the attention kernels: each workgroup forms the
      // queries of its columns and the K/V rows of this step in its range, and
      // stores each of its rows whose position lies there
      AttnArgs a{};
      a.q = nullptr; a.k = ly.k_cache; a.v = ly.v_cache; a.seq_stride = 0;
      a.Hq = Hq; a.Hkv = Hkv; a.GQ = Hq / Hkv;
      a.ring = full ? 0 : 1; a.R = m->ring; a.W = m->window;
      a.n_rows = n; a.S = full ? L.S_full : L.S_ring;
      a.scale_log2 = (full ? m->full_scale : m->sl_scale) * 1.4426950408889634f;
      a.sp = P.sp; a.part = P.apart;
      a.fin_on = 1;
      a.kvh_major = full ? 0 : 1;
      if (vrow) {
        a.vrow = 1; a.k = ly.v_cache; a.kw = ly.k_norm; a.theta = m->full_theta; a.krot = m->full_rot_pairs;
      }
      a.fin.qkv = P.qkv; a.fin.ldq = L.qkv_ld; a.fin.q_norm = ly.q_norm; a.fin.k_norm = ly.k_norm;
      a.fin.v_norm = ly.v_norm; a.fin.rot_pairs = full ? m->full_rot_pairs : m->sl_rot_pairs;
      a.fin.rope_cs = rope_l; a.fin.cs_ld = cs_ld; a.fin.eps = m->eps;
      a.fin.q_out = P.q16;
      // a block of rows: on a ring layer their columns share each tile of one
      // workgroup (16 / GQ rows); elsewhere every row is finished first
      if (B > 1) a.rpw = 16 % a.GQ == 0 ? 16 / a.GQ : 1;
      if (B == 1 || (!full && a.rpw > 1 && ring_ds_ok(a, D))) launch_fd(a, D, 1, nullptr, P.o, st);
      else enqueue_chunk_attn(m, L, P, ly, n, full, D, Hkv, vrow, rope_l, cs_ld, st);
    }
    // ---- output projection
    {
      GemvArgs a{};
      const GemvPlan& pl = full ? L.p_o_f : L.p_o_s;
      fill_seg(a.seg[0], ly.wo, H, Hq * D, 0, 0, fmt);
      a.nseg = 1;
      a.K = Hq * D; a.NQ = pl.NQ; a.W = pl.W; a.NQs = pl.NQs;
      a.x = P.o; a.ldx = Hq * D;
      a.y = P.y; a.ldy = H; a.y_split = (long)n * H; a.n_rows = n;
      a.ra0 = reinterpret_cast<const float4*>(ly.post_attn_norm);   // read by the next norm
      a.ra1 = reinterpret_cast<const float4*>(ly.pre_ff_norm);
      a.ra_n = H / 4;
      launch_gemv<B, EPI_STORE>(a, pl, a.seg[0].T, gemv_lds(B, pl), st);
    }
    // ---- gate/up with GELU(gate) * up; post-attention residual + pre-FF norm in the prologue
    if (!gemvs_only) {
      GemvArgs a{};
      const GemvPlan& pl = L.p_gu;
      fill_seg(a.seg[0], ly.wg, I, H, 0, 0, fmt);
      fill_seg(a.seg[1], ly.wu, I, H, 0, 0, fmt);
      a.nseg = 2;
      NormIn ni{};
      ni.h_src = P.hA; ni.y = P.y; ni.ny = (full ? L.p_o_f : L.p_o_s).S; ni.y_split = (long)n * H;
      ni.w_post = ly.post_attn_norm; ni.scalar = 1.0f;
      ni.w_in = ly.pre_ff_norm; ni.h_dst = P.hB; ni.H = H; ni.eps = m->eps;
      hipLaunchKernelGGL(k_norm_rows<4>, dim3(n), dim3(512), 0, st, ni, P.xf2);
      a.K = H; a.NQ = pl.NQ; a.W = pl.W; a.NQs = pl.NQs;
      a.x = P.xf2; a.ldx = H;
      a.a_out = P.a; a.inter = I; a.n_rows = n;
      launch_gemv<B, EPI_GATEUP>(a, pl, a.seg[0].T, gemv_lds(B, pl), st);
    }
    // ---- down projection
    {
      GemvArgs a{};
      const GemvPlan& pl = L.p_d;
      fill_seg(a.seg[0], ly.wd, H, I, 0, 0, fmt);
      a.nseg = 1;
      a.K = I; a.NQ = pl.NQ; a.W = pl.W; a.NQs = pl.NQs;
      a.x = P.a; a.ldx = I;
      a.y = P.y; a.ldy = H; a.y_split = (long)n * H; a.n_rows = n;
      a.ra0 = reinterpret_cast<const float4*>(ly.post_ff_norm);      // read by the next norm
      a.ra1 = reinterpret_cast<const float4*>(l + 1 < m->n_layers ? m->layers[l + 1].attn_norm : m->final_norm);
      a.ra_n = H / 4;
      launch_gemv<B, EPI_STORE>(a, pl, a.seg[0].T, gemv_lds(B, pl), st);
    }
  }
  if (gemvs_only) return launch_status();
  // ---- final norm (post-FF residual of the last layer), tied head, argmax
  {
    const q4dec_layer& last = m->layers[m->n_layers - 1];
    NormIn ni{};
    ni.h_src = P.hB; ni.y = P.y; ni.ny = L.p_d.S; ni.y_split = (long)n * H;
    ni.w_post = last.post_ff_norm; ni.scalar = last.layer_scalar;
    ni.w_in = m->final_norm; ni.h_dst = P.hA; ni.H = H; ni.eps = m->eps;
    hipLaunchKernelGGL(k_norm_rows<4>, dim3(n), dim3(512), 0, st, ni, P.xh);
  }
  {
    HeadArgs a{};
    a.E = m->embed; a.x = P.xh; a.V = m->vocab; a.H = H; a.softcap = m->softcap;
    a.sp = P.sp; a.best = P.best; a.n_rows = n;
    const int grid = head_grid(m->vocab, B == 1 ? 4 : 2);
    hipLaunchKernelGGL((k_head<B>), dim3(grid), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_argmax_out, dim3(1), dim3(256), 0, st, P.best, grid, n, nullptr, P.sp);
  }
  return launch_status();
}

q4_status check_model(const q4dec_model* m, int n, int pos0, const int32_t* tokens, int max_rows = kMaxRows) {
  if (!m || !m->layers || !m->embed || !m->final_norm || !tokens) return Q4_EINVAL;
  if (n < 1 || n > max_rows) return Q4_ESHAPE;
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
    const bool vrow = full && m->kv_format == 1;   // the K cache is not used
    if (!ly.attn_norm || !ly.q_norm || !ly.k_norm || !ly.post_attn_norm || !ly.pre_ff_norm ||
        !ly.post_ff_norm || (!ly.k_cache && !vrow) || !ly.v_cache)
      return Q4_EINVAL;
    if (vrow && !ly.v_norm) return Q4_EINVAL;         // K = RoPE(k_norm * V) needs the normed V
    const void* ps[] = {ly.wq, ly.wk, ly.wo, ly.wg, ly.wu, ly.wd, ly.attn_norm, ly.q_norm, ly.k_norm,
                        ly.post_attn_norm, ly.pre_ff_norm, ly.post_ff_norm, vrow ? ly.v_cache : ly.k_cache,
                        ly.v_cache};
    for (const void* p : ps)
      if (!al16(p)) return Q4_EALIGN;
    if (!full && !al16(ly.wv)) return Q4_EALIGN;
  }
  if (any_full && (long)pos0 + n - 1 >= (long)m->full_cap) return Q4_ERANGE;
  for (int i = 0; i < n; i++)
    if (tokens[i] < 0 || tokens[i] >= m->vocab) return Q4_ERANGE;
  return Q4_OK;
}

// ------------------------------------------------------ streaming read ----
// Reads n16 16-byte words with kStreamGrid x 256 threads: each wave takes 8
// consecutive 1 KB runs per pass (8 loads in flight per lane), then strides
// by all waves; workgroup b stores the XOR of the 32-bit words it read to
// sink[b].
constexpr int kStreamGrid = 4096;

__global__ void __launch_bounds__(256) k_stream_read(const u4v* p, long n16, uint32_t* sink) {
  __shared__ uint32_t wx[4];
  const int lane = threadIdx.x & 63;
  const long nw = (long)gridDim.x * 4;
  uint32_t s = 0;
  for (long w = blockIdx.x * 4L + (threadIdx.x >> 6); w * 512 < n16; w += nw) {
    u4v c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const long o = (w * 8 + j) * 64 + lane;
      c[j] = o < n16 ? __builtin_nontemporal_load(p + o) : (u4v){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 8; j++) s ^= c[j].x ^ c[j].y ^ c[j].z ^ c[j].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s ^= (uint32_t)__shfl_xor((int)s, o, 64);
  if (lane == 0) wx[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

// ----------------------------------------------------------- graph cache ----
// Captured step graphs, keyed by everything their kernel arguments hold: the
// model descriptor and layer table (weights, caches), the row count and the
// workspace.  Outputs and positions reach the graph through StepParams, so
// neither is part of the key.  At most kMaxGraphs are kept; the least recently
// used one is destroyed (after the stream it last ran on has finished it).
constexpr size_t kMaxGraphs = 16;

struct CachedGraph {
  hipGraphExec_t exec;
  hipStream_t last_stream;
  unsigned long long last_use;
};
std::map<std::string, CachedGraph> g_graphs;
unsigned long long g_use_clock = 0;

std::string graph_key(const q4dec_model* m, int n, const void* ws, size_t ws_bytes) {
  std::string k;
  k.append(reinterpret_cast<const char*>(m), sizeof(q4dec_model));
  k.append(reinterpret_cast<const char*>(m->layers), sizeof(q4dec_layer) * m->n_layers);
  k.append(reinterpret_cast<const char*>(&ws), sizeof(ws));
  k.append(reinterpret_cast<const char*>(&n), sizeof(n));
  k.append(reinterpret_cast<const char*>(&ws_bytes), sizeof(ws_bytes));
  return k;
}

// under g_mu: drop the least recently used graphs until one more fits
q4_status evict_graphs_locked() {
  q4_status rc = Q4_OK;
  while (g_graphs.size() >= kMaxGraphs) {
    auto victim = g_graphs.begin();
    for (auto it = g_graphs.begin(); it != g_graphs.end(); ++it)
      if (it->second.last_use < victim->second.last_use) victim = it;
    if (hipStreamSynchronize(victim->second.last_stream) != hipSuccess) rc = Q4_EHIP;
    if (hipGraphExecDestroy(victim->second.exec) != hipSuccess) rc = Q4_EHIP;
    g_graphs.erase(victim);
  }
  return rc;
}

q4_status begin_step(const q4dec_model* m, const StepPtrs& P, const int32_t* tokens, int n, int pos0,
                     float* logits, int32_t* argmax, hipStream_t st) {
  BeginArgs b{};
  b.sp = P.sp; b.pos0 = pos0; b.n = n;
  b.logits = logits; b.argmax = argmax;
  for (int i = 0; i < 4; i++) b.tokens[i] = i < n ? tokens[i] : 0;
  b.E = m->embed; b.H = m->hidden; b.emb_scale = (float)std::sqrt((double)m->hidden);
  b.h = P.hA;
  b.rope_cs = P.rope; b.ns = m->sl_rot_pairs; b.nf = m->full_rot_pairs;
  b.Ds = m->sl_head_dim; b.Df = m->full_head_dim; b.theta_s = m->sl_theta; b.theta_f = m->full_theta;
  hipLaunchKernelGGL(k_step_begin, dim3(n), dim3(256), 0, st, b);
  return launch_status();
}


// ------------------------------------------------------- prefill chunk ----
constexpr int kChunkSplits = 8;       // attention splits per (row, KV head) of a chunk
constexpr int kRows4Splits = 16;      // the same for the 4-row kernel of the full layers, and
constexpr int kRows4SplitsLong = 32;  // ... when the rows attend kRows4Long positions or more
constexpr int kRows4Long = 4096;

// A matrix product of a chunk: one 16-row tile per wave and S runs of K
// (S <= max_s; S > 1 writes partial products that the norm or finishing
// kernel reading them adds), chosen so that a launch has about 512
// workgroups: two per CU (x run in LDS 66.5 KB, 152 VGPRs), so that one
// workgroup's MFMAs run while the other waits for its next run.
struct ChunkPlan {
  int NQ, NQs, S, tpw;
};

ChunkPlan chunk_plan(int N, int K, int max_s = 8) {
  ChunkPlan p{};
  p.NQ = (int)ceil_div(K, 128);
  p.tpw = 1;
  const int base = (int)ceil_div(ceil_div(N, 16), 4);
  const int s = std::max(1, std::min(std::min(max_s, p.NQ), (int)ceil_div(512, base)));
  p.NQs = (int)ceil_div(p.NQ, s);
  p.S = (int)ceil_div(p.NQ, p.NQs);
  return p;
}

struct ChunkLayout {
  int qkv_ld, ymax;
  ChunkPlan p_qkv_s, p_qkv_f, p_o_s, p_o_f, p_d;
  size_t hA, hB, qkv, q16, o, y, a, xf, apart, best, total;
};

ChunkLayout chunk_layout(const q4dec_model* m) {
  ChunkLayout L{};
  const int H = m->hidden, I = m->inter, Hq = m->n_heads;
  const int Ds = m->sl_head_dim, Df = m->full_head_dim, Hs = m->sl_kv_heads;
  const int Dmax = std::max(Ds, Df);
  const int R = kChunkRows;
  L.qkv_ld = std::max(Hq * Ds + 2 * Hs * Ds, Hq * Df + Df);
  // the q, k and v products share one launch: plan on their joint workgroups
  L.p_qkv_s = chunk_plan(Hq * Ds + 2 * Hs * Ds, H);
  L.p_qkv_f = chunk_plan(Hq * Df + Df, H);
  L.p_o_s = chunk_plan(H, Hq * Ds);
  L.p_o_f = chunk_plan(H, Hq * Df);
  L.p_d = chunk_plan(H, I);
  L.ymax = std::max(std::max(L.p_o_s.S, L.p_o_f.S), L.p_d.S);
  const int Sq = std::max(L.p_qkv_s.S, L.p_qkv_f.S);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  L.best = take(sizeof(unsigned long long) * 4 * kHeadSlots);   // the head's per-workgroup slots
  L.hA = take(sizeof(float) * R * H);
  L.hB = take(sizeof(float) * R * H);
  L.qkv = take(sizeof(float) * Sq * R * L.qkv_ld);
  L.q16 = take(sizeof(uint16_t) * R * Hq * Dmax);
  L.o = take(sizeof(uint16_t) * R * Hq * Dmax);
  L.y = take(sizeof(float) * L.ymax * R * H);
  L.a = take(sizeof(uint16_t) * R * I);
  L.xf = take(sizeof(uint16_t) * R * H);
  const size_t apart_full = (size_t)R * std::max(kChunkSplits, kRows4SplitsLong) * Hq * (Df + 4);
  const size_t apart_ring = (size_t)R * Hs * kChunkSplits * (Hq / Hs) * (Ds + 4);
  L.apart = take(sizeof(float) * std::max(apart_full, apart_ring));
  L.total = off;
  return L;
}

void fill_gseg(GemmSeg& s, const void* packed, int N, int K, int wg0, int out_off) {
  const int T = (int)ceil_div(N, 16), NQ = (int)ceil_div(K, 128);
  s.codes = static_cast<const u4v*>(packed);
  s.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + (size_t)T * NQ * 64 * 16);
  s.N = N; s.T = T; s.wg0 = wg0; s.out_off = out_off;
}

int gseg_wgs(const GemmSeg& s, int tpw) { return (int)ceil_div(s.T, 4 * tpw); }

// One chunk of n rows at positions pos0 .. pos0 + n - 1 through the whole
// model, launched eagerly: embedding; per layer the input norm, the q/k/v
// products (one launch), q/k/v finishing with the cache writes of every row,
// split-K attention and combine (the rows read the caches only), the output
// product, the post-attention residual and pre-FF norm, gate/up with GELU * up,
// the down product; then the final norm of every row and the head of the last.
q4_status enqueue_chunk(const q4dec_model* m, const ChunkLayout& L, void* ws, const int32_t* tokens, int n,
                        int pos0, float* logits, int32_t* argmax, hipStream_t st) {
  uint8_t* wb = static_cast<uint8_t*>(ws);
  float* hA = reinterpret_cast<float*>(wb + L.hA);
  float* hB = reinterpret_cast<float*>(wb + L.hB);
  float* qkv = reinterpret_cast<float*>(wb + L.qkv);
  uint16_t* q16 = reinterpret_cast<uint16_t*>(wb + L.q16);
  uint16_t* o16 = reinterpret_cast<uint16_t*>(wb + L.o);
  float* y = reinterpret_cast<float*>(wb + L.y);
  uint16_t* a16 = reinterpret_cast<uint16_t*>(wb + L.a);
  uint16_t* xf = reinterpret_cast<uint16_t*>(wb + L.xf);
  float* apart = reinterpret_cast<float*>(wb + L.apart);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(wb + L.best);
  const int H = m->hidden, I = m->inter, Hq = m->n_heads;
  {
    ChunkEmbedArgs e{};
    e.E = m->embed; e.H = H; e.emb_scale = std::sqrt((float)H); e.h = hA;
    for (int i = 0; i < n; i++) e.tokens[i] = tokens[i];
    hipLaunchKernelGGL(k_chunk_embed, dim3(n), dim3(256), 0, st, e);
  }
  auto gemm = [&](GemmArgs& g, int wgs, const ChunkPlan& p) {
    g.NQ = p.NQ; g.NQs = p.NQs;
    if (p.tpw == 2) hipLaunchKernelGGL((k_q4_gemm<EPI_STORE, 2, kChunkRunQ>), dim3(wgs, p.S), dim3(256), kGemmLds, st, g);
    else hipLaunchKernelGGL((k_q4_gemm<EPI_STORE, 1, kChunkRunQ>), dim3(wgs, p.S), dim3(256), kGemmLds, st, g);
  };
  for (int l = 0; l < m->n_layers; l++) {
    const q4dec_layer& ly = m->layers[l];
    const bool full = ly.is_full != 0;
    const int D = full ? m->full_head_dim : m->sl_head_dim;
    const int Hkv = full ? 1 : m->sl_kv_heads;
    const ChunkPlan& pq = full ? L.p_qkv_f : L.p_qkv_s;
    const int Sq = pq.S;
    // ---- input norm (with the previous layer's post-FF residual), q/k/v products
    {
      NormIn ni{};
      if (l == 0) { ni.h_src = hA; ni.y = nullptr; ni.w_post = nullptr; ni.scalar = 1.0f; ni.h_dst = nullptr; }
      else {
        const q4dec_layer& prev = m->layers[l - 1];
        ni.h_src = hB; ni.y = y; ni.w_post = prev.post_ff_norm; ni.scalar = prev.layer_scalar; ni.h_dst = hA;
        ni.ny = L.p_d.S; ni.y_split = (long)n * H;
      }
      ni.w_in = ly.attn_norm; ni.H = H; ni.eps = m->eps;
      hipLaunchKernelGGL(k_norm_rows<8>, dim3(n), dim3(512), 0, st, ni, xf);
      GemmArgs g{};
      int wg = 0;
      fill_gseg(g.seg[0], ly.wq, Hq * D, H, wg, 0);
      wg += gseg_wgs(g.seg[0], pq.tpw);
      fill_gseg(g.seg[1], ly.wk, Hkv * D, H, wg, Hq * D);
      wg += gseg_wgs(g.seg[1], pq.tpw);
      g.nseg = 2;
      if (!full) {
        fill_gseg(g.seg[2], ly.wv, Hkv * D, H, wg, (Hq + Hkv) * D);
        wg += gseg_wgs(g.seg[2], pq.tpw);
        g.nseg = 3;
      }
      g.K = H;
      g.x = xf; g.ldx = H; g.n = n;
      g.y = qkv; g.ldy = L.qkv_ld; g.y_split = (long)n * L.qkv_ld;
      gemm(g, wg, pq);
    }
    // ---- finishing: q to q16, K/V rows of every row into the caches
    {
      ChunkFinArgs f{};
      f.qkv = qkv; f.ldq = L.qkv_ld; f.ny = Sq; f.y_split = (long)n * L.qkv_ld;
      f.Hq = Hq; f.Hkv = Hkv; f.ring = full ? 0 : 1; f.R = m->ring;
      f.v_norm = ly.v_norm; f.vrow = (full && m->kv_format == 1) ? 1 : 0;
      f.q_norm = ly.q_norm; f.k_norm = ly.k_norm;
      f.theta = full ? m->full_theta : m->sl_theta;
      f.rot_pairs = full ? m->full_rot_pairs : m->sl_rot_pairs;
      f.eps = m->eps; f.pos0 = pos0;
      f.q16 = q16; f.kc = ly.k_cache; f.vc = ly.v_cache;
      const dim3 grid(n, Hq + 2 * Hkv);
      switch (D) {
        case 64: hipLaunchKernelGGL(k_chunk_finish<64>, grid, dim3(64), 0, st, f); break;
        case 128: hipLaunchKernelGGL(k_chunk_finish<128>, grid, dim3(64), 0, st, f); break;
        case 256: hipLaunchKernelGGL(k_chunk_finish<256>, grid, dim3(64), 0, st, f); break;
        default: hipLaunchKernelGGL(k_chunk_finish<512>, grid, dim3(64), 0, st, f); break;
      }
    }
    // ---- attention over the caches (every row of the chunk is in them)
    {
      AttnArgs a{};
      a.q = q16; a.k = ly.k_cache; a.v = ly.v_cache; a.seq_stride = 0;
      a.Hq = Hq; a.Hkv = Hkv; a.GQ = Hq / Hkv;
      a.ring = full ? 0 : 1; a.R = m->ring; a.W = m->window;
      a.n_rows = n; a.S = kChunkSplits;
      a.scale_log2 = (full ? m->full_scale : m->sl_scale) * 1.4426950408889634f;
      a.sp = nullptr; a.part = apart;
      a.fin_on = 0;
      a.kvh_major = full ? 0 : 1;
      // the rows of the chunk share K/V tiles: as many rows per workgroup as
      // their query heads fill the 16 MFMA columns (8 on a ring layer)
      a.rpw = 16 % a.GQ == 0 ? 16 / a.GQ : 1;
      if (full && m->kv_format == 1) {
        a.vrow = 1; a.k = ly.v_cache; a.kw = ly.k_norm; a.theta = m->full_theta; a.krot = m->full_rot_pairs;
      }
      a.pos0[0] = pos0;
      if (full && a.rpw <= 1 && !a.vrow && (D == 256 || D == 512)) {
        // 16 query heads fill the columns: 4 rows share each K/V tile instead
        a.S = pos0 + n >= kRows4Long ? kRows4SplitsLong : kRows4Splits;
        if (D == 256) launch_rows4_d<256>(a, 1, o16, st);
        else launch_rows4_d<512>(a, 1, o16, st);
      } else {
        launch_fd(a, D, 1, nullptr, o16, st);
      }
    }
    // ---- output projection
    const ChunkPlan& po = full ? L.p_o_f : L.p_o_s;
    const int So = po.S;
    {
      GemmArgs g{};
      fill_gseg(g.seg[0], ly.wo, H, Hq * D, 0, 0);
      g.nseg = 1;
      g.K = Hq * D;
      g.x = o16; g.ldx = Hq * D; g.n = n;
      g.y = y; g.ldy = H; g.y_split = (long)n * H;
      gemm(g, gseg_wgs(g.seg[0], po.tpw), po);
    }
    // ---- post-attention residual + pre-FF norm, gate/up with GELU * up
    {
      NormIn ni{};
      ni.h_src = hA; ni.y = y; ni.ny = So; ni.y_split = (long)n * H;
      ni.w_post = ly.post_attn_norm; ni.scalar = 1.0f;
      ni.w_in = ly.pre_ff_norm; ni.h_dst = hB; ni.H = H; ni.eps = m->eps;
      hipLaunchKernelGGL(k_norm_rows<8>, dim3(n), dim3(512), 0, st, ni, xf);
      GemmArgs g{};
      fill_gseg(g.seg[0], ly.wg, I, H, 0, 0);
      fill_gseg(g.seg[1], ly.wu, I, H, 0, 0);
      g.nseg = 2;
      g.K = H; g.NQ = (int)ceil_div(H, 128); g.NQs = g.NQ;
      g.x = xf; g.ldx = H; g.n = n;
      g.a_out = a16; g.ld_a = I;
      hipLaunchKernelGGL((k_q4_gemm<EPI_GATEUP, 1, kChunkRunQ>), dim3(ceil_div(g.seg[0].T, 2), 1), dim3(256), kGemmLds, st, g);
    }
    // ---- down projection
    {
      GemmArgs g{};
      fill_gseg(g.seg[0], ly.wd, H, I, 0, 0);
      g.nseg = 1;
      g.K = I;
      g.x = a16; g.ldx = I; g.n = n;
      g.y = y; g.ldy = H; g.y_split = (long)n * H;
      gemm(g, gseg_wgs(g.seg[0], L.p_d.tpw), L.p_d);
    }
  }
  // ---- final norm of every row (the residual stream lands in hA), head of the last
  {
    const q4dec_layer& last = m->layers[m->n_layers - 1];
    NormIn ni{};
    ni.h_src = hB; ni.y = y; ni.ny = L.p_d.S; ni.y_split = (long)n * H;
    ni.w_post = last.post_ff_norm; ni.scalar = last.layer_scalar;
    ni.w_in = m->final_norm; ni.h_dst = hA; ni.H = H; ni.eps = m->eps;
    hipLaunchKernelGGL(k_norm_rows<8>, dim3(n), dim3(512), 0, st, ni, xf);
  }
  {
    HeadArgs a{};
    a.E = m->embed; a.x = xf + (size_t)(n - 1) * H; a.V = m->vocab; a.H = H; a.softcap = m->softcap;
    a.logits = logits; a.best = best; a.n_rows = 1;
    const int grid = head_grid(m->vocab, 4);
    hipLaunchKernelGGL((k_head<1>), dim3(grid), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_argmax_out, dim3(1), dim3(256), 0, st, best, grid, 1, argmax, nullptr);
  }
  return launch_status();
}

q4_status decode_step_impl(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                           int32_t* argmax, void* ws, size_t ws_bytes, void* stream, bool use_graph) {
  q4_status rc = check_model(m, n, pos0, tokens);
  if (rc != Q4_OK) return rc;
  if (!ws) return Q4_EINVAL;
  if (!al16(ws) || (logits && !al16(logits))) return Q4_EALIGN;
  const StepLayout L = step_layout(m);
  if (!L.ok) return Q4_ESHAPE;
  if (ws_bytes < L.total) return Q4_ENOSPACE;
  rc = set_attrs();
  if (rc != Q4_OK) return rc;
  const StepPtrs P = step_ptrs(L, ws);
  hipStream_t st = S(stream);
  rc = begin_step(m, P, tokens, n, pos0, logits, argmax, st);
  if (rc != Q4_OK) return rc;
  if (!use_graph || st == nullptr) {
    return n == 1 ? enqueue_layers<1>(m, L, P, n, st) : enqueue_layers<4>(m, L, P, n, st);
  }
  const std::string key = graph_key(m, n, ws, ws_bytes);
  hipGraphExec_t exec = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_graphs.find(key);
    if (it != g_graphs.end()) {
      exec = it->second.exec;
      it->second.last_stream = st;
      it->second.last_use = ++g_use_clock;
    }
  }
  if (!exec) {
    if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) return Q4_EHIP;
    q4_status r2 = n == 1 ? enqueue_layers<1>(m, L, P, n, st) : enqueue_layers<4>(m, L, P, n, st);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(st, &graph);
    if (r2 != Q4_OK || e != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      return Q4_EHIP;
    }
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return Q4_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (evict_graphs_locked() != Q4_OK) {
      (void)hipGraphExecDestroy(exec);
      return Q4_EHIP;
    }
    g_graphs[key] = CachedGraph{exec, st, ++g_use_clock};
  }
  if (hipGraphLaunch(exec, st) != hipSuccess) return Q4_EHIP;
  return Q4_OK;
}

// ------------------------------------------------------- stage export ----
// Buffer and size of a stage of the last layer a step ran (rows 0 .. n-1).
struct StageView {
  size_t off, bytes;
};

bool stage_view(const q4dec_model* m, const StepLayout& L, int n, int stage, StageView& v) {
  const int H = m->hidden;
  const bool full = m->layers[m->n_layers - 1].is_full != 0;
  const int D = full ? m->full_head_dim : m->sl_head_dim;
  switch (stage) {
    case Q4_STAGE_H_OUT: v = {L.hA, sizeof(float) * n * H}; return true;
    case Q4_STAGE_H_MID: v = {L.hB, sizeof(float) * n * H}; return true;
    case Q4_STAGE_X_ATTN: v = {L.xf, sizeof(uint16_t) * n * H}; return true;
    case Q4_STAGE_QKV: v = {L.qkv, sizeof(float) * n * L.qkv_ld}; return true;
    case Q4_STAGE_Q16: v = {L.q16, sizeof(uint16_t) * n * m->n_heads * D}; return true;
    case Q4_STAGE_O16: v = {L.o, sizeof(uint16_t) * n * m->n_heads * D}; return true;
    case Q4_STAGE_X_MLP: v = {L.xf2, sizeof(uint16_t) * n * H}; return true;
    case Q4_STAGE_A16: v = {L.a, sizeof(uint16_t) * n * m->inter}; return true;
    case Q4_STAGE_X_HEAD: v = {L.xh, sizeof(uint16_t) * n * H}; return true;
    default: return false;
  }
}

// ------------------------------------------------------ static scratch ----
// The split records of flash_decode_full_noalloc live in one file-scope device
// array instead of a caller's workspace: kNoAllocScratchBytes covers up to
// 256 splits of 16 query heads at D = 512 (every call with n_seq * n_rows <= 32,
// Hq <= 16).  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): the device address is taken
// once per device with hipGetSymbolAddress, with that device current, and
// kept in g_scratch.
constexpr size_t kNoAllocScratchBytes = (size_t)256 * 16 * (512 + 4) * sizeof(float);
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};

// the current device's scratch address (NULL on failure)
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
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

#ifndef Q4DEC_SRC_HASH
#define Q4DEC_SRC_HASH "unknown"
#endif
const char* q4dec_version(void) { return "q4dec 0.2 gfx950 src " Q4DEC_SRC_HASH; }

size_t q4_packed_bytes(int N, int K) {
  if (N < 1 || K < 32 || K % 32) return 0;
  return (size_t)ceil_div(N, 16) * 16 * ceil_div(K, 128) * 4 * 18;
}

q4_status q4_pack(const void* w, int w_dtype, int N, int K, void* packed, size_t packed_bytes,
                  int32_t* nonfinite, void* stream) {
  if (!w || !packed) return Q4_EINVAL;
  if (w_dtype != Q4_F32 && w_dtype != Q4_BF16) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32) return Q4_ESHAPE;
  if (packed_bytes < q4_packed_bytes(N, K)) return Q4_ENOSPACE;
  if (!al16(w) || !al16(packed)) return Q4_EALIGN;
  const int T = (int)ceil_div(N, 16);
  const long total = (long)T * ceil_div(K, 128) * 64;
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
  const int T = (int)ceil_div(N, 16);
  const size_t code_bytes = (size_t)T * ceil_div(K, 128) * 64 * 16;
  const u4v* codes = static_cast<const u4v*>(packed);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + code_bytes);
  const long total = (long)N * (K / 32);
  hipLaunchKernelGGL(k_q4_unpack, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, S(stream), codes,
                     scales, N, K, blocks);
  return launch_status();
}

q4_status q4_gemv(const void* packed, int N, int K, const uint16_t* x, int B, float* y, void* stream) {
  if (!packed || !x || !y) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32 || B < 1 || B > kMaxRows) return Q4_ESHAPE;
  const GemvPlan p = gemv_plan(N, K, B == 1 ? 16 : 8);
  if (p.W < 1 || gemv_lds(B == 1 ? 1 : 4, p) > (size_t)kMaxLds - 8 * 1024) return Q4_ESHAPE;
  if (!al16(packed) || !al16(x) || !al16(y)) return Q4_EALIGN;
  q4_status rc = set_attrs();
  if (rc != Q4_OK) return rc;
  GemvArgs a{};
  fill_seg(a.seg[0], packed, N, K, 0, 0);
  a.nseg = 1;
  a.K = K; a.NQ = p.NQ; a.W = p.W; a.NQs = p.NQs;
  a.x = x; a.ldx = K; a.y = y; a.ldy = N; a.n_rows = B;
  if (B == 1) launch_gemv<1, EPI_STORE>(a, p, p.T, gemv_lds(1, p), S(stream));
  else launch_gemv<4, EPI_STORE>(a, p, p.T, gemv_lds(4, p), S(stream));
  return launch_status();
}

size_t q8_packed_bytes(int N, int K) {
  if (N < 1 || K < 32 || K % 32) return 0;
  return (size_t)ceil_div(N, 16) * ceil_div(K, 64) * (64 * 16 + 32 * 2);
}

q4_status q8_pack(const void* w, int w_dtype, int N, int K, void* packed, size_t packed_bytes,
                  int32_t* nonfinite, void* stream) {
  if (!w || !packed) return Q4_EINVAL;
  if (w_dtype != Q4_F32 && w_dtype != Q4_BF16) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32) return Q4_ESHAPE;
  if (packed_bytes < q8_packed_bytes(N, K)) return Q4_ENOSPACE;
  if (!al16(w) || !al16(packed)) return Q4_EALIGN;
  const int T = (int)ceil_div(N, 16);
  const long pairs = (long)T * ceil_div(K, 64);
  u4v* codes = static_cast<u4v*>(packed);
  uint16_t* scales = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(packed) + (size_t)pairs * 64 * 16);
  const dim3 grid((unsigned)ceil_div(pairs * 32, 256));
  if (w_dtype == Q4_F32)
    hipLaunchKernelGGL(k_q8_pack<0>, grid, dim3(256), 0, S(stream), w, N, K, codes, scales, T, nonfinite);
  else
    hipLaunchKernelGGL(k_q8_pack<1>, grid, dim3(256), 0, S(stream), w, N, K, codes, scales, T, nonfinite);
  return launch_status();
}

q4_status q8_unpack(const void* packed, int N, int K, uint8_t* blocks, void* stream) {
  if (!packed || !blocks) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32) return Q4_ESHAPE;
  if (!al16(packed)) return Q4_EALIGN;
  const long pairs = (long)ceil_div(N, 16) * ceil_div(K, 64);
  const u4v* codes = static_cast<const u4v*>(packed);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(packed) + (size_t)pairs * 64 * 16);
  const long total = (long)N * (K / 32);
  hipLaunchKernelGGL(k_q8_unpack, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, S(stream), codes,
                     scales, N, K, blocks);
  return launch_status();
}

q4_status q8_gemv(const void* packed, int N, int K, const uint16_t* x, int B, float* y, void* stream) {
  if (!packed || !x || !y) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32 || B < 1 || B > kMaxRows) return Q4_ESHAPE;
  // the smallest CQ that keeps W within 8 (the grid of a 12B shape is then
  // resident at once: 15360 x 3840 in 12.0 us against 12.4-12.8 us with 15
  // waves of 4 pairs), else within 16
  GemvPlan p = gemv_plan(N, K, 8, 0, 1);
  if (p.W < 1) p = gemv_plan(N, K, 16, 0, 1);
  if (p.W < 1 || gemv_lds(B == 1 ? 1 : 4, p) > (size_t)kMaxLds - 8 * 1024) return Q4_ESHAPE;
  if (!al16(packed) || !al16(x) || !al16(y)) return Q4_EALIGN;
  q4_status rc = set_attrs();
  if (rc != Q4_OK) return rc;
  GemvArgs a{};
  fill_seg(a.seg[0], packed, N, K, 0, 0, 1);
  a.nseg = 1;
  a.K = K; a.NQ = p.NQ; a.W = p.W; a.NQs = p.NQs;
  a.x = x; a.ldx = K; a.y = y; a.ldy = N; a.n_rows = B;
  if (B == 1) launch_gemv<1, EPI_STORE>(a, p, p.T, gemv_lds(1, p), S(stream));
  else launch_gemv<4, EPI_STORE>(a, p, p.T, gemv_lds(4, p), S(stream));
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

// host-only checks of a full-attention call (everything but the workspace)
static q4_status full_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride, int cap,
                           int Hq, int D, const int32_t* pos0, int n_seq, int n_rows, float* out, long& maxlen) {
  if (!q || !k || !v || !pos0 || !out) return Q4_EINVAL;
  if (n_seq < 1 || n_seq > 64 || n_rows < 1 || n_rows > kMaxRows) return Q4_ESHAPE;
  if (Hq < 1 || Hq > 16 || !valid_d(D) || seq_stride < 0 || cap < 1) return Q4_ESHAPE;
  if (n_seq > 1 && (seq_stride == 0 || seq_stride < (int64_t)cap * D)) return Q4_ESHAPE;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(out) || (seq_stride * 2) % 16) return Q4_EALIGN;
  maxlen = 1;
  for (int s = 0; s < n_seq; s++) {
    if (pos0[s] < 0 || (long)pos0[s] + n_rows - 1 >= cap) return Q4_ERANGE;
    maxlen = std::max(maxlen, (long)pos0[s] + n_rows);
  }
  return Q4_OK;
}

static q4_status full_run(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride, int cap,
                          int Hq, int D, const int32_t* pos0, int n_seq, int n_rows, float scale, float* out,
                          void* ws, long maxlen, void* stream) {
  q4_status rc = set_attrs();
  if (rc != Q4_OK) return rc;
  AttnArgs a{};
  a.q = q; a.k = const_cast<uint16_t*>(k); a.v = const_cast<uint16_t*>(v); a.seq_stride = seq_stride;
  a.Hq = Hq; a.Hkv = 1; a.GQ = Hq; a.ring = 0; a.R = cap; a.W = cap;
  a.n_rows = n_rows;
  a.S = (int)std::min<long>(fd_split_cap(n_seq, n_rows), std::max<long>(1, ceil_div(maxlen, kTilePos)));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sp = nullptr; a.part = static_cast<float*>(ws);
  for (int s = 0; s < n_seq; s++) a.pos0[s] = pos0[s];
  launch_fd(a, D, n_seq, out, nullptr, S(stream));
  return launch_status();
}

q4_status flash_decode_full(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride,
                            int cap, int Hq, int D, const int32_t* pos0, int n_seq, int n_rows, float scale,
                            float* out, void* ws, size_t ws_bytes, void* stream) {
  long maxlen = 1;
  q4_status rc = full_args(q, k, v, seq_stride, cap, Hq, D, pos0, n_seq, n_rows, out, maxlen);
  if (rc != Q4_OK) return rc;
  if (!ws) return Q4_EINVAL;
  if (ws_bytes < flash_decode_workspace_size(n_seq, n_rows, Hq, D)) return Q4_ENOSPACE;
  if (!al16(ws)) return Q4_EALIGN;
  return full_run(q, k, v, seq_stride, cap, Hq, D, pos0, n_seq, n_rows, scale, out, ws, maxlen, stream);
}

size_t flash_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

q4_status flash_decode_full_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_stride,
                                    int cap, int Hq, int D, const int32_t* pos0, int n_seq, int n_rows,
                                    float scale, float* out, void* stream) {
  long maxlen = 1;
  q4_status rc = full_args(q, k, v, seq_stride, cap, Hq, D, pos0, n_seq, n_rows, out, maxlen);
  if (rc != Q4_OK) return rc;
  if (flash_decode_workspace_size(n_seq, n_rows, Hq, D) > kNoAllocScratchBytes) return Q4_ENOSPACE;
  // the first call on a device (with it current) records its scratch address
  void* ws = scratch_ptr();
  if (!ws) return Q4_EHIP;
  return full_run(q, k, v, seq_stride, cap, Hq, D, pos0, n_seq, n_rows, scale, out, ws, maxlen, stream);
}

q4_status flash_decode_full_vrow(const uint16_t* q, const uint16_t* vrow, int64_t seq_stride, int cap, int Hq,
                                 int D, const float* kw, double theta, int rot_pairs, const int32_t* pos0,
                                 int n_seq, int n_rows, float scale, float* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  q4_status rc = fd_common(q, vrow, vrow, seq_stride, Hq, 1, D, pos0, n_seq, n_rows, out, ws, ws_bytes);
  if (rc != Q4_OK) return rc;
  if (!kw) return Q4_EINVAL;
  if (!vrow_dims_ok(D, rot_pairs) || !(theta > 0.0) || cap < 1) return Q4_ESHAPE;
  if (!al16(kw)) return Q4_EALIGN;
  if (n_seq > 1 && seq_stride < (int64_t)cap * D) return Q4_ESHAPE;
  long maxlen = 1;
  for (int s = 0; s < n_seq; s++) {
    if (pos0[s] < 0 || (long)pos0[s] + n_rows - 1 >= cap) return Q4_ERANGE;
    maxlen = std::max(maxlen, (long)pos0[s] + n_rows);
  }
  rc = set_attrs();
  if (rc != Q4_OK) return rc;
  AttnArgs a{};
  a.q = q; a.k = const_cast<uint16_t*>(vrow); a.v = const_cast<uint16_t*>(vrow); a.seq_stride = seq_stride;
  a.Hq = Hq; a.Hkv = 1; a.GQ = Hq; a.ring = 0; a.R = cap; a.W = cap;
  a.n_rows = n_rows;
  a.S = (int)std::min<long>(fd_split_cap(n_seq, n_rows), std::max<long>(1, ceil_div(maxlen, kTilePos)));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sp = nullptr; a.part = static_cast<float*>(ws);
  a.vrow = 1; a.kw = kw; a.theta = theta; a.krot = rot_pairs;
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
  if (R < 32) return Q4_ESHAPE;   // a tile's 32 positions wrap the ring at most once
  if (n_seq > 1 && seq_stride < (int64_t)Hkv * R * D) return Q4_ESHAPE;
  for (int s = 0; s < n_seq; s++)
    if (pos0[s] < 0 || (long)pos0[s] + n_rows - 1 > 0x7FFFFFFFL) return Q4_ERANGE;
  rc = set_attrs();
  if (rc != Q4_OK) return rc;
  AttnArgs a{};
  a.q = q; a.k = const_cast<uint16_t*>(k_ring); a.v = const_cast<uint16_t*>(v_ring); a.seq_stride = seq_stride;
  a.Hq = Hq; a.Hkv = Hkv; a.GQ = Hq / Hkv; a.ring = 1; a.R = R; a.W = W;
  a.n_rows = n_rows;
  // one 32-position tile per split when the split cap allows it (the waves
  // then share each tile's head dimension), else 4 tiles per split
  const long cap_s = fd_split_cap(n_seq, n_rows);
  a.S = (int)std::min<long>(cap_s, std::max<long>(1, ceil_div(W, kTilePos)));
  if (D >= 128 && ceil_div(W, 32) <= cap_s) a.S = (int)ceil_div(W, 32);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sp = nullptr; a.part = static_cast<float*>(ws);
  for (int s = 0; s < n_seq; s++) a.pos0[s] = pos0[s];
  launch_fd(a, D, n_seq, out, nullptr, S(stream));
  return launch_status();
}

size_t decode_step_workspace_size(const q4dec_model* m, int n) {
  if (!m || n < 1 || n > kMaxRows || !model_dims_ok(m)) return 0;
  const StepLayout L = step_layout(m);
  return L.ok ? L.total : 0;
}

q4_status decode_step_hidden(const q4dec_model* m, const void* ws, size_t ws_bytes, int n, float* h_out,
                             void* stream) {
  if (!m || !ws || !h_out) return Q4_EINVAL;
  if (n < 1 || n > kMaxRows || !model_dims_ok(m)) return Q4_ESHAPE;
  const StepLayout L = step_layout(m);
  if (ws_bytes < L.total) return Q4_ENOSPACE;
  const void* src = static_cast<const uint8_t*>(ws) + L.hA;
  if (hipMemcpyAsync(h_out, src, sizeof(float) * n * m->hidden, hipMemcpyDeviceToDevice, S(stream)) != hipSuccess)
    return Q4_EHIP;
  return Q4_OK;
}

size_t decode_step_stage_bytes(const q4dec_model* m, int n, int stage) {
  if (!m || n < 1 || n > kMaxRows || !model_dims_ok(m)) return 0;
  const StepLayout L = step_layout(m);
  StageView v{};
  if (!L.ok || !stage_view(m, L, n, stage, v)) return 0;
  return v.bytes;
}

q4_status decode_step_stage(const q4dec_model* m, const void* ws, size_t ws_bytes, int n, int stage, void* dst,
                            size_t dst_bytes, void* stream) {
  if (!m || !m->layers || !ws || !dst) return Q4_EINVAL;
  if (n < 1 || n > kMaxRows || !model_dims_ok(m)) return Q4_ESHAPE;
  const StepLayout L = step_layout(m);
  StageView v{};
  if (!L.ok) return Q4_ESHAPE;
  if (!stage_view(m, L, n, stage, v)) return Q4_EINVAL;
  if (ws_bytes < L.total || dst_bytes < v.bytes) return Q4_ENOSPACE;
  const void* src = static_cast<const uint8_t*>(ws) + v.off;
  if (hipMemcpyAsync(dst, src, v.bytes, hipMemcpyDeviceToDevice, S(stream)) != hipSuccess) return Q4_EHIP;
  return Q4_OK;
}

q4_status decode_step_gemvs(const q4dec_model* m, int n, void* ws, size_t ws_bytes, void* stream) {
  if (!m || !m->layers || !ws) return Q4_EINVAL;
  if (n < 1 || n > kMaxRows || !model_dims_ok(m)) return Q4_ESHAPE;
  const StepLayout L = step_layout(m);
  if (!L.ok) return Q4_ESHAPE;
  if (ws_bytes < L.total) return Q4_ENOSPACE;
  if (!al16(ws)) return Q4_EALIGN;
  q4_status rc = set_attrs();
  if (rc != Q4_OK) return rc;
  const StepPtrs P = step_ptrs(L, ws);
  return n == 1 ? enqueue_layers<1>(m, L, P, n, S(stream), true) : enqueue_layers<4>(m, L, P, n, S(stream), true);
}

int q4dec_graph_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int)g_graphs.size();
}

q4_status decode_step(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                      int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(m, tokens, n, pos0, logits, argmax, ws, ws_bytes, stream, true);
}

q4_status decode_step_eager(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                            int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(m, tokens, n, pos0, logits, argmax, ws, ws_bytes, stream, false);
}

q4_status q4_gemm(const void* packed, int N, int K, const uint16_t* x, int n, float* y, void* stream) {
  if (!packed || !x || !y) return Q4_EINVAL;
  if (N < 1 || K < 32 || K % 32 || n < 1 || n > kChunkRows) return Q4_ESHAPE;
  if (!al16(packed) || !al16(x) || !al16(y) || K % 8) return Q4_EALIGN;
  q4_status rc = set_attrs();
  if (rc != Q4_OK) return rc;
  GemmArgs g{};
  fill_gseg(g.seg[0], packed, N, K, 0, 0);
  g.nseg = 1;
  const ChunkPlan p = chunk_plan(N, K, 1);       // one run of K: y is the whole product
  g.K = K; g.NQ = p.NQ; g.NQs = p.NQs;
  g.x = x; g.ldx = K; g.n = n;
  g.y = y; g.ldy = N; g.y_split = 0;
  const dim3 grid(gseg_wgs(g.seg[0], p.tpw), 1);
  if (p.tpw == 2) hipLaunchKernelGGL((k_q4_gemm<EPI_STORE, 2, kGemmRunQ>), grid, dim3(256), kGemmLds, S(stream), g);
  else hipLaunchKernelGGL((k_q4_gemm<EPI_STORE, 1, kGemmRunQ>), grid, dim3(256), kGemmLds, S(stream), g);
  return launch_status();
}

size_t prefill_chunk_workspace_size(const q4dec_model* m) {
  if (!m || !model_dims_ok(m)) return 0;
  return chunk_layout(m).total;
}

q4_status prefill_chunk(const q4dec_model* m, const int32_t* tokens, int n, int pos0, float* logits,
                        int32_t* argmax, float* h_out, void* ws, size_t ws_bytes, void* stream) {
  q4_status rc = check_model(m, n, pos0, tokens, kChunkRows);
  if (rc != Q4_OK) return rc;
  if (m->weight_format != 0) return Q4_ESHAPE;          // the chunk products take q4 weights
  if (!ws) return Q4_EINVAL;
  if (!al16(ws) || (logits && !al16(logits))) return Q4_EALIGN;
  const ChunkLayout L = chunk_layout(m);
  if (ws_bytes < L.total) return Q4_ENOSPACE;
  rc = set_attrs();
  if (rc != Q4_OK) return rc;
  hipStream_t st = S(stream);
  rc = enqueue_chunk(m, L, ws, tokens, n, pos0, logits, argmax, st);
  if (rc != Q4_OK) return rc;
  if (h_out) {
    const void* src = static_cast<const uint8_t*>(ws) + L.hA;
    if (hipMemcpyAsync(h_out, src, sizeof(float) * n * m->hidden, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return Q4_EHIP;
  }
  return Q4_OK;
}

q4_status q4_spec_accept(const int32_t* block, const int32_t* argmax, int n, int32_t* emitted,
                         int* n_emitted) {
  if (!block || !argmax || !emitted || !n_emitted) return Q4_EINVAL;
  if (n < 1 || n > kMaxRows) return Q4_ESHAPE;
  int a = 0;
  while (a < n - 1 && block[a + 1] == argmax[a]) {
    emitted[a] = block[a + 1];
    a++;
  }
  emitted[a] = argmax[a];
  *n_emitted = a + 1;
  return Q4_OK;
}

int q4_stream_read_sink_words(void) { return kStreamGrid; }

q4_status q4_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return Q4_EINVAL;
  if (bytes == 0 || bytes % 16) return Q4_ESHAPE;
  if (!al16(src) || !al16(sink)) return Q4_EALIGN;
  hipLaunchKernelGGL(k_stream_read, dim3(kStreamGrid), dim3(256), 0, S(stream),
                     static_cast<const u4v*>(src), (long)(bytes / 16), sink);
  return launch_status();
}

q4_status q4dec_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  q4_status rc = Q4_OK;
  for (auto& kv : g_graphs) {
    if (hipStreamSynchronize(kv.second.last_stream) != hipSuccess) rc = Q4_EHIP;
    if (hipGraphExecDestroy(kv.second.exec) != hipSuccess) rc = Q4_EHIP;
  }
  g_graphs.clear();
  return rc;
}

}  // extern "C"
