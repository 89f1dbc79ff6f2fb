// attn_kernels.h -- split-K flash-decode attention for gfx950 (full layers
// and sliding-window ring layers), plus the log-sum-exp combine.
//
// Per KV head, the query heads that share it (16 for a full layer, 2 for a
// sliding layer) are the columns of one MFMA tile, so every K/V element is
// loaded once for all of them (the GQA fold of the gemma-4-E4B-CoreAI card,
// ring3/).  Per 32-position tile a wave computes
//   S^T = K Q^T   with v_mfma_f32_16x16x32_f16 (A = K rows straight from HBM),
// an fp32 online softmax per column (gemma4-12b card, "The fix": fp32 online
// softmax, scale 1.0), and
//   O += P V      with v_mfma_f32_16x16x32_f16, V staged through LDS and P
//                 split into fp16 hi + lo parts (about 22 significant bits).
// Positions are dealt to workgroups in contiguous splits computed on the
// device from the live position (never from the capacity); each workgroup
// merges its 4 waves and writes one (m, l, O) record per query head; the
// combine kernel merges the splits in fixed order.
//
// Ring: row at position P attends positions max(0, P-W+1) .. P, held at slot
// p mod R (Gemma-4-12B-CoreAI card, "v5/ -- ring extent R = 2W": a slot's
// implied position p = P - ((P - j) mod R) is admitted iff P - p < W; it must
// also have been written, p >= 0).  Full: positions 0 .. P at row p.
//
// Inside the decode step the kernel also finishes q/k/v from the raw
// projections (per-head RMSNorm, RoPE, the scale-free V norm; gemma4-12b
// card, architecture notes): every workgroup forms the queries of its
// columns, the rows of the current step are formed in LDS by the workgroups
// whose range holds them (no other workgroup reads them), and the workgroup
// owning a row's own position writes that row to the cache.
#pragma once
#include "device_common.h"
#include "gemv_kernels.h"

namespace q4k {

struct AttnFin {
  const float* qkv;       // [rows][ldq]: q (Hq*D) | k (Hkv*D) | v (Hkv*D, ring layers)
  int ldq;
  const float* q_norm;
  const float* k_norm;
  int v_norm;
  int rot_pairs;
  const float2* rope_cs;  // [row][cs_ld]: (cos, sin) of pair i < D/2 at the row's position
  int cs_ld;
  float eps;
};

struct AttnArgs {
  const uint16_t* q;      // [n_seq][n_rows][Hq][D] (when fin_on == 0)
  uint16_t* k;            // sequence s at + s * seq_stride
  uint16_t* v;
  long seq_stride;
  int Hq, Hkv, GQ;        // GQ = Hq / Hkv query heads per KV head (<= 16)
  int ring, R, W;
  int n_rows;             // rows per sequence (grid extent)
  int S;                  // splits per (sequence, row, KV head)
  float scale_log2;       // softmax scale * log2(e)
  const StepParams* sp;   // decode step: positions on the device
  float* part;            // records [n_seq][n_rows][Hkv][S][GQ][D + 4]
  int fin_on;
  int kvh_major;          // grids enumerate KV heads fastest (the splits of one KV head, and
                          // the combine of its query heads, then share an XCD when Hkv = 8)
  int rpw;                // rows per workgroup (fin_on == 0 only; 0 or 1: one): the MFMA
                          // columns are (row, query head) pairs, GQ * rpw <= 16, so a K/V
                          // tile is read once for rpw rows (a prefill chunk's ring layers)
  AttnFin fin;
  // Full layers that cache one row per position (kernel template VR): the
  // key of cached row t is RoPE_t(kw * v_t), formed in registers from the V
  // row (gemma4-12b card, architecture notes: V is the scale-free norm of the
  // raw k projection and K its k_norm-weighted norm, rotated, so K = RoPE(kw *
  // V); Gemma-4-12B-CoreAI card, "The per-tier cost": the full-layer pair is
  // the KV term that grows with the context).  a.k is then unused.
  int vrow;               // host-side dispatch flag for VR
  const float* kw;        // [D] the layer's k_norm multiplier (16-byte aligned)
  double theta;           // RoPE base of the layer kind
  int krot;               // rotated pairs, at most vr_max_rot<D>()
  int pos0[64];
};

// Pairs (i, i + D/2) that a VR kernel can rotate: those of its first
// min(2, D/64) k steps (64 pairs for D >= 128).
template <int D>
constexpr int vr_rsteps() { return D / 64 < 2 ? D / 64 : 2; }
template <int D>
constexpr int vr_max_rot() { return 32 * vr_rsteps<D>(); }

Q4_DEV long attn_rec(const AttnArgs& a, int seq, int row, int kvh, int split, int col, int D) {
  return (((((long)seq * a.n_rows + row) * a.Hkv + kvh) * a.S + split) * a.GQ + col) * (long)(D + 4);
}

// LDS of k_fd_partial: V rows [4 waves][32][pitch], rows of this step newK /
// newV [4][D], finished queries q16 [16][D].  The V rows are written by direct
// global-to-LDS loads of 1 KB per instruction.  Each 16-lane group of the PV
// step's transposing reads touches 4 rows x 32 bytes, which must fall in
// distinct banks.  D <= 256: several rows per instruction, so the rows are
// unpadded and the 16-byte chunk c of tile row r sits at chunk c ^ 2 vswz(r)
// (which also separates the two groups of a 32-lane half).  D = 512: one row
// per instruction, padded by 32 bytes (rows 8 banks apart), unswizzled;
// 159,744 bytes in all.
template <int D>
constexpr int fd_vpitch() { return D == 512 ? D + 16 : D; }

// swizzle of tile row r, in units of two 16-byte chunks (< D / 16)
template <int D>
Q4_DEV int vswz(int r) { return D == 512 ? 0 : ((r & 3) | (((r >> 3) & 1) << 2)) & (D / 16 - 1); }

template <int D>
constexpr size_t fd_lds_vbytes() { return (size_t)4 * 32 * fd_vpitch<D>() * 2; }

template <int D>
constexpr size_t fd_lds_bytes() {
  return (size_t)4 * 32 * fd_vpitch<D>() * 2 + (size_t)2 * 4 * D * 2 + (size_t)16 * D * 2;
}

// Layout of a head vector (D elements) spread over one wave for finishing:
// lane l holds H = D / 128 consecutive elements of each half, l*H .. l*H+H-1
// and D/2 + l*H .. D/2 + l*H+H-1 (v[0..H) and v[H..2H)), so the rotated pairs
// (i, i + D/2) sit in one lane and each half is one vector load; D = 64 keeps
// one element per lane (element l), its pairs in lanes l and l + 32.
template <int D> constexpr int fin_h() { return D >= 128 ? D / 128 : 1; }

template <int N> struct fvec;            // N consecutive floats as one load
template <> struct fvec<1> { using t = float; };
template <> struct fvec<2> { using t = float2; };
template <> struct fvec<4> { using t = float4; };

// loads the wave's share of a D-float vector in the finishing layout
template <int D>
Q4_DEV void fin_load(float (&v)[D / 64], const float* src) {
  const int lane = threadIdx.x & 63;
  if constexpr (D == 64) {
    v[0] = src[lane];
  } else {
    constexpr int H = fin_h<D>();
    using V = typename fvec<H>::t;
    const V lo = *reinterpret_cast<const V*>(src + lane * H);
    const V hi = *reinterpret_cast<const V*>(src + D / 2 + lane * H);
    const float* pl = reinterpret_cast<const float*>(&lo);
    const float* ph = reinterpret_cast<const float*>(&hi);
#pragma unroll
    for (int e = 0; e < H; e++) { v[e] = pl[e]; v[H + e] = ph[e]; }
  }
}

// stores the wave's share (finishing layout) as fp16 to dst (LDS)
template <int D>
Q4_DEV void fin_store(const float (&v)[D / 64], uint16_t* dst) {
  const int lane = threadIdx.x & 63;
  if constexpr (D == 64) {
    dst[lane] = f2h(v[0]);
  } else {
    constexpr int H = fin_h<D>();
#pragma unroll
    for (int e = 0; e < H; e++) {
      dst[lane * H + e] = f2h(v[e]);
      dst[D / 2 + lane * H + e] = f2h(v[H + e]);
    }
  }
}

// Per-head RMSNorm (weights wv, or scale-free) and RoPE on one head vector in
// the finishing layout; fp16 result to dst (LDS).  cs holds (cos, sin) of
// this lane's pairs (l*H + e; D = 64: l mod 32) at the vector's position;
// pairs past rot_pairs are not rotated.
template <int D>
Q4_DEV void finish_vals(float (&v)[D / 64], const float (&wv)[D / 64], bool weighted, bool rope,
                        const float2 (&cs)[fin_h<D>()], int rot_pairs, float eps, uint16_t* dst) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; e++) ss += v[e] * v[e];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int e = 0; e < E; e++) v[e] = v[e] * inv * (weighted ? wv[e] : 1.0f);
  auto rot = [&](int i, float2 t, float& x0, float& x1) {
    if (rope && i < rot_pairs) {
      const float c = t.x, s = t.y;
      const float y0 = x0 * c - x1 * s;
      const float y1 = x1 * c + x0 * s;
      x0 = y0; x1 = y1;
    }
  };
  if constexpr (E == 1) {
    const float other = __shfl_xor(v[0], 32, 64);
    float x0 = lane < 32 ? v[0] : other, x1 = lane < 32 ? other : v[0];
    rot(lane & 31, cs[0], x0, x1);
    v[0] = lane < 32 ? x0 : x1;
  } else {
    constexpr int H = fin_h<D>();
#pragma unroll
    for (int e = 0; e < H; e++) rot(lane * H + e, cs[e], v[e], v[H + e]);
  }
  fin_store<D>(v, dst);
}

// D <= 256 fits two waves per SIMD (<= 256 registers), so two workgroups
// share a CU when the grid is larger than the chip (many sequences).
//
// VR (one cached row per position): the V row of a tile is loaded twice, into
// registers as the QK operand and into LDS for PV (the second read is served
// by the L2), so HBM carries 1 KB per position at D = 512.  In k steps whose
// dims rotate (pairs below vr_max_rot: steps s < RS and their partners
// s + D/64), the lane rebuilds its key elements k = RoPE_t(kw * v) in fp32 and
// splits them into fp16 hi + lo; in the other steps the key is kw * v, so kw
// is folded into the query (q * kw split into fp16 hi + lo).  Either way the
// scores carry about 22 significant bits of the key, which is never rounded
// to fp16.  The angle t * theta^(-2i/D) is formed in fp64 revolutions and
// reduced to [0, 1) before the hardware sine and cosine; the row 4 positions
// on is turned by the precomputed (cos, sin) of 4 * theta^(-2i/D).
//
// MR (several rows per workgroup, a.rpw; without the finishing prologue): the
// MFMA columns are (row, query head) pairs, each masked to its own row's
// window, and the splits divide the union of the rows' ranges.
template <int D, bool VR = false, bool MR = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 256 ? 2 : 1))) k_fd_partial(AttnArgs a) {
  constexpr int VROW = fd_vpitch<D>();        // LDS row pitch of the V rows (halves)
  constexpr int NDS = D / 16;                 // PV dim steps
  constexpr int NKS = D / 32;                 // QK k steps
  constexpr int HS = D / 64;                  // k steps per half head: step s pairs with s + HS
  constexpr int RS = vr_rsteps<D>();          // VR: rotating k steps of the first half
  constexpr int NR = VR ? 32 * RS : 1;        // VR: rotatable pairs
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* vlds = reinterpret_cast<uint16_t*>(smem);
  uint16_t* newK = vlds + 4 * 32 * VROW;      // [4][D] rows of this step (decode step)
  uint16_t* newV = newK + 4 * D;
  uint16_t* q16 = newV + 4 * D;               // [16][D] finished queries (decode step)
  __shared__ float wm[4][16], wl[4][16];
  // VR tables of the rotatable pairs i: revolutions per position of pair i
  // (0 past krot), (cos, sin) of 4 positions' turn, kw at dims i and i + D/2
  __shared__ double vr_f[NR];
  __shared__ float2 vr_c4[NR];
  __shared__ float vr_w[2 * NR];
  static_assert(fd_lds_bytes<D>() + sizeof(wm) + sizeof(wl) + sizeof(vr_f) + sizeof(vr_c4) + sizeof(vr_w) <=
                    160 * 1024, "LDS of one workgroup");
  auto rebuilt = [](int s) { return VR && (s < RS || (s >= HS && s < HS + RS)); };

  const int split = a.kvh_major ? blockIdx.y : blockIdx.x, kvh = a.kvh_major ? blockIdx.x : blockIdx.y;
  // rows of this workgroup: row .. rlast (one unless MR)
  const int rpw = MR && a.rpw > 1 ? a.rpw : 1;
  int seq, row;
  if constexpr (MR) {
    const int nrg = (a.n_rows + rpw - 1) / rpw;
    seq = blockIdx.z / nrg;
    row = (blockIdx.z - seq * nrg) * rpw;
  } else {
    seq = blockIdx.z / a.n_rows;
    row = blockIdx.z - seq * a.n_rows;
  }
  if (row >= a.n_rows) return;
  const int rlast = MR ? min(a.n_rows, row + rpw) - 1 : row;
  // the wave index as a scalar: tile origins and cache rows derived from it
  // are then computed once per wave, not per lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

  // ---- the step's first position, before any other load: a global load
  // (not a generic one through a pointer that may also point at the
  // arguments), so waiting for it does not wait for the loads issued after it
  int base;
  if (a.sp) base = *(const __attribute__((address_space(1))) int*)(&a.sp->pos0);
  else base = a.pos0[seq];

  // ---- inputs of the finishing prologue (decode step), issued first: they
  // do not depend on the position, so they travel while the step
  // parameters are read.  Jobs are dealt round-robin to the waves: the query
  // heads of this workgroup's columns, then k and v of every row 0 .. row of
  // the step (after the position is known, only the rows in this
  // workgroup's range are finished).
  constexpr int FE = D / 64, FEH = fin_h<D>();
  constexpr int MAXJ = (16 + 2 * 4 + 3) / 4;
  const int njobs = a.fin_on ? a.GQ + 2 * (row + 1) : 0;
  float raw[MAXJ][FE], wq[FE], wk[FE];
  float2 fcs[MAXJ][FEH];
  if (a.fin_on) {
    const AttnFin& f = a.fin;
    fin_load<D>(wq, f.q_norm);
    fin_load<D>(wk, f.k_norm);
#pragma unroll
    for (int k = 0; k < MAXJ; k++) {
      const int jb = wave + 4 * k;
      if (jb >= njobs) break;                                // wave-uniform
      const int r = jb < a.GQ ? row : (jb - a.GQ) >> 1;    // row of the step the job belongs to
      const float* rr = f.qkv + (long)r * f.ldq;
      const float* src;
      if (jb < a.GQ) src = rr + (long)(kvh * a.GQ + jb) * D;
      else if (((jb - a.GQ) & 1) == 0 || !a.ring) src = rr + (long)(a.Hq + kvh) * D;   // k (full: V from raw k)
      else src = rr + (long)(a.Hq + a.Hkv + kvh) * D;                                   // v
      fin_load<D>(raw[k], src);
      // (cos, sin) of this lane's pairs: the table row holds D / 2 pairs
      const float2* cr = f.rope_cs + (long)r * f.cs_ld + (D == 64 ? (lane & 31) : lane * FEH);
      if constexpr (FEH == 4) {
        const float4 c0 = *reinterpret_cast<const float4*>(cr), c1 = *reinterpret_cast<const float4*>(cr + 2);
        fcs[k][0] = make_float2(c0.x, c0.y); fcs[k][1] = make_float2(c0.z, c0.w);
        fcs[k][2] = make_float2(c1.x, c1.y); fcs[k][3] = make_float2(c1.z, c1.w);
      } else if constexpr (FEH == 2) {
        const float4 c0 = *reinterpret_cast<const float4*>(cr);
        fcs[k][0] = make_float2(c0.x, c0.y); fcs[k][1] = make_float2(c0.z, c0.w);
      } else {
        fcs[k][0] = *cr;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  base = __builtin_amdgcn_readfirstlane(base);   // uniform: the split bounds and rows are scalar
  const int P = base + row;
  const int lo = a.ring ? max(0, P - a.W + 1) : 0;
  const int Pl = MR ? base + rlast : P;               // MR: the union of the rows' ranges
  const int L = Pl - lo + 1;
  const int chunk = (L + a.S - 1) / a.S;
  const int st = lo + split * chunk;
  const int en = min(st + chunk, Pl + 1);
  const int P0new = a.fin_on ? base : 0x7FFFFFFF;   // first position formed in this step

  const int j = lane & 15, g = lane >> 4;
  // column j: row row + jr, query head jh of this KV head; it admits
  // positions lo_j .. P_j (its own window and causal bound)
  const int jr = MR ? j / a.GQ : 0, jh = MR ? j - jr * a.GQ : j;
  const bool col_ok = MR ? (j < a.GQ * rpw && row + jr <= rlast) : j < a.GQ;
  const int Pj = P + jr, loj = a.ring ? Pj - a.W + 1 : 0;

  uint16_t* vb = a.v + seq * a.seq_stride + (a.ring ? (long)kvh * a.R * D : 0);
  uint16_t* kb = VR ? vb : a.k + seq * a.seq_stride + (a.ring ? (long)kvh * a.R * D : 0);

  // ---- K and V of this wave's first tile, issued before anything waits.
  // MFMA row r of half h <-> tile position 8*(r/4) + 4h + r%4, so lane
  // (column j, group g) ends up holding positions 8g .. 8g+7 of the tile.
  // Rows formed in this step (p >= P0new) are not in the cache yet: their
  // lanes load cache row 0 and are patched from LDS after the prologue.
  constexpr bool EK = D <= 256;               // K of the first tile is loaded before the
                                              // prologue (D = 512: its 128 registers wait
                                              // for the prologue's); V always goes
                                              // straight into this wave's LDS rows
  uint16_t* vl = vlds + wave * 32 * VROW;
  h8_t KA[NKS], KB[NKS];
  h8_t KAl[NKS], KBl[NKS];                    // VR: fp16 lo parts of the rebuilt key elements
  // Cache rows of a tile.  Rows [0, nv) of the tile at t0 come from the cache
  // (the rest are masked out or formed in this step: they read row 0).  On a
  // ring layer, tile row r lives at slot (t0 + r) mod R; rings hold at least
  // 32 slots (the host checks), so the 32 rows of a tile wrap at most once: a
  // lane takes one remainder for its first row and steps from there with one
  // compare per row, with no division and no branch per row.
  const bool ringf = a.ring != 0;
  const int Rr = ringf ? a.R : 1;
  const int nv_end = min(en, P0new);
  // scalar tile geometry: slot of the tile's first position and the number
  // of tile rows read from the cache
  auto tile_geom = [&](int t0, int& s0, int& nv) {
    s0 = __builtin_amdgcn_readfirstlane(ringf ? t0 % Rr : t0);
    nv = __builtin_amdgcn_readfirstlane(nv_end - t0);
  };
  // cache row (in elements) of tile row r (r < 32)
  auto row_at = [&](int s0, int nv, int r) -> long {
    const int sl = ringf && r >= Rr - s0 ? s0 + r - Rr : s0 + r;
    return r < nv ? (long)sl * D : 0l;
  };
  auto load_k = [&](int t0) {
    int s0, nv;
    tile_geom(t0, s0, nv);
    const int ra = 8 * (j >> 2) + (j & 3);
    const uint16_t* ka = kb + row_at(s0, nv, ra) + 8 * g;
    const uint16_t* kc = kb + row_at(s0, nv, ra + 4) + 8 * g;
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      // VR: plain loads, so that the lines stay in the L2 for the V read
      const u4v* pa_ = reinterpret_cast<const u4v*>(ka + 32 * s);
      const u4v* pb_ = reinterpret_cast<const u4v*>(kc + 32 * s);
      KA[s] = __builtin_bit_cast(h8_t, VR ? *pa_ : __builtin_nontemporal_load(pa_));
      KB[s] = __builtin_bit_cast(h8_t, VR ? *pb_ : __builtin_nontemporal_load(pb_));
    }
  };
  // V: each instruction fills 1 KB of LDS, RPI = 512 / D consecutive tile
  // rows; lane l writes chunk position l mod (D / 8) of row l / (D / 8) and
  // so loads the global chunk that the swizzle puts there (D = 512: one row
  // per instruction, its address scalar)
  auto load_v = [&](int t0) {
    int s0, nv;
    tile_geom(t0, s0, nv);
    constexpr int CPR = D / 8, RPI = 64 / CPR;
    const int rl = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; i++) {
      const int r = RPI * i + rl;
      const int c = pc ^ (2 * vswz<D>(r));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(vb + row_at(s0, nv, r) + c * 8),
                                       reinterpret_cast<uint32_t*>(vl + RPI * i * VROW), 16, 0, 0);
    }
  };
  // the first tile: V, and for D <= 256 also K, before the prologue (with the
  // prologue's inputs that stays under the 63 vector loads a wave may have in
  // flight); K of D = 512 (128 registers) waits for the prologue's registers
  int t0 = st + 32 * wave;
  if (t0 < en) {
    if (EK) load_k(t0);
    load_v(t0);
  }
  if constexpr (VR) {
    const int i = threadIdx.x;
    if (i < NR) {
      const double f = i < a.krot ? pow(a.theta, -2.0 * (double)i / (double)D) : 0.0;
      const double r4 = 4.0 * f;
      vr_f[i] = f * 0.15915494309189535;                       // revolutions per position
      vr_c4[i] = make_float2((float)cos(r4), (float)sin(r4));
      vr_w[i] = a.kw[i];
      vr_w[NR + i] = a.kw[D / 2 + i];
    }
  }

  // ---- queries of this workgroup's columns as the MFMA B operand (VR: in
  // the steps whose key is kw * v, q * kw as fp16 hi in qb; the lo parts are
  // parked in LDS over the finished queries, qlo [NKS][64 lanes][8])
  h8_t qb[NKS], qlo[NKS];
  uint16_t* qlo_l = q16;
  auto set_q = [&](int s, u4v t) {
    if (VR && !rebuilt(s)) {
      const float4 w0 = *reinterpret_cast<const float4*>(a.kw + 32 * s + 8 * g);
      const float4 w1 = *reinterpret_cast<const float4*>(a.kw + 32 * s + 8 * g + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const h8_t qh = __builtin_bit_cast(h8_t, t);
      h8_t hi, lo;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float x = (float)qh[e] * wv[e];
        hi[e] = (_Float16)x;
        lo[e] = (_Float16)(x - (float)hi[e]);
      }
      qb[s] = hi;
      qlo[s] = lo;
    } else {
      qb[s] = __builtin_bit_cast(h8_t, t);
    }
  };
  if (a.fin_on) {
    const AttnFin& f = a.fin;
    // finish the jobs: every query head, and k and v of the rows of this
    // step that lie in [st, en) and that this row attends (rows r0 .. r1)
    const int r0 = max(0, st - base), r1 = min(row, en - 1 - base);
#pragma unroll
    for (int k = 0; k < MAXJ; k++) {
      const int jb = wave + 4 * k;
      if (jb >= njobs) break;
      if (jb < a.GQ) {
        finish_vals<D>(raw[k], wq, true, true, fcs[k], f.rot_pairs, f.eps, q16 + jb * D);
        continue;
      }
      const int r = (jb - a.GQ) >> 1;
      if (r < r0 || r > r1) continue;
      if (((jb - a.GQ) & 1) == 0) {
        if (!VR) finish_vals<D>(raw[k], wk, true, true, fcs[k], f.rot_pairs, f.eps, newK + r * D);
      } else if (f.v_norm) {
        finish_vals<D>(raw[k], wk, false, false, fcs[k], f.rot_pairs, f.eps, newV + r * D);
      } else {
        fin_store<D>(raw[k], newV + r * D);
      }
    }
    __syncthreads();
    // the workgroup whose own row lies in its range stores that row
    if (P >= st && P < en) {
      const long so = (long)(a.ring ? P % a.R : P) * D;
      for (int d = threadIdx.x; d < D; d += 256) {
        if (!VR) kb[so + d] = newK[row * D + d];
        vb[so + d] = newV[row * D + d];
      }
    }
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(q16 + (col_ok ? j : 0) * D + 32 * s + 8 * g);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      set_q(s, t);
    }
  } else {
    const uint16_t* qp = MR ? a.q + (((long)seq * a.n_rows + row + (col_ok ? jr : 0)) * a.Hq +
                                     (col_ok ? kvh * a.GQ + jh : 0)) * D + 8 * g
                            : a.q + (((long)seq * a.n_rows + row) * a.Hq + (col_ok ? kvh * a.GQ + j : 0)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(qp + 32 * s);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      set_q(s, t);
    }
  }
  if constexpr (VR) {
    __syncthreads();                          // every wave has read q16; the VR tables are in
    if (wave == 0) {
#pragma unroll
      for (int s = 0; s < NKS; s++)
        if (!rebuilt(s)) *reinterpret_cast<h8_t*>(qlo_l + (s * 64 + lane) * 8) = qlo[s];
    }
    __syncthreads();
  }

  float m_run = -INFINITY, l_part = 0.f;
  f4_t O[NDS];
#pragma unroll
  for (int d = 0; d < NDS; d++) O[d] = (f4_t){0.f, 0.f, 0.f, 0.f};

  for (bool first = true; t0 < en; t0 += 128, first = false) {
    if (!first || !EK) load_k(t0);
    if (!first) load_v(t0);
    if (t0 + 31 >= P0new) {                   // patch the rows formed in this step
      const int pa = t0 + 8 * (j >> 2) + (j & 3), pb = pa + 4;
      const uint16_t* nk = VR ? newV : newK;  // VR: the key is formed from the V row
#pragma unroll
      for (int s = 0; s < NKS; s++) {
        if (pa >= P0new && pa < en) KA[s] = *reinterpret_cast<const h8_t*>(nk + (pa - P0new) * D + 32 * s + 8 * g);
        if (pb >= P0new && pb < en) KB[s] = *reinterpret_cast<const h8_t*>(nk + (pb - P0new) * D + 32 * s + 8 * g);
      }
    }
    if constexpr (VR) {
      // key elements of the rotating steps: lane (j, g) holds positions
      // pa (KA) and pa + 4 (KB) at dims 32 s + 8 g + e and that + D/2
      const int pa = t0 + 8 * (j >> 2) + (j & 3);
#pragma unroll
      for (int s = 0; s < RS; s++) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int i = 32 * s + 8 * g + e;
          double r = (double)pa * vr_f[i];
          r -= floor(r);
          const float rv = (float)r;
          const float ca = __builtin_amdgcn_cosf(rv), sa = __builtin_amdgcn_sinf(rv);
          const float2 c4 = vr_c4[i];
          const float cb = ca * c4.x - sa * c4.y, sb = sa * c4.x + ca * c4.y;
          const float w0 = vr_w[i], w1 = vr_w[NR + i];
          auto form = [&](h8_t& X0, h8_t& X1, h8_t& L0, h8_t& L1, float c, float sn) {
            const float u0 = w0 * (float)X0[e], u1 = w1 * (float)X1[e];
            const float k0 = c * u0 - sn * u1, k1 = sn * u0 + c * u1;
            const _Float16 h0 = (_Float16)k0, h1 = (_Float16)k1;
            X0[e] = h0; L0[e] = (_Float16)(k0 - (float)h0);
            X1[e] = h1; L1[e] = (_Float16)(k1 - (float)h1);
          };
          form(KA[s], KA[s + HS], KAl[s], KAl[s + HS], ca, sa);
          form(KB[s], KB[s + HS], KBl[s], KBl[s + HS], cb, sb);
        }
      }
    }
    f4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA[s], qb[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB[s], qb[s], s1, 0, 0, 0);
      if (VR && rebuilt(s)) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KAl[s], qb[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KBl[s], qb[s], s1, 0, 0, 0);
      } else if (VR) {
        const h8_t ql = *reinterpret_cast<const h8_t*>(qlo_l + (s * 64 + lane) * 8);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA[s], ql, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB[s], ql, s1, 0, 0, 0);
      }
    }
    // lane (j, g): reg i of s0 -> position t0 + 8g + i; of s1 -> t0 + 8g + 4 + i
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (MR) {
        const int pa = t0 + 8 * g + i, pb = pa + 4;
        sv[i] = (pa < en && pa <= Pj && pa >= loj) ? s0[i] * a.scale_log2 : -INFINITY;
        sv[4 + i] = (pb < en && pb <= Pj && pb >= loj) ? s1[i] * a.scale_log2 : -INFINITY;
      } else {
        sv[i] = (t0 + 8 * g + i < en) ? s0[i] * a.scale_log2 : -INFINITY;
        sv[4 + i] = (t0 + 8 * g + 4 + i < en) ? s1[i] * a.scale_log2 : -INFINITY;
      }
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    // a column none of whose positions so far is admitted keeps m = -inf
    // and weights 0 (its rows' windows may start past this tile)
    const bool none = MR && m_new == -INFINITY;
    const float alpha = MR ? (none ? 1.f : exp2f(m_run - m_new)) : exp2f(m_run - m_new);
    m_run = m_new;
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      p[i] = MR ? (none ? 0.f : exp2f(sv[i] - m_new)) : exp2f(sv[i] - m_new);
      ps += p[i];
    }
    l_part = l_part * alpha + ps;
    // rescale O rows (heads 4g+i): their alpha lives in lane 4g+i
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; i++) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
    for (int d = 0; d < NDS; d++)
#pragma unroll
      for (int i = 0; i < 4; i++) O[d][i] *= al[i];
    h8_t Ahi, Alo;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const _Float16 hi = (_Float16)p[i];
      Ahi[i] = hi;
      Alo[i] = (_Float16)(p[i] - (float)hi);
    }
    // the tile's direct V loads have landed (waiting for them here, not
    // before QK, lets the scores go ahead as soon as K is in); rows formed in
    // this step overwrite theirs
    __builtin_amdgcn_s_waitcnt(0);
    __asm__ __volatile__("" ::: "memory");
    if (t0 + 31 >= P0new) {
      for (int r = 0; r < 32; r++) {
        const int pr = t0 + r;
        if (pr >= P0new && pr < en && lane < D / 8)
          *reinterpret_cast<u4v*>(vl + r * VROW + (lane ^ (2 * vswz<D>(r))) * 8) =
              *reinterpret_cast<const u4v*>(newV + (pr - P0new) * D + lane * 8);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // O += P V: B operand lane (dim 16d + j, group g) = V[8g .. 8g+7][dim].
    // A transposing 8-byte read gives lane j of a 16-lane group element j % 4
    // of the 4-half chunks addressed by lanes j / 4 + 4i of the group, as its
    // element i; so lane j addresses row 8g + 4h + j / 4 at column
    // 16d + 4 (j % 4) (16-byte chunk 2d + (j % 4) / 2, stored at chunk
    // position 2 (d ^ vswz) + (j % 4) / 2 of the row), and reads h = 0, 1
    // return elements 4h .. 4h+3.  Both rows share the swizzle.
    const int sw = vswz<D>(8 * g + (j >> 2));
    const uint16_t* vt = vl + (8 * g + (j >> 2)) * VROW + 4 * (j & 3);
#pragma unroll
    for (int d = 0; d < NDS; d++) {
      typedef short v4s_t __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s_t lds_v4s;
      const int cd = 16 * (d ^ sw);
      const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vt + cd));
      const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vt + 4 * VROW + cd));
      // joined as one vector: filling Bv element by element from lo and hi
      // compiled to a wrong operand (the low half of each read repeated)
      const h8_t Bv = __builtin_bit_cast(h8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[d], 0, 0, 0);
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[d], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  // column totals of l over the 4 lane groups
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  // record of column col, or NULL for columns without a row and head
  auto rec_of = [&](int col) -> float* {
    int rr = row, hh = col;
    if (MR) {
      rr = row + col / a.GQ;
      hh = col - (col / a.GQ) * a.GQ;
      if (col >= a.GQ * rpw || rr > rlast) return nullptr;
    } else if (col >= a.GQ) {
      return nullptr;
    }
    return a.part + attn_rec(a, seq, rr, kvh, split, hh, D);
  };
  // ---- a split of at most one tile: wave 0 holds the whole record and
  // stores it from registers (the merge below would give the same values:
  // the other waves' weights are 0 and wave 0's is 1)
  if (en - st <= 32) {
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float* rec = MR ? rec_of(4 * g + i)
                      : (4 * g + i < a.GQ ? a.part + attn_rec(a, seq, row, kvh, split, 4 * g + i, D) : nullptr);
      if (rec) {
#pragma unroll
        for (int d = 0; d < NDS; d++) rec[16 * d + j] = O[d][i];
      }
    }
    if (lane < (MR ? 16 : a.GQ)) {
      float* rec = MR ? rec_of(lane) : a.part + attn_rec(a, seq, row, kvh, split, lane, D);
      if (rec) {
        rec[D] = m_run;
        rec[D + 1] = l_tot;
      }
    }
    return;
  }

  // ---- merge the 4 waves (the V rows are free now): per head the wave
  // maxima meet in LDS; each wave rescales its own O rows in registers and
  // stores them as one float4 per (dim step, lane), the 4 heads of that lane
  // (conflict-free 16-byte LDS writes); then every thread adds the four
  // waves' float4s of its items in a fixed order and stores them to the
  // records.  LDS: 4 * NDS * 64 float4 (D = 512: 128 KB, inside the V rows).
  __syncthreads();
  if (lane < 16) { wm[wave][lane] = m_run; wl[wave][lane] = l_tot; }
  __syncthreads();
  static_assert((size_t)4 * 32 * VROW * 2 >= (size_t)4 * NDS * 64 * 16, "merge buffer inside the V rows");
  f4_t* ow = reinterpret_cast<f4_t*>(smem);       // [4][NDS][64]
  {
    float fw[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int hc = 4 * g + i;
      const float M = fmaxf(fmaxf(wm[0][hc], wm[1][hc]), fmaxf(wm[2][hc], wm[3][hc]));
      fw[i] = (M == -INFINITY) ? 0.f : exp2f(wm[wave][hc] - M);
    }
#pragma unroll
    for (int d = 0; d < NDS; d++)
      ow[(wave * NDS + d) * 64 + lane] = (f4_t){O[d][0] * fw[0], O[d][1] * fw[1], O[d][2] * fw[2], O[d][3] * fw[3]};
  }
  __syncthreads();
  {
    // items (d, lane) with d = wave + 4k: heads 4g + i at dim 16d + j
    constexpr int NI = NDS / 4;
    f4_t acc[NI];
#pragma unroll
    for (int k = 0; k < NI; k++) {
      const int d = wave + 4 * k;
      const f4_t v0 = ow[(0 * NDS + d) * 64 + lane], v1 = ow[(1 * NDS + d) * 64 + lane];
      const f4_t v2 = ow[(2 * NDS + d) * 64 + lane], v3 = ow[(3 * NDS + d) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; i++) acc[k][i] = ((v0[i] + v1[i]) + v2[i]) + v3[i];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float* rec = MR ? rec_of(4 * g + i)
                      : (4 * g + i < a.GQ ? a.part + attn_rec(a, seq, row, kvh, split, 4 * g + i, D) : nullptr);
      if (rec) {
#pragma unroll
        for (int k = 0; k < NI; k++) rec[16 * (wave + 4 * k) + j] = acc[k][i];
      }
    }
  }
  if (MR ? (threadIdx.x < 16 && rec_of(threadIdx.x)) : threadIdx.x < a.GQ) {
    const int col = threadIdx.x;
    const float M = fmaxf(fmaxf(wm[0][col], wm[1][col]), fmaxf(wm[2][col], wm[3][col]));
    float l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; w++) l += exp2f(wm[w][col] - M) * wl[w][col];
    }
    float* rec = MR ? rec_of(col) : a.part + attn_rec(a, seq, row, kvh, split, col, D);
    rec[D] = M;
    rec[D + 1] = l;
  }
}

// out[seq][row][h][d] = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// Grid (n_seq * n_rows * Hq, D / 64), 256 threads: lane = output dim, wave w
// takes splits w, w + 4, ... (S <= MAXS).  Every load of the workgroup is
// issued before the first use (split indices past S are clamped and their
// weight is zero), and the four wave sums meet in LDS in a fixed order.
constexpr int kMaxSplits = 256;

template <int D, int MAXS>
__global__ void __launch_bounds__(256) k_fd_combine(AttnArgs a, float* out32, uint16_t* out16) {
  constexpr int PER = MAXS / 4;
  __shared__ float wsp[MAXS];
  __shared__ float red[4][64];
  __shared__ float rm[4], rl[4];
  const int idx = blockIdx.x;
  const int h = a.kvh_major ? (idx % a.Hkv) * a.GQ + (idx / a.Hkv) % a.GQ : idx % a.Hq, sr = idx / a.Hq;
  const int seq = sr / a.n_rows, row = sr - seq * a.n_rows;
  const int kvh = h / a.GQ, col = h - kvh * a.GQ;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long r0 = attn_rec(a, seq, row, kvh, 0, col, D);
  const long rs = (long)a.GQ * (D + 4);                // stride between splits
  const int d = blockIdx.y * 64 + lane;
  const int S = a.S;
  const bool own = tid < S;
  const long mo = r0 + (long)min(tid, S - 1) * rs + D;
  const float m_raw = a.part[mo], l_raw = a.part[mo + 1];
  float ov[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) ov[i] = a.part[r0 + (long)min(wave + 4 * i, S - 1) * rs + d];
  const float m = own ? m_raw : -INFINITY;
  float M = wave_max(m);
  if (lane == 0) rm[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
  const float w = (own && m != -INFINITY) ? exp2f(m - M) : 0.f;
  if (tid < MAXS) wsp[tid] = w;
  float L = wave_sum(w * (own ? l_raw : 0.f));
  if (lane == 0) rl[wave] = L;
  __syncthreads();
  L = ((rl[0] + rl[1]) + rl[2]) + rl[3];
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < PER; i++) o += wsp[wave + 4 * i] * ov[i];
  red[wave][lane] = o;
  __syncthreads();
  if (wave == 0) {
    o = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    o *= (L > 0.f) ? 1.0f / L : 0.f;
    const long oi = (((long)seq * a.n_rows + row) * a.Hq + h) * D + d;
    if (out32) out32[oi] = o;
    if (out16) out16[oi] = f2h(o);
  }
}

}  // namespace q4k
