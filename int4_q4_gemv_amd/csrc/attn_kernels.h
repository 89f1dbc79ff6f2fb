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
  uint16_t* q_out;        // [rows][Hq][D] or NULL: split 0 also stores its finished queries
                          // (the step's stage export reads them)
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
    if (f.q_out && split == 0) {
      constexpr int CH = D / 8;               // 16-byte chunks per head
      for (int i = threadIdx.x; i < a.GQ * CH; i += 256) {
        const int jq = i / CH, c = i - jq * CH;
        *reinterpret_cast<u4v*>(f.q_out + ((long)row * a.Hq + kvh * a.GQ + jq) * D + c * 8) =
            *reinterpret_cast<const u4v*>(q16 + jq * D + c * 8);
      }
    }
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
    mt = rows_max(mt);
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
  float l_tot = rows_sum(l_part);

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

// The step's first position, read in two parts: pos_issue loads the word
// that holds it with the step parameters on the device (else any valid word:
// the records), by a vector load through an address the compiler cannot prove
// uniform, and pos_take picks the value where it is first used.  A scalar
// load would be waited for together with the kernel's argument loads, before
// the loads that do not need the position are issued; a vector load is waited
// for only where the position is used, by a count that leaves the loads
// issued after it in flight.
Q4_DEV int pos_issue(const AttnArgs& a) {
  int z = 0;
  __asm__ __volatile__("" : "+v"(z));   // an opaque zero
  const int* w = a.sp ? &a.sp->pos0 : reinterpret_cast<const int*>(a.part);
  return ((const __attribute__((address_space(1))) int*)w)[z];
}
Q4_DEV int pos_take(const AttnArgs& a, int loaded, int seq) {
  return __builtin_amdgcn_readfirstlane(a.sp ? loaded : a.pos0[seq]);
}

// Ring layers whose splits hold at most one 32-position tile (S * 32 >= W).
// With one tile per workgroup, k_fd_partial streams it from one wave while
// the other three wait; here the head dimension is dealt to the 4 waves
// instead.  Wave w loads the keys' dims [w D/4, (w+1) D/4) of all 32
// positions (its D/128 QK k steps) and V rows 8w .. 8w+7 of the tile into
// one shared LDS tile; the waves' partial scores meet in LDS and are added
// in a fixed order, every wave runs the same softmax on the sums, and wave w
// forms O for its own D/4 dims over the 32 rows.  A wave then has a quarter
// of the tile in flight (8 KB at D = 256) rather than one wave holding all of
// it, and that is what keeps the memory pipeline full when a CU holds one
// workgroup.  Splits, masking, the finishing prologue (FIN), the records and
// the combine are those of k_fd_partial (one tile, no merge of waves).  The
// LDS objects the kernel uses, static and separate, total ds_lds_bytes.
//
// MR (a.rpw rows per workgroup, with the finishing prologue): as in
// k_fd_partial, the MFMA columns are (row, query head) pairs masked to their
// own row's window.  The splits divide the first row's window (S * 32 >=
// W); a later row's own positions past it (formed in this step, at most
// rpw - 1) are added by the combine (k_fd_combine, TAIL) from the cache.  The
// workgroup forms the queries of all its columns and the K/V rows of the
// step in its range; the split holding the first row's position finishes and
// stores all the workgroup's rows: a block of rows then needs no launch of
// its own to finish them.
template <int D>
constexpr size_t ds_lds_bytes() {
  return (size_t)32 * fd_vpitch<D>() * 2 + (size_t)2 * 4 * D * 2 + (size_t)16 * D * 2 + (size_t)4 * 2 * 64 * 16;
}

template <int D, bool MR = false, bool FIN = false>
__global__ void __launch_bounds__(256) k_fd_ring_ds(AttnArgs a) {
  static_assert(D >= 128 && D <= 512, "a wave takes whole QK k steps");
  static_assert(sizeof(AttnArgs) >= 128 + 4, "argument lines fetched below lie inside the struct");
  kernarg_fetch<0, 64, 128>();                // the argument lines this kernel reads
  constexpr int VROW = fd_vpitch<D>();
  constexpr int KS = D / 128;                 // QK k steps of a wave
  constexpr int DS = D / 64;                  // PV dim steps of a wave
  constexpr int DW = D / 4;                   // dims of a wave
  // LDS objects of their own: the compiler then knows that the accesses to
  // the step's rows, the queries and the scores do not touch the V rows still
  // arriving, and waits for those only where they are read
  __shared__ __align__(16) uint16_t vl[32 * VROW];     // the tile's V rows
  __shared__ __align__(16) uint16_t nkv[2 * 4 * D];    // rows of this step: K [4][D], V [4][D]
  __shared__ __align__(16) uint16_t q16[16 * D];       // finished queries
  __shared__ f4_t sx[4 * 2 * 64];                      // [4 waves][2][64] partial scores
  uint16_t* newK = nkv;
  uint16_t* newV = nkv + 4 * D;
  static_assert(ds_lds_bytes<D>() <= 160 * 1024, "LDS of one workgroup");

  // ---- the step's first position, issued before anything else (a valid
  // word for every workgroup, so also ahead of the early exit below)
  const int pos_w = pos_issue(a);

  const int split = a.kvh_major ? blockIdx.y : blockIdx.x, kvh = a.kvh_major ? blockIdx.x : blockIdx.y;
  // rows of this workgroup: row .. rlast (one unless MR); its columns.  All
  // the rows in one workgroup (or one row): no division ahead of the loads
  const int rpw = MR && a.rpw > 1 ? a.rpw : 1;
  int seq = blockIdx.z, row = 0;
  if (a.n_rows > rpw) {
    if constexpr (MR) {
      const int nrg = (a.n_rows + rpw - 1) / rpw;
      seq = blockIdx.z / nrg;
      row = (blockIdx.z - seq * nrg) * rpw;
    } else {
      seq = blockIdx.z / a.n_rows;
      row = blockIdx.z - seq * a.n_rows;
    }
  }
  if (row >= a.n_rows) return;
  const int rlast = MR ? min(a.n_rows, row + rpw) - 1 : row;
  const int ncols = a.GQ * (rlast - row + 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

  // ---- inputs of the finishing prologue (FIN): jobs dealt round-robin to
  // the waves (this workgroup's columns, then k and v of rows 0 .. rlast).
  // Every wave loads MAXJ jobs' inputs, those past the last job repeating
  // job 0's, so the count of loads is the same on every path.
  constexpr int FE = D / 64, FEH = fin_h<D>();
  constexpr int MAXJ = (16 + 2 * 4 + 3) / 4;
  const int njobs = FIN ? ncols + 2 * (rlast + 1) : 0;
  float raw[MAXJ][FE], wq[FE], wk[FE];
  float2 fcs[MAXJ][FEH];
  if constexpr (FIN) {
    const AttnFin& f = a.fin;
    fin_load<D>(wq, f.q_norm);
    fin_load<D>(wk, f.k_norm);
#pragma unroll
    for (int k = 0; k < MAXJ; k++) {
      const int jb = wave + 4 * k < njobs ? wave + 4 * k : 0;
      const int jq = MR ? jb / a.GQ : 0;      // a column's row offset
      const int r = jb < ncols ? row + jq : (jb - ncols) >> 1;
      const float* rr = f.qkv + (long)r * f.ldq;
      const float* src;
      if (jb < ncols) src = rr + (long)(kvh * a.GQ + jb - jq * a.GQ) * D;
      else if (((jb - ncols) & 1) == 0) src = rr + (long)(a.Hq + kvh) * D;
      else src = rr + (long)(a.Hq + a.Hkv + kvh) * D;
      fin_load<D>(raw[k], src);
      const float2* cr = f.rope_cs + (long)r * f.cs_ld + lane * FEH;
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

  const int base = pos_take(a, pos_w, seq);
  const int P = base + row;
  const int lo = max(0, P - a.W + 1);
  const int Pl = base + rlast;                // MR: the union of the rows' ranges
  // splits of chunk positions over the first row's window (chunk <= 32: the
  // host launches this kernel only then).  MR: the later rows' positions past
  // it (P + 1 .. Pl, formed in this step) are left to the combine; the split
  // holding P finishes and stores those rows.
  const int chunk = (P - lo + a.S) / a.S;
  const int st = lo + split * chunk;
  const int en = min(st + chunk, P + 1);
  const bool has = st < en;                   // workgroup-uniform
  const bool holds_p = P >= st && P < en;
  const int P0new = FIN ? base : 0x7FFFFFFF;

  const int j = lane & 15, g = lane >> 4;
  // column j: row row + jr, query head jh; it admits positions loj .. Pj
  const int jr = MR ? j / a.GQ : 0, jh = j - jr * a.GQ;
  const bool col_ok = j < ncols;
  const int Pj = P + jr, loj = Pj - a.W + 1;
  uint16_t* vb = a.v + seq * a.seq_stride + (long)kvh * a.R * D;
  uint16_t* kb = a.k + seq * a.seq_stride + (long)kvh * a.R * D;

  // ---- a tile's K elements and V rows.  Row r of the tile at t0 lives at
  // slot (t0 + r) mod R (R >= 32: one wrap at most); rows past nv are masked
  // or formed in this step and read slot 0.  Lane (column j, group g) holds
  // positions 8g .. 8g+7 of the tile (MFMA row r of half h <-> tile position
  // 8 (r / 4) + 4h + r % 4).  The V rows travel through registers (RPI rows
  // per instruction, lane l holding 16-byte chunk l mod CPR of its row, the
  // one the swizzle puts there) and are written to LDS once the scores are
  // formed: with loads into registers only, and the same loads on every path
  // (an empty split loads row 0), the compiler's waits are counts, so the
  // prologue's finishing and the scores wait for their own inputs, not for
  // the whole tile.
  constexpr int CPR = D / 8, RPI = 64 / CPR;   // 16-byte chunks per row, rows per instruction
  h8_t KA[KS], KB[KS];
  u4v vr[8 / RPI];
  auto load_tile = [&](int t0) {
    const int s0 = __builtin_amdgcn_readfirstlane(t0 % a.R);
    const int nv = __builtin_amdgcn_readfirstlane(min(en, P0new) - t0);
    auto row_at = [&](int r) -> long {
      const int sl = r >= a.R - s0 ? s0 + r - a.R : s0 + r;
      return r < nv ? (long)sl * D : 0l;
    };
    const int ra = 8 * (j >> 2) + (j & 3);
    const uint16_t* ka = kb + row_at(ra) + DW * wave + 8 * g;
    const uint16_t* kc = kb + row_at(ra + 4) + DW * wave + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      KA[s] = __builtin_bit_cast(h8_t, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(ka + 32 * s)));
      KB[s] = __builtin_bit_cast(h8_t, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(kc + 32 * s)));
    }
    const int rl = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < 8 / RPI; i++) {
      const int r = 8 * wave + RPI * i + rl;
      const int c = pc ^ (2 * vswz<D>(r));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(vb + row_at(r) + c * 8));
    }
  };
  load_tile(st);                              // issued before anything waits

  // ---- queries (as the MFMA B operand, this wave's k steps)
  h8_t qb[KS];
  if constexpr (FIN) {
    const AttnFin& f = a.fin;
    const int r0 = max(0, st - base), r1 = holds_p ? rlast : min(rlast, en - 1 - base);
#pragma unroll
    for (int k = 0; k < MAXJ; k++) {
      const int jb = wave + 4 * k;
      if (jb >= njobs) break;
      if (jb < ncols) {
        finish_vals<D>(raw[k], wq, true, true, fcs[k], f.rot_pairs, f.eps, q16 + jb * D);
        continue;
      }
      const int r = (jb - ncols) >> 1;
      if (r < r0 || r > r1) continue;
      if (((jb - ncols) & 1) == 0) finish_vals<D>(raw[k], wk, true, true, fcs[k], f.rot_pairs, f.eps, newK + r * D);
      else if (f.v_norm) finish_vals<D>(raw[k], wk, false, false, fcs[k], f.rot_pairs, f.eps, newV + r * D);
      else fin_store<D>(raw[k], newV + r * D);
    }
    lds_barrier();
    if (f.q_out && split == 0) {
      constexpr int CH = D / 8;
      for (int i = threadIdx.x; i < ncols * CH; i += 256) {
        const int jq = i / CH, c = i - jq * CH, qr = jq / a.GQ;
        *reinterpret_cast<u4v*>(f.q_out + ((long)(row + qr) * a.Hq + kvh * a.GQ + jq - qr * a.GQ) * D + c * 8) =
            *reinterpret_cast<const u4v*>(q16 + jq * D + c * 8);
      }
    }
#pragma unroll
    for (int s = 0; s < KS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(q16 + (col_ok ? j : 0) * D + DW * wave + 32 * s + 8 * g);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      qb[s] = __builtin_bit_cast(h8_t, t);
    }
  } else {
    const uint16_t* qp = a.q + (((long)seq * a.n_rows + row + (col_ok ? jr : 0)) * a.Hq +
                                (col_ok ? kvh * a.GQ + jh : 0)) * D + DW * wave + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(qp + 32 * s);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      qb[s] = __builtin_bit_cast(h8_t, t);
    }
  }

  // ---- the split's tile: scores, softmax, O += P V
  f4_t O[DS];
#pragma unroll
  for (int d = 0; d < DS; d++) O[d] = (f4_t){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l_tot = 0.f;
  if (has) {
    // keys of the rows formed in this step come from LDS
    if (st + 31 >= P0new) {
      const int pa = st + 8 * (j >> 2) + (j & 3), pb = pa + 4;
#pragma unroll
      for (int s = 0; s < KS; s++) {
        const int off = DW * wave + 32 * s + 8 * g;
        if (pa >= P0new && pa < en) KA[s] = *reinterpret_cast<const h8_t*>(newK + (pa - P0new) * D + off);
        if (pb >= P0new && pb < en) KB[s] = *reinterpret_cast<const h8_t*>(newK + (pb - P0new) * D + off);
      }
    }
    f4_t p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; s++) {
      p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA[s], qb[s], p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB[s], qb[s], p1, 0, 0, 0);
    }
    sx[(2 * wave) * 64 + lane] = p0;
    sx[(2 * wave + 1) * 64 + lane] = p1;
    // this wave's V rows to LDS (lane l: bytes 16 l .. of RPI rows from row
    // 8 wave + RPI i); rows formed in this step overwrite theirs
#pragma unroll
    for (int i = 0; i < 8 / RPI; i++)
      *reinterpret_cast<u4v*>(vl + (8 * wave + RPI * i) * VROW + lane * 8) = vr[i];
    if (st + 31 >= P0new) {
#pragma unroll
      for (int r = 8 * wave; r < 8 * wave + 8; r++) {
        const int pr = st + r;
        if (pr >= P0new && pr < en && lane < D / 8)
          *reinterpret_cast<u4v*>(vl + r * VROW + (lane ^ (2 * vswz<D>(r))) * 8) =
              *reinterpret_cast<const u4v*>(newV + (pr - P0new) * D + lane * 8);
      }
    }
  }
  lds_barrier();
  if (has) {
    // full scores: the 4 waves' parts added in a fixed order
    f4_t c0 = sx[0 * 64 + lane], c1 = sx[1 * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; w++) {
      const f4_t e0 = sx[(2 * w) * 64 + lane], e1 = sx[(2 * w + 1) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; i++) { c0[i] += e0[i]; c1[i] += e1[i]; }
    }
    // lane (j, g): reg i of c0 -> position st + 8g + i; of c1 -> st + 8g + 4 + i
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int pa = st + 8 * g + i, pb = pa + 4;
      sv[i] = (pa < en && (!MR || pa >= loj)) ? c0[i] * a.scale_log2 : -INFINITY;
      sv[4 + i] = (pb < en && (!MR || pb >= loj)) ? c1[i] * a.scale_log2 : -INFINITY;
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mt = fmaxf(mt, sv[i]);
    mt = rows_max(mt);
    m = mt;                                   // one row: finite, position st is admitted
    // MR: a column that admits none of the tile's positions (its row's
    // window starts past it) keeps m = -inf, l = 0 and O = 0
    const bool none = MR && m == -INFINITY;
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      p[i] = none ? 0.f : exp2f(sv[i] - m);
      ps += p[i];
    }
    l_tot = rows_sum(ps);
    h8_t Ahi, Alo;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const _Float16 hi = (_Float16)p[i];
      Ahi[i] = hi;
      Alo[i] = (_Float16)(p[i] - (float)hi);
    }
    // O += P V over this wave's dims (the transposing reads of k_fd_partial)
    const int sw = vswz<D>(8 * g + (j >> 2));
    const uint16_t* vt = vl + (8 * g + (j >> 2)) * VROW + 4 * (j & 3);
#pragma unroll
    for (int dd = 0; dd < DS; dd++) {
      typedef short v4s_t __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s_t lds_v4s;
      const int cd = 16 * ((DS * wave + dd) ^ sw);
      const v4s_t vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vt + cd));
      const v4s_t vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vt + 4 * VROW + cd));
      const h8_t Bv = __builtin_bit_cast(h8_t, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
      O[dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[dd], 0, 0, 0);
      O[dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[dd], 0, 0, 0);
    }
  }
  // ---- records: wave w stores its dims of every column; wave 0 also m and
  // l (an empty split stores O = 0, m = -inf, l = 0).  Column c's record lies
  // c / GQ rows and c mod GQ heads past the workgroup's first: lane c holds
  // that offset (32 bits, from the column split above), the other lanes
  // fetch it, and one scalar base serves every store.  With one wave per
  // SIMD the wave issues every instruction itself, and 64-bit index
  // arithmetic per record would take longer than the stores.
  // All four offsets are formed before the first store, so no register of
  // a store in flight is reused (which would wait for the store).
  float* rbase = a.part + attn_rec(a, seq, row, kvh, split, 0, D);
  const unsigned my_off = (unsigned)(jr * (a.Hkv * a.S * a.GQ * (D + 4)) + jh * (D + 4));
  unsigned offs[4];
#pragma unroll
  for (int i = 0; i < 4; i++) offs[i] = (unsigned)__shfl((int)my_off, 4 * g + i, 64) + 16 * DS * wave + j;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (4 * g + i < ncols) {
#pragma unroll
      for (int dd = 0; dd < DS; dd++) rbase[offs[i] + 16 * dd] = O[dd][i];
    }
  }
  if (wave == 0 && lane < ncols) {
    rbase[my_off + D] = m;
    rbase[my_off + D + 1] = l_tot;
  }
  // the split holding P stores the rows of this workgroup (P .. Pl), last:
  // nothing waits for these stores
  if constexpr (FIN) {
    for (int rr = row; rr <= rlast; rr++) {
      const int Pr = base + rr;
      if (holds_p) {
        const long so = (long)(Pr % a.R) * D;
        for (int d = threadIdx.x; d < D; d += 256) {
          kb[so + d] = newK[rr * D + d];
          vb[so + d] = newV[rr * D + d];
        }
      }
    }
  }
}

// Full layers (positions 0 .. P, one KV head per cache): 8 waves as 2 groups
// of 4.  The 32-position tiles covering 0 .. P are dealt to the S splits
// round-robin (split s: tiles s, s + S, s + 2S, ...), so in each round the
// workgroups together read one contiguous stretch of the cache.  In round r
// group c takes the split's tile 2r + c.  Inside a group the head dimension
// is dealt to the waves as in k_fd_ring_ds, but by QK k step round-robin
// (wave w: steps w, w + 4, ...): the RoPE partner of a dim lies D/64 k steps
// on, a multiple of 4, so with one cached row per position (VR) a wave
// rebuilds its keys from its own V elements.  The partial scores meet in
// LDS, every wave of a group runs the group's online softmax on the sums and
// forms O for its own D/4 dims.  At the end group 1 hands its rescaled O to
// group 0 through LDS, which writes the split's records.
//
// Loads in flight: a round's K elements (to registers) and V rows (straight
// to LDS) are issued as soon as the previous round's scores are formed, so
// they arrive during that round's softmax and PV; the even rounds' V rows
// sit in one array, the odd rounds' in another.  A round starts by waiting
// for all of its wave's loads, then a barrier.  With one row per position the
// keys are read from the tile's V rows in LDS once every wave's rows have
// landed, so the cache is read once and no key load is on the round's path.
// The V arrays are LDS objects of their own, and the direct loads and the PV
// reads go through restrict pointers (lds_dma16, lds_tr8): the compiler then
// knows that the LDS accesses to the scores, the queries, the step's rows
// and the round's own V rows do not touch the rows still arriving in the
// other array, and does not wait for those (it otherwise waited for every
// load in flight before the PV reads, so the next round's tiles could not
// overlap this round's PV).  Every
// round issues the same loads whether or not the group has such a tile
// (without one, all lanes read row 0: one line per instruction), so the
// count of loads in flight, and with it each wait, is the same on every path.
//
// V rows in LDS are unpadded: the 16-byte chunk c of tile row r sits at chunk
// position c ^ 2 fds_swz(r), the swizzle k_fd_partial uses for D <= 256 (the
// transposing reads of a 16-lane group then touch distinct banks for any row
// pitch that is a multiple of 512 bytes).
Q4_DEV int fds_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

// waits until at most N vector memory instructions of this wave are in flight
template <int N>
Q4_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __asm__ __volatile__("" ::: "memory");
}

template <int N> struct fds_ic { static constexpr int v = N; };

// queries [16][D], reused for the partial scores [2 groups][4 waves][2][64] float4
template <int D>
constexpr int fds_qx_halves() { return 16 * D > 8192 ? 16 * D : 8192; }

// LDS accesses through restrict pointers of inlined helpers carry alias-scope
// metadata, which the compiler's wait insertion needs before it will tell a
// read of one LDS buffer from a direct-to-LDS load into another buffer (it
// then waits for the loads into the buffer read only; without the metadata it
// waits for every direct load in flight).  The waits that make a buffer's
// loads complete before it is read stay explicit in the kernels.
// One 16-byte direct-to-LDS load per lane.
__device__ __attribute__((always_inline)) inline void lds_dma16(const uint16_t* src, uint16_t* __restrict__ dst) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), 16, 0, 0);
}
// Transposing reads of two 4 x 16-bit groups (rows p and p + off_hi) as one
// 8-half MFMA operand.
__device__ __attribute__((always_inline)) inline h8_t lds_tr8(const uint16_t* __restrict__ p, int off_hi) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4_t lds_s4;
  const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
  const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p + off_hi));
  return __builtin_bit_cast(h8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D, bool VR>
__global__ void __launch_bounds__(512) k_fd_full_ds(AttnArgs a) {
  static_assert(D == 256 || D == 512, "a wave's k steps pair with their RoPE partners");
  static_assert(sizeof(AttnArgs) >= 192 + 4, "argument lines fetched below lie inside the struct");
  kernarg_fetch<0, 64, 128, 192>();           // the argument lines this kernel reads
  constexpr int G = 2;                        // wave groups
  constexpr int KS = D / 128;                 // QK k steps of a wave (global step w + 4k)
  constexpr int DS = D / 64;                  // PV dim steps of a wave (global DS w + dd)
  constexpr int HS = D / 64;                  // k steps per half head
  constexpr int RS = vr_rsteps<D>();          // VR: rotating k steps of the first half
  constexpr int NR = VR ? 32 * RS : 1;
  constexpr int CPR = D / 8, RPI = 64 / CPR;  // V: 16-byte chunks per row, rows per instruction
  constexpr int NVS = 8 / RPI;                // V loads of a wave per tile (its 8 rows)
  __shared__ __align__(16) uint16_t vA[G * 32 * D];   // V rows of the even rounds' tiles [G][32][D]
  __shared__ __align__(16) uint16_t vB[G * 32 * D];   // ... of the odd rounds' tiles
  __shared__ __align__(16) uint16_t qx[fds_qx_halves<D>()];
  __shared__ __align__(16) uint16_t nkv[2 * 4 * D];   // rows of this step: K [4][D], V [4][D]
  __shared__ float wm[G][16], wl[G][16];
  __shared__ double vr_f[NR];
  __shared__ float2 vr_c4[NR];
  __shared__ float vr_w[2 * NR];
  static_assert((size_t)G * 32 * D * 2 >= (size_t)4 * DS * 64 * 16, "merge buffer inside the V rows");
  uint16_t* newK = nkv;
  uint16_t* newV = nkv + 4 * D;
  uint16_t* q16 = qx;                         // [16][D] finished queries, then
  f4_t* sx = reinterpret_cast<f4_t*>(qx);     // [G][4 waves][2][64] partial scores
  auto rebuilt = [](int s) { return VR && (s < RS || (s >= HS && s < HS + RS)); };

  const int pos_w = pos_issue(a);             // the step's first position, issued first

  const int split = blockIdx.x, kvh = blockIdx.y;
  int seq = blockIdx.z, row = 0;              // one row: no division ahead of the loads
  if (a.n_rows > 1) {
    seq = blockIdx.z / a.n_rows;
    row = blockIdx.z - seq * a.n_rows;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = wave >> 2, w = wave & 3;
  const int j = lane & 15, g = lane >> 4;
  const bool col_ok = j < a.GQ;

  // ---- queries of a call without the finishing prologue: issued first, so
  // that no K/V load is ahead of them
  u4v qraw[KS];
  if (!a.fin_on) {
    const uint16_t* qp =
        a.q + (((long)seq * a.n_rows + row) * a.Hq + (col_ok ? kvh * a.GQ + j : 0)) * D + 8 * g;
#pragma unroll
    for (int k = 0; k < KS; k++) qraw[k] = *reinterpret_cast<const u4v*>(qp + 32 * (w + 4 * k));
  }
  // ---- finishing inputs, dealt round-robin to the 8 waves: this
  // workgroup's query heads, then k and v of rows 0 .. row (both from the
  // raw k projection on a full layer)
  constexpr int FE = D / 64, FEH = fin_h<D>();
  constexpr int MAXJ = (16 + 2 * 4 + 7) / 8;
  const int njobs = a.fin_on ? a.GQ + 2 * (row + 1) : 0;
  float raw[MAXJ][FE], wq[FE], wk[FE];
  float2 fcs[MAXJ][FEH];
  if (a.fin_on) {
    const AttnFin& f = a.fin;
    fin_load<D>(wq, f.q_norm);
    fin_load<D>(wk, f.k_norm);
#pragma unroll
    for (int k = 0; k < MAXJ; k++) {
      const int jb = wave + 8 * k;
      if (jb >= njobs) break;
      const int r = jb < a.GQ ? row : (jb - a.GQ) >> 1;
      const float* rr = f.qkv + (long)r * f.ldq;
      const float* src = jb < a.GQ ? rr + (long)(kvh * a.GQ + jb) * D : rr + (long)(a.Hq + kvh) * D;
      fin_load<D>(raw[k], src);
      const float2* cr = f.rope_cs + (long)r * f.cs_ld + lane * FEH;
      if constexpr (FEH == 4) {
        const float4 c0 = *reinterpret_cast<const float4*>(cr), c1 = *reinterpret_cast<const float4*>(cr + 2);
        fcs[k][0] = make_float2(c0.x, c0.y); fcs[k][1] = make_float2(c0.z, c0.w);
        fcs[k][2] = make_float2(c1.x, c1.y); fcs[k][3] = make_float2(c1.z, c1.w);
      } else {
        const float4 c0 = *reinterpret_cast<const float4*>(cr);
        fcs[k][0] = make_float2(c0.x, c0.y); fcs[k][1] = make_float2(c0.z, c0.w);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const int base = pos_take(a, pos_w, seq);
  const int P = base + row;
  // this split's tiles: split, split + S, ... of the 32-position tiles
  // covering 0 .. P (positions past P are masked)
  const int en = P + 1;
  const int ntile = split <= (P >> 5) ? ((P >> 5) - split) / a.S + 1 : 0;
  const int nround = (ntile + G - 1) / G;
  auto tile0 = [&](int i) { return 32 * (split + a.S * i); };
  auto owns = [&](int p) { return p <= P && (p >> 5) % a.S == split; };
  const int P0new = a.fin_on ? base : 0x7FFFFFFF;
  const int nv_end = min(en, P0new);

  uint16_t* vb = a.v + seq * a.seq_stride;
  uint16_t* kb = VR ? vb : a.k + seq * a.seq_stride;
  // cache row (elements) of tile row r; rows past nv_end are masked or
  // formed in this step and read row 0
  auto row_at = [&](int t0, int r) -> long { return t0 + r < nv_end ? (long)(t0 + r) * D : 0l; };

  h8_t KA[KS], KB[KS], KAl[KS], KBl[KS];
  // K elements of this wave's k steps from global memory (the K/V pair layout)
  auto load_k = [&](int t0, bool real) {
    if constexpr (VR) return;
    const int ra = 8 * (j >> 2) + (j & 3);
    const uint16_t* ka = real ? kb + row_at(t0, ra) + 8 * g : kb;
    const uint16_t* kc = real ? kb + row_at(t0, ra + 4) + 8 * g : kb;
#pragma unroll
    for (int k = 0; k < KS; k++) {
      const int s = w + 4 * k;
      const u4v* pa_ = reinterpret_cast<const u4v*>(ka + 32 * s);
      const u4v* pb_ = reinterpret_cast<const u4v*>(kc + 32 * s);
      KA[k] = __builtin_bit_cast(h8_t, __builtin_nontemporal_load(pa_));
      KB[k] = __builtin_bit_cast(h8_t, __builtin_nontemporal_load(pb_));
    }
  };
  // VR: the same elements from the group's V rows of the tile in LDS (lane
  // (j, g) reads rows 8 (j / 4) + j % 4 and that + 4 at dims 32 s + 8 g ..
  // + 7, chunk 4 s + g of the row, stored at position (4 s + g) ^ 2 fds_swz)
  auto lds_k = [&](const uint16_t* vl) {
    const int ra = 8 * (j >> 2) + (j & 3);
#pragma unroll
    for (int k = 0; k < KS; k++) {
      const int c = 4 * (w + 4 * k) + g;
      KA[k] = *reinterpret_cast<const h8_t*>(vl + ra * D + (c ^ (2 * fds_swz(ra))) * 8);
      KB[k] = *reinterpret_cast<const h8_t*>(vl + (ra + 4) * D + (c ^ (2 * fds_swz(ra + 4))) * 8);
    }
  };
  // this wave's 8 V rows of a tile into its group's rows of X: lane l writes
  // chunk position l % CPR of row 8w + RPI i + l / CPR, so loads the chunk
  // that the swizzle puts there
  auto load_v = [&](uint16_t* X, int t0, bool real) {
    uint16_t* vl = X + grp * 32 * D;
    const int rl = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < NVS; i++) {
      const int r0 = 8 * w + RPI * i, r = r0 + rl;
      const uint16_t* src = real ? vb + row_at(t0, r) + (pc ^ (2 * fds_swz(r))) * 8 : vb;
      lds_dma16(src, vl + r0 * D);
    }
  };
  load_k(tile0(grp), grp < ntile);
  load_v(vA, tile0(grp), grp < ntile);
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

  if (a.fin_on) {
    const AttnFin& f = a.fin;
#pragma unroll
    for (int k = 0; k < MAXJ; k++) {
      const int jb = wave + 8 * k;
      if (jb >= njobs) break;
      if (jb < a.GQ) {
        finish_vals<D>(raw[k], wq, true, true, fcs[k], f.rot_pairs, f.eps, q16 + jb * D);
        continue;
      }
      const int r = (jb - a.GQ) >> 1;        // rows this workgroup attends and holds
      if (r > row || !owns(base + r)) continue;
      if (((jb - a.GQ) & 1) == 0) {
        if (!VR) finish_vals<D>(raw[k], wk, true, true, fcs[k], f.rot_pairs, f.eps, newK + r * D);
      } else if (f.v_norm) {
        finish_vals<D>(raw[k], wk, false, false, fcs[k], f.rot_pairs, f.eps, newV + r * D);
      } else {
        fin_store<D>(raw[k], newV + r * D);
      }
    }
  }
  lds_barrier();                              // finished rows and the VR tables are in
  // split 0 exports the finished queries, from registers at the end (the
  // scores take their LDS; stores issued here would be waited for by every
  // later wait of the wave): thread t holds 16-byte chunks t and t + 512
  constexpr int QCH = 16 * D / 8;             // chunks of 16 finished heads
  u4v qexp[(QCH + 511) / 512];
  const bool q_exp = a.fin_on && a.fin.q_out && split == 0;
  if (q_exp) {
#pragma unroll
    for (int e = 0; e < (QCH + 511) / 512; e++) {
      const int ci = threadIdx.x + 512 * e;
      qexp[e] = ci < a.GQ * (D / 8) ? *reinterpret_cast<const u4v*>(q16 + ci * 8) : (u4v){0u, 0u, 0u, 0u};
    }
  }
  // ---- queries of this wave's k steps as the MFMA B operand (VR: in the
  // steps whose key is kw * v, q * kw split into fp16 hi and lo)
  h8_t qb[KS], qlo[KS];
#pragma unroll
  for (int k = 0; k < KS; k++) {
    const int s = w + 4 * k;
    u4v t = a.fin_on ? *reinterpret_cast<const u4v*>(q16 + (col_ok ? j : 0) * D + 32 * s + 8 * g) : qraw[k];
    if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
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
      qb[k] = hi;
      qlo[k] = lo;
    } else {
      qb[k] = __builtin_bit_cast(h8_t, t);
    }
  }
  if (a.fin_on) lds_barrier();                // every wave has its queries: the scores take their place

  float m_run = -INFINITY, l_part = 0.f;
  f4_t O[DS];
#pragma unroll
  for (int d = 0; d < DS; d++) O[d] = (f4_t){0.f, 0.f, 0.f, 0.f};
  f4_t* sxw = sx + (grp * 4 + w) * 2 * 64;
  const f4_t* sxg = sx + grp * 4 * 2 * 64;

  auto body = [&](auto bc, int rd) {
    constexpr int b = decltype(bc)::v;
    uint16_t* X = b ? vB : vA;
    uint16_t* vl = X + grp * 32 * D;
    const int ti = G * rd + grp;
    const bool act = ti < ntile;              // group-uniform
    const int t0 = tile0(ti);
    // this round's K and V rows have landed (they were issued with the last
    // round's scores; nothing of the next round is in flight yet)
    wait_vm<0>();
    if constexpr (VR) {
      lds_barrier();                          // every wave's V rows of the tile are in
      if (act) lds_k(vl);
    }
    if (act) {
      if (t0 + 31 >= P0new) {                 // rows formed in this step: keys, then V rows
        const int pa = t0 + 8 * (j >> 2) + (j & 3), pb = pa + 4;
        const uint16_t* nk = VR ? newV : newK;
#pragma unroll
        for (int k = 0; k < KS; k++) {
          const int off = 32 * (w + 4 * k) + 8 * g;
          if (pa >= P0new && pa < en) KA[k] = *reinterpret_cast<const h8_t*>(nk + (pa - P0new) * D + off);
          if (pb >= P0new && pb < en) KB[k] = *reinterpret_cast<const h8_t*>(nk + (pb - P0new) * D + off);
        }
#pragma unroll
        for (int r = 8 * w; r < 8 * w + 8; r++) {
          const int pr = t0 + r;
          if (pr >= P0new && pr < en && lane < D / 8)
            *reinterpret_cast<u4v*>(vl + r * D + (lane ^ (2 * fds_swz(r))) * 8) =
                *reinterpret_cast<const u4v*>(newV + (pr - P0new) * D + lane * 8);
        }
      }
      if (VR && w < RS) {
        // keys of the rotating steps w and w + HS (local 0 and HS / 4):
        // lane (j, g) holds positions pa (KA) and pa + 4 (KB)
        const int pa = t0 + 8 * (j >> 2) + (j & 3);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int i = 32 * w + 8 * g + e;
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
          form(KA[0], KA[HS / 4], KAl[0], KAl[HS / 4], ca, sa);
          form(KB[0], KB[HS / 4], KBl[0], KBl[HS / 4], cb, sb);
        }
      }
      f4_t p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; k++) {
        const int s = w + 4 * k;
        p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA[k], qb[k], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB[k], qb[k], p1, 0, 0, 0);
        if (VR && rebuilt(s)) {
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KAl[k], qb[k], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KBl[k], qb[k], p1, 0, 0, 0);
        } else if (VR) {
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA[k], qlo[k], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB[k], qlo[k], p1, 0, 0, 0);
        }
      }
      sxw[lane] = p0;
      sxw[64 + lane] = p1;
    }
    // the next round's K and V rows, in flight through this round's softmax
    // and PV: the K registers are free once the scores are formed, and the
    // other V buffer since the last round's final barrier (its direct loads
    // do not hold up the PV reads of this buffer: both go through restrict
    // pointers, lds_dma16 and lds_tr8)
    load_k(tile0(ti + G), ti + G < ntile);
    load_v(b ? vA : vB, tile0(ti + G), ti + G < ntile);
    lds_barrier();
    if (act) {
      // full scores: the group's 4 parts added in a fixed order
      f4_t c0 = sxg[lane], c1 = sxg[64 + lane];
#pragma unroll
      for (int u = 1; u < 4; u++) {
        const f4_t e0 = sxg[u * 128 + lane], e1 = sxg[u * 128 + 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; i++) { c0[i] += e0[i]; c1[i] += e1[i]; }
      }
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        sv[i] = (t0 + 8 * g + i < en) ? c0[i] * a.scale_log2 : -INFINITY;
        sv[4 + i] = (t0 + 8 * g + 4 + i < en) ? c1[i] * a.scale_log2 : -INFINITY;
      }
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 8; i++) mt = fmaxf(mt, sv[i]);
      mt = rows_max(mt);
      const float m_new = fmaxf(m_run, mt);   // finite: position t0 is admitted
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float p[8], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        p[i] = exp2f(sv[i] - m_new);
        ps += p[i];
      }
      l_part = l_part * alpha + ps;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; i++) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int d = 0; d < DS; d++)
#pragma unroll
        for (int i = 0; i < 4; i++) O[d][i] *= al[i];
      h8_t Ahi, Alo;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const _Float16 hi = (_Float16)p[i];
        Ahi[i] = hi;
        Alo[i] = (_Float16)(p[i] - (float)hi);
      }
      // O += P V over this wave's dims (lane (j, g) addresses row 8g + j/4
      // (and + 4) at dims 16d + 4 (j % 4), as in k_fd_partial)
      const int sw = fds_swz(8 * g + (j >> 2));
      const uint16_t* vt = vl + (8 * g + (j >> 2)) * D + 4 * (j & 3);
#pragma unroll
      for (int dd = 0; dd < DS; dd++) {
        const int cd = 16 * ((DS * w + dd) ^ sw);
        const h8_t Bv = lds_tr8(vt + cd, 4 * D);
        O[dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[dd], 0, 0, 0);
        O[dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[dd], 0, 0, 0);
      }
    }
    lds_barrier();                            // these V rows and the scores are free again
  };
  for (int rd = 0; rd < nround; rd += 2) {
    body(fds_ic<0>{}, rd);
    if (rd + 1 < nround) body(fds_ic<1>{}, rd + 1);
  }

  // ---- merge the two groups: maxima and sums per head meet in LDS; group 1
  // stores its rescaled O (one float4 of 4 heads per dim step and lane) into
  // the even rounds' V rows, group 0 adds it to its own in a fixed order and
  // writes the records
  float l_tot = rows_sum(l_part);
  if (w == 0 && lane < 16) { wm[grp][lane] = m_run; wl[grp][lane] = l_tot; }
  __syncthreads();
  float fw[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int hc = 4 * g + i;
    const float M = fmaxf(wm[0][hc], wm[1][hc]);
    fw[i] = wm[grp][hc] == -INFINITY ? 0.f : exp2f(wm[grp][hc] - M);
  }
  f4_t* ob = reinterpret_cast<f4_t*>(vA);     // [4 waves][DS][64]
  if (grp == 1) {
#pragma unroll
    for (int dd = 0; dd < DS; dd++)
      ob[(w * DS + dd) * 64 + lane] = (f4_t){O[dd][0] * fw[0], O[dd][1] * fw[1], O[dd][2] * fw[2], O[dd][3] * fw[3]};
  }
  __syncthreads();
  if (grp == 0) {
    // one scalar base, 32-bit offsets (head c's record lies c (D + 4) on);
    // O / l in fp16 (k_fd_combine, H16), m and l in fp32
    float* rbase = a.part + attn_rec(a, seq, row, kvh, split, 0, D);
    uint16_t* rb16 = reinterpret_cast<uint16_t*>(rbase);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int hc = 4 * g + i;
      const float M = fmaxf(wm[0][hc], wm[1][hc]);
      const float lh = M == -INFINITY ? 0.f : exp2f(wm[0][hc] - M) * wl[0][hc] + exp2f(wm[1][hc] - M) * wl[1][hc];
      const float inv = lh > 0.f ? 1.0f / lh : 0.f;
      if (hc < a.GQ) {
        const unsigned o = (unsigned)(2 * hc * (D + 4) + 16 * DS * w + j);
#pragma unroll
        for (int dd = 0; dd < DS; dd++)
          rb16[o + 16 * dd] = f2h((O[dd][i] * fw[i] + ob[(w * DS + dd) * 64 + lane][i]) * inv);
      }
    }
    if (w == 0 && lane < a.GQ) {
      const float M = fmaxf(wm[0][lane], wm[1][lane]);
      float l = 0.f;
      if (M != -INFINITY) l = exp2f(wm[0][lane] - M) * wl[0][lane] + exp2f(wm[1][lane] - M) * wl[1][lane];
      rbase[lane * (D + 4) + D] = M;
      rbase[lane * (D + 4) + D + 1] = l;
    }
  }
  // ---- last, so that nothing waits for them: the queries' export and the
  // row's own position into the cache
  if (q_exp) {
#pragma unroll
    for (int e = 0; e < (QCH + 511) / 512; e++) {
      const int ci = threadIdx.x + 512 * e;
      if (ci < a.GQ * (D / 8))
        *reinterpret_cast<u4v*>(a.fin.q_out + ((long)row * a.Hq + kvh * a.GQ) * D + ci * 8) = qexp[e];
    }
  }
  if (a.fin_on && owns(P)) {
    const long so = (long)P * D;
    for (int d = threadIdx.x; d < D; d += 512) {
      if (!VR) kb[so + d] = newK[row * D + d];
      vb[so + d] = newV[row * D + d];
    }
  }
}

// out[seq][row][h][d] = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// The output pointers come before the argument struct: after it they would
// lie in a 64-byte argument line of their own (the struct ends in the
// positions of the API path), one more memory round trip of the kernel.
// Grid (Hkv, GQ, n_seq * n_rows * D / 64), 256 threads: lane = output dim, wave w
// takes splits w, w + 4, ... (S <= MAXS).  Every load of the workgroup is
// issued before the first use (split indices past S are clamped and their
// weight is zero), and the four wave sums meet in LDS in a fixed order.
//
// TAIL (a block of rows whose ring splits cover each group of a.rpw rows up
// to the position P of its first row; one sequence, the finished queries in
// a.fin.q_out): row r also attends positions P + 1 .. P + (r mod rpw), rows
// formed in this step and already in the cache.  Each is one more term of
// the sums, with m its score, l = 1 and O its V row; the score is q . k
// over the whole head (dims dealt to the 256 threads, the wave sums added
// in a fixed order), scaled as the partial kernels scale theirs.
//
// H16 (the full layers' kernels k_fd_full_ds and k_fd_rows4): a record holds
// O / l in fp16 at its start (m and l stay fp32 at D, D + 1), half the bytes
// of the records written and read; split s then weighs 2^(m_s - M) l_s.
constexpr int kMaxSplits = 256;
constexpr int kMaxTail = 3;                    // rows of a block (at most 4) past its first

template <int D, int MAXS, bool TAIL = false, bool H16 = false>
__global__ void __launch_bounds__(256) k_fd_combine(float* out32, uint16_t* out16, AttnArgs a) {
  constexpr int PER = MAXS / 4;
  constexpr int TD = (D + 255) / 256;          // TAIL: head dims per thread
  __shared__ float wsp[MAXS];
  __shared__ float red[4][64];
  __shared__ float rm[4], rl[4];
  __shared__ float tred[4][kMaxTail];
  const int pos_w = TAIL ? pos_issue(a) : 0;
  // grid (Hkv, GQ, rows x D / 64), KV heads fastest: with 8 KV heads the
  // workgroups of one KV head run on the XCD whose L2 holds its records (the
  // ring partial enumerates KV heads fastest too; workgroups go round-robin
  // over the 8 XCDs).  No index needs a division by a runtime value but the
  // row's, and only with several rows: the divisions otherwise ran ahead of
  // the first load
  constexpr int NDC = D / 64;
  const int kvh = blockIdx.x, col = blockIdx.y, h = kvh * a.GQ + col;
  const int sr = blockIdx.z / NDC, dc = blockIdx.z % NDC;
  int seq = sr, row = 0;
  if (a.n_rows > 1) {
    seq = sr / a.n_rows;
    row = sr - seq * a.n_rows;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // one scalar base and 32-bit offsets (a split's records lie rs floats
  // apart, S rs < 2^31): the split index of each load is wave-uniform, so
  // its offset is scalar arithmetic, not a per-lane 64-bit multiply
  const float* rb = a.part + attn_rec(a, seq, row, kvh, 0, col, D);
  const int rs = a.GQ * (D + 4);                       // stride between splits
  const int d = dc * 64 + lane;
  const int S = a.S;
  const bool own = tid < S;
  const unsigned mo = (unsigned)(min(tid, S - 1) * rs + D);
  const float m_raw = rb[mo], l_raw = rb[mo + 1];
  float ov[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const unsigned ro = (unsigned)(min(wave + 4 * i, S - 1) * rs);
    ov[i] = H16 ? h2f(reinterpret_cast<const uint16_t*>(rb + ro)[d]) : rb[ro + d];
  }
  // TAIL: the query, and the keys and this lane's V elements of the rows
  // past the group's first
  int nt = 0;
  float tq[TD], tk[kMaxTail][TD], tv[kMaxTail];
  if constexpr (TAIL) {
    nt = row % a.rpw;
    const int Pf = pos_take(a, pos_w, seq) + row - nt;
    const uint16_t* qr = a.fin.q_out + ((long)row * a.Hq + h) * D;
    const uint16_t* kb = a.k + (long)kvh * a.R * D;
    const uint16_t* vb = a.v + (long)kvh * a.R * D;
    // loads without conditions (a dim past D reads dim D - 1 and its query
    // element is zeroed after the load), so none waits inside a branch
#pragma unroll
    for (int i = 0; i < TD; i++) {
      const float qv = h2f(qr[min(tid + 256 * i, D - 1)]);
      tq[i] = tid + 256 * i < D ? qv : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kMaxTail; e++) {
      const long so = (long)((Pf + 1 + min(e, max(nt - 1, 0))) % a.R) * D;
#pragma unroll
      for (int i = 0; i < TD; i++) tk[e][i] = h2f(kb[so + min(tid + 256 * i, D - 1)]);
      tv[e] = h2f(vb[so + d]);
    }
    // every load above is issued before the first sum waits (left to itself
    // the compiler moves each load down to its use, past the cross-lane sums,
    // and the loads then wait for one another)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < kMaxTail; e++) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < TD; i++) part = fmaf(tq[i], tk[e][i], part);
      part = wave_sum(part);
      if (lane == 0) tred[wave][e] = part;
    }
  }
  const float m = own ? m_raw : -INFINITY;
  float M = wave_max(m);
  if (lane == 0) rm[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
  float ts[kMaxTail];
  if constexpr (TAIL) {
#pragma unroll
    for (int e = 0; e < kMaxTail; e++) {
      ts[e] = e < nt ? (((tred[0][e] + tred[1][e]) + tred[2][e]) + tred[3][e]) * a.scale_log2 : -INFINITY;
      M = fmaxf(M, ts[e]);
    }
  }
  const float w = (own && m != -INFINITY) ? exp2f(m - M) : 0.f;
  if (tid < MAXS) wsp[tid] = H16 ? w * l_raw : w;     // H16: the records hold O / l
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
    if constexpr (TAIL) {
#pragma unroll
      for (int e = 0; e < kMaxTail; e++) {
        if (e < nt) {
          const float we = exp2f(ts[e] - M);
          L += we;
          o = fmaf(we, tv[e], o);
        }
      }
    }
    o *= (L > 0.f) ? 1.0f / L : 0.f;
    const long oi = (((long)seq * a.n_rows + row) * a.Hq + h) * D + d;
    if (out32) out32[oi] = o;
    if (out16) out16[oi] = f2h(o);
  }
}

}  // namespace q4k
