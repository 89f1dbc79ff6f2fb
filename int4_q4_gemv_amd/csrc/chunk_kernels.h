// chunk_kernels.h -- the kernels of a prefill chunk: up to 64 rows (tokens at
// consecutive positions) through the decoder in one pass (Gemma-4-12B-CoreAI
// card, "v5/ -- ring extent R = 2W": a block of rows is written into the ring
// before it is read, and the slot rule keeps it causal while R >= W + rows - 1;
// gemma-4-E4B-CoreAI card, ring/: only written, causal, in-window slots are
// attended).
//
// k_q4_gemm: Y[b][n] = sum_k x[b][k] * (d * q)[n][k] for the rows b < 64 of a
// chunk, on v_mfma_f32_16x16x32_f16.  The weights stay in the q4 device layout
// of pack_kernels.h: lane l of a wave-wide load holds row l & 15 and block
// l >> 4 of a quad (16 rows x 4 blocks).  The MFMA's k index is permuted so
// that every lane multiplies its own data: MFMA w of a quad takes, in lane
// group g, elements 8w .. 8w+7 of block g (the A operand of lane (r, g) is
// word w of its own 16 bytes), and the x operand of lane (c, g) is read at
// the same columns, 128 q + 32 g + 8 w.  One MFMA thus spans four blocks with
// four scales, so the scale goes into the operand: d * q is split exactly into
// fp16 hi + lo (d has 11 significant bits and |q| <= 8, so d * q has at most 15
// and its lowest bit is at least 2^-24; packed fp16 multiply and fma), and each
// product is two MFMAs.  Sums are fp32 in the MFMA accumulators.  The chunk's
// x rows are staged in LDS 128 or 256 columns at a time (direct global-to-LDS loads,
// 2 or 4 rows per instruction; 16-byte chunk p of row b at position p ^ (b & 15),
// so the 16 rows a 16-lane group reads fall in distinct banks).
//
// A workgroup is 4 waves; each wave owns TPW row tiles and all 64 chunk rows
// (4 column groups of 16), accumulating TPW x 4 MFMA tiles.  STORE: the 4
// waves take 64 TPW consecutive rows, and blockIdx.y picks one of S runs of
// K, written as S partial products side by side (the next kernel adds them in
// order).  GATEUP: waves 0, 1 take 16 TPW gate rows each and waves 2, 3 the
// same rows of up; the epilogue writes fp16(gelu_tanh(gate) * up).
//
// Limits: the dequantised weights d * q must be finite in fp16 (block absmax
// below 65504); the decode path, which scales in fp32, has no such limit.
#pragma once
#include "device_common.h"
#include "gemv_kernels.h"
#include "attn_kernels.h"

namespace q4k {

constexpr int kChunkRows = 64;                 // rows of a chunk
constexpr int kChunkRunQ = 1;                  // quads per staged x run in the chunk's products
constexpr int kGemmRunQ = 2;                   // ... in q4_gemm (one workgroup per CU: longer runs)
constexpr size_t kGemmLds = 0;                 // the x runs live in two static LDS arrays

// One matrix of a launch.  STORE launches may hold up to 3 (the q, k and v
// projections), laid out along blockIdx.x from workgroup wg0 on; GATEUP holds
// gate (seg[0]) and up (seg[1]) over the same rows.
struct GemmSeg {
  const u4v* codes;        // q4 device layout
  const uint16_t* scales;
  int N, T;                // rows, 16-row tiles
  int wg0;                 // first workgroup (STORE)
  int out_off;             // first output column (STORE)
};

struct GemmArgs {
  GemmSeg seg[3];
  int nseg;
  int K, NQ;               // columns, quads per row
  int NQs;                 // quads per run of K (blockIdx.y = run)
  const uint16_t* x;       // fp16 [n][ldx], ldx >= K >= 8
  int ldx, n;
  float* y;                // STORE: run s at y + s * y_split: fp32 [n][ldy], columns out_off ..
  int ldy;
  long y_split;
  uint16_t* a_out;         // GATEUP: fp16 [n][ld_a]
  int ld_a;
};

// TPW: 16-row tiles per wave (STORE: 4 TPW x 16 rows per workgroup; GATEUP:
// the gate waves 0, 1 and the up waves 2, 3 on the same 32 TPW rows).  The K
// loop is pipelined over runs of CQ quads (128 CQ columns): while run r is computed from
// one LDS array, the weights of run r + 1 are loaded into registers and its x
// rows straight into the other array (two distinct arrays, so that the
// compiler can tell the next run's global-to-LDS writes from this run's LDS
// reads and does not wait for them first).  The scales are kept one per
// 32-bit register (packing two into one made the compiler wait for the load
// in flight).
template <int EPI, int TPW, int CQ>
__global__ void __launch_bounds__(256) k_q4_gemm(GemmArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const bool up = EPI == EPI_GATEUP && wave >= 2;
  // the segment of this workgroup, selected without a dependent load
  const GemmSeg s0 = a.seg[0], s1 = a.seg[1], s2 = a.seg[2];
  int si = up ? 1 : 0;
  if constexpr (EPI != EPI_GATEUP)
    si = (a.nseg > 1 && (int)blockIdx.x >= s1.wg0 ? 1 : 0) + (a.nseg > 2 && (int)blockIdx.x >= s2.wg0 ? 1 : 0);
  const GemmSeg sg = si == 0 ? s0 : (si == 1 ? s1 : s2);
  const int bx = EPI == EPI_GATEUP ? (int)blockIdx.x : (int)blockIdx.x - sg.wg0;
  const int tile0 = EPI == EPI_GATEUP ? (bx * 2 + (wave & 1)) * TPW : (bx * 4 + wave) * TPW;
  const u4v* codes = sg.codes;
  const uint16_t* scales = sg.scales;
  // tiles past the matrix read tile 0 and are not stored
  int tl[TPW];
#pragma unroll
  for (int t = 0; t < TPW; t++) tl[t] = tile0 + t < sg.T ? tile0 + t : 0;
  const int q_begin = blockIdx.y * a.NQs, q_end = min(a.NQ, q_begin + a.NQs);

  f4_t acc[TPW][4];
#pragma unroll
  for (int t = 0; t < TPW; t++)
#pragma unroll
    for (int c = 0; c < 4; c++) acc[t][c] = (f4_t){0.f, 0.f, 0.f, 0.f};

  // one run: the weights (TPW tiles x CQ quads, a 16-byte load and a scale
  // per lane each; quads past the run reload the run's first) and the x rows
  // 16 wave .. +15 from column 128 qc, 16 CQ chunks of 8 columns per row, one
  // chunk per lane and 64 / (16 CQ) rows per load (chunks are clamped into
  // the row and rows past n repeat row n - 1; neither is used)
  // double-buffered x runs of CQ quads in two distinct LDS arrays, filled by
  // global-to-LDS loads; row b at pitch 128 CQ columns, 16-byte chunk p of
  // row b at position p ^ (b & 15)
  constexpr int DQ = CQ;
  constexpr int RW = 128 * DQ, CPR = 16 * DQ, RPI = 64 / CPR;   // halves and chunks per row, rows per load
  __shared__ __align__(16) uint16_t xa[64 * RW];
  __shared__ __align__(16) uint16_t xb2[64 * RW];
  static_assert(EPI != EPI_GATEUP || 2 * TPW * 4 * 64 * 16 <= 64 * RW * 2, "exchange fits in xa");
  auto load_w = [&](int qc, u4v (&cw)[TPW][CQ], uint32_t (&sw)[TPW][CQ]) {
    const int nq = min(DQ, q_end - qc);
#pragma unroll
    for (int i = 0; i < DQ; i++) {
      const int qi = qc + (i < nq ? i : 0);
#pragma unroll
      for (int t = 0; t < TPW; t++) {
        const long o = ((long)tl[t] * a.NQ + qi) * 64 + lane;
        cw[t][i] = __builtin_nontemporal_load(codes + o);
        sw[t][i] = (uint32_t)scales[o];
      }
    }
  };
  auto load_x = [&](int qc, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < 16 / RPI; i++) {
      const int b = 16 * wave + RPI * i + lane / CPR;
      const int bs = min(b, a.n - 1);
      const int p = lane % CPR;
      const int col = min(qc * 128 + (p ^ (b & 15)) * 8, a.K - 8);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(a.x + (long)bs * a.ldx + col),
                                       reinterpret_cast<uint32_t*>(buf + (16 * wave + RPI * i) * RW), 16, 0, 0);
    }
  };
  auto compute = [&](const uint16_t* buf, const u4v (&cw)[TPW][CQ], const uint32_t (&sw)[TPW][CQ], int nq) {
#pragma unroll
    for (int i = 0; i < DQ; i++) {
      if (i >= nq) break;
#pragma unroll
      for (int t = 0; t < TPW; t++) {
        const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)sw[t][i]);
        const h2_t d2 = {d, d};
        const uint32_t qw[4] = {cw[t][i].x, cw[t][i].y, cw[t][i].z, cw[t][i].w};
#pragma unroll
        for (int w = 0; w < 4; w++) {
          h2_t v0, v1, v2, v3;
          dq_word(qw[w], v0, v1, v2, v3);
          const h2_t h0 = v0 * d2, h1 = v1 * d2, h2 = v2 * d2, h3 = v3 * d2;
          const h2_t l0 = __builtin_elementwise_fma(v0, d2, -h0), l1 = __builtin_elementwise_fma(v1, d2, -h1);
          const h2_t l2 = __builtin_elementwise_fma(v2, d2, -h2), l3 = __builtin_elementwise_fma(v3, d2, -h3);
          const h8_t hi = __builtin_shufflevector(__builtin_shufflevector(h0, h1, 0, 1, 2, 3),
                                                  __builtin_shufflevector(h2, h3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
          const h8_t lo = __builtin_shufflevector(__builtin_shufflevector(l0, l1, 0, 1, 2, 3),
                                                  __builtin_shufflevector(l2, l3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
          h8_t xv[4];
#pragma unroll
          for (int c = 0; c < 4; c++) {
            const int b = 16 * c + r;
            const int p = (16 * i + 4 * g + w) ^ (b & 15);
            xv[c] = *reinterpret_cast<const h8_t*>(buf + b * RW + p * 8);
          }
#pragma unroll
          for (int c = 0; c < 4; c++) acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, xv[c], acc[t][c], 0, 0, 0);
#pragma unroll
          for (int c = 0; c < 4; c++) acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, xv[c], acc[t][c], 0, 0, 0);
        }
      }
    }
  };
  u4v cw[TPW][CQ], cn[TPW][CQ];
  uint32_t sw[TPW][CQ], sn[TPW][CQ];
  if (q_begin < q_end) {
    load_w(q_begin, cw, sw);
    load_x(q_begin, xa);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // two phases per iteration with swapped roles (no register copies: a copy
  // of a load in flight would wait for it)
  for (int qc = q_begin; qc < q_end; qc += 2 * DQ) {
    {
      const bool more = qc + DQ < q_end;
      if (more) { load_w(qc + DQ, cn, sn); load_x(qc + DQ, xb2); }
      compute(xa, cw, sw, min(DQ, q_end - qc));
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (!more) break;
    }
    {
      const int q1 = qc + DQ;
      const bool more = q1 + DQ < q_end;
      if (more) { load_w(q1 + DQ, cw, sw); load_x(q1 + DQ, xa); }
      compute(xb2, cn, sn, min(DQ, q_end - q1));
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (!more) break;
    }
  }
  // lane (c, g) of tile t, column group cg holds rows 16 tile + 4 g + i of
  // chunk row 16 cg + c
  if constexpr (EPI == EPI_GATEUP) {
    f4_t* ex = reinterpret_cast<f4_t*>(xa);   // [2 waves][TPW tiles][4 groups][64 lanes]
    if (up) {
#pragma unroll
      for (int t = 0; t < TPW; t++)
#pragma unroll
        for (int c = 0; c < 4; c++) ex[(((wave - 2) * TPW + t) * 4 + c) * 64 + lane] = acc[t][c];
    }
    __syncthreads();
    if (!up) {
#pragma unroll
      for (int t = 0; t < TPW; t++) {
        const int tile = tile0 + t;
        if (tile >= sg.T) continue;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int b = 16 * c + r;
          const f4_t u = ex[((wave * TPW + t) * 4 + c) * 64 + lane];
          if (b < a.n) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int row = tile * 16 + 4 * g + i;
              if (row < sg.N) a.a_out[(long)b * a.ld_a + row] = f2h(gelu_tanh(acc[t][c][i]) * u[i]);
            }
          }
        }
      }
    }
  } else {
    float* yb = a.y + blockIdx.y * a.y_split + sg.out_off;
#pragma unroll
    for (int t = 0; t < TPW; t++) {
      const int tile = tile0 + t;
      if (tile >= sg.T) continue;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const int b = 16 * c + r;
        if (b >= a.n) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int row = tile * 16 + 4 * g + i;
          if (row < sg.N) yb[(long)b * a.ldy + row] = acc[t][c][i];
        }
      }
    }
  }
}

// ------------------------------------------------------- chunk attention ----
// Rows of a chunk over shared K/V tiles (layers whose query heads already fill
// the 16 MFMA columns, so rows cannot share a tile as columns): a workgroup's
// 4 waves take 4 consecutive rows, and every 32-position tile of its split is
// staged once in LDS for all four -- K rows at pitch D with 16-byte chunk c of
// row r at c ^ kswz(r) (the 16 rows one 16-lane group reads fall in distinct
// banks), V rows in the layout of k_fd_partial's transposing PV reads.  Each
// wave runs the online softmax of its own row over the union of the 4 rows'
// ranges (positions outside its row's range are masked) and writes its row's
// (O, m, l) records; the combine is k_fd_combine's.  NB = 2: two tiles in
// flight, the next one staged while the current one is computed (132 KB of
// LDS at D = 512, one workgroup per CU: for grids up to one workgroup per
// CU).  NB = 1: one tile at a time (66 KB), so two workgroups share a CU and
// one's loads overlap the other's arithmetic (larger grids: a prefill chunk).
Q4_DEV int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

template <int D, int NB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 2 : 1))) k_fd_rows4(AttnArgs a) {
  static_assert(NB == 1 || NB == 2, "one or two tile buffers");
  static_assert(D >= 128, "a K row holds at least 16 chunks");
  constexpr int VROW = fd_vpitch<D>();
  constexpr int NDS = D / 16, NKS = D / 32;
  constexpr int CPR = D / 8, RPI = 64 / CPR;      // 16-byte chunks per row, rows per 1 KB load
  __shared__ __align__(16) uint16_t kA[32 * D];        // tile buffer A: K rows [32][D]
  __shared__ __align__(16) uint16_t vA[32 * VROW];     // ... V rows [32][VROW]
  __shared__ __align__(16) uint16_t kB[NB == 2 ? 32 * D : 8];   // tile buffer B (NB = 2)
  __shared__ __align__(16) uint16_t vB[NB == 2 ? 32 * VROW : 8];
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int ngrp = (a.n_rows + 3) / 4;
  const int seq = blockIdx.z / ngrp, row0 = (blockIdx.z - seq * ngrp) * 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rlast = min(a.n_rows, row0 + 4) - 1;
  const bool live = row0 + wave <= rlast;              // wave-uniform
  const int row = live ? row0 + wave : rlast;
  // first position: from the decode step's parameters on the device, else the host's
  const int base = __builtin_amdgcn_readfirstlane(
      a.sp ? *(const __attribute__((address_space(1))) int*)(&a.sp->pos0) : a.pos0[seq]);
  const int P = base + row;
  const int lo = a.ring ? max(0, base + row0 - a.W + 1) : 0;
  const int Pl = base + rlast;
  const int L = Pl - lo + 1;
  const int chunk = (L + a.S - 1) / a.S;
  const int st = lo + split * chunk;
  const int en = min(st + chunk, Pl + 1);
  const int loj = a.ring ? P - a.W + 1 : 0;
  const int j = lane & 15, g = lane >> 4;
  const bool col_ok = live && j < a.GQ;

  const uint16_t* kb = a.k + seq * a.seq_stride + (a.ring ? (long)kvh * a.R * D : 0);
  const uint16_t* vb = a.v + seq * a.seq_stride + (a.ring ? (long)kvh * a.R * D : 0);
  const bool ringf = a.ring != 0;
  const int Rr = ringf ? a.R : 1;

  h8_t qb[NKS];
  {
    const uint16_t* qp = a.q + (((long)seq * a.n_rows + row) * a.Hq + (col_ok ? kvh * a.GQ + j : 0)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(qp + 32 * s);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      qb[s] = __builtin_bit_cast(h8_t, t);
    }
  }
  float m_run = -INFINITY, l_part = 0.f;
  f4_t O[NDS];
#pragma unroll
  for (int d = 0; d < NDS; d++) O[d] = (f4_t){0.f, 0.f, 0.f, 0.f};

  // Two tile buffers, each a pair of LDS objects of its own: the next tile's
  // rows are loaded straight to LDS while the current one is computed.  The
  // loop is unrolled by two so that every LDS access names its buffer (the
  // compiler then waits for the other buffer's loads only where they are
  // read: the explicit counts below).  Every round issues its loads, a tile
  // past the split's end reading row 0, so the counts are the same on every
  // path.  (The queries' registers are first used with tiles in flight: that
  // first use waits for both.)
  constexpr int NL = 2 * (8 / RPI);                // loads of a tile per thread
  auto issue = [&](uint16_t* kt, uint16_t* vt, int t0) {
    // cache rows of the tile: tile row r at slot (t0 + r) mod R (rings hold
    // at least 32 slots), rows past en read row 0 and are masked
    const int s0 = __builtin_amdgcn_readfirstlane(ringf ? t0 % Rr : t0);
    const int nv = __builtin_amdgcn_readfirstlane(en - t0);
    auto row_at = [&](int r) -> long {
      const int sl = ringf && r >= Rr - s0 ? s0 + r - Rr : s0 + r;
      return r < nv ? (long)sl * D : 0l;
    };
    // wave w stages tile rows 8w .. 8w+7 of K and of V, 1 KB per instruction
    const int rl = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < 8 / RPI; i++) {
      const int r = 8 * wave + RPI * i + rl;
      const int ck = pc ^ kswz(r);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(kb + row_at(r) + ck * 8),
                                       reinterpret_cast<uint32_t*>(kt + (8 * wave + RPI * i) * D), 16, 0, 0);
      const int cv = pc ^ (2 * vswz<D>(r));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(vb + row_at(r) + cv * 8),
                                       reinterpret_cast<uint32_t*>(vt + (8 * wave + RPI * i) * VROW), 16, 0, 0);
    }
  };
  auto compute = [&](const uint16_t* kt, const uint16_t* vt, int t0) {
    // S^T = K Q^T: MFMA row r of half h <-> tile position 8 (r / 4) + 4h + r % 4
    const int ra = 8 * (j >> 2) + (j & 3);
    f4_t s0v = {0.f, 0.f, 0.f, 0.f}, s1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      const int cc = 4 * s + g;                    // 16-byte chunk of dims 32 s + 8 g
      const h8_t KA = *reinterpret_cast<const h8_t*>(kt + ra * D + (cc ^ kswz(ra)) * 8);
      const h8_t KB = *reinterpret_cast<const h8_t*>(kt + (ra + 4) * D + (cc ^ kswz(ra + 4)) * 8);
      s0v = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA, qb[s], s0v, 0, 0, 0);
      s1v = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB, qb[s], s1v, 0, 0, 0);
    }
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int pa = t0 + 8 * g + i, pb = pa + 4;
      sv[i] = (pa < en && pa <= P && pa >= loj) ? s0v[i] * a.scale_log2 : -INFINITY;
      sv[4 + i] = (pb < en && pb <= P && pb >= loj) ? s1v[i] * a.scale_log2 : -INFINITY;
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mt = fmaxf(mt, sv[i]);
    mt = rows_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const bool none = m_new == -INFINITY;          // nothing of this row admitted yet
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    m_run = m_new;
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      p[i] = none ? 0.f : exp2f(sv[i] - m_new);
      ps += p[i];
    }
    l_part = l_part * alpha + ps;
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
    // O += P V with the transposing reads of k_fd_partial
    const int sw = vswz<D>(8 * g + (j >> 2));
    const uint16_t* vp = vt + (8 * g + (j >> 2)) * VROW + 4 * (j & 3);
#pragma unroll
    for (int d = 0; d < NDS; d++) {
      typedef short v4s_t __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s_t lds_v4s;
      const int cd = 16 * (d ^ sw);
      const v4s_t vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vp + cd));
      const v4s_t vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vp + 4 * VROW + cd));
      const h8_t Bv = __builtin_bit_cast(h8_t, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[d], 0, 0, 0);
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[d], 0, 0, 0);
    }
  };
  const int ntile = st < en ? (en - st + 31) / 32 : 0;
  if constexpr (NB == 1) {
    for (int t = 0; t < ntile; t++) {
      issue(kA, vA, st + 32 * t);
      wait_vm<0>();
      lds_barrier();
      if (live) compute(kA, vA, st + 32 * t);
      lds_barrier();                                // the tile's reads are done
    }
  } else {
  issue(kA, vA, st);
  for (int t = 0; t < ntile; t += 2) {
    issue(kB, vB, st + 32 * (t + 1));               // tile t + 1 (or row 0 past the end)
    wait_vm<NL>();                                  // this wave's rows of tile t are in
    lds_barrier();
    if (live) compute(kA, vA, st + 32 * t);         // wave-uniform; every wave joins every barrier
    lds_barrier();                                  // buffer A is free
    if (t + 1 >= ntile) break;
    issue(kA, vA, st + 32 * (t + 2));
    wait_vm<NL>();
    lds_barrier();
    if (live) compute(kB, vB, st + 32 * (t + 1));
    lds_barrier();
  }
  }
  __builtin_amdgcn_s_waitcnt(0);                    // no load past the end still in flight at exit
  if (!live) return;
  float l_tot = rows_sum(l_part);
  // records with O / l in fp16 (k_fd_combine, H16): half the bytes of the
  // 4 rows' records, which this kernel writes and the combine reads
  float* rbase = a.part + attn_rec(a, seq, row, kvh, split, 0, D);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int col = 4 * g + i;
    const float lc = __shfl(l_tot, col, 64);
    const float inv = lc > 0.f ? 1.0f / lc : 0.f;
    if (col < a.GQ) {
      uint16_t* rec = reinterpret_cast<uint16_t*>(rbase + col * (D + 4));
#pragma unroll
      for (int d = 0; d < NDS; d++) rec[16 * d + j] = f2h(O[d][i] * inv);
    }
  }
  if (lane < a.GQ) {
    rbase[lane * (D + 4) + D] = m_run;
    rbase[lane * (D + 4) + D + 1] = l_tot;
  }
}

// ------------------------------------------------------------ embedding ----
struct ChunkEmbedArgs {
  const uint16_t* E;       // [vocab][H] fp16
  int H;
  float emb_scale;         // sqrt(H)
  float* h;                // [n][H]
  int tokens[kChunkRows];
};

// One workgroup per row: h = fp32(E[token]) * sqrt(H).
__global__ void __launch_bounds__(256) k_chunk_embed(ChunkEmbedArgs a) {
  const int b = blockIdx.x;
  const uint16_t* e = a.E + (long)a.tokens[b] * a.H;
  float* h = a.h + (long)b * a.H;
  for (int i = threadIdx.x; i < a.H; i += 256) h[i] = h2f(e[i]) * a.emb_scale;
}

// ------------------------------------------------------------ finishing ----
// (cos, sin) of the RoPE angle pos * theta^(-2i/D) for pair i (i < rot_pairs;
// (1, 0) beyond): the angle in fp64, reduced mod 2 pi in fp64, then fp32
// sincos, as k_step_begin forms its table.
Q4_DEV float2 rope_cs(int pos, int i, int D, double theta, int rot_pairs) {
  if (i >= rot_pairs) return make_float2(1.0f, 0.0f);
  const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)D);
  const double k = rint(ang * 0.15915494309189535);
  const float rr = (float)fma(-k, 6.283185307179586, ang);
  float sn, cn;
  sincosf(rr, &sn, &cn);
  return make_float2(cn, sn);
}

struct ChunkFinArgs {
  const float* qkv;        // [n][ldq]: q (Hq*D) | k (Hkv*D) | v (Hkv*D, sliding), ny runs y_split apart
  int ldq, ny;
  long y_split;
  int Hq, Hkv;
  int ring, R;             // ring layer: slot p mod R of KV head h at (h * R + slot) * D
  int v_norm, vrow;        // vrow: a full layer keeps only the V row
  const float* q_norm;
  const float* k_norm;
  double theta;
  int rot_pairs;
  float eps;
  int pos0;
  const StepParams* sp;    // decode step: the first position is read here instead of pos0
  const float2* rope_cs;   // decode step: (cos, sin) per row and pair [row][cs_ld] (k_step_begin's
  int cs_ld;               // table, the same values rope_cs() forms); NULL: formed here
  uint16_t* q16;           // [n][Hq][D]
  uint16_t* kc;
  uint16_t* vc;
};

// Grid (rows, Hq + 2 Hkv jobs), one wave each: query head j (per-head
// RMSNorm with q_norm, RoPE) to q16; then for KV head h, job Hq + 2h the key
// (k_norm, RoPE) and job Hq + 2h + 1 the value (the scale-free norm of V, or
// of the raw k on a full layer, or V as it is), written to the caches at the
// row's position.  The products' S runs are added in order first.
template <int D>
__global__ void __launch_bounds__(64) k_chunk_finish(ChunkFinArgs a) {
  static_assert(sizeof(ChunkFinArgs) >= 128 + 4, "argument lines fetched below lie inside the struct");
  kernarg_fetch<0, 64, 128>();                // the argument lines this kernel reads
  constexpr int FE = D / 64, FEH = fin_h<D>();
  const int row = blockIdx.x, job = blockIdx.y;
  const int lane = threadIdx.x;
  const int pos = (a.sp ? a.sp->pos0 : a.pos0) + row;
  int kind, head;                                 // 0 q, 1 k, 2 v
  if (job < a.Hq) { kind = 0; head = job; }
  else { kind = 1 + ((job - a.Hq) & 1); head = (job - a.Hq) >> 1; }
  if (kind == 1 && a.vrow) return;
  const float* rr = a.qkv + (long)row * a.ldq;
  long off;
  if (kind == 0) off = (long)head * D;
  else if (kind == 1 || !a.ring) off = (long)(a.Hq + head) * D;     // full: V from the raw k
  else off = (long)(a.Hq + a.Hkv + head) * D;
  float v[FE], t[FE];
  fin_load<D>(v, rr + off);
  for (int s = 1; s < a.ny; s++) {
    fin_load<D>(t, rr + s * a.y_split + off);
#pragma unroll
    for (int e = 0; e < FE; e++) v[e] += t[e];
  }
  float wv[FE];
#pragma unroll
  for (int e = 0; e < FE; e++) wv[e] = 1.0f;
  float2 cs[FEH];
#pragma unroll
  for (int e = 0; e < FEH; e++) {
    const int pr = D == 64 ? (lane & 31) : lane * FEH + e;
    cs[e] = a.rope_cs ? a.rope_cs[(long)row * a.cs_ld + pr] : rope_cs(pos, pr, D, a.theta, kind == 2 ? 0 : a.rot_pairs);
  }
  const long slot = a.ring ? ((long)head * a.R + pos % a.R) * D : (long)pos * D;
  if (kind == 0) {
    fin_load<D>(wv, a.q_norm);
    finish_vals<D>(v, wv, true, true, cs, a.rot_pairs, a.eps, a.q16 + ((long)row * a.Hq + head) * D);
  } else if (kind == 1) {
    fin_load<D>(wv, a.k_norm);
    finish_vals<D>(v, wv, true, true, cs, a.rot_pairs, a.eps, a.kc + slot);
  } else if (a.v_norm) {
    finish_vals<D>(v, wv, false, false, cs, a.rot_pairs, a.eps, a.vc + slot);
  } else {
    fin_store<D>(v, a.vc + slot);
  }
}

}  // namespace q4k
