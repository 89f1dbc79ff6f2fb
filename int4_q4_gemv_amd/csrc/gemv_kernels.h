// gemv_kernels.h -- int4 q4_0 matrix-vector products for gfx950, and the fp16
// tied-head product with softcap and argmax.
//
// Work split: one workgroup owns a 16-row tile of a matrix over one of S
// runs of K (S = 1 for most products).  Partial sums never meet across
// workgroups inside a kernel (on gfx950 the L2 writeback such a handoff
// needs costs more than the product itself): with S > 1 the S partial
// products are written side by side and the next kernel, which reads the
// product anyway, adds them in a fixed order.  The W waves of a workgroup
// split its run into CQ quads each (a quad = 16 rows x 4 q4 blocks = one
// 1 KB wave-wide load, see pack_kernels.h); partial sums meet in LDS in a
// fixed order, so results are deterministic.  Every wave issues all of its
// weight loads before anything else, and the grid is sized so that all of
// its waves are resident at once: the whole matrix is in flight from the
// first microseconds of the kernel.
//
// Batch 1: lane l works on row (l & 15) and block (l >> 4) of each quad; the
// activation comes from LDS; dequantisation is the fp16 magic-number trick
// (1024 + u, 64 + u) minus the bias, exact, then v_dot2_f32_f16.
// Batch 2..4 (the width-4 verify block): v_mfma_f32_4x4x4_16b_f16 with the
// 64 lanes as 16 blocks of 4 rows and the batch as the 4 columns; each lane
// still dequantises only its own 32 weights and the per-block scale is
// applied to the fp32 accumulator, so the dequantised weights stay exact.
//
// The activation comes in as fp16; where it is a normalised residual stream
// it is formed once per row by k_norm_rows (RMSNorm of the previous product
// added to the residual, then the input RMSNorm).
#pragma once
#include "device_common.h"

namespace q4k {

struct StepParams {       // written on the device at the start of every step
  int pos0;
  int n;
  int tokens[4];
  float* logits;          // this step's outputs (logits may be NULL): the captured
  int32_t* argmax;        // step graph reads them here, so it is output-independent
};

struct GemvSeg {
  const u4v* codes;
  const uint16_t* scales;
  int N;        // rows of this matrix
  int T;        // 16-row tiles
  int tile0;    // first global tile index (segments are laid end to end)
  int out_off;  // first output column in the concatenated output row
};

// x = fp16(RMSNorm(h_new) * w_in), h_new = (h_src + RMSNorm(y) * w_post) * scalar
// (y == NULL: h_new = h_src * scalar), where y is the sum, in order, of ny
// (<= MAXY of the kernel) partial products laid y_split floats apart.  h_new
// goes to h_dst.
struct NormIn {
  const float* h_src;
  const float* y;
  int ny;
  long y_split;
  const float* w_post;
  float scalar;
  const float* w_in;
  float* h_dst;
  int H;
  float eps;
};

enum { EPI_STORE = 0, EPI_GATEUP = 1 };

// The fields are ordered without padding holes, so that the arguments fill
// three 64-byte lines: the kernel reads them in one round, where a fourth
// line, fetched later, was one more memory round trip of every launch.
struct GemvArgs {
  GemvSeg seg[3];
  int nseg;
  int K, NQ, W;           // K, quads per row, waves per matrix tile
  int NQs;                // quads per split (blockIdx.y = split; NQ when unsplit)
  int ra_n;               // read-ahead: float4 per array (below)
  long y_split;           // EPI_STORE: floats between the partial products
  const uint16_t* x;      // fp16 [rows][ldx]
  float* y;               // EPI_STORE: fp32 [rows][ldy]
  uint16_t* a_out;        // EPI_GATEUP: fp16 [rows][inter] = GELU(gate) * up
  // Read-ahead for the one-workgroup launch that follows (the RMSNorm rows):
  // two fp32 arrays of ra_n float4 (its norm weights) are read by workgroups
  // 0, 8, 16, .. so that they sit in the L2 of the XCD that runs workgroup 0
  // of every launch (workgroups go round-robin over the 8 XCDs, and L2
  // contents outlive a launch).  Performance only; NULL: none.
  const float4* ra0;
  const float4* ra1;
  int ldx;
  int ldy;
  int inter;
  int n_rows;             // rows of x (<= B)
};
static_assert(sizeof(GemvArgs) <= 192, "GemvArgs fills at most three 64-byte lines");

Q4_DEV float gelu_tanh(float g) {
  const float k0 = 0.7978845608028654f;
  return 0.5f * g * (1.0f + tanhf(k0 * (g + 0.044715f * g * g * g)));
}

// (a & m) | c in one VALU op (the pattern is not selected from plain C).
Q4_DEV uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

// Dequantises one 32-bit code word (8 weights) into 4 exact fp16 pairs.
Q4_DEV void dq_word(uint32_t q, h2_t& v0, h2_t& v1, h2_t& v2, h2_t& v3) {
  const uint32_t t = q >> 8;
  const h2_t b1024 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2_t b64 = {(_Float16)72.0f, (_Float16)72.0f};
  v0 = as_h2(and_or(q, 0x000F000Fu, 0x64006400u)) - b1024;
  v1 = as_h2(and_or(q, 0x00F000F0u, 0x54005400u)) - b64;
  v2 = as_h2(and_or(t, 0x000F000Fu, 0x64006400u)) - b1024;
  v3 = as_h2(and_or(t, 0x00F000F0u, 0x54005400u)) - b64;
}

// Block-wide sum of NT threads (NT / 64 waves) in a fixed order, through LDS
// slots red[0 .. NT/64) that no other sum of the kernel uses (so no barrier
// guards their reuse), behind a barrier that orders LDS only (the global
// loads still in flight stay in flight).
template <int NT>
Q4_DEV float block_sum_once(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; i++) s += red[i];
  return s;
}

// fp16 pair (1024 + u_a, 1024 + u_b) of two code bytes of an int8 code word
Q4_DEV h2_t q8_pair(uint32_t w, uint32_t sel) { return as_h2(__builtin_amdgcn_perm(0x64646464u, w, sel)); }

// ------------------------------------------------------------ the kernel ----
// Grid: (tiles, S).  Block: 64 * W threads (EPI_GATEUP: 64 * 2W, the first W
// waves on the gate tile, the rest on the up tile; S = 1).  Dynamic LDS:
// B rows of NQs * UC halves of activation (plus 8 halves of padding per row
// when B > 1).
// FMT 0: q4 weights, a unit is a quad (16 rows x 4 blocks, UC = 128 columns),
// lane l holds row l & 15 and block l >> 4.  FMT 1: int8 weights
// (q8_kernels.h), a unit is a pair (16 rows x 2 blocks, UC = 64 columns), lane
// l holds row l & 15 and columns 16 (l >> 4) .. +15; its scales are laid out
// [unit][block][row].  NQ / NQs / CQ count units.
// (int8 at batch 4 allows 16 waves: a standalone product with K up to 16384
// needs them at 16 units per wave)
template <int B, int EPI, int CQ, int FMT>
__global__ void __launch_bounds__((B == 1 || FMT == 1) ? 1024 : 512) k_q4_gemv(GemvArgs a) {
  constexpr int UC = FMT == 0 ? 128 : 64;       // columns per unit
  extern __shared__ __align__(16) unsigned char smem_g[];
  const int ldxs = a.NQs * UC;                  // staged activation row (halves)
  // row pitch: batch rows start 16 B apart modulo the 256-byte bank period,
  // so the 4 rows one MFMA read spans fall in different LDS banks
  const int ldxp = ldxs + (B > 1 ? 8 : 0);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem_g);
  __shared__ float red[16 * B * 16];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int half = (EPI == EPI_GATEUP && wave >= a.W) ? 1 : 0;   // wave < 2 W
  const int wq = wave - half * a.W;
  const int tile = blockIdx.x, split = blockIdx.y;
  // every segment descriptor is read in one round of scalar loads and the
  // one this tile needs is selected without a dependent load
  const GemvSeg sg0 = a.seg[0], sg1 = a.seg[1], sg2 = a.seg[2];
  int s = half;
  if constexpr (EPI != EPI_GATEUP)
    s = (a.nseg > 1 && tile >= sg1.tile0 ? 1 : 0) + (a.nseg > 2 && tile >= sg2.tile0 ? 1 : 0);
  const u4v* seg_codes = s == 0 ? sg0.codes : (s == 1 ? sg1.codes : sg2.codes);
  const uint16_t* seg_scales = s == 0 ? sg0.scales : (s == 1 ? sg1.scales : sg2.scales);
  const int seg_N = s == 0 ? sg0.N : (s == 1 ? sg1.N : sg2.N);
  const int seg_off = s == 0 ? sg0.out_off : (s == 1 ? sg1.out_off : sg2.out_off);
  const int lt = (EPI == EPI_GATEUP) ? tile : tile - (s == 0 ? sg0.tile0 : (s == 1 ? sg1.tile0 : sg2.tile0));
  const int qs0 = split * a.NQs;                // first quad of this split
  const int qend = min(a.NQ, qs0 + a.NQs);
  const int q0raw = qs0 + wq * CQ;
  const int nq = max(0, min(CQ, qend - q0raw));
  const int q0 = nq > 0 ? q0raw : qs0;          // idle waves load (and ignore) valid quads
  const long tq = (long)lt * a.NQ + q0;

  // ---- loads, in the order their data is used: this thread's share of the
  // activation run, then the scales, then the codes.  Loads return in order,
  // so the activation reaches LDS as soon as its own load lands and quad i
  // is worked on as soon as its codes land, while the later quads are still
  // in flight.  A share beyond one u4v per thread and row (only very long
  // unsplit runs) is staged after the weights.
  const int nrow = a.n_rows;
  const int n8 = ldxs / 8;
  // threads of the workgroup, from the arguments (the launch derives the
  // block from them too): blockDim is an argument past the struct, in a line
  // the kernel would fetch on its own
  const int nthr = 64 * (EPI == EPI_GATEUP ? 2 * a.W : a.W);
  const int kx = qs0 * UC + threadIdx.x * 8;
  u4v xr[B];
#pragma unroll
  for (int bb = 0; bb < B; bb++) {
    const int br = min(bb, nrow - 1);
    xr[bb] = *reinterpret_cast<const u4v*>(a.x + (long)br * a.ldx + min(kx, a.K - 8));
  }
  __builtin_amdgcn_sched_barrier(0);
  u4v c[CQ];
  uint16_t sr[CQ];   // batch 1: this lane's scales
  u2v s4[CQ];        // batch 4: the scales of this lane's 4 MFMA rows
  {
    constexpr int SU = FMT == 0 ? 64 : 32;      // scales per unit
    const uint16_t* spp = FMT == 0 ? seg_scales + tq * 64 + (B == 1 ? lane : (lane & ~3))
                                   : seg_scales + tq * 32 + (g >> 1) * 16 + (B == 1 ? (lane & 15) : (lane & 12));
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      const long o = (long)(i < nq ? i : 0) * SU;
      if constexpr (B == 1) sr[i] = spp[o];
      else s4[i] = *reinterpret_cast<const u2v*>(spp + o);
    }
    const u4v* cp = seg_codes + tq * 64 + lane;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      c[i] = __builtin_nontemporal_load(cp + (long)(i < nq ? i : 0) * 64);
      __builtin_amdgcn_sched_barrier(0);   // keep the issue order
    }
  }
  // read-ahead, issued after this wave's own loads: one 64-byte line per lane
  // of wave 0 of workgroups 0, 8, 16, ..
  float rav = 0.f;
  {
    // (the launches that read ahead have one segment, whose tiles are the
    // grid's x extent: the grid size itself is an argument past the struct)
    const int id = blockIdx.y * sg0.T + blockIdx.x;
    const int line = (id >> 3) * 64 + lane;
    if (a.ra0 && (id & 7) == 0 && threadIdx.x < 64 && line * 4 < a.ra_n)
      rav = a.ra0[line * 4].x + a.ra1[line * 4].x;
  }
  {
    const bool in = threadIdx.x < n8;
    const bool kin = kx < a.K;
#pragma unroll
    for (int bb = 0; bb < B; bb++) {
      const u4v z = {0u, 0u, 0u, 0u};
      if (in) *reinterpret_cast<u4v*>(&xs[bb * ldxp + threadIdx.x * 8]) = (bb < nrow && kin) ? xr[bb] : z;
    }
#pragma unroll
    for (int bb = 0; bb < B; bb++)
      for (int i = threadIdx.x + nthr; i < n8; i += nthr) {
        const int k = qs0 * UC + i * 8;
        u4v v = {0u, 0u, 0u, 0u};
        if (bb < nrow && k < a.K) v = *reinterpret_cast<const u4v*>(a.x + (long)bb * a.ldx + k);
        *reinterpret_cast<u4v*>(&xs[bb * ldxp + i * 8]) = v;
      }
  }
  __syncthreads();

  const int qx = q0 - qs0;                      // unit index inside the staged run
  const h2_t b8 = {(_Float16)1152.0f, (_Float16)1152.0f};   // int8: 1024 + 128
  if constexpr (B == 1) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      const int ii = i < nq ? i : 0;
      const uint32_t qw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      float bs = 0.f;
      if constexpr (FMT == 0) {
        const u4v* xv = reinterpret_cast<const u4v*>(xs + ((qx + ii) * 4 + g) * 32);
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const u4v xx = xv[w];
          h2_t v0, v1, v2, v3;
          dq_word(qw[w], v0, v1, v2, v3);
          bs = __builtin_amdgcn_fdot2(v0, as_h2(xx.x), bs, false);
          bs = __builtin_amdgcn_fdot2(v1, as_h2(xx.y), bs, false);
          bs = __builtin_amdgcn_fdot2(v2, as_h2(xx.z), bs, false);
          bs = __builtin_amdgcn_fdot2(v3, as_h2(xx.w), bs, false);
        }
      } else {
        const u4v* xv = reinterpret_cast<const u4v*>(xs + (qx + ii) * 64 + g * 16);
        const u4v x0 = xv[0], x1 = xv[1];
        const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const h2_t lo = q8_pair(qw[w], 0x04010400u) - b8;
          const h2_t hi = q8_pair(qw[w], 0x04030402u) - b8;
          bs = __builtin_amdgcn_fdot2(lo, as_h2(xw[2 * w]), bs, false);
          bs = __builtin_amdgcn_fdot2(hi, as_h2(xw[2 * w + 1]), bs, false);
        }
      }
      const float d = i < nq ? h2f(sr[i]) : 0.f;
      acc = fmaf(d, bs, acc);
    }
    // the 4 lane groups hold the same 16 rows over different columns
    acc = rows_sum(acc);
    if (lane < 16) red[wave * 16 + lane] = acc;
  } else {
    // MFMA block m = lane / 4 holds rows 4m..4m+3 (mod 16) of lane group m / 4
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xl = xs + (lane & 3) * ldxp;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      const int ii = i < nq ? i : 0;
      const uint32_t qw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      f4_t cb = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FMT == 0) {
        const uint16_t* xb = xl + ((qx + ii) * 4 + g) * 32;
#pragma unroll
        for (int w = 0; w < 4; w++) {
          h2_t v0, v1, v2, v3;
          dq_word(qw[w], v0, v1, v2, v3);
          const u2v xa = *reinterpret_cast<const u2v*>(xb + 8 * w);
          const u2v xc = *reinterpret_cast<const u2v*>(xb + 8 * w + 4);
          const h4_t A0 = {v0.x, v0.y, v1.x, v1.y};
          const h4_t A1 = {v2.x, v2.y, v3.x, v3.y};
          cb = __builtin_amdgcn_mfma_f32_4x4x4f16(A0, __builtin_bit_cast(h4_t, xa), cb, 0, 0, 0);
          cb = __builtin_amdgcn_mfma_f32_4x4x4f16(A1, __builtin_bit_cast(h4_t, xc), cb, 0, 0, 0);
        }
      } else {
        const uint16_t* xb = xl + (qx + ii) * 64 + g * 16;
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const h2_t lo = q8_pair(qw[w], 0x04010400u) - b8;
          const h2_t hi = q8_pair(qw[w], 0x04030402u) - b8;
          const h4_t A = {lo.x, lo.y, hi.x, hi.y};
          const u2v xa = *reinterpret_cast<const u2v*>(xb + 4 * w);
          cb = __builtin_amdgcn_mfma_f32_4x4x4f16(A, __builtin_bit_cast(h4_t, xa), cb, 0, 0, 0);
        }
      }
      const bool ok = i < nq;
      const uint32_t s01 = s4[i].x, s23 = s4[i].y;
      acc[0] = fmaf(ok ? h2f((uint16_t)(s01 & 0xFFFF)) : 0.f, cb[0], acc[0]);
      acc[1] = fmaf(ok ? h2f((uint16_t)(s01 >> 16)) : 0.f, cb[1], acc[1]);
      acc[2] = fmaf(ok ? h2f((uint16_t)(s23 & 0xFFFF)) : 0.f, cb[2], acc[2]);
      acc[3] = fmaf(ok ? h2f((uint16_t)(s23 >> 16)) : 0.f, cb[3], acc[3]);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      acc[r] = rows_sum(acc[r]);
    }
    if (lane < 16) {
      const int bb = lane & 3;
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (bb < B) red[(wave * B + bb) * 16 + (lane & ~3) + r] = acc[r];
    }
  }
  __asm__ __volatile__("" :: "v"(rav));   // keeps the read-ahead loads
  __syncthreads();
  // ---- sum the waves in fixed order, then the epilogue
  const int t = threadIdx.x;
  if (t < B * 16) {
    const int bb = t >> 4, rr = t & 15;
    const int row = lt * 16 + rr;
    if constexpr (EPI == EPI_GATEUP) {
      float gv = 0.f, uv = 0.f;
      for (int w = 0; w < a.W; w++) {
        gv += red[(w * B + bb) * 16 + rr];
        uv += red[((a.W + w) * B + bb) * 16 + rr];
      }
      if (row < a.inter && bb < nrow) a.a_out[(long)bb * a.inter + row] = f2h(gelu_tanh(gv) * uv);
    } else {
      float v = 0.f;
      for (int w = 0; w < a.W; w++) v += red[(w * B + bb) * 16 + rr];
      if (row < seg_N && bb < nrow) a.y[split * a.y_split + (long)bb * a.ldy + seg_off + row] = v;
    }
  }
}

// ------------------------------------------------------------- RMSNorm ----
// One workgroup of 512 threads per row (H <= 4096, H % 4 == 0): h_new as in
// NormIn, stored to h_dst (when set), and x = fp16(RMSNorm(h_new) * w_in),
// the input of the next product.  Thread t handles elements 4 (t + 512 c) ..
// +3 through 16-byte loads, and every global load of the row is issued up
// front (a lone workgroup is bound by its CU's load issue: 16-byte loads
// move the row in a quarter of the instructions).  Partial products past ny
// alias the first and are added times 0, so no load waits for another; the
// two mean squares are block sums in a fixed order.
template <int MAXY>
__global__ void __launch_bounds__(512) k_norm_rows(NormIn p, uint16_t* x) {
  constexpr int NT = 512, C = 4096 / 4 / NT;
  __shared__ float nred[16];
  const int b = blockIdx.x;               // grid: the rows of the step
  const int H = p.H, tid = threadIdx.x, n4 = H / 4;
  // scalar bases and 32-bit element offsets (rows x H and the partials'
  // stride stay far below 2^31): 64-bit pointer arithmetic per partial took
  // most of the scalar instructions ahead of the first load
  const bool hy = p.y != nullptr;
  const float* y = hy ? p.y : nullptr;
  const float* ybase = hy ? p.y : p.h_src;   // partials past ny read the residual, times 0
  const unsigned rb = (unsigned)(b * H);     // this row's first element
  const unsigned ys = (unsigned)p.y_split;
  unsigned yo[MAXY];
  float mj[MAXY];
#pragma unroll
  for (int j = 0; j < MAXY; j++) {
    yo[j] = p.ny > j ? j * ys : 0u;
    mj[j] = p.ny > j ? 1.f : 0.f;
  }
  const float* wpb = hy ? p.w_post : p.w_in;
  float4 hv[C], ay[MAXY][C], wp[C], wi[C];
#pragma unroll
  for (int c = 0; c < C; c++) {
    const unsigned k4 = 4u * (unsigned)min(tid + NT * c, n4 - 1);
    hv[c] = *reinterpret_cast<const float4*>(p.h_src + (rb + k4));
#pragma unroll
    for (int j = 0; j < MAXY; j++) ay[j][c] = *reinterpret_cast<const float4*>(ybase + (yo[j] + rb + k4));
    wp[c] = *reinterpret_cast<const float4*>(wpb + k4);
    wi[c] = *reinterpret_cast<const float4*>(p.w_in + k4);
  }
  __builtin_amdgcn_sched_barrier(0);
  // partial sums in the order ((a0 + a1) + a2) + ..; out-of-range elements 0
  float yv[C][4], hh[C][4];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < C; c++) {
    const bool in = tid + NT * c < n4;
    const float HV[4] = {hv[c].x, hv[c].y, hv[c].z, hv[c].w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float v = ay[0][c][e];
#pragma unroll
      for (int j = 1; j < MAXY; j++) v = v + mj[j] * ay[j][c][e];
      yv[c][e] = (y && in) ? v : 0.f;
      hh[c][e] = in ? HV[e] : 0.f;
      ss += yv[c][e] * yv[c][e];
    }
  }
  float inv_y = 0.f;
  if (y) {
    ss = block_sum_once<NT>(ss, nred);
    inv_y = 1.0f / sqrtf(ss / (float)H + p.eps);
  }
  float ss2 = 0.f;
#pragma unroll
  for (int c = 0; c < C; c++) {
    const float WP[4] = {wp[c].x, wp[c].y, wp[c].z, wp[c].w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float v = hh[c][e];
      if (y) v += yv[c][e] * inv_y * WP[e];
      v *= p.scalar;
      hh[c][e] = v;
      ss2 += v * v;
    }
  }
  ss2 = block_sum_once<NT>(ss2, nred + NT / 64);
  const float inv_h = 1.0f / sqrtf(ss2 / (float)H + p.eps);
  float4* hd = p.h_dst ? reinterpret_cast<float4*>(p.h_dst + (long)b * H) : nullptr;
  uint2* xo = reinterpret_cast<uint2*>(x + (long)b * H);
#pragma unroll
  for (int c = 0; c < C; c++) {
    const int k = tid + NT * c;
    if (k < n4) {
      const float WI[4] = {wi[c].x, wi[c].y, wi[c].z, wi[c].w};
      if (hd) hd[k] = make_float4(hh[c][0], hh[c][1], hh[c][2], hh[c][3]);
      uint2 o;
      o.x = (uint32_t)f2h(hh[c][0] * inv_h * WI[0]) | ((uint32_t)f2h(hh[c][1] * inv_h * WI[1]) << 16);
      o.y = (uint32_t)f2h(hh[c][2] * inv_h * WI[2]) | ((uint32_t)f2h(hh[c][3] * inv_h * WI[3]) << 16);
      xo[k] = o;
    }
  }
}

// ------------------------------------------------------- fp16 tied head ----
// z[b][r] = E[r] . x[b]; logits = c * tanh(z / c); greedy argmax with the
// lowest index on ties (gemma4-12b card: tied embeddings, final softcap;
// 128k card, Limitations: the head emits a greedy argmax id).  Each
// workgroup stores its largest (order key << 32 | ~index) per row to a slot
// of its own, and k_argmax_out takes the maximum over the workgroups (one
// atomicMax per workgroup on a single word serialised ~1000 atomics at the
// kernel's end).  The maximum does not depend on the order, so the lowest
// index still wins ties.
constexpr int kHeadSlots = 4096;   // head workgroups at most (slots of 4 rows each)
struct HeadArgs {
  const uint16_t* E;       // [V][H]
  const uint16_t* x;       // [4][H]
  int V, H;
  float softcap;
  float* logits;           // [n][V] or NULL (when sp is NULL)
  const StepParams* sp;    // decode step: the logits pointer is read from here
  unsigned long long* best;  // [gridDim.x][4]: each workgroup's best key per row
  int n_rows;
};

template <int B>
__global__ void __launch_bounds__(256) k_head(HeadArgs a) {
  __shared__ unsigned long long sbest[4][4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = a.n_rows;
  float* const logits = a.sp ? a.sp->logits : a.logits;
  const int nchunk = a.H >> 3;           // 16-byte chunks per row
  const int J = (nchunk + 63) >> 6;      // chunks per lane (<= 8)
  u4v xr[B][8];
#pragma unroll
  for (int bb = 0; bb < B; bb++)
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int c = lane + 64 * j;
      xr[bb][j] = (j < J && c < nchunk && bb < n)
                      ? *reinterpret_cast<const u4v*>(a.x + (long)bb * a.H + c * 8)
                      : (u4v){0u, 0u, 0u, 0u};
    }
  unsigned long long best[B];
#pragma unroll
  for (int bb = 0; bb < B; bb++) best[bb] = 0ull;
  // wave gw takes rows 2 gw, 2 gw + 1, then 2 (gw + nw), ...: in each
  // iteration the grid's waves together read one contiguous stretch of E
  const long gw = (long)blockIdx.x * 4 + wave, nw = (long)gridDim.x * 4;
  for (long ra = 2 * gw; ra < a.V; ra += 2 * nw) {
    const long rb = ra + 1;
    const bool hasb = rb < a.V;
    u4v ea[8], eb[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int c = lane + 64 * j;
      const bool ok = j < J && c < nchunk;
      ea[j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u4v*>(a.E + ra * a.H) + c) : (u4v){0u, 0u, 0u, 0u};
      eb[j] = (ok && hasb) ? __builtin_nontemporal_load(reinterpret_cast<const u4v*>(a.E + rb * a.H) + c) : (u4v){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int bb = 0; bb < B; bb++) {
      float za = 0.f, zb = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t xe[4] = {xr[bb][j].x, xr[bb][j].y, xr[bb][j].z, xr[bb][j].w};
        const uint32_t ae[4] = {ea[j].x, ea[j].y, ea[j].z, ea[j].w};
        const uint32_t be[4] = {eb[j].x, eb[j].y, eb[j].z, eb[j].w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
          za = __builtin_amdgcn_fdot2(as_h2(ae[q]), as_h2(xe[q]), za, false);
          zb = __builtin_amdgcn_fdot2(as_h2(be[q]), as_h2(xe[q]), zb, false);
        }
      }
      za = wave_sum(za);
      zb = wave_sum(zb);
      if (bb < n) {
        const float la = a.softcap * tanhf(za / a.softcap);
        const float lb = a.softcap * tanhf(zb / a.softcap);
        if (lane == 0 && logits) {
          logits[(long)bb * a.V + ra] = la;
          if (hasb) logits[(long)bb * a.V + rb] = lb;
        }
        unsigned long long ka = ((unsigned long long)f32_order_key(la) << 32) | (0xFFFFFFFFu - (uint32_t)ra);
        best[bb] = ka > best[bb] ? ka : best[bb];
        if (hasb) {
          unsigned long long kb = ((unsigned long long)f32_order_key(lb) << 32) | (0xFFFFFFFFu - (uint32_t)rb);
          best[bb] = kb > best[bb] ? kb : best[bb];
        }
      }
    }
  }
  if (lane == 0)
#pragma unroll
    for (int bb = 0; bb < B; bb++) sbest[wave][bb] = best[bb];
  __syncthreads();
  if (threadIdx.x < B && threadIdx.x < n) {
    unsigned long long m = 0ull;
    for (int w = 0; w < 4; w++) m = sbest[w][threadIdx.x] > m ? sbest[w][threadIdx.x] : m;
    a.best[(long)blockIdx.x * 4 + threadIdx.x] = m;
  }
}

// The greedy id of each row from the head's per-workgroup slots (nb
// workgroups; the output from sp when it is set, else argmax).  The slots are
// written whole by every head launch, so nothing is cleared.
__global__ void __launch_bounds__(256) k_argmax_out(const unsigned long long* best, int nb, int n_rows,
                                                     int32_t* argmax, const StepParams* sp) {
  // the maximum of the nb workgroups' keys per row (256 threads, every load
  // issued before the first maximum), then the index it holds
  __shared__ unsigned long long red[4][4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (sp) argmax = sp->argmax;
  unsigned long long m[4] = {0ull, 0ull, 0ull, 0ull};
  for (int i = tid; i < nb; i += 256)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const unsigned long long v = r < n_rows ? best[(long)i * 4 + r] : 0ull;
      m[r] = v > m[r] ? v : m[r];
    }
#pragma unroll
  for (int r = 0; r < 4; r++) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long v = __shfl_xor(m[r], o, 64);
      m[r] = v > m[r] ? v : m[r];
    }
    if (lane == 0) red[wave][r] = m[r];
  }
  __syncthreads();
  if (tid < 4 && tid < n_rows && argmax) {
    unsigned long long k = 0ull;
    for (int w = 0; w < 4; w++) k = red[w][tid] > k ? red[w][tid] : k;
    argmax[tid] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
  }
}

}  // namespace q4k
