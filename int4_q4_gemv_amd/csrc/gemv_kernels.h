// gemv_kernels.h -- int4 q4_0 matrix-vector products for gfx950, and the fp16
// tied-head product with softcap and argmax.
//
// Work split: a 64-row tile of one matrix is cut along K into chunks of CB
// blocks; each wave streams one chunk (one 16-byte load per lane per block,
// so every wave-wide load is 1 KB contiguous) and a workgroup of 4 waves
// takes 4 consecutive chunks of the same tile.  Partial sums meet in LDS
// (fixed order), and when a tile spans G > 1 workgroups the last one to
// finish adds the G partials in fixed order, so results are deterministic.
//
// Batch 1: each lane owns one row; the activation is wave-uniform and is read
// through the scalar cache; dequantisation is the fp16 magic-number trick
// (1024 + u, 64 + u) minus the bias, exact, then v_dot2_f32_f16.
// Batch 2..4 (the width-4 verify block): v_mfma_f32_4x4x4_16b_f16 with the
// 64 rows as 16 blocks of 4, the batch as the 4 columns; each lane still
// dequantises only its own row, and per-block scales are applied to the
// fp32 accumulator, so the dequantised weights stay exact.
#pragma once
#include "device_common.h"

namespace q4k {


struct GemvSeg {
  const u4v* codes;
  const uint16_t* scales;
  int N;        // rows of this matrix
  int T;        // 64-row tiles
  int tile0;    // first global tile index
  int out_off;  // first output column in the concatenated output row
};

enum { EPI_STORE = 0, EPI_QKV = 1, EPI_GATEUP = 2, EPI_RESID = 3 };

struct StepParams {       // written on the device at the start of every step
  int pos0;
  int n;
  int tokens[4];
};

struct EpiArgs {
  const StepParams* sp;   // decode step: positions and row count (NULL otherwise)
  unsigned* grp_cnt;      // per output group completion counters
  int grp_tiles;          // tiles per group
  // QKV
  int Hq, Hkv, D, is_full, v_norm, rot_pairs, R;
  double theta;
  float eps;
  const float* q_norm;
  const float* k_norm;
  uint16_t* q_out;        // fp16 [4][Hq][D]
  uint16_t* k_cache;
  uint16_t* v_cache;
  // GATEUP
  int inter;
  uint16_t* a_out;        // fp16 [4][inter]
  // RESID
  int H;
  float* h;               // fp32 [4][H]
  const float* w_post;
  const float* w_next;
  float scalar;
  uint16_t* x_out;        // fp16 [4][H]
};

struct GemvArgs {
  GemvSeg seg[3];
  int nseg;
  int K, NB, CB, G;
  const uint16_t* x;      // fp16 [B][ldx]
  int ldx;
  float* y;               // fp32 output / stage, [B][ldy]
  int ldy;
  float* partial;         // [tiles][G][B][64]
  unsigned* tile_cnt;     // [tiles]
  int n_rows;             // rows of x actually used (<= B); ignored when sp given
  EpiArgs e;
};

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

// ------------------------------------------------------------ epilogues ----
// Per-head q/k/v finishing of the decode step (gemma4-12b card, architecture
// notes): q, k get RMSNorm with learned scale then RoPE; V on full layers is
// the raw k projection after a scale-free RMSNorm (attention_k_eq_v).
Q4_DEV void epi_head(const GemvArgs& a, int head, float* lds) {
  const EpiArgs& e = a.e;
  const int D = e.D, tid = threadIdx.x;
  const int n = e.sp->n;
  float* buf = lds;          // D floats
  float* red = lds + 512;    // 4 floats
  for (int b = 0; b < n; b++) {
    const int P = e.sp->pos0 + b;
    const float* src;
    int kind;   // 0 q, 1 k, 2 v
    int g;
    if (head < e.Hq) { kind = 0; g = head; src = a.y + (long)b * a.ldy + head * D; }
    else if (head < e.Hq + e.Hkv) { kind = 1; g = head - e.Hq; src = a.y + (long)b * a.ldy + head * D; }
    else { kind = 2; g = head - e.Hq - e.Hkv; src = a.y + (long)b * a.ldy + head * D; }
    float v0 = tid < D ? src[tid] : 0.f;
    float v1 = tid + 256 < D ? src[tid + 256] : 0.f;
    const float ss = block_sum<256>(v0 * v0 + v1 * v1, red);
    const float inv = 1.0f / sqrtf(ss / (float)D + e.eps);
    long slot_off;
    if (e.is_full) slot_off = (long)P * D;
    else slot_off = ((long)g * e.R + (P % e.R)) * D;
    if (kind == 2) {      // sliding V row
      uint16_t* dst = e.v_cache + slot_off;
      if (e.v_norm) {
        if (tid < D) dst[tid] = f2h(v0 * inv);
        if (tid + 256 < D) dst[tid + 256] = f2h(v1 * inv);
      } else {
        if (tid < D) dst[tid] = f2h(v0);
        if (tid + 256 < D) dst[tid + 256] = f2h(v1);
      }
      __syncthreads();
      continue;
    }
    if (kind == 1 && e.is_full) {   // V = scale-free RMSNorm of the raw key row
      uint16_t* dst = e.v_cache + slot_off;
      if (tid < D) dst[tid] = f2h(e.v_norm ? v0 * inv : v0);
      if (tid + 256 < D) dst[tid + 256] = f2h(e.v_norm ? v1 * inv : v1);
    }
    const float* wn = kind == 0 ? e.q_norm : e.k_norm;
    if (tid < D) buf[tid] = v0 * inv * wn[tid];
    if (tid + 256 < D) buf[tid + 256] = v1 * inv * wn[tid + 256];
    __syncthreads();
    const int half = D >> 1;
    uint16_t* dst = (kind == 0) ? e.q_out + ((long)b * e.Hq + g) * D : e.k_cache + slot_off;
    if (tid < half) {
      float x0 = buf[tid], x1 = buf[tid + half];
      if (tid < e.rot_pairs) {
        // angle P * theta^(-2i/D) in fp64, cos/sin rounded to fp32
        const double inv_freq = pow(e.theta, -2.0 * (double)tid / (double)D);
        const double ang = (double)P * inv_freq;
        const float c = (float)cos(ang), s = (float)sin(ang);
        const float y0 = x0 * c - x1 * s;
        const float y1 = x1 * c + x0 * s;
        x0 = y0; x1 = y1;
      }
      dst[tid] = f2h(x0);
      dst[tid + half] = f2h(x1);
    }
    __syncthreads();
  }
}

// h <- (h + RMSNorm(y) * w_post) * scalar;  x_out <- fp16(RMSNorm(h) * w_next)
Q4_DEV void epi_resid(const GemvArgs& a, float* lds) {
  const EpiArgs& e = a.e;
  const int H = e.H, tid = threadIdx.x;
  const int n = e.sp->n;
  float* red = lds + 512;
  for (int b = 0; b < n; b++) {
    const float* y = a.y + (long)b * a.ldy;
    float* h = e.h + (long)b * H;
    float ss = 0.f;
    for (int i = tid; i < H; i += 256) { float v = y[i]; ss += v * v; }
    ss = block_sum<256>(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)H + e.eps);
    float ss2 = 0.f;
    for (int i = tid; i < H; i += 256) {
      float hn = (h[i] + y[i] * inv * e.w_post[i]) * e.scalar;
      h[i] = hn;
      ss2 += hn * hn;
    }
    ss2 = block_sum<256>(ss2, red);
    const float inv2 = 1.0f / sqrtf(ss2 / (float)H + e.eps);
    uint16_t* xo = e.x_out + (long)b * H;
    for (int i = tid; i < H; i += 256) xo[i] = f2h(h[i] * inv2 * e.w_next[i]);
    __syncthreads();
  }
}

// ------------------------------------------------------------ the kernel ----
template <int B, int EPI, int CB>
__global__ void __launch_bounds__(256) k_q4_gemv(GemvArgs a) {
  __shared__ float red[4 * B * 64];
  __shared__ float elds[520];
  __shared__ int flag;
  __shared__ __align__(16) uint16_t xs[B * 4 * CB * 32];   // [B][4 waves * CB * 32]

  const int tile = blockIdx.x / a.G;
  const int g = blockIdx.x - tile * a.G;
  int s = 0;
  if (a.nseg > 1 && tile >= a.seg[1].tile0) s = 1;
  if (a.nseg > 2 && tile >= a.seg[2].tile0) s = 2;
  const GemvSeg& sg = a.seg[s];
  const int lt = tile - sg.tile0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int chunk = g * 4 + wave;
  const int b0raw = chunk * CB;
  const int nb = max(0, min(CB, a.NB - b0raw));
  const int b0 = nb > 0 ? b0raw : 0;
  const long tb = (long)lt * a.NB + b0;
  const u4v* cp = sg.codes + tb * 64 + lane;
  const int nrow = a.e.sp ? a.e.sp->n : a.n_rows;

  // this workgroup's slice of x (every batch row): fetched first, stored to
  // LDS after the weight loads are in flight
  constexpr int span = 4 * CB * 32;
  constexpr int XPT = (B * span / 8 + 255) / 256;
  uint4 xv_stage[XPT];
  {
    const int kw0 = g * span;
    const int kwn = min(span, a.K - kw0);
#pragma unroll
    for (int r = 0; r < XPT; r++) {
      const int i = threadIdx.x + 256 * r;
      const int bb = i / (span / 8);
      const int kk = (i - bb * (span / 8)) * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (i < B * span / 8 && bb < nrow && kk < kwn)
        v = *reinterpret_cast<const uint4*>(a.x + (long)bb * a.ldx + kw0 + kk);
      xv_stage[r] = v;
    }
  }
  auto stage_x = [&]() {
#pragma unroll
    for (int r = 0; r < XPT; r++) {
      const int i = threadIdx.x + 256 * r;
      if (i < B * span / 8) {
        const int bb = i / (span / 8);
        const int kk = (i - bb * (span / 8)) * 8;
        *reinterpret_cast<uint4*>(&xs[bb * span + kk]) = xv_stage[r];
      }
    }
    __syncthreads();
  };

  if constexpr (B == 1) {
    const uint16_t* sp = sg.scales + tb * 64 + lane;
    u4v c[CB];
    uint16_t sraw[CB];
#pragma unroll
    for (int i = 0; i < CB; i++) {
      const int ii = i < nb ? i : 0;
      c[i] = __builtin_nontemporal_load(cp + (long)ii * 64);
      sraw[i] = sp[(long)ii * 64];
    }
    stage_x();
    float acc = 0.f;
    const uint16_t* xl = xs + wave * CB * 32;
#pragma unroll
    for (int i = 0; i < CB; i++) {
      const u4v* xv = reinterpret_cast<const u4v*>(xl + i * 32);
      const uint32_t qw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      float bs = 0.f;
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
      const float d = i < nb ? h2f(sraw[i]) : 0.f;
      acc = fmaf(d, bs, acc);
    }
    red[wave * 64 + lane] = acc;
  } else {
    const uint16_t* sp = sg.scales + tb * 64 + (lane & ~3);
    u4v c[CB];
    u2v sc4[CB];
#pragma unroll
    for (int i = 0; i < CB; i++) {
      const int ii = i < nb ? i : 0;
      c[i] = __builtin_nontemporal_load(cp + (long)ii * 64);
      sc4[i] = *reinterpret_cast<const u2v*>(sp + (long)ii * 64);
    }
    stage_x();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xl = xs + (lane & 3) * span + wave * CB * 32;
#pragma unroll
    for (int i = 0; i < CB; i++) {
      const uint32_t qw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      f4_t cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; w++) {
        h2_t v0, v1, v2, v3;
        dq_word(qw[w], v0, v1, v2, v3);
        const u2v xa = *reinterpret_cast<const u2v*>(xl + i * 32 + 8 * w);
        const u2v xb = *reinterpret_cast<const u2v*>(xl + i * 32 + 8 * w + 4);
        const h4_t A0 = {v0.x, v0.y, v1.x, v1.y};
        const h4_t A1 = {v2.x, v2.y, v3.x, v3.y};
        cb = __builtin_amdgcn_mfma_f32_4x4x4f16(A0, __builtin_bit_cast(h4_t, xa), cb, 0, 0, 0);
        cb = __builtin_amdgcn_mfma_f32_4x4x4f16(A1, __builtin_bit_cast(h4_t, xb), cb, 0, 0, 0);
      }
      const bool ok = i < nb;
      const uint32_t s01 = sc4[i].x, s23 = sc4[i].y;
      acc[0] = fmaf(ok ? h2f((uint16_t)(s01 & 0xFFFF)) : 0.f, cb[0], acc[0]);
      acc[1] = fmaf(ok ? h2f((uint16_t)(s01 >> 16)) : 0.f, cb[1], acc[1]);
      acc[2] = fmaf(ok ? h2f((uint16_t)(s23 & 0xFFFF)) : 0.f, cb[2], acc[2]);
      acc[3] = fmaf(ok ? h2f((uint16_t)(s23 >> 16)) : 0.f, cb[3], acc[3]);
    }
    // lane holds rows 4*(lane/4)+r for batch lane%4
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int row = (lane & ~3) + r, bb = lane & 3;
      if (bb < B) red[(wave * B + bb) * 64 + row] = acc[r];
    }
  }
  __syncthreads();

  // ---- reduce the 4 waves, then the G workgroups of the tile
  const int t = threadIdx.x;
  float v = 0.f;
  if (t < B * 64) {
    const int bb = t >> 6, row = t & 63;
#pragma unroll
    for (int w = 0; w < 4; w++) v += red[(w * B + bb) * 64 + row];
  }
  if (a.G > 1) {
    float* pt = a.partial + (long)tile * a.G * B * 64;
    if (t < B * 64) pt[g * B * 64 + t] = v;
    if (!last_arrival(a.tile_cnt + tile, (unsigned)a.G, &flag)) return;
    if (t < B * 64) {
      v = 0.f;
      for (int j = 0; j < a.G; j++) v += __builtin_nontemporal_load(pt + j * B * 64 + t);
    }
  }
  // ---- epilogue
  if (t < B * 64) {
    const int bb = t >> 6, row = lt * 64 + (t & 63);
    if (row < sg.N && bb < nrow) a.y[(long)bb * a.ldy + sg.out_off + row] = v;
  }
  if constexpr (EPI == EPI_STORE) return;
  int grp;
  unsigned expect;
  if constexpr (EPI == EPI_QKV) { grp = (sg.out_off + lt * 64) / (a.e.grp_tiles * 64); expect = a.e.grp_tiles; }
  else if constexpr (EPI == EPI_GATEUP) { grp = lt; expect = 2; }
  else { grp = 0; expect = (unsigned)(a.seg[0].T); }
  if (!last_arrival(a.e.grp_cnt + grp, expect, &flag)) return;
  if constexpr (EPI == EPI_QKV) {
    epi_head(a, grp, elds);
  } else if constexpr (EPI == EPI_GATEUP) {
    const int n = a.e.sp->n;
    for (int i = threadIdx.x; i < n * 64; i += 256) {
      const int bb = i >> 6, row = grp * 64 + (i & 63);
      if (row < a.e.inter) {
        const float gv = a.y[(long)bb * a.ldy + row];
        const float uv = a.y[(long)bb * a.ldy + a.e.inter + row];
        a.e.a_out[(long)bb * a.e.inter + row] = f2h(gelu_tanh(gv) * uv);
      }
    }
  } else {
    epi_resid(a, elds);
  }
}

// ------------------------------------------------------- fp16 tied head ----
// z[b][r] = E[r] . x[b]; logits = c * tanh(z / c); greedy argmax with the
// lowest index on ties (gemma4-12b card: tied embeddings, final softcap;
// 128k card, Limitations: the head emits a greedy argmax id).
struct HeadArgs {
  const uint16_t* E;       // [V][H]
  const uint16_t* x;       // [4][H]
  int V, H;
  float softcap;
  float* logits;           // [n][V] or NULL
  unsigned long long* best;  // [4] packed (key << 32 | ~idx), zeroed before
  unsigned* cnt;
  int32_t* argmax;         // [n] or NULL
  const StepParams* sp;
  int n_rows;
  int rows_per_wave;
};

template <int B>
__global__ void __launch_bounds__(256) k_head(HeadArgs a) {
  __shared__ unsigned long long sbest[4][4];
  __shared__ int flag;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = a.sp ? a.sp->n : a.n_rows;
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
  const long gw = (long)blockIdx.x * 4 + wave;
  const long r0 = gw * a.rows_per_wave;
  for (int rr = 0; rr < a.rows_per_wave; rr += 2) {
    const long ra = r0 + rr, rb = r0 + rr + 1;
    if (ra >= a.V) break;
    const bool hasb = (rr + 1 < a.rows_per_wave) && rb < a.V;
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
        if (lane == 0 && a.logits) {
          a.logits[(long)bb * a.V + ra] = la;
          if (hasb) a.logits[(long)bb * a.V + rb] = lb;
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
    atomicMax(a.best + threadIdx.x, m);
  }
  if (!last_arrival(a.cnt, gridDim.x, &flag)) return;
  if (threadIdx.x < n) {
    const unsigned long long m = atomicExch(a.best + threadIdx.x, 0ull);
    if (a.argmax) a.argmax[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
  }
}

}  // namespace q4k
