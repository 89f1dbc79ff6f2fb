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
  const double* inv_freq; // [rot_pairs]: theta^(-2i/D) in fp64
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
  AttnFin fin;
  int pos0[64];
};

Q4_DEV long attn_rec(const AttnArgs& a, int seq, int row, int kvh, int split, int col, int D) {
  return (((((long)seq * a.n_rows + row) * a.Hkv + kvh) * a.S + split) * a.GQ + col) * (long)(D + 4);
}

template <int D>
constexpr size_t fd_lds_bytes() {
  return (size_t)4 * 32 * (D + 2) * 2 + (size_t)2 * 4 * D * 2;
}

// Per-head RMSNorm (weight w, or scale-free when w == NULL) and RoPE at
// position pos on one head vector, done by one wave; src fp32 [D] -> dst
// fp16 [D].  scratch: D floats of this wave's LDS.
template <int D>
Q4_DEV void finish_head(const float* src, const float* w, bool rope, int pos, const AttnFin& f,
                        float* scratch, uint16_t* dst) {
  const int lane = threadIdx.x & 63;
  float v[D / 64 > 0 ? D / 64 : 1];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; e++) { v[e] = src[lane + 64 * e]; ss += v[e] * v[e]; }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D + f.eps);
#pragma unroll
  for (int e = 0; e < D / 64; e++) {
    const int d = lane + 64 * e;
    scratch[d] = v[e] * inv * (w ? w[d] : 1.0f);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  constexpr int half = D / 2;
  for (int i = lane; i < half; i += 64) {
    float x0 = scratch[i], x1 = scratch[i + half];
    if (rope && i < f.rot_pairs) {
      // angle pos * theta^(-2i/D) in fp64, reduced to [-pi, pi] in fp64 by
      // one fma with the double nearest 2 pi (k * 2.5e-16 rad of error, under
      // 1e-10 for positions below 2^20), then cos/sin in fp32
      const double ang = (double)pos * f.inv_freq[i];
      const double k = rint(ang * 0.15915494309189535);
      const float r = (float)fma(-k, 6.283185307179586, ang);
      float s, c;
      sincosf(r, &s, &c);
      const float y0 = x0 * c - x1 * s;
      const float y1 = x1 * c + x0 * s;
      x0 = y0; x1 = y1;
    }
    dst[i] = f2h(x0);
    dst[i + half] = f2h(x1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int D>
__global__ void __launch_bounds__(256) k_fd_partial(AttnArgs a) {
  constexpr int VROW = D + 2;                 // LDS row pitch (halves): 1-dword pad
  constexpr int NDS = D / 16;                 // PV dim steps
  constexpr int NKS = D / 32;                 // QK k steps
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* vlds = reinterpret_cast<uint16_t*>(smem);
  uint16_t* newK = vlds + 4 * 32 * VROW;      // [4][D] rows of this step (decode step)
  uint16_t* newV = newK + 4 * D;
  __shared__ float wm[4][16], wl[4][16];

  const int split = blockIdx.x, kvh = blockIdx.y;
  const int seq = blockIdx.z / a.n_rows, row = blockIdx.z - seq * a.n_rows;
  const int nlive = a.sp ? a.sp->n : a.n_rows;
  if (row >= nlive) return;
  const int base = a.sp ? a.sp->pos0 : a.pos0[seq];
  const int P = base + row;
  const int lo = a.ring ? max(0, P - a.W + 1) : 0;
  const int L = P - lo + 1;
  const int chunk = (L + a.S - 1) / a.S;
  const int st = lo + split * chunk;
  const int en = min(st + chunk, P + 1);
  const int P0new = a.fin_on ? base : 0x7FFFFFFF;   // first position formed in this step

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const bool col_ok = j < a.GQ;

  uint16_t* kb = a.k + seq * a.seq_stride + (a.ring ? (long)kvh * a.R * D : 0);
  uint16_t* vb = a.v + seq * a.seq_stride + (a.ring ? (long)kvh * a.R * D : 0);

  // ---- queries of this workgroup's columns as the MFMA B operand
  h8_t qb[NKS];
  if (a.fin_on) {
    const AttnFin& f = a.fin;
    uint16_t* q16 = vlds;                                   // [16][D], aliases the V rows
    float* scratch = reinterpret_cast<float*>(vlds + 16 * D) + wave * D;
    for (int c = wave; c < a.GQ; c += 4) {
      const int h = kvh * a.GQ + c;
      finish_head<D>(f.qkv + (long)row * f.ldq + (long)h * D, f.q_norm, true, P, f, scratch, q16 + c * D);
    }
    // rows of this step inside [st, en): wave r forms row r (k, then v)
    if (wave < nlive && wave <= row) {
      const int p = base + wave;
      if (p >= st && p < en) {
        const float* raw = f.qkv + (long)wave * f.ldq;
        const float* rk = raw + (long)(a.Hq + kvh) * D;
        finish_head<D>(rk, f.k_norm, true, p, f, scratch, newK + wave * D);
        const float* rv = a.ring ? raw + (long)(a.Hq + a.Hkv + kvh) * D : rk;  // full: V from raw k
        if (f.v_norm) {
          finish_head<D>(rv, nullptr, false, p, f, scratch, newV + wave * D);
        } else {
          for (int d = lane; d < D; d += 64) newV[wave * D + d] = f2h(rv[d]);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
        if (wave == row) {     // this workgroup owns position p: store the row
          const long so = (long)(a.ring ? p % a.R : p) * D;
          for (int d = lane; d < D; d += 64) {
            kb[so + d] = newK[wave * D + d];
            vb[so + d] = newV[wave * D + d];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(q16 + (col_ok ? j : 0) * D + 32 * s + 8 * g);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      qb[s] = __builtin_bit_cast(h8_t, t);
    }
    __syncthreads();
  } else {
    const uint16_t* qp = a.q + (((long)seq * a.n_rows + row) * a.Hq + (col_ok ? kvh * a.GQ + j : 0)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      u4v t = *reinterpret_cast<const u4v*>(qp + 32 * s);
      if (!col_ok) t = (u4v){0u, 0u, 0u, 0u};
      qb[s] = __builtin_bit_cast(h8_t, t);
    }
  }
  uint16_t* vl = vlds + wave * 32 * VROW;

  float m_run = -INFINITY, l_part = 0.f;
  f4_t O[NDS];
#pragma unroll
  for (int d = 0; d < NDS; d++) O[d] = (f4_t){0.f, 0.f, 0.f, 0.f};

  for (int t0 = st + 32 * wave; t0 < en; t0 += 128) {
    // MFMA row r of half h <-> tile position 8*(r/4) + 4h + r%4, so lane
    // (column j, group g) ends up holding positions 8g .. 8g+7 of the tile.
    const bool fresh = t0 + 31 >= P0new;      // this tile may hold rows of this step
    const int pa = t0 + 8 * (j >> 2) + (j & 3);
    const int pb = pa + 4;
    const int pac = pa < en ? pa : st, pbc = pb < en ? pb : st;
    const int sa = a.ring ? pac % a.R : pac;
    const int sb = a.ring ? pbc % a.R : pbc;
    f4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t* ka = (fresh && pac >= P0new) ? newK + (pac - P0new) * D + 8 * g : kb + (long)sa * D + 8 * g;
      const uint16_t* kc = (fresh && pbc >= P0new) ? newK + (pbc - P0new) * D + 8 * g : kb + (long)sb * D + 8 * g;
      h8_t KA[NKS], KB[NKS];
      if (!fresh) {
#pragma unroll
        for (int s = 0; s < NKS; s++) {
          KA[s] = __builtin_bit_cast(h8_t, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(ka + 32 * s)));
          KB[s] = __builtin_bit_cast(h8_t, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(kc + 32 * s)));
        }
      } else {
#pragma unroll
        for (int s = 0; s < NKS; s++) {
          KA[s] = __builtin_bit_cast(h8_t, *reinterpret_cast<const u4v*>(ka + 32 * s));
          KB[s] = __builtin_bit_cast(h8_t, *reinterpret_cast<const u4v*>(kc + 32 * s));
        }
      }
      // stage the V tile (32 positions) into this wave's LDS rows
#pragma unroll 4
      for (int c = lane; c < 32 * (D / 8); c += 64) {
        const int r = c / (D / 8), cc = c - r * (D / 8);
        const int p = t0 + r;
        const int pc = p < en ? p : st;
        u4v vv;
        if (fresh && pc >= P0new) vv = *reinterpret_cast<const u4v*>(newV + (pc - P0new) * D + cc * 8);
        else {
          const int sl = a.ring ? pc % a.R : pc;
          vv = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(vb + (long)sl * D + cc * 8));
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(vl + r * VROW + cc * 8);
        dst[0] = vv.x; dst[1] = vv.y; dst[2] = vv.z; dst[3] = vv.w;
      }
#pragma unroll
      for (int s = 0; s < NKS; s++) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KA[s], qb[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(KB[s], qb[s], s1, 0, 0, 0);
      }
    }
    // lane (j, g): reg i of s0 -> position t0 + 8g + i; of s1 -> t0 + 8g + 4 + i
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sv[i] = (t0 + 8 * g + i < en) ? s0[i] * a.scale_log2 : -INFINITY;
      sv[4 + i] = (t0 + 8 * g + 4 + i < en) ? s1[i] * a.scale_log2 : -INFINITY;
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) { p[i] = exp2f(sv[i] - m_new); ps += p[i]; }
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // O += P V: B operand lane (dim 16d + j, group g) = V[8g .. 8g+7][dim]
#pragma unroll
    for (int d = 0; d < NDS; d++) {
      const uint16_t* vc = vl + 8 * g * VROW + 16 * d + j;
      h8_t Bv;
#pragma unroll
      for (int e = 0; e < 8; e++) Bv[e] = __builtin_bit_cast(_Float16, vc[e * VROW]);
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

  // ---- merge the 4 waves through LDS (the V rows are free now)
  __syncthreads();
  float* ow = reinterpret_cast<float*>(smem);     // [4][16][D]
  if (lane < 16) { wm[wave][lane] = m_run; wl[wave][lane] = l_tot; }
#pragma unroll
  for (int d = 0; d < NDS; d++)
#pragma unroll
    for (int i = 0; i < 4; i++) ow[(wave * 16 + 4 * g + i) * D + 16 * d + j] = O[d][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.GQ * D; idx += 256) {
    const int col = idx / D, dim = idx - col * D;
    float M = wm[0][col];
#pragma unroll
    for (int w = 1; w < 4; w++) M = fmaxf(M, wm[w][col]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const float f = exp2f(wm[w][col] - M);
        o += f * ow[(w * 16 + col) * D + dim];
        l += f * wl[w][col];
      }
    }
    float* rec = a.part + attn_rec(a, seq, row, kvh, split, col, D);
    rec[dim] = o;
    if (dim == 0) { rec[D] = M; rec[D + 1] = l; }
  }
}

// out[seq][row][h][d] = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// Grid (n_seq * n_rows * Hq, D / 64); one wave per 64 output dims.
template <int D>
__global__ void __launch_bounds__(64) k_fd_combine(AttnArgs a, float* out32, uint16_t* out16) {
  __shared__ float wsp[256];
  const int idx = blockIdx.x;
  const int h = idx % a.Hq, sr = idx / a.Hq;
  const int seq = sr / a.n_rows, row = sr - seq * a.n_rows;
  const int nlive = a.sp ? a.sp->n : a.n_rows;
  if (row >= nlive) return;
  const int kvh = h / a.GQ, col = h - kvh * a.GQ;
  const int lane = threadIdx.x;
  const long r0 = attn_rec(a, seq, row, kvh, 0, col, D);
  const long rs = (long)a.GQ * (D + 4);                // stride between splits
  float M = -INFINITY;
  for (int s = lane; s < a.S; s += 64) M = fmaxf(M, a.part[r0 + s * rs + D]);
  M = wave_max(M);
  float L = 0.f;
  for (int s = lane; s < a.S; s += 64) {
    const float m = a.part[r0 + s * rs + D];
    const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
    wsp[s] = w;
    L += w * a.part[r0 + s * rs + D + 1];
  }
  L = wave_sum(L);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const int d = blockIdx.y * 64 + lane;
  float o = 0.f;
#pragma unroll 8
  for (int s = 0; s < a.S; s++) o += wsp[s] * a.part[r0 + s * rs + d];
  o *= (L > 0.f) ? 1.0f / L : 0.f;
  const long oi = (((long)seq * a.n_rows + row) * a.Hq + h) * D + d;
  if (out32) out32[oi] = o;
  if (out16) out16[oi] = f2h(o);
}

}  // namespace q4k
