// q8_kernels.h -- int8 ("int8lin") weights: quantisation into the device
// layout, export to the canonical block format, and the matrix-vector
// product.
//
// Grid (gemma4-12b card, intro and Throughput: the int8lin ship beside
// int4linsym; its block format is not given, so the int4 rule is taken on the
// int8 grid): per block of 32 weights d = fp16_rne(absmax / 127) and
// q = clamp(round_half_away(w / d), -127, 127), the quotient an IEEE fp32
// division against the stored fp16 scale.
//
// Device layout (this library's): one wave-wide 16-byte load fetches a
// "pair" = 16 consecutive rows x 2 consecutive blocks (64 columns), lane l
// holding row (l & 15) and the 16-column segment s = l >> 4 (block s >> 1,
// half s & 1):
//   codes  [T = ceil(N/16)][NP = ceil(K/64)][64 lanes][16 bytes]
//   scales [T][NP][2 blocks][16 rows] fp16, right after the codes.
// Code byte j of a lane is u = q + 128 of column 16 s + j of the pair, so that
//   perm(0x64646464, word, 0x04010400) -> fp16 pair (1024 + u0, 1024 + u1)
//   perm(0x64646464, word, 0x04030402) -> fp16 pair (1024 + u2, 1024 + u3)
// and subtracting 1152 gives the codes exactly.  Rows past N and blocks past
// K/32 are padding with zero scale and zero codes.
#pragma once
#include "device_common.h"

namespace q4k {

// One thread per (tile, pair, row, block of the pair).
template <int DT>   // 0: fp32 input, 1: bf16 input
__global__ void __launch_bounds__(256) k_q8_pack(const void* __restrict__ w, int N, int K,
                                                 u4v* __restrict__ codes,
                                                 uint16_t* __restrict__ scales, int T,
                                                 int32_t* nonfinite) {
  const int NB = K >> 5, NP = (NB + 1) >> 1;
  const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
  const long total = (long)T * NP * 32;
  if (gid >= total) return;
  const int lr = (int)(gid & 31), row = lr & 15, blk = lr >> 4;
  const long tp = gid >> 5;            // t * NP + p
  const int p = (int)(tp % NP);
  const int t = (int)(tp / NP);
  const int n = t * 16 + row;
  const int b = p * 2 + blk;
  uint32_t wd[8] = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u,
                    0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
  uint16_t d16 = 0;
  if (n < N && b < NB) {
    float v[32];
    if (DT == 0) {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(w) + (long)n * K + b * 32);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + (long)n * K + b * 32);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 u = src[i];
        const uint32_t a[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[8 * i + 2 * j] = __builtin_bit_cast(float, a[j] << 16);
          v[8 * i + 2 * j + 1] = __builtin_bit_cast(float, a[j] & 0xFFFF0000u);
        }
      }
    }
    float amax = 0.f;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 32; i++) {
      bad |= !__builtin_isfinite(v[i]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    d16 = bad ? (uint16_t)0 : f2h(amax / 127.0f);
    const float d = h2f(d16);
    if (bad || !__builtin_isfinite(d)) {
      d16 = 0;
      if (nonfinite) atomicAdd(nonfinite, 1);
    } else if (d != 0.f) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          float rr = roundf(v[4 * i + k] / d);  // correctly rounded fp32 division
          rr = fminf(fmaxf(rr, -127.f), 127.f);
          acc |= (uint32_t)((int)rr + 128) << (8 * k);
        }
        wd[i] = acc;
      }
    }
  }
  u4v* dst = codes + tp * 64 + blk * 32 + row;   // lanes (2 blk) * 16 + row and +16
  dst[0] = (u4v){wd[0], wd[1], wd[2], wd[3]};
  dst[16] = (u4v){wd[4], wd[5], wd[6], wd[7]};
  scales[(tp * 2 + blk) * 16 + row] = d16;
}

// One thread per (row, block): device layout -> canonical 34-byte block.
__global__ void __launch_bounds__(256) k_q8_unpack(const u4v* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int N,
                                                   int K, uint8_t* __restrict__ blocks) {
  const int NB = K >> 5, NP = (NB + 1) >> 1;
  const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (gid >= (long)N * NB) return;
  const int n = (int)(gid / NB), b = (int)(gid % NB);
  const long tp = (long)(n >> 4) * NP + (b >> 1);
  const int blk = b & 1, row = n & 15;
  const u4v c0 = codes[tp * 64 + blk * 32 + row], c1 = codes[tp * 64 + blk * 32 + 16 + row];
  const uint32_t wd[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const uint16_t d16 = scales[(tp * 2 + blk) * 16 + row];
  uint8_t* o = blocks + gid * 34;
  o[0] = (uint8_t)(d16 & 0xFF);
  o[1] = (uint8_t)(d16 >> 8);
#pragma unroll
  for (int i = 0; i < 32; i++) o[2 + i] = (uint8_t)(((wd[i >> 2] >> (8 * (i & 3))) & 0xFFu) - 128u);
}

struct Q8Args {
  const u4v* codes;
  const uint16_t* scales;
  int N, K, NP, W;        // rows, columns, 64-column pairs per row, waves per tile
  const uint16_t* x;      // fp16 [rows][ldx]
  int ldx;
  float* y;               // fp32 [rows][ldy]
  int ldy;
  int n_rows;             // rows of x (<= B)
};

// fp16 pair (1024 + u_a, 1024 + u_b) of two code bytes of a word
Q4_DEV h2_t q8_pair(uint32_t w, uint32_t sel) { return as_h2(__builtin_amdgcn_perm(0x64646464u, w, sel)); }

// Grid: tiles.  Block: 64 * W threads, wave w streaming pairs w*CQ ..
// w*CQ + CQ - 1 of its 16-row tile (loads in the order used: activation run,
// scales, codes).  Dynamic LDS: B * NP * 64 halves of activation.  Batch 1:
// v_dot2_f32_f16 per lane; batch 2..4: v_mfma_f32_4x4x4_16b_f16 with the 64
// lanes as 16 blocks of 4 rows and the batch as the 4 columns, the block
// scale applied to the fp32 accumulator.
template <int B, int CQ>
__global__ void __launch_bounds__(1024) k_q8_gemv(Q8Args a) {
  extern __shared__ __align__(16) unsigned char smem_g[];
  const int ldxs = a.NP * 64;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem_g);
  __shared__ float red[16 * B * 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int q0raw = wave * CQ;
  const int nq = max(0, min(CQ, a.NP - q0raw));
  const int q0 = nq > 0 ? q0raw : 0;            // idle waves load (and ignore) valid pairs
  const long tq = (long)tile * a.NP + q0;
  const int nrow = a.n_rows;
  const int n8 = ldxs / 8;
  const int kx = threadIdx.x * 8;
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
    const uint16_t* spp = a.scales + tq * 32 + (g >> 1) * 16 + (B == 1 ? (lane & 15) : (lane & 12));
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      const long o = (long)(i < nq ? i : 0) * 32;
      if constexpr (B == 1) sr[i] = spp[o];
      else s4[i] = *reinterpret_cast<const u2v*>(spp + o);
    }
    const u4v* cp = a.codes + tq * 64 + lane;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      c[i] = __builtin_nontemporal_load(cp + (long)(i < nq ? i : 0) * 64);
      __builtin_amdgcn_sched_barrier(0);   // keep the issue order
    }
  }
  {
    const bool in = threadIdx.x < n8;
    const bool kin = kx < a.K;
#pragma unroll
    for (int bb = 0; bb < B; bb++) {
      const u4v z = {0u, 0u, 0u, 0u};
      if (in) *reinterpret_cast<u4v*>(&xs[bb * ldxs + threadIdx.x * 8]) = (bb < nrow && kin) ? xr[bb] : z;
    }
#pragma unroll
    for (int bb = 0; bb < B; bb++)
      for (int i = threadIdx.x + blockDim.x; i < n8; i += blockDim.x) {
        const int k = i * 8;
        u4v v = {0u, 0u, 0u, 0u};
        if (bb < nrow && k < a.K) v = *reinterpret_cast<const u4v*>(a.x + (long)bb * a.ldx + k);
        *reinterpret_cast<u4v*>(&xs[bb * ldxs + i * 8]) = v;
      }
  }
  __syncthreads();

  const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  if constexpr (B == 1) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      const int ii = i < nq ? i : 0;
      const u4v* xv = reinterpret_cast<const u4v*>(xs + (q0 + ii) * 64 + g * 16);
      const u4v x0 = xv[0], x1 = xv[1];
      const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const uint32_t cw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      float bs = 0.f;
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const h2_t lo = q8_pair(cw[w], 0x04010400u) - bias;
        const h2_t hi = q8_pair(cw[w], 0x04030402u) - bias;
        bs = __builtin_amdgcn_fdot2(lo, as_h2(xw[2 * w]), bs, false);
        bs = __builtin_amdgcn_fdot2(hi, as_h2(xw[2 * w + 1]), bs, false);
      }
      const float d = i < nq ? h2f(sr[i]) : 0.f;
      acc = fmaf(d, bs, acc);
    }
    // the 4 lane groups hold the same 16 rows over different segments
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    if (lane < 16) red[wave * 16 + lane] = acc;
  } else {
    // MFMA block m = lane / 4 holds rows 4m..4m+3 (mod 16) of lane group m / 4
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xl = xs + (lane & 3) * ldxs;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
      const int ii = i < nq ? i : 0;
      const uint16_t* xb = xl + (q0 + ii) * 64 + g * 16;
      const uint32_t cw[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      f4_t cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const h2_t lo = q8_pair(cw[w], 0x04010400u) - bias;
        const h2_t hi = q8_pair(cw[w], 0x04030402u) - bias;
        const h4_t A = {lo.x, lo.y, hi.x, hi.y};
        const u2v xa = *reinterpret_cast<const u2v*>(xb + 4 * w);
        cb = __builtin_amdgcn_mfma_f32_4x4x4f16(A, __builtin_bit_cast(h4_t, xa), cb, 0, 0, 0);
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
      acc[r] += __shfl_xor(acc[r], 16, 64);
      acc[r] += __shfl_xor(acc[r], 32, 64);
    }
    if (lane < 16) {
      const int bb = lane & 3;
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (bb < B) red[(wave * B + bb) * 16 + (lane & ~3) + r] = acc[r];
    }
  }
  __syncthreads();
  // ---- sum the waves in fixed order
  const int t = threadIdx.x;
  if (t < B * 16) {
    const int bb = t >> 4, rr = t & 15;
    const int row = tile * 16 + rr;
    float v = 0.f;
    for (int w = 0; w < a.W; w++) v += red[(w * B + bb) * 16 + rr];
    if (row < a.N && bb < nrow) a.y[(long)bb * a.ldy + row] = v;
  }
}

}  // namespace q4k
