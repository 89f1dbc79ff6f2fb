// q8_kernels.h -- int8 ("int8lin") weights: quantisation into the device
// layout and export to the canonical block format.
//
// Grid (gemma4-12b card, intro and Throughput: the int8lin ship beside
// int4linsym; its block format is not given, so the int4 rule is taken on the
// int8 grid): per block of 32 weights d = fp16_rne(absmax / 127) and
// q = clamp(round_half_away(w / d), -127, 127), the quotient an IEEE fp32
// division against the stored fp16 scale.
//
// The product runs in k_q4_gemv (gemv_kernels.h) with FMT = 1.
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

}  // namespace q4k
