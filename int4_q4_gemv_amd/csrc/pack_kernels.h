// pack_kernels.h -- q4_0 quantisation into the device layout, and export to
// the canonical block format.
//
// q4_0 grid (gemma4-12b card, intro: per-block-32 absmax symmetric int4;
// gemma-4-E4B-CoreAI card, Provenance: symmetric with clipping, [-8, 7]):
// d = fp16_rne(absmax / 8); q = clamp(round_half_away(w / d), -8, 7), the
// quotient an IEEE fp32 division against the stored fp16 scale.
//
// Device layout (this library's): one wave-wide 16-byte load fetches a
// "quad" = 16 consecutive rows x 4 consecutive q4 blocks, lane l holding row
// (l & 15) and block (l >> 4) of the quad:
//   codes  [T = ceil(N/16)][NQ = ceil(K/128)][64 lanes][16 bytes]
//   scales [T][NQ][64 lanes] fp16, right after the codes.
// Rows past N and blocks past K/32 are padding with zero scale.
// Inside a block's 16 bytes, 32-bit word w holds elements 8w..8w+7 with the
// nibble of element 8w+k at bit (k & 1) * 16 + (k >> 1) * 4, so that
//   (word & 0x000F000F) | 0x64006400  -> fp16 pair (1024 + u0, 1024 + u1)
//   (word & 0x00F000F0) | 0x54005400  -> fp16 pair (  64 + u2,   64 + u3)
// and the same on word >> 8 for elements 4..7 (u = q + 8).
#pragma once
#include "device_common.h"

namespace q4k {

Q4_DEV int nib_shift(int k) { return (k & 1) * 16 + (k >> 1) * 4; }

template <int DT>   // 0: fp32 input, 1: bf16 input
__global__ void __launch_bounds__(256) k_q4_pack(const void* __restrict__ w, int N, int K,
                                                 u4v* __restrict__ codes,
                                                 uint16_t* __restrict__ scales, int T,
                                                 int32_t* nonfinite) {
  const int NB = K >> 5, NQ = (NB + 3) >> 2;
  const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
  const long total = (long)T * NQ * 64;
  if (gid >= total) return;
  const int l = (int)(gid & 63);
  const long tq = gid >> 6;            // t * NQ + q
  const int q = (int)(tq % NQ);
  const int t = (int)(tq / NQ);
  const int n = t * 16 + (l & 15);
  const int b = q * 4 + (l >> 4);
  uint32_t wd[4] = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
  uint16_t d16 = 0;
  if (n < N && b < NB) {
    float v[32];
    if (DT == 0) {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(w) + (long)n * K + b * 32);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + (long)n * K + b * 32);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        uint4 u = src[i];
        uint32_t a[4] = {u.x, u.y, u.z, u.w};
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
    d16 = f2h(amax / 8.0f);
    const float d = h2f(d16);
    if (bad || !__builtin_isfinite(d)) {
      d16 = 0;
      if (nonfinite) atomicAdd(nonfinite, 1);
    } else if (d != 0.f) {
      uint32_t acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 32; i++) {
        float rr = roundf(v[i] / d);          // correctly rounded fp32 division
        rr = fminf(fmaxf(rr, -8.f), 7.f);
        uint32_t u = (uint32_t)((int)rr + 8);
        acc[i >> 3] |= u << nib_shift(i & 7);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) wd[i] = acc[i];
    }
  }
  codes[tq * 64 + l] = (u4v){wd[0], wd[1], wd[2], wd[3]};
  scales[tq * 64 + l] = d16;
}

// One thread per (row, block): device layout -> canonical 18-byte block.
__global__ void __launch_bounds__(256) k_q4_unpack(const u4v* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int N,
                                                   int K, uint8_t* __restrict__ blocks) {
  const int NB = K >> 5, NQ = (NB + 3) >> 2;
  const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (gid >= (long)N * NB) return;
  const int n = (int)(gid / NB), b = (int)(gid % NB);
  const long src = ((long)(n >> 4) * NQ + (b >> 2)) * 64 + (b & 3) * 16 + (n & 15);
  const u4v c = codes[src];
  const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
  const uint16_t d16 = scales[src];
  uint8_t* o = blocks + gid * 18;
  o[0] = (uint8_t)(d16 & 0xFF);
  o[1] = (uint8_t)(d16 >> 8);
#pragma unroll
  for (int j = 0; j < 16; j++) {
    uint32_t lo = (wd[j >> 3] >> nib_shift(j & 7)) & 15u;
    uint32_t hi = (wd[(j + 16) >> 3] >> nib_shift((j + 16) & 7)) & 15u;
    o[2 + j] = (uint8_t)(lo | (hi << 4));
  }
}

}  // namespace q4k
