// step_kernels.h -- the kernel that opens a decode step: device-side step
// parameters, counter reset, embedding gather and the first RMSNorm.
#pragma once
#include "device_common.h"
#include "gemv_kernels.h"

namespace q4k {

struct BeginArgs {
  StepParams* sp;
  int pos0, n;
  int tokens[4];
  float* logits;            // the step's outputs, published in sp
  int32_t* argmax;
  const uint16_t* E;        // [vocab][H] fp16
  int H;
  float emb_scale;          // sqrt(H)
  float* h;                 // [4][H]
  float2* rope_cs;          // [4][Ds/2 + Df/2]: (cos, sin) per row and pair, sliding then full
  int ns, nf, Ds, Df;
  double theta_s, theta_f;
};

// One workgroup per row: h = fp32(E[token]) * sqrt(H) (reading of the
// embedding scale) and the RoPE rotations of the row's position p: for pair
// i of a layer kind with head size D and base theta, the angle p * theta^(-2i/D)
// is formed in fp64 (power and product), reduced to [-pi, pi] in fp64 by one
// fma with the double nearest 2 pi (k * 2.5e-16 rad of error, under 1e-10 for
// positions below 2^20), and its cos and sin are taken in fp32.  Every
// attention workgroup of the step reads them from this table instead of
// recomputing them.  Workgroup 0 also publishes the step parameters.  The
// embedding row (H <= 4096, H % 32 == 0: at most two 16-byte chunks per
// thread) is loaded first, so its latency overlaps the table's arithmetic.
__global__ void __launch_bounds__(256) k_step_begin(BeginArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const u4v* e8 = reinterpret_cast<const u4v*>(a.E + (long)a.tokens[b] * a.H);
  const int nch = a.H / 8;
  u4v ev[2];
#pragma unroll
  for (int c = 0; c < 2; c++) ev[c] = e8[min(tid + 256 * c, nch - 1)];
  if (b == 0) {
    if (tid == 0) {
      a.sp->pos0 = a.pos0;
      a.sp->n = a.n;
      for (int i = 0; i < 4; i++) a.sp->tokens[i] = a.tokens[i];
      a.sp->logits = a.logits;
      a.sp->argmax = a.argmax;
    }
  }
  // every pair slot of both kinds is written (pairs past rot_pairs, which
  // are not rotated, get (1, 0)), so readers may load whole runs of it
  const int pos = a.pos0 + b;
  const int hs = a.Ds / 2, ld = a.Ds / 2 + a.Df / 2;
  for (int i = tid; i < ld; i += 256) {
    const bool sl = i < hs;
    const int ii = sl ? i : i - hs;
    float2 c = make_float2(1.0f, 0.0f);
    if (ii < (sl ? a.ns : a.nf)) {
      const double fr = sl ? pow(a.theta_s, -2.0 * (double)ii / (double)a.Ds)
                           : pow(a.theta_f, -2.0 * (double)ii / (double)a.Df);
      const double ang = (double)pos * fr;
      const double k = rint(ang * 0.15915494309189535);
      const float r = (float)fma(-k, 6.283185307179586, ang);
      float sn, cn;
      sincosf(r, &sn, &cn);
      c = make_float2(cn, sn);
    }
    a.rope_cs[(long)b * ld + i] = c;
  }
  float4* h4 = reinterpret_cast<float4*>(a.h + (long)b * a.H);
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int k = tid + 256 * c;
    if (k < nch) {
      const uint32_t w[4] = {ev[c].x, ev[c].y, ev[c].z, ev[c].w};
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        f[2 * q] = h2f((uint16_t)(w[q] & 0xFFFF)) * a.emb_scale;
        f[2 * q + 1] = h2f((uint16_t)(w[q] >> 16)) * a.emb_scale;
      }
      h4[2 * k] = make_float4(f[0], f[1], f[2], f[3]);
      h4[2 * k + 1] = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
}

}  // namespace q4k
