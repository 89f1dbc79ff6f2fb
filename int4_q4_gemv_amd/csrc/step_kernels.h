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
  unsigned* cnt;            // counters to clear
  int ncnt;
  unsigned long long* best; // [4] argmax slots
  const uint16_t* E;        // [vocab][H] fp16
  int H;
  float emb_scale;          // sqrt(H)
  float* h;                 // [4][H]
  const float* w_norm;      // first layer's attention-input norm
  float eps;
  uint16_t* x;              // [4][H]
};

// One workgroup per row.  h = fp32(E[token]) * sqrt(H) (reading of the
// embedding scale), x = fp16(RMSNorm(h) * w).
__global__ void __launch_bounds__(256) k_step_begin(BeginArgs a) {
  __shared__ float red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b == 0) {
    if (tid == 0) {
      a.sp->pos0 = a.pos0;
      a.sp->n = a.n;
      for (int i = 0; i < 4; i++) a.sp->tokens[i] = a.tokens[i];
    }
    for (int i = tid; i < a.ncnt; i += 256) a.cnt[i] = 0u;
    if (tid < 4) a.best[tid] = 0ull;
  }
  const int tok = a.tokens[b];
  const uint16_t* e = a.E + (long)tok * a.H;
  float* h = a.h + (long)b * a.H;
  float ss = 0.f;
  for (int i = tid; i < a.H; i += 256) {
    const float v = h2f(e[i]) * a.emb_scale;
    h[i] = v;
    ss += v * v;
  }
  ss = block_sum<256>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)a.H + a.eps);
  for (int i = tid; i < a.H; i += 256) a.x[(long)b * a.H + i] = f2h(h[i] * inv * a.w_norm[i]);
}

}  // namespace q4k
