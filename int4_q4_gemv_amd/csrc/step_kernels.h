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
  unsigned long long* best; // [4] argmax slots
  const uint16_t* E;        // [vocab][H] fp16
  int H;
  float emb_scale;          // sqrt(H)
  float* h;                 // [4][H]
  double* inv_freq;         // [ns + nf]: RoPE inverse frequencies, sliding then full
  int ns, nf, Ds, Df;
  double theta_s, theta_f;
};

// One workgroup per row: h = fp32(E[token]) * sqrt(H) (reading of the
// embedding scale); workgroup 0 also publishes the step parameters and the
// RoPE inverse frequencies theta^(-2i/D) in fp64 (one table per layer kind).
__global__ void __launch_bounds__(256) k_step_begin(BeginArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b == 0) {
    if (tid == 0) {
      a.sp->pos0 = a.pos0;
      a.sp->n = a.n;
      for (int i = 0; i < 4; i++) a.sp->tokens[i] = a.tokens[i];
    }
    if (tid < 4) a.best[tid] = 0ull;
    for (int i = tid; i < a.ns + a.nf; i += 256)
      a.inv_freq[i] = i < a.ns ? pow(a.theta_s, -2.0 * (double)i / (double)a.Ds)
                               : pow(a.theta_f, -2.0 * (double)(i - a.ns) / (double)a.Df);
  }
  const uint16_t* e = a.E + (long)a.tokens[b] * a.H;
  float* h = a.h + (long)b * a.H;
  for (int i = tid; i < a.H; i += 256) h[i] = h2f(e[i]) * a.emb_scale;
}

}  // namespace q4k
