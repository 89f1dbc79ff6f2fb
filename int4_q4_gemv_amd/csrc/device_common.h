// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

#define Q4_DEV __device__ __forceinline__

Q4_DEV float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
Q4_DEV uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }  // RNE
Q4_DEV h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
Q4_DEV uint32_t as_u32(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Sum over the 64 lanes of a wave (every lane gets the result).
Q4_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
Q4_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x == NT (multiple of 64); `red` holds NT/64 floats.
template <int NT>
Q4_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; i++) s += red[i];
  return s;
}

// Release the block's global writes, bump `counter`, and report whether this
// block was the `expected`-th (last) arrival; the last one resets the counter
// to zero and acquires every earlier arrival's writes.  Whole block must call.
Q4_DEV bool last_arrival(unsigned* counter, unsigned expected, int* flag_lds) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    unsigned prev = atomicAdd(counter, 1u);
    int last = (prev == expected - 1);
    if (last) {
      atomicExch(counter, 0u);
      __threadfence();
    }
    *flag_lds = last;
  }
  __syncthreads();
  bool last = *flag_lds != 0;
  if (last) __threadfence();
  return last;
}

// Orderable key of an fp32 value (larger value -> larger key).
Q4_DEV uint32_t f32_order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
