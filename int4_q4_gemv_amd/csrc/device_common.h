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

// Reductions over the 64 lanes of a wave (every lane gets the result).  Each
// 16-lane row folds its lanes with four DPP shifts on the VALU (row_shr 1,
// 2, 4, 8: the row's total lands in its last lane; a lane whose source lies
// outside the row takes the identity), then the four row results are read
// as scalars and combined in order.  Butterfly shuffles through
// ds_bpermute cost an LDS round trip per step.  The wave must be fully
// active: every caller runs in wave-uniform control flow.
template <int CTRL>
Q4_DEV float dpp_row_shr(float v, float identity) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                               __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
Q4_DEV float lane_f(float v, int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); }
Q4_DEV float wave_sum(float v) {
  v += dpp_row_shr<0x111>(v, 0.f);
  v += dpp_row_shr<0x112>(v, 0.f);
  v += dpp_row_shr<0x114>(v, 0.f);
  v += dpp_row_shr<0x118>(v, 0.f);
  return ((lane_f(v, 15) + lane_f(v, 31)) + lane_f(v, 47)) + lane_f(v, 63);
}
// Sum / maximum over the four 16-lane rows of a wave, per column (lane mod
// 16), returned in every lane: v_permlane16_swap with both operands v gives
// rows (0, 0, 2, 2) and (1, 1, 3, 3), so their sum is each row pair's sum in
// both rows; v_permlane32_swap then does the same for the two halves.  The
// same values a butterfly over lanes l ^ 16 and l ^ 32 gives, on the VALU
// instead of through LDS.  The wave must be fully active.  The two results
// are copied out as unsigned before the bit cast: a bit cast straight from
// the returned vector's second element compiled to a second read of the
// first (a wrong sum, caught by the parity tests).
template <bool MAX>
Q4_DEV float rows_fold(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned p0 = p[0], p1 = p[1];
  const float a = __builtin_bit_cast(float, p0), b = __builtin_bit_cast(float, p1);
  v = MAX ? fmaxf(a, b) : a + b;
  const unsigned w = __builtin_bit_cast(unsigned, v);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const unsigned q0 = q[0], q1 = q[1];
  const float c = __builtin_bit_cast(float, q0), d = __builtin_bit_cast(float, q1);
  return MAX ? fmaxf(c, d) : c + d;
}
Q4_DEV float rows_sum(float v) { return rows_fold<false>(v); }
Q4_DEV float rows_max(float v) { return rows_fold<true>(v); }
Q4_DEV float wave_max(float v) {
  v = fmaxf(v, dpp_row_shr<0x111>(v, -INFINITY));
  v = fmaxf(v, dpp_row_shr<0x112>(v, -INFINITY));
  v = fmaxf(v, dpp_row_shr<0x114>(v, -INFINITY));
  v = fmaxf(v, dpp_row_shr<0x118>(v, -INFINITY));
  return fmaxf(fmaxf(lane_f(v, 15), lane_f(v, 31)), fmaxf(lane_f(v, 47), lane_f(v, 63)));
}

// Orderable key of an fp32 value (larger value -> larger key).
Q4_DEV uint32_t f32_order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Fetches the 64-byte lines of the kernel's arguments that hold the fields a
// kernel reads, in one round of scalar loads (one byte offset inside each
// line), waited for inside the same asm block.  Left to itself the compiler
// requests the argument fields in several rounds, each waiting for the one
// before (an early exit test first, or fields far down a large argument
// struct only where they are used), and every round that touches a line not
// yet fetched is a memory round trip of its own, ~0.3 us on the path to the
// kernel's first load.  After this call every argument read is a scalar
// cache hit.  Call it first in the kernel: the scheduling barrier keeps the
// kernel's own argument loads after it.
template <int O0, int O1, int O2>
Q4_DEV void kernarg_fetch() {
  const auto kp = __builtin_amdgcn_kernarg_segment_ptr();
  uint32_t t0, t1, t2;
  asm volatile(
      "s_load_dword %0, %3, %4\n\t"
      "s_load_dword %1, %3, %5\n\t"
      "s_load_dword %2, %3, %6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(t0), "=&s"(t1), "=&s"(t2)
      : "s"(kp), "i"(O0), "i"(O1), "i"(O2));
  __builtin_amdgcn_sched_barrier(0);          // the kernel's own argument loads stay below
}
template <int O0, int O1, int O2, int O3>
Q4_DEV void kernarg_fetch() {
  const auto kp = __builtin_amdgcn_kernarg_segment_ptr();
  uint32_t t0, t1, t2, t3;
  asm volatile(
      "s_load_dword %0, %4, %5\n\t"
      "s_load_dword %1, %4, %6\n\t"
      "s_load_dword %2, %4, %7\n\t"
      "s_load_dword %3, %4, %8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(t0), "=&s"(t1), "=&s"(t2), "=&s"(t3)
      : "s"(kp), "i"(O0), "i"(O1), "i"(O2), "i"(O3));
  __builtin_amdgcn_sched_barrier(0);          // the kernel's own argument loads stay below
}

// A workgroup barrier that orders LDS only: this wave's LDS operations
// have completed (lgkmcnt 0) before it arrives.  __syncthreads' release fence
// would also wait for every global load in flight, the prefetches included.
Q4_DEV void lds_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);         // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}
