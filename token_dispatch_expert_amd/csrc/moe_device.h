// Device-side helpers shared by the HIP kernels of the MoE hot path (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  // round to nearest even (gfx950: one v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf2f(p->bits); }
  __device__ static __forceinline__ void store(bf16_t* p, float v) { p->bits = f2bf(v); }
};

__device__ __forceinline__ float sigmoidf_(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Wave-wide (64 lanes) sum.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave-wide inclusive prefix sum; every lane of the wave must be active.
// Data-parallel-primitive moves only (no LDS round trips): shifts by 1, 2, 4
// and 8 inside each row of 16 lanes give the row scans, then the last lane
// of row 0 is added to row 1 and of row 2 to row 3 (row_bcast:15), and the
// last lane of row 1 to rows 2 and 3 (row_bcast:31).  Lanes without a source
// add 0 (the `old` operand).
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Block-wide (256 threads = 4 waves) inclusive scan; *total gets the block
// sum.  `scratch` holds at least 4 ints of LDS.  Contains two barriers.
__device__ __forceinline__ int block256_incl_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = wave_incl_scan(v, lane);
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  int add = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int s = scratch[w];
    if (w < wave) add += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return inc + add;
}

// Number of non-zero bytes in a 32-bit word.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return (int)((w & 0xffu) != 0) + (int)((w & 0xff00u) != 0) + (int)((w & 0xff0000u) != 0) +
         (int)((w & 0xff000000u) != 0);
}

}  // namespace moe
