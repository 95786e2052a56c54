// gfx950 matrix-core helpers shared by the MFMA chunk-prep and state kernels.
//
// v_mfma_f32_16x16x32_{f16,bf16}: D(16x16) += A(16x32) B(32x16), one wavefront.
// Lane l (r = l % 16, g = l / 16) holds
//   A: row r, k = 8g .. 8g+7        B: column r, k = 8g .. 8g+7
//   C/D: rows 4g .. 4g+3 of column r (4 fp32).
// A contraction may use any order of k as long as A and B agree. These kernels
// feed lane group g the k values {4g..4g+3} and {16+4g..16+4g+3} of each 32-wide
// k step ("kperm"), because that is what a lane holds of two vertically stacked
// D tiles: the fp32 results of one product then serve as the B (or A) operand of
// the next product without any data movement across lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
namespace mfma {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma_f16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 16x16x4: lane l holds A[l%16][l/16], B[l/16][l%16]; D as above.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not
// for its outstanding global loads and stores (a plain __syncthreads() also fences
// global memory, which would drain the next chunk's prefetch at every barrier).
// Valid only where no thread reads global memory written by another thread of the
// workgroup.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Position inside a 32-wide k step of element j (0..7) held by lane group g.
__device__ __forceinline__ constexpr int kperm(int g, int j) {
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += ((u >> 16) & 1u) + 0x7FFFu;
  return (uint16_t)(u >> 16);
}

// Two bf16 (bits) -> packed vector pieces.
__device__ __forceinline__ bf16x8 bf16x8_from_u32x4(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ half8 half8_from_u32x4(u32x4 v) { return __builtin_bit_cast(half8, v); }

__device__ __forceinline__ half4 to_half4(f32x4 x) {
  half4 h;
  h[0] = (_Float16)x[0];
  h[1] = (_Float16)x[1];
  h[2] = (_Float16)x[2];
  h[3] = (_Float16)x[3];
  return h;
}

__device__ __forceinline__ half8 cat(half4 a, half4 b) {
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Row fragment in kperm order: row `row`, elements col0 + kperm(g, 0..7).
__device__ __forceinline__ u32x4 row_frag_kperm(const uint16_t* base, int ld, int row, int col0,
                                                int g) {
  const uint16_t* p = base + row * ld + col0 + 4 * g;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
  u32x4 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
  return r;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Column fragment of a row-major LDS tile: column col0 + m, rows 32s + kperm(g, 0..7),
// from two transpose reads. Within a group of 16 lanes, ds_read_b64_tr_b16 hands lane
// 4a + c element c of the 8-byte chunks that lanes a, a + 4, a + 8, a + 12 address, so
// lane (a + 4j) points at row 4g + j (+ 16), columns col0 + 4a .. col0 + 4a + 3.
__device__ __forceinline__ u32x4 col_frag_tr(const uint16_t* base, int ld, int col0, int s, int g,
                                             int m) {
  const int a = m & 3, j = m >> 2;
  const uint16_t* p = base + (32 * s + 4 * g + j) * ld + col0 + 4 * a;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * ld));
  u32x4 r;
  r[0] = (uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  r[1] = (uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  r[2] = (uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  r[3] = (uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return r;
}

}  // namespace mfma
}  // namespace gdn
