// Device helpers shared by the HIP kernel files of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lane pairs on the vector ALU, with no LDS round trip (a
// __shfl_xor compiles to ds_bpermute, which goes through LDS). Both lanes of
// a pair get op(value of the lower lane, value of the upper lane):
//  - lanes l and l ^ 32: v_permlane32_swap of x with itself leaves the low
//    half's values in both halves of one result and the high half's in both
//    halves of the other;
//  - lanes l and l ^ 16 (16-lane rows 0/1 and 2/3): v_permlane16_swap, alike;
//  - lanes l and l ^ 1, l ^ 2: DPP quad permutations.
// With max and + the results equal those of the shuffles bit for bit (the
// two operands only change places).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// DPP sources (each lane reads the lane named, within its 16-lane row)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]: lane l ^ 1
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]: lane l ^ 2
constexpr int kDppRowRor8 = 0x128;      // row_ror 8: lane l ^ 8
constexpr int kDppRowRor4 = 0x124;      // row_ror 4: lane l ^ 4 once lanes l and l ^ 8 agree
constexpr int kDppRowRor2 = 0x122;      // row_ror 2: lane l ^ 2 once lanes l, l ^ 4, l ^ 8 agree
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane l ^ 4 once quads agree
template <int kCtrl>
__device__ __forceinline__ float dpp_read(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), on
// the vector ALU: DPP row shifts by 1, 2, 4 and 8 sum within each 16-lane row
// (lanes shifted in from outside the row add 0), then row 0's total is
// broadcast into row 1 and row 2's into row 3 (row_bcast 15), and the total
// of rows 0-1 into rows 2 and 3 (row_bcast 31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr 1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr 2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr 4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr 8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast 15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast 31 -> rows 2, 3
  return x;
}

// Order a wave's own LDS writes before its later LDS reads (and reads before
// later writes). LDS requests of one wave are served in order, so only the
// compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace
}  // namespace pkv
