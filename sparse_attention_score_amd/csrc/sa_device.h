// Device helpers shared by the gfx950 kernels of the sparse-attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_launch.h"

namespace sa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kHeads = 64;
constexpr int kDim = 512;
constexpr int kWindow = 128;
constexpr int kTopK = 512;
constexpr int kIdxHeads = 16;
constexpr int kIdxDim = 128;
constexpr int kBlock = 8;
constexpr int kCandBlocks = 2048;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// bf16 bits <-> fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two fp32 -> two bf16 (nearest, ties to even; lo in the low half) by one v_cvt_pk_bf16_f32.
// The kernels run with fp32 denormals kept and round-to-nearest-even, so the conversion is
// the exact rounding of each value, denormals included. Inputs here are finite.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

// Four OCP e4m3 codes (one dword) -> four bf16 values in two dwords, codes 0-1 in the
// first (code 0 in its low half), 2-3 in the second. Exact: every e4m3 value, subnormals
// included, is a bf16 value, so the hardware's scaled conversion with scale 1 returns it
// unchanged (one instruction per pair of codes).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t codes, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true));
}

// E8M0 code -> fp32 scale 2^(e-127) (e = 0 is the fp32 subnormal 2^-127, 255 is NaN).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : e << 23));
}

// max(x, 0) as one integer max: negative floats (sign bit set) are negative int32s, and
// +0, positive floats and +inf keep their bits. Exact for every non-NaN input.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// The wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Order-preserving map fp32 -> u32 (larger float -> larger key); -0 maps to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] with the gfx950 row-swap instructions (VALU, no
// LDS round trip). Both lanes of a pair add the same two values, so they agree bitwise.
__device__ __forceinline__ float add_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP (VALU, no LDS round trip):
// shifts by 1, 2, 4, 8 inside each row of 16 (lanes shifted in from outside the row add
// 0), then the total of row 0 broadcast into rows 1 and 3 and the total of rows 0-1 into
// rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);    // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);    // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);    // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);    // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Min and max of a u32 over the 64 lanes of a wave, in every lane (DPP inside rows of 16,
// then the row-swap instructions across rows).
__device__ __forceinline__ void wave_minmax_u32(uint32_t& lo, uint32_t& hi) {
#define SA_DPP_MINMAX(ctrl)                                                                     \
  lo = min(lo, (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, ctrl, 0xF, 0xF, false)); \
  hi = max(hi, (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, ctrl, 0xF, 0xF, false));
  SA_DPP_MINMAX(0xB1)    // quad_perm 1,0,3,2
  SA_DPP_MINMAX(0x4E)    // quad_perm 2,3,0,1
  SA_DPP_MINMAX(0x141)   // row_half_mirror
  SA_DPP_MINMAX(0x140)   // row_mirror
#undef SA_DPP_MINMAX
  auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  lo = min(l16[0], l16[1]);
  hi = max(h16[0], h16[1]);
  auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  lo = min(l32[0], l32[1]);
  hi = max(h32[0], h32[1]);
}

// Max over each aligned group of 8 lanes (DPP quad permutes, then the half-row mirror).
__device__ __forceinline__ float max8_lanes(float v) {
  float m = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));
  return m;
}

// Page id of compressed position j of sequence seq in a paged store (clamped into the pool).
__device__ __forceinline__ int64_t page_of(const PageTable& pt, int seq, int j) {
  int64_t pg = pt.table[(int64_t)seq * pt.stride + (j >> pt.log2_page)];
  pg = pg < 0 ? 0 : pg;
  return pg < pt.num_pages ? pg : pt.num_pages - 1;
}
// Pool row of position j given its page id.
__device__ __forceinline__ int64_t pool_row(const PageTable& pt, int64_t page, int j) {
  return (page << pt.log2_page) + (j & ((1 << pt.log2_page) - 1));
}

}  // namespace sa
