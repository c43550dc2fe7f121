// S0 softmax-gate compressor: the work of one 256-thread work-group, as device functions
// shared by the compressor's own kernels and by the indexer kernels, which can run a
// compressor job in extra work-groups of their launch.
//
// For each group of r raw latents (r = 2 in the compressing layers that collapse two
// positions into one, "DeepSeek-V4.1 Flash" Miles docs, section 1) and each channel c:
//   pi_k = softmax_k(gate[k][c] + bias[k][c]),   out[c] = sum_k pi_k * raw[k][c]
// (latents pooled by a learned softmax gate, vLLM recipe, Overview, two-tier sparse
// attention bullet). Ratio 1 is the identity copy.
//
// bf16 rows: elementwise and HBM-bound; each thread handles 8 channels of one group with
// 16-byte loads and stores; arithmetic in fp32, output rounded to bf16 (nearest even).
//
// Code rows (the FP8 and FP4 caches of "SGLang and Miles Add Day-0 Support for DeepSeek-V4.1",
// Miles Day-0 Support table, Quantization row): one wave per group quantises the fp32 row it
// computed. e4m3: scale s = amax / 448 over the row (1 for an all-zero row), code = nearest
// e4m3 of x / s (ties to the even code). MXFP4: per block of 32 channels, E8M0 exponent
// X = floor(log2 amax) - 2 (-127 for an all-zero block, clamped to [-127, 127]), element =
// nearest E2M1 of x * 2^-X (ties to the even code, saturating at 6). Divisions are IEEE fp32.
#pragma once
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kCThreads = 256;               // threads of every work-group that runs a job
constexpr int kCChunks = kDim / 8;           // 64 chunks of 8 channels per group
constexpr int kCGroupsPerWG = kCThreads / 64;   // code rows: one wave per group

// Work-groups a job wants (grid-stride beyond 64 per CU for bf16 rows).
inline int64_t compress_blocks_wanted(const CompressArgs& a) {
  if (a.kv_mode != 0) return (a.G + kCGroupsPerWG - 1) / kCGroupsPerWG;
  const int64_t b = (a.G * kCChunks + kCThreads - 1) / kCThreads;
  return b < 1 ? 1 : (b > 256 * 64 ? 256 * 64 : b);
}

namespace cdetail {

// bf16 rows: items (group, chunk of 8 channels) first, first + stride, ...
template <int R>
__device__ __forceinline__ void bf16_items(const CompressArgs& a, int64_t first, int64_t stride) {
  const int64_t total = a.G * kCChunks;
  for (int64_t item = first; item < total; item += stride) {
    const int64_t grp = item / kCChunks;
    const int ch = (int)(item % kCChunks) * 8;
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.raw) + grp * a.raw_stride + ch;
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + grp * a.out_stride + ch;
    if constexpr (R == 1) {
      *reinterpret_cast<u32x4*>(o) = *reinterpret_cast<const u32x4*>(x);
    } else {
      const uint16_t* z = reinterpret_cast<const uint16_t*>(a.gate) + grp * a.gate_stride + ch;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(x);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(x + kDim);
      const u32x4 z0 = *reinterpret_cast<const u32x4*>(z);
      const u32x4 z1 = *reinterpret_cast<const u32x4*>(z + kDim);
      const float* b0 = a.bias + ch;
      const float* b1 = a.bias + kDim + ch;
      u32x4 ov;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float r[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int cc = 2 * w + h;
          const float xa = h ? bf16_hi(x0[w]) : bf16_lo(x0[w]);
          const float xb = h ? bf16_hi(x1[w]) : bf16_lo(x1[w]);
          const float a0 = (h ? bf16_hi(z0[w]) : bf16_lo(z0[w])) + b0[cc];
          const float a1 = (h ? bf16_hi(z1[w]) : bf16_lo(z1[w])) + b1[cc];
          // pi_0 = 1 / (1 + exp(a1 - a0)); out = xb + pi_0 * (xa - xb)
          const float e = __builtin_amdgcn_exp2f((a1 - a0) * 1.4426950408889634f);
          const float p0 = 1.0f / (1.0f + e);
          r[h] = fmaf(p0, xa - xb, xb);
        }
        ov[w] = pack_bf16x2(r[0], r[1]);
      }
      *reinterpret_cast<u32x4*>(o) = ov;
    }
  }
}

// Nearest OCP e4m3 code of y (|y| clamped to 448, ties to the even code), y's sign kept.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);   // subnormals: 2^-9 steps
  int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;                   // floor(log2 a)
  float m = __builtin_rintf(__builtin_ldexpf(a, 3 - e));                       // 8 .. 16
  if (m >= 16.0f) {
    m = 8.0f;
    e += 1;
  }
  const uint32_t code = ((uint32_t)(e + 7) << 3) | ((uint32_t)m - 8u);
  return sign | (code < 0x7Eu ? code : 0x7Eu);
}

// Nearest FP4 E2M1 code of y (0, 0.5, 1, 1.5, 2, 3, 4, 6; ties to the even code; saturating).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 0x8u;
  const float a = fabsf(y);
  uint32_t c;
  if (a < 2.0f) c = (uint32_t)__builtin_rintf(2.0f * a);      // steps of 0.5: codes 0..4
  else if (a < 4.0f) c = (uint32_t)__builtin_rintf(a) + 2u;   // steps of 1: codes 4..6
  else if (a < 6.0f) c = a > 5.0f ? 7u : 6u;                  // 4 or 6 (5 ties to 4)
  else c = 7u;
  return sign | c;
}

__device__ __forceinline__ float wave_max(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Code rows: group grp by one wave; lane l computes channels 8l .. 8l+7 (the bf16 path's
// arithmetic, kept in fp32) and quantises them.
template <int KVM, int R>
__device__ __forceinline__ void code_group(const CompressArgs& a, int64_t grp, int lane) {
  const int ch = 8 * lane;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.raw) + grp * a.raw_stride + ch;
  const u32x4 x0 = *reinterpret_cast<const u32x4*>(x);
  float r[8];
  if constexpr (R == 2) {
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(x + kDim);
    const uint16_t* z = reinterpret_cast<const uint16_t*>(a.gate) + grp * a.gate_stride + ch;
    const u32x4 z0 = *reinterpret_cast<const u32x4*>(z);
    const u32x4 z1 = *reinterpret_cast<const u32x4*>(z + kDim);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int w = k >> 1, h = k & 1;
      const float xa = h ? bf16_hi(x0[w]) : bf16_lo(x0[w]);
      const float xb = h ? bf16_hi(x1[w]) : bf16_lo(x1[w]);
      const float a0 = (h ? bf16_hi(z0[w]) : bf16_lo(z0[w])) + a.bias[ch + k];
      const float a1 = (h ? bf16_hi(z1[w]) : bf16_lo(z1[w])) + a.bias[kDim + ch + k];
      const float e = __builtin_amdgcn_exp2f((a1 - a0) * 1.4426950408889634f);
      r[k] = fmaf(1.0f / (1.0f + e), xa - xb, xb);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = (k & 1) ? bf16_hi(x0[k >> 1]) : bf16_lo(x0[k >> 1]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(r[k]));
  uint8_t* out = reinterpret_cast<uint8_t*>(a.out) + grp * a.out_stride;
  uint8_t* sc = reinterpret_cast<uint8_t*>(a.scales) + grp * a.scales_stride;
  if constexpr (KVM == 1) {
    amax = wave_max(amax, 64);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= e4m3_code(r[k] / s) << (8 * k);
      hi |= e4m3_code(r[k + 4] / s) << (8 * k);
    }
    *reinterpret_cast<uint2*>(out + ch) = uint2{lo, hi};
    if (lane == 0) *reinterpret_cast<float*>(sc) = s;
  } else {
    amax = wave_max(amax, 4);   // the block: lanes 4b .. 4b+3
    int X = -127;
    if (amax > 0.0f) {
      int e;
      frexpf(amax, &e);        // amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
      X = min(max(e - 3, -127), 127);
    }
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) packed |= e2m1_code(__builtin_ldexpf(r[k], -X)) << (4 * k);
    *reinterpret_cast<uint32_t*>(out + 4 * lane) = packed;
    if ((lane & 3) == 0) sc[lane >> 2] = (uint8_t)(X + 127);
  }
}

template <int KVM, int R>
__device__ __forceinline__ void code_groups(const CompressArgs& a, int64_t block, int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  for (int64_t grp = block * kCGroupsPerWG + (threadIdx.x >> 6); grp < a.G; grp += nblocks * kCGroupsPerWG)
    code_group<KVM, R>(a, grp, lane);
}

}  // namespace cdetail

// Work-group `block` of `nblocks` (256 threads each) does its share of the job: bf16 items
// block * 256 + thread, strided by nblocks * 256; code rows one group per wave, strided by
// nblocks * 4. Any nblocks >= 1 covers the whole job.
__device__ __forceinline__ void compress_blocks(const CompressArgs& a, int64_t block, int64_t nblocks) {
  if (a.kv_mode == 0) {
    const int64_t first = block * kCThreads + threadIdx.x, stride = nblocks * kCThreads;
    if (a.ratio == 2) cdetail::bf16_items<2>(a, first, stride);
    else cdetail::bf16_items<1>(a, first, stride);
  } else if (a.kv_mode == 1) {
    if (a.ratio == 2) cdetail::code_groups<1, 2>(a, block, nblocks);
    else cdetail::code_groups<1, 1>(a, block, nblocks);
  } else {
    if (a.ratio == 2) cdetail::code_groups<2, 2>(a, block, nblocks);
    else cdetail::code_groups<2, 1>(a, block, nblocks);
  }
}

}  // namespace sa
