// S0 softmax-gate compressor on gfx950.
//
// For each group of r raw latents (r = 2 in the compressing layers that collapse two
// positions into one, "DeepSeek-V4.1 Flash" Miles docs, section 1) and each channel c:
//   pi_k = softmax_k(gate[k][c] + bias[k][c]),   out[c] = sum_k pi_k * raw[k][c]
// (latents "pooled by a learned softmax gate", vLLM recipe, Overview, two-tier sparse
// attention bullet). Ratio 1 is the identity copy.
//
// Elementwise and HBM-bound: each thread handles 8 channels of one group with 16-byte
// loads and stores; arithmetic in fp32, output rounded to bf16 (nearest even).
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kCThreads = 256;
constexpr int kChunks = kDim / 8;  // 64 chunks of 8 channels per group

__global__ __launch_bounds__(kCThreads) void compress2_kernel(CompressArgs a) {
  const int64_t total = a.G * kChunks;
  for (int64_t item = (int64_t)blockIdx.x * kCThreads + threadIdx.x; item < total;
       item += (int64_t)gridDim.x * kCThreads) {
    const int64_t grp = item / kChunks;
    const int ch = (int)(item % kChunks) * 8;
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.raw) + grp * a.raw_stride + ch;
    const uint16_t* z = reinterpret_cast<const uint16_t*>(a.gate) + grp * a.gate_stride + ch;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(x);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(x + kDim);
    const u32x4 z0 = *reinterpret_cast<const u32x4*>(z);
    const u32x4 z1 = *reinterpret_cast<const u32x4*>(z + kDim);
    const float* b0 = a.bias + ch;
    const float* b1 = a.bias + kDim + ch;
    u32x4 o;
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
      o[w] = pack_bf16x2(r[0], r[1]);
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + grp * a.out_stride + ch) = o;
  }
}

__global__ __launch_bounds__(kCThreads) void copy1_kernel(CompressArgs a) {
  const int64_t total = a.G * kChunks;
  for (int64_t item = (int64_t)blockIdx.x * kCThreads + threadIdx.x; item < total;
       item += (int64_t)gridDim.x * kCThreads) {
    const int64_t grp = item / kChunks;
    const int ch = (int)(item % kChunks) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.raw) +
                                                    grp * a.raw_stride + ch);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + grp * a.out_stride + ch) = v;
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  const int64_t items = a.G * kChunks;
  int64_t blocks = (items + kCThreads - 1) / kCThreads;
  if (blocks > 256 * 64) blocks = 256 * 64;   // grid-stride beyond 64 work-groups per CU
  if (blocks < 1) blocks = 1;
  if (a.ratio == 2)
    hipLaunchKernelGGL(compress2_kernel, dim3((unsigned)blocks), dim3(kCThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(copy1_kernel, dim3((unsigned)blocks), dim3(kCThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
