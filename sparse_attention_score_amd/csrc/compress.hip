// S0 softmax-gate compressor kernels on gfx950: one launch over all groups. The per-group
// arithmetic (and its sources) is in sa_compress.h, which the indexer kernels share when a
// compressor job rides in their launch.
#include "sa_compress.h"

namespace sa {
namespace {

__global__ __launch_bounds__(kCThreads) void compress_kernel(CompressArgs a) {
  compress_blocks(a, blockIdx.x, gridDim.x);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  const int64_t blocks = compress_blocks_wanted(a);
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)blocks), dim3(kCThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
