// S2 candidate blocks and S3 top-512 on gfx950.
//
// Both stages keep the first k elements of a set in the order (value descending, id
// ascending) and emit their ids in ascending order ("deepseek-ai/DeepSeek-V4.1-Flash"
// recipe, Overview, two-tier sparse attention bullet: 2048 candidate blocks of 8, then the
// best 512 positions per query). One work-group handles one query:
//   S2  elements = block maxima of the query's ceil(n/8) blocks, k = 2048;
//   S3  elements = scores of the visible positions inside the kept blocks, k = 512.
// Each thread holds a contiguous run of elements in registers (so id order = thread order).
// A most-significant-digit radix select over order-preserving u32 keys (11/11/10 bits)
// finds the k-th key v with LDS histograms; then every element with key > v is kept,
// plus the lowest-id elements with key == v until k are taken. Two work-group prefix
// sums place the kept ids in ascending order.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesSel = kThreads / 64;
constexpr int kBins = 2048;

struct SelShared {
  uint32_t hist[kBins];
  int wave_sum[kWavesSel];
  int bin;           // selected digit of the current pass
  int above;         // elements with a larger digit in the current pass
};

__device__ __forceinline__ int64_t visible_n(const QueryMeta& m, int t) {
  int seq = m.seq_id[t], pos = m.pos[t];
  if (seq < 0 || seq >= m.num_seqs || pos < 0) return 0;
  int64_t n = ((int64_t)pos + 1) / m.ratio;
  n = n < m.max_visible ? n : m.max_visible;
  return n < m.compressed_cap ? n : m.compressed_cap;
}

// Inclusive prefix sum over the work-group; `total` receives the sum over all threads.
__device__ __forceinline__ int wg_inclusive_scan(int v, SelShared& sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) sh.wave_sum[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWavesSel; ++w) {
    int s = sh.wave_sum[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

// The elements of one thread: keys in registers plus either a contiguous id run
// (id = base + e, valid while id < limit) or explicit ids with validity flags.
template <int EPT>
struct ContigIds {
  int base, limit;
  __device__ __forceinline__ bool ok(int e) const { return base + e < limit; }
  __device__ __forceinline__ int32_t id(int e) const { return base + e; }
};
template <int EPT>
struct ListIds {
  int32_t ids[EPT];
  bool valid[EPT];
  __device__ __forceinline__ bool ok(int e) const { return valid[e]; }
  __device__ __forceinline__ int32_t id(int e) const { return ids[e]; }
};

// Radix select over the EPT keys of each thread. Returns the k-th largest key v and,
// through `take_eq`, how many elements equal to v are to be kept.
template <int EPT, class Ids>
__device__ uint32_t radix_kth(const uint32_t (&key)[EPT], const Ids& I, int k,
                              SelShared& sh, int& take_eq) {
  uint32_t prefix = 0, mask = 0;
  int kk = k;
  const int shifts[3] = {21, 10, 0};
  const uint32_t dmask[3] = {0x7FFu, 0x7FFu, 0x3FFu};
#pragma unroll
  for (int ps = 0; ps < 3; ++ps) {
    const int sh_ = shifts[ps];
    const uint32_t dm = dmask[ps];
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
      sh.bin = 0;
      sh.above = 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (I.ok(e) && (key[e] & mask) == prefix) atomicAdd(&sh.hist[(key[e] >> sh_) & dm], 1u);
    __syncthreads();
    // Suffix sums from the top digit: thread i owns digits 2047-2i and 2046-2i.
    const int d_hi = kBins - 1 - 2 * threadIdx.x, d_lo = d_hi - 1;
    int c_hi = (int)sh.hist[d_hi], c_lo = (int)sh.hist[d_lo];
    int tot;
    int incl = wg_inclusive_scan(c_hi + c_lo, sh, tot);
    int above_hi = incl - c_hi - c_lo;   // elements with digit > d_hi
    if (above_hi < kk && kk <= above_hi + c_hi) {
      sh.bin = d_hi;
      sh.above = above_hi;
    } else if (above_hi + c_hi < kk && kk <= above_hi + c_hi + c_lo) {
      sh.bin = d_lo;
      sh.above = above_hi + c_hi;
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sh.bin;
    kk -= sh.above;
    prefix |= d << sh_;
    mask |= dm << sh_;
    __syncthreads();
  }
  take_eq = kk;
  return prefix;
}

// Keep the first k of the thread-ordered elements by (key desc, id asc) and write their
// ids ascending to out[0..k). Every thread's ids must be ascending and precede the next
// thread's.
template <int EPT, class Ids>
__device__ void select_and_emit(const uint32_t (&key)[EPT], const Ids& I, int k, SelShared& sh,
                                int32_t* out) {
  int take_eq;
  const uint32_t v = radix_kth<EPT, Ids>(key, I, k, sh, take_eq);
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gt += (I.ok(e) && key[e] > v) ? 1 : 0;
    eq += (I.ok(e) && key[e] == v) ? 1 : 0;
  }
  int tot;
  int eq_before = wg_inclusive_scan(eq, sh, tot) - eq;
  int my_eq = take_eq - eq_before;
  my_eq = my_eq < 0 ? 0 : (my_eq > eq ? eq : my_eq);
  int cnt = gt + my_eq;
  int off = wg_inclusive_scan(cnt, sh, tot) - cnt;
  int seen_eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!I.ok(e)) continue;
    bool keep = key[e] > v;
    if (key[e] == v) {
      keep = seen_eq < my_eq;
      ++seen_eq;
    }
    if (keep && off < k) out[off++] = I.id(e);
  }
}

// ---------------------------------------------------------------------------------------
// S2: one work-group per query. Block maxima come from block_max, or from scores.
// ---------------------------------------------------------------------------------------
template <int EPT>
__global__ __launch_bounds__(kThreads) void select_blocks_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const int64_t n = visible_n(a.m, t);
  const int nb = (int)((n + kBlock - 1) / kBlock);
  int32_t* cand = a.cand + (int64_t)t * kCandBlocks;

  if (nb <= kCandBlocks) {  // every block is a candidate
    for (int i = threadIdx.x; i < kCandBlocks; i += kThreads) cand[i] = i < nb ? i : -1;
    return;
  }
  uint32_t key[EPT];
  ContigIds<EPT> I{(int)threadIdx.x * EPT, nb};
  if (a.block_max) {
    const float* row = a.block_max + (int64_t)t * a.ld_block_max;
#pragma unroll
    for (int e = 0; e < EPT; ++e) key[e] = I.ok(e) ? order_key(row[I.base + e]) : 0u;
  } else {
    const float* row = a.scores + (int64_t)t * a.ld_scores;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      float m = neg_inf();
      if (I.ok(e)) {
        for (int j = 0; j < kBlock; ++j) {
          int64_t p = (int64_t)(I.base + e) * kBlock + j;
          if (p < n) m = fmaxf(m, row[p]);
        }
      }
      key[e] = I.ok(e) ? order_key(m) : 0u;
    }
  }
  select_and_emit<EPT>(key, I, kCandBlocks, sh, cand);
}

// ---------------------------------------------------------------------------------------
// S3: one work-group per query; thread i holds the 16 positions of candidates 2i, 2i+1.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void select_topk_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const int64_t n = visible_n(a.m, t);
  int32_t* out = a.topk + (int64_t)t * kTopK;

  if (n <= kTopK) {  // every visible position is selected
    for (int i = threadIdx.x; i < kTopK; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  constexpr int EPT = 16;
  const int32_t* cand = a.cand + (int64_t)t * kCandBlocks;
  const float* row = a.scores + (int64_t)t * a.ld_scores;
  uint32_t key[EPT];
  ListIds<EPT> I;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cb = cand[2 * threadIdx.x + h];
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
      const int e = h * kBlock + j;
      const int64_t p = (int64_t)cb * kBlock + j;
      I.valid[e] = cb >= 0 && p < n;
      I.ids[e] = (int32_t)p;
      key[e] = I.valid[e] ? order_key(row[p]) : 0u;
    }
  }
  select_and_emit<EPT>(key, I, kTopK, sh, out);
  // n > 512 here, so exactly 512 ids were written.
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  const int64_t nbmax = (a.m.max_visible + kBlock - 1) / kBlock;
  const dim3 grid((unsigned)a.m.T);
  if (nbmax <= 8 * kThreads)
    hipLaunchKernelGGL(select_blocks_kernel<8>, grid, dim3(kThreads), 0, stream, a);
  else if (nbmax <= 16 * kThreads)
    hipLaunchKernelGGL(select_blocks_kernel<16>, grid, dim3(kThreads), 0, stream, a);
  else if (nbmax <= 32 * kThreads)
    hipLaunchKernelGGL(select_blocks_kernel<32>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(select_blocks_kernel<64>, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_topk_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
