// S2 candidate blocks and S3 top-512 on gfx950 (one fused kernel).
//
// Both stages keep the first k elements of a set in the order (value descending, id
// ascending) and emit their ids in ascending order ("deepseek-ai/DeepSeek-V4.1-Flash"
// recipe, Overview, two-tier sparse attention bullet: 2048 candidate blocks of 8, then the
// best 512 positions per query). One work-group handles one query:
//   S2  elements = block maxima of the query's ceil(n/8) blocks, k = 2048;
//   S3  elements = scores of the visible positions inside the kept blocks, k = 512.
// Each thread holds a contiguous run of elements in registers (so id order = thread order),
// as order-preserving u32 keys. The k-th largest key v is found by rounds of LDS
// histograms over linear bins of the remaining key range (each round keeps the bin that
// holds the k-th key and shrinks the range to it), so a skewed score distribution does not
// pile onto a few bins. Then every element with key > v is kept, plus the lowest-id
// elements with key == v until k are taken; two work-group prefix sums place the kept ids
// in ascending order.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesSel = kThreads / 64;
constexpr int kBins = 2048;

constexpr int kMaxSel = 2;      // selections sharing one histogram (candidate and core blocks)
constexpr int kColl = 256;      // most elements of a threshold bin the fast path collects

struct SelShared {
  uint32_t hist[kBins];
  uint32_t wmin[kWavesSel], wmax[kWavesSel];
  int wave_sum[kWavesSel];
  int wave_sum2[kWavesSel];
  int bin;           // selected bin of the current round (refinement path)
  int above;         // elements in higher bins (refinement path)
  // fast path, per selection
  int tb[kMaxSel], tabove[kMaxSel], ncoll[kMaxSel];
  uint32_t vkey[kMaxSel];
  int32_t vid[kMaxSel];
  uint32_t ckey[kMaxSel][kColl];
  int32_t cid[kMaxSel][kColl];
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

// Two inclusive prefix sums over the work-group in one pass (one pair of barriers).
__device__ __forceinline__ void wg_inclusive_scan2(int& a, int& b, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int oa = __shfl_up(a, d, 64), ob = __shfl_up(b, d, 64);
    if (lane >= d) {
      a += oa;
      b += ob;
    }
  }
  if (lane == 63) {
    sh.wave_sum[wave] = a;
    sh.wave_sum2[wave] = b;
  }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < kWavesSel; ++w) {
    ba += (w < wave) ? sh.wave_sum[w] : 0;
    bb += (w < wave) ? sh.wave_sum2[w] : 0;
  }
  __syncthreads();
  a += ba;
  b += bb;
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

// Work-group min and max of one u32 per thread.
__device__ __forceinline__ void wg_minmax(uint32_t lo, uint32_t hi, SelShared& sh, uint32_t& glo,
                                          uint32_t& ghi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, d, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, d, 64));
  }
  if (lane == 0) {
    sh.wmin[wave] = lo;
    sh.wmax[wave] = hi;
  }
  __syncthreads();
  glo = sh.wmin[0];
  ghi = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < kWavesSel; ++w) {
    glo = min(glo, sh.wmin[w]);
    ghi = max(ghi, sh.wmax[w]);
  }
  __syncthreads();
}

// Value of an order-preserving key (inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Monotone map of keys in [lo, hi] onto kBins bins: linear in the score value when the
// value range is finite and not tiny, else linear in the key. Every step is a monotone
// rounding, so a higher bin holds strictly larger keys; lo falls in bin 0 and hi in the
// top bin.
struct Binner {
  bool by_value;
  float lo_f, scale;
  uint32_t lo_k;
  __device__ __forceinline__ Binner(uint32_t lo, uint32_t hi) {
    lo_k = lo;
    lo_f = key_value(lo);
    const float range = key_value(hi) - lo_f;
    // range is finite and large enough that scale stays finite (checked on the bits, as
    // NaN/inf comparisons are not reliable under -fno-honor-nans)
    by_value = ((__float_as_uint(range) >> 23) & 0xFFu) >= 0x10u && ((__float_as_uint(range) >> 23) & 0xFFu) < 0xFFu;
    scale = by_value ? (float)kBins / range : (float)kBins / ((float)(hi - lo) + 1.0f);
  }
  __device__ __forceinline__ uint32_t operator()(uint32_t x) const {
    const float d = by_value ? key_value(x) - lo_f : (float)(x - lo_k);
    const uint32_t b = (uint32_t)(d * scale);
    return b < (uint32_t)(kBins - 1) ? b : (uint32_t)(kBins - 1);
  }
};

// The k-th largest key of the valid elements, and through `take_eq` how many elements
// equal to it are kept. Each round histograms the remaining candidates (keys in [lo, hi])
// over kBins linear bins of that range, keeps the bin that holds the k-th key, and shrinks
// [lo, hi] to the keys in that bin; the range strictly shrinks every round (lo and hi
// always fall in different bins), and spread data needs two or three rounds.
template <int EPT, class Ids>
__device__ uint32_t kth_key(const uint32_t (&key)[EPT], const Ids& I, int k, SelShared& sh,
                            int& take_eq) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (I.ok(e)) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  wg_minmax(lo, hi, sh, lo, hi);
  int kk = k;
  while (lo != hi) {
    const Binner bin(lo, hi);
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
      sh.bin = 0;
      sh.above = 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (I.ok(e) && key[e] >= lo && key[e] <= hi) atomicAdd(&sh.hist[bin(key[e])], 1u);
    __syncthreads();
    // Suffix sums from the top bin: thread i owns bins 2047-2i and 2046-2i.
    const int d_hi = kBins - 1 - 2 * threadIdx.x, d_lo = d_hi - 1;
    const int c_hi = (int)sh.hist[d_hi], c_lo = (int)sh.hist[d_lo];
    int tot;
    const int incl = wg_inclusive_scan(c_hi + c_lo, sh, tot);
    const int above_hi = incl - c_hi - c_lo;   // elements in bins above d_hi
    if (above_hi < kk && kk <= above_hi + c_hi) {
      sh.bin = d_hi;
      sh.above = above_hi;
    } else if (above_hi + c_hi < kk && kk <= above_hi + c_hi + c_lo) {
      sh.bin = d_lo;
      sh.above = above_hi + c_hi;
    }
    __syncthreads();
    const uint32_t tb = (uint32_t)sh.bin;
    kk -= sh.above;
    uint32_t lo2 = 0xFFFFFFFFu, hi2 = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (I.ok(e) && key[e] >= lo && key[e] <= hi && bin(key[e]) == tb) {
        lo2 = min(lo2, key[e]);
        hi2 = max(hi2, key[e]);
      }
    wg_minmax(lo2, hi2, sh, lo, hi);   // also orders the reads of sh.bin before the next round
  }
  take_eq = kk;
  return lo;
}

// Keep the first k of the thread-ordered elements by (key desc, id asc) and write their
// ids ascending to out[0..k). Every thread's ids must be ascending and precede the next
// thread's.
template <int EPT, class Ids>
__device__ void select_and_emit(const uint32_t (&key)[EPT], const Ids& I, int k, SelShared& sh,
                                int32_t* out) {
  int take_eq;
  const uint32_t v = kth_key<EPT, Ids>(key, I, k, sh, take_eq);
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

// NS selections of k[s] elements from the same thread-ordered elements, ids written
// ascending to out[s][0..k[s]). Fast path: one histogram over kBins linear bins of the
// key range gives, for every selection, the bin tb holding its k-th key; the few
// elements of that bin are collected in LDS and one wave ranks them by (key desc, id
// asc) to find the k-th element (v, id_v) exactly. An element is then kept iff
// key > v or (key == v and id <= id_v). Selections whose threshold bin holds more than
// kColl elements (long runs of equal or clustered keys) fall back to the refinement
// path above.
template <int EPT, int NS, class Ids>
__device__ void multi_select(const uint32_t (&key)[EPT], const Ids& I, const int (&k)[NS],
                             int32_t* const (&out)[NS], SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (I.ok(e)) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  wg_minmax(lo, hi, sh, lo, hi);
  bool fast = lo != hi;
  const Binner bin(lo, fast ? hi : lo + 1u);
  if (fast) {
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    if (tid < NS) {
      sh.tb[tid] = 0;
      sh.tabove[tid] = 0;
      sh.ncoll[tid] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (I.ok(e)) atomicAdd(&sh.hist[bin(key[e])], 1u);
    __syncthreads();
    const int d_hi = kBins - 1 - 2 * tid, d_lo = d_hi - 1;
    const int c_hi = (int)sh.hist[d_hi], c_lo = (int)sh.hist[d_lo];
    int tot;
    const int above_hi = wg_inclusive_scan(c_hi + c_lo, sh, tot) - c_hi - c_lo;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      if (above_hi < k[q] && k[q] <= above_hi + c_hi) {
        sh.tb[q] = d_hi;
        sh.tabove[q] = above_hi;
      } else if (above_hi + c_hi < k[q] && k[q] <= above_hi + c_hi + c_lo) {
        sh.tb[q] = d_lo;
        sh.tabove[q] = above_hi + c_hi;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NS; ++q) fast = fast && (int)sh.hist[sh.tb[q]] <= kColl;
  }
  if (!fast) {
#pragma unroll
    for (int q = 0; q < NS; ++q) select_and_emit<EPT, Ids>(key, I, k[q], sh, out[q]);
    return;
  }
  // collect the threshold bins' elements
  int tbq[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) tbq[q] = sh.tb[q];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!I.ok(e)) continue;
    const int b = (int)bin(key[e]);
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (b == tbq[q]) {
        const int slot = atomicAdd(&sh.ncoll[q], 1);
        sh.ckey[q][slot] = key[e];
        sh.cid[q][slot] = I.id(e);
      }
  }
  __syncthreads();
  // wave q ranks selection q's collected elements: the one with rank kk-1 is the k-th
  if (wave < NS) {
    const int q = wave;
    const int kk = k[q] - sh.tabove[q];
    const int mcol = sh.ncoll[q];
    for (int i = lane; i < mcol; i += 64) {
      const uint32_t ki = sh.ckey[q][i];
      const int32_t ii = sh.cid[q][i];
      int rank = 0;
      for (int j = 0; j < mcol; ++j) {
        const uint32_t kj = sh.ckey[q][j];
        rank += (kj > ki || (kj == ki && sh.cid[q][j] < ii)) ? 1 : 0;
      }
      if (rank == kk - 1) {
        sh.vkey[q] = ki;
        sh.vid[q] = ii;
      }
    }
  }
  __syncthreads();
  // emit: one prefix sum per selection (two at a time)
  uint32_t v[NS];
  int32_t vi[NS];
  int cnt[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    v[q] = sh.vkey[q];
    vi[q] = sh.vid[q];
    cnt[q] = 0;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!I.ok(e)) continue;
#pragma unroll
    for (int q = 0; q < NS; ++q) cnt[q] += (key[e] > v[q] || (key[e] == v[q] && I.id(e) <= vi[q])) ? 1 : 0;
  }
  int off[NS];
  if constexpr (NS == 2) {
    int a = cnt[0], b = cnt[1];
    wg_inclusive_scan2(a, b, sh);
    off[0] = a - cnt[0];
    off[1] = b - cnt[1];
  } else {
    int tot;
    off[0] = wg_inclusive_scan(cnt[0], sh, tot) - cnt[0];
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!I.ok(e)) continue;
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if ((key[e] > v[q] || (key[e] == v[q] && I.id(e) <= vi[q])) && off[q] < k[q]) out[q][off[q]++] = I.id(e);
  }
}

// ---------------------------------------------------------------------------------------
// S2 + S3 in one work-group per query.
//   S2: the 2048 candidate blocks (block maxima from block_max, or recomputed from scores).
//   S3: the top-512 positions inside the candidates. By the candidate-stage lemma (a
//       position among the best k of a union of blocks lies in one of the best k blocks,
//       blocks ranked by (block max desc, block id asc)), the top-512 inside the 2048
//       candidates lie inside the best 512 blocks, so S3 only reads those 512 "core"
//       blocks (4096 scores) and returns the same set.
// ---------------------------------------------------------------------------------------
template <int EPT>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ int32_t core[kTopK];
  const int t = blockIdx.x;
  const int64_t n = visible_n(a.m, t);
  const int nb = (int)((n + kBlock - 1) / kBlock);
  int32_t* cand = a.cand + (int64_t)t * kCandBlocks;

  // ---- S2: candidate blocks, and the 512 core blocks ----
  if (nb <= kCandBlocks)
    for (int i = threadIdx.x; i < kCandBlocks; i += kThreads) cand[i] = i < nb ? i : -1;
  if (nb <= kTopK) {
    for (int i = threadIdx.x; i < kTopK; i += kThreads) core[i] = i < nb ? i : -1;
  } else {
    uint32_t key[EPT];
    ContigIds<EPT> I{(int)threadIdx.x * EPT, nb};
    if (a.block_max) {
      // rows are 16-byte aligned (ld_block_max % 4 == 0) and hold at least nb entries
      const float* row = a.block_max + (int64_t)t * a.ld_block_max + I.base;
#pragma unroll
      for (int q = 0; q < EPT / 4; ++q) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (I.base + 4 * q < nb) v = *reinterpret_cast<const f32x4*>(row + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * q + e] = order_key(v[e]);
      }
    } else {
      const float* row = a.scores + (int64_t)t * a.ld_scores;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float m = neg_inf();
        if (I.ok(e)) {
          for (int j = 0; j < kBlock; ++j) {
            const int64_t p = (int64_t)(I.base + e) * kBlock + j;
            if (p < n) m = fmaxf(m, row[p]);
          }
        }
        key[e] = I.ok(e) ? order_key(m) : 0u;
      }
    }
    if (nb > kCandBlocks) {
      const int ks[2] = {kCandBlocks, kTopK};
      int32_t* const outs[2] = {cand, core};
      multi_select<EPT, 2>(key, I, ks, outs, sh);
    } else {
      const int ks[1] = {kTopK};
      int32_t* const outs[1] = {core};
      multi_select<EPT, 1>(key, I, ks, outs, sh);
    }
  }
  __syncthreads();

  // ---- S3: top-512 positions; thread i holds 4 positions of core block i/2 ----
  int32_t* out = a.topk + (int64_t)t * kTopK;
  if (n <= kTopK) {  // every visible position is selected
    for (int i = threadIdx.x; i < kTopK; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  constexpr int E3 = 4;
  const float* row = a.scores + (int64_t)t * a.ld_scores;
  const int cb = core[threadIdx.x >> 1];
  const int half = threadIdx.x & 1;
  uint32_t key[E3];
  ListIds<E3> I;
  // a block's 8 scores are contiguous and 32-byte aligned inside the row
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (cb >= 0) v = *reinterpret_cast<const f32x4*>(row + (int64_t)cb * kBlock + 4 * half);
#pragma unroll
  for (int j = 0; j < E3; ++j) {
    const int64_t p = (int64_t)cb * kBlock + 4 * half + j;
    I.valid[j] = cb >= 0 && p < n;
    I.ids[j] = (int32_t)p;
    key[j] = order_key(v[j]);
  }
  {
    const int ks[1] = {kTopK};
    int32_t* const outs[1] = {out};
    multi_select<E3, 1>(key, I, ks, outs, sh);
  }
  // n > 512 here and the core holds at least 512 visible positions: 512 ids written.
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  const int64_t nbmax = (a.m.max_visible + kBlock - 1) / kBlock;
  const dim3 grid((unsigned)a.m.T);
  if (nbmax <= 8 * kThreads)
    hipLaunchKernelGGL(select_kernel<8>, grid, dim3(kThreads), 0, stream, a);
  else if (nbmax <= 16 * kThreads)
    hipLaunchKernelGGL(select_kernel<16>, grid, dim3(kThreads), 0, stream, a);
  else if (nbmax <= 32 * kThreads)
    hipLaunchKernelGGL(select_kernel<32>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
