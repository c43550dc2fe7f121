// S2 candidate blocks and S3 top-512 on gfx950.
//
// Both stages keep the first k elements of a set in the order (value descending, id
// ascending) and emit their ids in ascending order ("deepseek-ai/DeepSeek-V4.1-Flash"
// recipe, Overview, two-tier sparse attention bullet: 2048 candidate blocks of 8, then the
// best 512 positions per query). One work-group (4 waves) handles one query:
//   S2  elements = block maxima of the query's ceil(n/8) blocks, k = 2048;
//   S3  elements = scores of the visible positions inside the kept blocks, k = 512.
// Each thread holds a contiguous run of elements in registers (so id order = thread order),
// as order-preserving u32 keys. The k-th largest key v is found by rounds of LDS
// histograms over linear bins of the remaining key range (each round keeps the bin that
// holds the k-th key and shrinks the range to it), so a skewed score distribution does not
// pile onto a few bins. Then every element with key > v is kept, plus the lowest-id
// elements with key == v until k are taken; work-group prefix sums place the kept ids in
// ascending order.
// Above 8192 blocks S2 runs in two levels: parts of 8192 blocks (16384 for rows past 65536
// blocks, so at most 8 parts up to 1,048,576 positions) each keep their own best 2048 (a
// block among the best 2048 of the union is among the best 2048 of its part, with the same
// order), then one work-group per query selects among the survivors.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

// Work-group sizes: 1024 threads when few queries run (latency of one query matters),
// 512 when many do (more work-groups per CU).
constexpr int kMaxWaves = 16;
constexpr int kBins = 2048;

constexpr int kMaxSel = 2;      // selections sharing one histogram (candidate and core blocks)
constexpr int kColl = 256;      // most elements of a threshold bin the fast path collects
constexpr int kTwoRoleQueries = 256;   // batches up to this size run two work-groups per query

struct SelShared {
  uint32_t hist[kBins];
  uint32_t wmin[kMaxWaves], wmax[kMaxWaves];
  int wave_sum[kMaxWaves];
  int wave_sum2[kMaxWaves];
  int bin;           // selected bin of the current round (refinement path)
  int above;         // elements in higher bins (refinement path)
  // fast path, per selection
  int tb[kMaxSel], tabove[kMaxSel], ncoll[kMaxSel];
  uint32_t vkey[kMaxSel];
  int32_t vid[kMaxSel];
  uint32_t ckey[kMaxSel][kColl];
  int32_t cid[kMaxSel][kColl];
  int32_t stage[kCandBlocks + kTopK] __attribute__((aligned(16)));   // kept ids before they go out
};
static_assert(kBins >= kCandBlocks, "the histogram doubles as key staging once the threshold is known");

__device__ __forceinline__ int64_t visible_n(const QueryMeta& m, int t) {
  int seq = m.seq_id[t], pos = m.pos[t];
  if (seq < 0 || seq >= m.num_seqs || pos < 0) return 0;
  int64_t n = ((int64_t)pos + 1) / m.ratio;
  n = n < m.max_visible ? n : m.max_visible;
  return n < m.compressed_cap ? n : m.compressed_cap;
}

// Inclusive prefix sum over the work-group; `total` receives the sum over all threads.
template <int NT>
__device__ __forceinline__ int wg_inclusive_scan(int v, SelShared& sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) sh.wave_sum[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int s = sh.wave_sum[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

// Two inclusive prefix sums over the work-group in one pass (one pair of barriers).
template <int NT>
__device__ __forceinline__ void wg_inclusive_scan2(int& a, int& b, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_incl_scan(a);
  b = wave_incl_scan(b);
  if (lane == 63) {
    sh.wave_sum[wave] = a;
    sh.wave_sum2[wave] = b;
  }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
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
template <int NT>
__device__ __forceinline__ void wg_minmax(uint32_t lo, uint32_t hi, SelShared& sh, uint32_t& glo,
                                          uint32_t& ghi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_minmax_u32(lo, hi);
  if (lane == 0) {
    sh.wmin[wave] = lo;
    sh.wmax[wave] = hi;
  }
  __syncthreads();
  glo = sh.wmin[0];
  ghi = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
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

// Bins of the histogram in LDS, from the top: thread i owns bins kBins-1-kBPT*i down to
// kBins-kBPT*(i+1). For each selection q, the bin holding its k[q]-th element and the
// number of elements in the bins above it are stored to tb[q] / tabove[q] by the thread
// that owns that bin (a k beyond the total leaves them untouched).
template <int NT, int NS>
__device__ __forceinline__ void find_threshold(const uint32_t* hist, const int (&k)[NS], int* tb,
                                               int* tabove, SelShared& sh) {
  constexpr int kBPT = kBins / NT;   // bins per thread
  const int top = kBins - 1 - kBPT * (int)threadIdx.x;
  int c[kBPT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kBPT; ++j) {
    c[j] = (int)hist[top - j];
    sum += c[j];
  }
  int tot;
  int above = wg_inclusive_scan<NT>(sum, sh, tot) - sum;
#pragma unroll
  for (int j = 0; j < kBPT; ++j) {
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (above < k[q] && k[q] <= above + c[j]) {
        tb[q] = top - j;
        tabove[q] = above;
      }
    above += c[j];
  }
}

// The k-th largest key of the valid elements, and through `take_eq` how many elements
// equal to it are kept. Each round histograms the remaining candidates (keys in [lo, hi])
// over kBins linear bins of that range, keeps the bin that holds the k-th key, and shrinks
// [lo, hi] to the keys in that bin; the range strictly shrinks every round (lo and hi
// always fall in different bins), and spread data needs two or three rounds.
template <int NT, int EPT, class Ids>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&key)[EPT], const Ids& I, int k, SelShared& sh,
                            int& take_eq) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (I.ok(e)) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  wg_minmax<NT>(lo, hi, sh, lo, hi);
  int kk = k;
  while (lo != hi) {
    const Binner bin(lo, hi);
    for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
      sh.bin = 0;
      sh.above = 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (I.ok(e) && key[e] >= lo && key[e] <= hi) atomicAdd(&sh.hist[bin(key[e])], 1u);
    __syncthreads();
    {
      const int kq[1] = {kk};
      find_threshold<NT, 1>(sh.hist, kq, &sh.bin, &sh.above, sh);
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
    wg_minmax<NT>(lo2, hi2, sh, lo, hi);   // also orders the reads of sh.bin before the next round
  }
  take_eq = kk;
  return lo;
}

// Keep the first k of the thread-ordered elements by (key desc, id asc) and write their
// ids ascending to out[0..k). Every thread's ids must be ascending and precede the next
// thread's.
template <int NT, int EPT, class Ids>
__device__ __forceinline__ void select_and_emit(const uint32_t (&key)[EPT], const Ids& I, int k, SelShared& sh,
                                int32_t* out, uint32_t* kout) {
  int take_eq;
  const uint32_t v = kth_key<NT, EPT, Ids>(key, I, k, sh, take_eq);
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gt += (I.ok(e) && key[e] > v) ? 1 : 0;
    eq += (I.ok(e) && key[e] == v) ? 1 : 0;
  }
  int tot;
  int eq_before = wg_inclusive_scan<NT>(eq, sh, tot) - eq;
  int my_eq = take_eq - eq_before;
  my_eq = my_eq < 0 ? 0 : (my_eq > eq ? eq : my_eq);
  int cnt = gt + my_eq;
  int off = wg_inclusive_scan<NT>(cnt, sh, tot) - cnt;
  int seen_eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!I.ok(e)) continue;
    bool keep = key[e] > v;
    if (key[e] == v) {
      keep = seen_eq < my_eq;
      ++seen_eq;
    }
    if (keep && off < k) {
      if (kout) kout[off] = key[e];
      out[off++] = I.id(e);
    }
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
template <int NT, int EPT, int NS, class Ids>
__device__ __forceinline__ void multi_select(const uint32_t (&key)[EPT], const Ids& I, const int (&k)[NS],
                             int32_t* const (&out)[NS], SelShared& sh, uint32_t* kout0 = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (I.ok(e)) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  wg_minmax<NT>(lo, hi, sh, lo, hi);
  bool fast = lo != hi;
  const Binner bin(lo, fast ? hi : lo + 1u);
  if (fast) {
    for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0;
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
    find_threshold<NT, NS>(sh.hist, k, sh.tb, sh.tabove, sh);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NS; ++q) fast = fast && (int)sh.hist[sh.tb[q]] <= kColl;
  }
  if (!fast) {
#pragma unroll
    for (int q = 0; q < NS; ++q) select_and_emit<NT, EPT, Ids>(key, I, k[q], sh, out[q], q == 0 ? kout0 : nullptr);
    return;
  }
  // collect the threshold bins' elements
  int tbq[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) tbq[q] = sh.tb[q];
  // (wave-level compaction: one LDS atomic per wave and element index that has matches)
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int b = I.ok(e) ? (int)bin(key[e]) : -1;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      const bool match = b == tbq[q];
      const uint64_t bal = __ballot(match);
      if (bal != 0) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&sh.ncoll[q], __popcll(bal));
        base = __builtin_amdgcn_readfirstlane(base);
        if (match) {
          const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          sh.ckey[q][slot] = key[e];
          sh.cid[q][slot] = I.id(e);
        }
      }
    }
  }
  __syncthreads();
  // wave q ranks selection q's collected elements: the one with rank kk-1 is the k-th
  if (wave < NS) {
    const int q = wave;
    const int kk = k[q] - sh.tabove[q];
    const int mcol = sh.ncoll[q];
    if (mcol <= 64) {
      // one element per lane; the others arrive by lane reads (no LDS round trips)
      const uint32_t ki = lane < mcol ? sh.ckey[q][lane] : 0u;
      const int32_t ii = lane < mcol ? sh.cid[q][lane] : 0;
      int rank = 0;
#pragma unroll 4
      for (int j = 0; j < mcol; ++j) {
        const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)ki, j);
        const int32_t ij = __builtin_amdgcn_readlane(ii, j);
        rank += (kj > ki || (kj == ki && ij < ii)) ? 1 : 0;
      }
      if (lane < mcol && rank == kk - 1) {
        sh.vkey[q] = ki;
        sh.vid[q] = ii;
      }
    } else {
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
    wg_inclusive_scan2<NT>(a, b, sh);
    off[0] = a - cnt[0];
    off[1] = b - cnt[1];
  } else {
    int tot;
    off[0] = wg_inclusive_scan<NT>(cnt[0], sh, tot) - cnt[0];
  }
  // kept ids go to their offsets in an LDS staging area, then out in 16-byte stores
  int sbase[NS];
  sbase[0] = 0;
  if constexpr (NS == 2) sbase[1] = k[0];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!I.ok(e)) continue;
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if ((key[e] > v[q] || (key[e] == v[q] && I.id(e) <= vi[q])) && off[q] < k[q])
      {
        if (q == 0 && kout0) sh.hist[off[q]] = key[e];   // the histogram is no longer read
        sh.stage[sbase[q] + off[q]++] = I.id(e);
      }
  }
  __syncthreads();
  // exactly k[q] ids were kept (the k-th element exists); k and the outputs are 16-byte aligned
#pragma unroll
  for (int q = 0; q < NS; ++q)
    for (int i = 4 * tid; i < k[q]; i += 4 * NT)
      *reinterpret_cast<int4*>(out[q] + i) = *reinterpret_cast<const int4*>(&sh.stage[sbase[q] + i]);
  if (kout0)
    for (int i = 4 * tid; i < k[0]; i += 4 * NT)
      *reinterpret_cast<uint4*>(kout0 + i) = *reinterpret_cast<const uint4*>(&sh.hist[i]);
}

// ---------------------------------------------------------------------------------------
// S3: the top-512 positions inside the candidates. By the candidate-stage lemma (a
// position among the best k of a union of blocks lies in one of the best k blocks, blocks
// ranked by (block max desc, block id asc)), the top-512 inside the 2048 candidates lie
// inside the best 512 blocks, so S3 only reads those 512 "core" blocks (4096 scores) and
// returns the same set. Each thread holds 8 (or 4) consecutive positions of the core.
// ---------------------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void select_core(const SelectArgs& a, int t, int64_t n, const int32_t* core, SelShared& sh) {
  int32_t* out = a.topk + (int64_t)t * kTopK;
  if (n <= kTopK) {  // every visible position is selected
    for (int i = threadIdx.x; i < kTopK; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  constexpr int E3 = (kTopK * kBlock) / NT;   // positions per thread: 8 (512 threads) or 4
  const float* row = a.scores + (int64_t)t * a.ld_scores;
  uint32_t key[E3];
  ListIds<E3> I;
  // a block's 8 scores are contiguous and 32-byte aligned inside the row
  auto load4 = [&](int cb, int half, int e0) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (cb >= 0) v = *reinterpret_cast<const f32x4*>(row + (int64_t)cb * kBlock + 4 * half);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = (int64_t)cb * kBlock + 4 * half + j;
      I.valid[e0 + j] = cb >= 0 && p < n;
      I.ids[e0 + j] = (int32_t)p;
      key[e0 + j] = order_key(v[j]);
    }
  };
  if constexpr (E3 >= kBlock) {   // whole core blocks E3/8 * tid ..
#pragma unroll
    for (int u = 0; u < E3 / kBlock; ++u) {
      const int cb = core[(E3 / kBlock) * threadIdx.x + u];
      load4(cb, 0, 8 * u);
      load4(cb, 1, 8 * u + 4);
    }
  } else {                        // half of core block tid/2
    load4(core[threadIdx.x >> 1], threadIdx.x & 1, 0);
  }
  const int ks[1] = {kTopK};
  int32_t* const outs[1] = {out};
  multi_select<NT, E3, 1>(key, I, ks, outs, sh);
  // n > 512 here and the core holds at least 512 visible positions: 512 ids written.
}

// Block max of block b of query t (from block_max, or recomputed from the scores).
__device__ __forceinline__ float block_value(const SelectArgs& a, int t, int64_t n, int b) {
  if (a.block_max) return a.block_max[(int64_t)t * a.ld_block_max + b];
  const float* row = a.scores + (int64_t)t * a.ld_scores + (int64_t)b * kBlock;
  float m = neg_inf();
  for (int j = 0; j < kBlock; ++j)
    if ((int64_t)b * kBlock + j < n) m = fmaxf(m, row[j]);
  return m;
}

// Keys of the contiguous blocks I.base .. I.base+EPT-1 (invalid ones 0).
template <int EPT>
__device__ __forceinline__ void load_block_keys(const SelectArgs& a, int t, int64_t n, const ContigIds<EPT>& I,
                                                uint32_t (&key)[EPT]) {
  static_assert(EPT % 4 == 0, "runs of whole 16-byte loads");
  if (a.block_max) {
    // rows are 16-byte aligned (ld_block_max % 4 == 0), runs start at multiples of 4
    const float* row = a.block_max + (int64_t)t * a.ld_block_max + I.base;
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (I.base + 4 * q < I.limit) v = *reinterpret_cast<const f32x4*>(row + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * q + e] = I.ok(4 * q + e) ? order_key(v[e]) : 0u;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) key[e] = I.ok(e) ? order_key(block_value(a, t, n, I.base + e)) : 0u;
  }
}

// S2 + S3 for at most NT * EPT blocks per query. ROLES = 1: one work-group of NT threads
// per query selects the candidate and core blocks together, then the top-512 positions.
// ROLES = 2 (batches of few queries, where the latency of one query is the kernel time):
// two work-groups per query work independently, role 0 selecting the 2048 candidate
// blocks and role 1 the 512 core blocks and then the top-512 positions.
// 512-thread work-groups (large batches) are held to 80 registers so that three fit a CU
// beside each other (six waves per SIMD instead of four): the phases of one query are short
// and latency-bound, and a third work-group hides more of them (prefill chunk: 183 -> 153
// us, though the 8192-block variant then keeps a few values in scratch).
template <int NT, int EPT, int ROLES>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 512 ? 6 : 1, 8)))
void select_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) int32_t core[kTopK];
  // one work-group doing both stages keeps the candidate list in LDS until the end: a
  // barrier after global stores waits for them to complete (~10 us per query under load)
  __shared__ __attribute__((aligned(16))) int32_t cand_lds[ROLES == 1 ? kCandBlocks : 4];
  const int role = ROLES == 1 ? -1 : (int)blockIdx.x;
  const int t = ROLES == 1 ? blockIdx.x : blockIdx.y;
  const int64_t n = visible_n(a.m, t);
  const int nb = (int)((n + kBlock - 1) / kBlock);
  int32_t* cand = a.cand + (int64_t)t * kCandBlocks;

  if (role != 1 && nb <= kCandBlocks)
    for (int i = threadIdx.x; i < kCandBlocks; i += NT) cand[i] = i < nb ? i : -1;
  if (role == 0 && nb <= kCandBlocks) return;
  if (role != 0 && nb <= kTopK) {
    for (int i = threadIdx.x; i < kTopK; i += NT) core[i] = i < nb ? i : -1;
  } else {
    uint32_t key[EPT];
    const ContigIds<EPT> I{(int)threadIdx.x * EPT, nb};
    load_block_keys<EPT>(a, t, n, I, key);
    if (role == -1 && nb > kCandBlocks) {
      const int ks[2] = {kCandBlocks, kTopK};
      int32_t* const outs[2] = {cand_lds, core};
      multi_select<NT, EPT, 2>(key, I, ks, outs, sh);
    } else {
      const int ks[1] = {role == 0 ? kCandBlocks : kTopK};
      int32_t* const outs[1] = {role == 0 ? cand : core};
      multi_select<NT, EPT, 1>(key, I, ks, outs, sh);
      if (role == 0) return;
    }
  }
  __syncthreads();
  select_core<NT>(a, t, n, core, sh);
  if (ROLES == 1 && nb > kCandBlocks)
    for (int i = 4 * threadIdx.x; i < kCandBlocks; i += 4 * NT)
      *reinterpret_cast<int4*>(cand + i) = *reinterpret_cast<const int4*>(&cand_lds[i]);
}

// Two-level S2, first level: work-group (t, p) keeps the best 2048 of blocks
// [p * size, (p + 1) * size) and writes their ids ascending to its part list (-1 after the
// last), with each block's key (its order-preserving block max) beside it, so the second
// level reads its elements contiguously instead of gathering block maxima.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) void select_part_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  static_assert(NT * EPT == kPartBlocks || NT * EPT == 2 * kPartBlocks, "one part per work-group");
  const int t = blockIdx.y, p = blockIdx.x;
  const int64_t n = visible_n(a.m, t);
  const int nb = (int)((n + kBlock - 1) / kBlock);
  const int b0 = p * (NT * EPT);
  const int b1 = min(nb, b0 + NT * EPT);
  const int64_t li = ((int64_t)t * a.parts + p) * kCandBlocks;
  int32_t* out = a.part_ids + li;
  uint32_t* kout = a.part_keys + li;
  if (b1 - b0 <= kCandBlocks) {
    for (int i = threadIdx.x; i < kCandBlocks; i += NT) {
      const bool v = b0 + i < b1;
      out[i] = v ? b0 + i : -1;
      kout[i] = v ? order_key(block_value(a, t, n, b0 + i)) : 0u;
    }
    return;
  }
  uint32_t key[EPT];
  const ContigIds<EPT> I{b0 + (int)threadIdx.x * EPT, b1};
  load_block_keys<EPT>(a, t, n, I, key);
  const int ks[1] = {kCandBlocks};
  int32_t* const outs[1] = {out};
  multi_select<NT, EPT, 1>(key, I, ks, outs, sh, kout);
}

// Two-level S2, second level, in two work-groups per query: the union of the query's part
// lists (ids ascending part after part, keys beside them) holds its best 2048 blocks.
// Role 0 selects them into cand; role 1 selects the best 512 (the core blocks) and then
// the top-512 positions inside them (S3), independently of role 0.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) void select_merge_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) int32_t core[kTopK];
  const int role = blockIdx.x, t = blockIdx.y;
  const int64_t n = visible_n(a.m, t);
  const int nb = (int)((n + kBlock - 1) / kBlock);
  int32_t* cand = a.cand + (int64_t)t * kCandBlocks;
  if (nb <= kCandBlocks) {
    if (role == 0) {
      for (int i = threadIdx.x; i < kCandBlocks; i += NT) cand[i] = i < nb ? i : -1;
      return;
    }
    if (nb <= kTopK) {
      for (int i = threadIdx.x; i < kTopK; i += NT) core[i] = i < nb ? i : -1;
    } else {
      // nb in (512, 2048]: all blocks are candidates, the best 512 are the core
      constexpr int E = kCandBlocks / NT < 4 ? 4 : kCandBlocks / NT;
      uint32_t key[E];
      const ContigIds<E> I{(int)threadIdx.x * E, nb};
      load_block_keys<E>(a, t, n, I, key);
      const int ks[1] = {kTopK};
      int32_t* const outs[1] = {core};
      multi_select<NT, E, 1>(key, I, ks, outs, sh);
    }
  } else {
    const int64_t l0 = (int64_t)t * a.parts * kCandBlocks;
    const int32_t* lists = a.part_ids + l0;
    const uint32_t* lkeys = a.part_keys + l0;
    const int total = a.parts * kCandBlocks;
    uint32_t key[EPT];
    ListIds<EPT> I;
    // a thread's EPT entries are contiguous and 16-byte aligned (total is a multiple of 16)
    static_assert(EPT % 4 == 0, "whole 16-byte loads");
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
      const int i = (int)threadIdx.x * EPT + 4 * q;
      const bool in = i < total;
      const int4 v = in ? *reinterpret_cast<const int4*>(lists + i) : int4{-1, -1, -1, -1};
      const uint4 kv = in ? *reinterpret_cast<const uint4*>(lkeys + i) : uint4{0u, 0u, 0u, 0u};
      I.ids[4 * q] = v.x;
      I.ids[4 * q + 1] = v.y;
      I.ids[4 * q + 2] = v.z;
      I.ids[4 * q + 3] = v.w;
      key[4 * q] = kv.x;
      key[4 * q + 1] = kv.y;
      key[4 * q + 2] = kv.z;
      key[4 * q + 3] = kv.w;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      I.valid[e] = I.ids[e] >= 0;
      key[e] = I.valid[e] ? key[e] : 0u;
    }
    const int ks[1] = {role == 0 ? kCandBlocks : kTopK};
    int32_t* const outs[1] = {role == 0 ? cand : core};
    multi_select<NT, EPT, 1>(key, I, ks, outs, sh);
    if (role == 0) return;
  }
  __syncthreads();
  select_core<NT>(a, t, n, core, sh);
}

// Candidate mode: the top-512 positions inside a query's carried candidate blocks. Slot i
// is block cand[i] (ascending, -1 padded); the re-scored entries are in slot order (entry
// 8i + r is position 8 cand[i] + r) with slot maxima in block_max. The 512 best slots by
// (slot max desc, block id asc) hold the 512 best positions (the candidate-stage lemma),
// so, as in select_kernel, the final selection reads only those slots. Slot ids ascend
// with block ids and positions, so ties between slots and between positions resolve as
// in the two-stage path; the ids passed to the selection are the positions themselves.
template <int NT>
__global__ __launch_bounds__(NT) void select_cand_kernel(SelectArgs a) {
  static_assert(NT == 512, "4 slots and one core slot per thread");
  constexpr int ES = kCandBlocks / NT;   // slots per thread
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) int32_t core[kTopK];
  __shared__ int32_t cids[kCandBlocks];  // block id of every valid slot, else -1
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t n = visible_n(a.m, t);
  const int32_t* crow = a.cand + (int64_t)t * kCandBlocks;
  int32_t* out = a.topk + (int64_t)t * kTopK;
  const float* row = a.scores + (int64_t)t * a.ld_scores;
  const float* bm = a.block_max + (int64_t)t * a.ld_block_max;

  // slots tid*ES .. +ES-1; a slot is valid when its block holds a visible position
  uint32_t key[ES];
  ListIds<ES> I;
  int nv_mine = 0;
  {
    const int4 b4 = *reinterpret_cast<const int4*>(crow + tid * ES);
    const f32x4 m4 = *reinterpret_cast<const f32x4*>(bm + tid * ES);
    const int b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int e = 0; e < ES; ++e) {
      const bool v = b[e] >= 0 && (int64_t)b[e] * kBlock < n;
      cids[tid * ES + e] = v ? b[e] : -1;
      I.valid[e] = v;
      I.ids[e] = tid * ES + e;
      key[e] = v ? order_key(m4[e]) : 0u;
      nv_mine += v ? 1 : 0;
    }
  }
  int nvs;
  const int vbefore = wg_inclusive_scan<NT>(nv_mine, sh, nvs) - nv_mine;
  if (nvs <= kTopK) {   // every valid slot, in slot order
    int o = vbefore;
#pragma unroll
    for (int e = 0; e < ES; ++e)
      if (I.valid[e]) core[o++] = I.ids[e];
    for (int i = nvs + tid; i < kTopK; i += NT) core[i] = -1;
  } else {
    const int ks[1] = {kTopK};
    int32_t* const outs[1] = {core};
    multi_select<NT, ES, 1>(key, I, ks, outs, sh);
  }
  __syncthreads();

  // positions of core slot `tid`: 8 entries, ids = positions
  uint32_t pkey[kBlock];
  ListIds<kBlock> P;
  int np_mine = 0;
  {
    const int cs = core[tid];
    const int b = cs >= 0 ? cids[cs] : -1;
    f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
    if (b >= 0) {
      v0 = *reinterpret_cast<const f32x4*>(row + (int64_t)cs * kBlock);
      v1 = *reinterpret_cast<const f32x4*>(row + (int64_t)cs * kBlock + 4);
    }
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
      const int64_t p = (int64_t)b * kBlock + r;
      P.valid[r] = b >= 0 && p < n;
      P.ids[r] = (int32_t)p;
      pkey[r] = order_key(r < 4 ? v0[r] : v1[r - 4]);
      np_mine += P.valid[r] ? 1 : 0;
    }
  }
  int np;
  const int before = wg_inclusive_scan<NT>(np_mine, sh, np) - np_mine;
  if (np <= kTopK) {   // every candidate position is selected, in slot (= position) order
    int o = before;
#pragma unroll
    for (int r = 0; r < kBlock; ++r)
      if (P.valid[r]) out[o++] = P.ids[r];
    for (int i = np + tid; i < kTopK; i += NT) out[i] = -1;
    return;
  }
  const int ks[1] = {kTopK};
  int32_t* const outs[1] = {out};
  multi_select<NT, kBlock, 1>(pkey, P, ks, outs, sh);
}

template <int NT>
hipError_t launch_select_nt(const SelectArgs& a, hipStream_t stream) {
  const int64_t nbmax = (a.m.max_visible + kBlock - 1) / kBlock;
  const dim3 grid((unsigned)a.m.T);
  // blocks per thread: a multiple of 4 (16-byte loads), at least 4
  constexpr int E1 = 2048 / NT < 4 ? 4 : 2048 / NT, E2 = 4096 / NT < 4 ? 4 : 4096 / NT;
  if (a.parts <= 1) {
    if (a.m.T <= kTwoRoleQueries) {   // two work-groups per query
      const dim3 g2(2u, (unsigned)a.m.T);
      if (nbmax <= NT * E1)
        hipLaunchKernelGGL((select_kernel<NT, E1, 2>), g2, dim3(NT), 0, stream, a);
      else if (nbmax <= NT * E2)
        hipLaunchKernelGGL((select_kernel<NT, E2, 2>), g2, dim3(NT), 0, stream, a);
      else
        hipLaunchKernelGGL((select_kernel<NT, kPartBlocks / NT, 2>), g2, dim3(NT), 0, stream, a);
      return hipGetLastError();
    }
    if (nbmax <= NT * E1)
      hipLaunchKernelGGL((select_kernel<NT, E1, 1>), grid, dim3(NT), 0, stream, a);
    else if (nbmax <= NT * E2)
      hipLaunchKernelGGL((select_kernel<NT, E2, 1>), grid, dim3(NT), 0, stream, a);
    else
      hipLaunchKernelGGL((select_kernel<NT, kPartBlocks / NT, 1>), grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 pgrid((unsigned)a.parts, (unsigned)a.m.T);
  if (a.part_blocks == kPartBlocks)
    hipLaunchKernelGGL((select_part_kernel<NT, kPartBlocks / NT>), pgrid, dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL((select_part_kernel<NT, 2 * kPartBlocks / NT>), pgrid, dim3(NT), 0, stream, a);
  // the merge reads the part lists: enqueue it only if the part launch was accepted
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid(2u, (unsigned)a.m.T);   // role, query
  const int per_thread = a.parts * kCandBlocks / NT;
  if (per_thread <= 16 * 256 / NT)
    hipLaunchKernelGGL((select_merge_kernel<NT, 16 * 256 / NT>), mgrid, dim3(NT), 0, stream, a);
  else if (per_thread <= 32 * 256 / NT)
    hipLaunchKernelGGL((select_merge_kernel<NT, 32 * 256 / NT>), mgrid, dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL((select_merge_kernel<NT, 64 * 256 / NT>), mgrid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

PartSplit select_parts(int64_t max_visible) {
  const int64_t nb = (max_visible + kBlock - 1) / kBlock;
  if (nb <= kPartBlocks) return {1, kPartBlocks};
  const int size = nb <= (int64_t)kMaxParts * kPartBlocks ? kPartBlocks : 2 * kPartBlocks;
  return {(int)((nb + size - 1) / size), size};
}

hipError_t launch_select_cand(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(select_cand_kernel<512>, dim3((unsigned)a.m.T), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  // few queries: one large work-group each (the latency of a query is the kernel time);
  // many queries: 512-thread work-groups, three per CU (measured against 256 and 1024
  // threads on a 4096-query chunk: 193 us against 258 and 292 at two per CU; 768 queries
  // of a multi-token step: 31 us against 50 with 1024 threads)
  return a.m.T < 512 ? launch_select_nt<1024>(a, stream) : launch_select_nt<512>(a, stream);
}

}  // namespace sa
