// S4 joint-softmax gather attention on gfx950 MFMA.
//
// For query t (sequence b, raw position p) and each of its 64 heads h:
//   X = [latents[b][j] for j in topk[t] (those in [0, n))] ++ [window rows of u = max(0,p-127)..p]
//   s_i = scale * <q_h, X_i>,  o_h = sum_i softmax(s)_i * X_i,  lse_h = log sum_i exp(s_i)
// Every 512-wide latent is both key and value and all 64 heads share it ("DeepSeek-V4.1
// Flash" Miles docs, section 1 Model Introduction; one softmax over both tiers, recipe
// Overview, two-tier sparse attention bullet).
//
// One work-group (8 waves, two per SIMD) per query, so every gathered row is read from
// memory once for all 64 heads. Rows are gathered 32 per step into LDS tiles by direct
// global-to-LDS loads (no registers), kDepth steps ahead of the step being computed.
//   softmax: in the log2 domain against a fixed reference per head, the max of the first
//           step's scores (softmax does not depend on the reference, and P and the fp32 sums
//           have the range of fp32), so the output is never rescaled and waves holding
//           different keys of a head need not exchange maxima. If a later score exceeds the
//           reference by more than kSafe, the query is run again with the true max.
// The waves have two roles; waves w and w+4 share a SIMD, one of each:
//   score waves 0-3: wave (kh, hp) = (w % 2, w / 2) takes keys 16kh..16kh+15 of the step and
//           head groups 2hp, 2hp+1 (16 heads each): S^T with v_mfma_f32_16x16x32_bf16, A =
//           key rows from LDS (read once for both groups), B = the query heads held in
//           registers (16 k-steps over the 512 dims); lane (c, g) ends with keys 4g..4g+3 of
//           head c. Its 4 probabilities, packed, are half of the P^T operand of the head
//           group (the MFMA k order is free as long as A uses the same one); they go to LDS.
//   value waves 4-7: wave 4+v owns output dims 128v..128v+127 of all 64 heads: O^T += V^T
//           P^T with A = V^T built from LDS rows by byte permutes (8 keys x 1 dim per lane),
//           each value element read from LDS once per step, and B = P^T of each head group.
// The values of step s and the scores of step s+1 are independent and run in the same
// loop iteration, with one barrier per step. Each wave requests its rows of step s+3 after
// its MFMAs of the iteration are issued: the operand reads start right at the barrier, and
// the 32 direct loads of a step, which the CU's load path takes one at a time, queue while
// the matrix cores work.
// Small batches spread each query's key list over kMaxSplits work-groups; the last to
// finish combines their partial results. Mid-size batches (33 to 128 queries) split each
// query's 64 heads over two work-groups instead, which need no combining: both gather the
// same rows, and as neighbours in the grid they normally share an XCD, so the second
// read comes from its L2.
#include <atomic>
#include <mutex>

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kAW = 8;              // waves
constexpr int kSW = 4;              // score waves (the other four weigh the values)
constexpr int kVW = kAW - kSW;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, 32-bit data (gfx9 family)
constexpr int kCoherent = 16;            // buffer cache policy sc1: device-scope coherent
constexpr int64_t kAttnPartBytesO = 64 * 512 * 4;   // one partial O
constexpr int kMaxSplits = kMaxAttnSplits;
constexpr int kAThreads = 64 * kAW;
constexpr int kHG = 4;              // head groups of 16
constexpr int kKT = 32;             // keys per step
constexpr int kRowsPerWave = kKT / kAW;
constexpr int kRow = kDim * 2 + 32; // padded LDS row bytes (+32: conflict-free 16-row reads)
constexpr int kMaxKeys = kTopK + kWindow;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSafe = 64.0f;      // largest score above the reference a pass accepts (log2)
constexpr int kDepth = 3;           // steps whose rows are in flight ahead of the current one
constexpr int kBufs = kDepth + 1;   // LDS tiles
// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8;
// expcnt and lgkmcnt left at their maxima = no wait)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLater = waitcnt_vm(kRowsPerWave * (kDepth - 1));   // all but kDepth-1 later steps
constexpr int kWaitNext = waitcnt_vm(kRowsPerWave * (kDepth - 2));    // all but kDepth-2 later steps
constexpr int kWaitAll = waitcnt_vm(0);

struct AttnShared {
  uint8_t tile[kBufs][kKT * kRow];     // 135,168 B
  const uint16_t* rows[kMaxKeys];      // global row of every key slot
  int32_t topk[kTopK];                 // the query's selection, loaded straight into LDS
  u32x4 P[2][kHG][64];                 // P^T operand of each head group per lane, two steps
  float tmax[2][kHeads];               // step-0 maxima per key half / partial normalisers
  float norm[kHeads];                  // final normaliser of each head
  float rscale[kMaxKeys];              // code rows: the fp32 row scale of every key slot
                                       // (1 for MXFP4 rows and slots past the list)
  const float* sptr[kMaxKeys];         // code rows: where each slot's fp32 scale (e4m3) or
                                       // 16 E8M0 block scales (MXFP4) live
  int wave_cnt[kAW];
  int redo[kAW];                       // per wave: a score exceeded its reference by > kSafe
  int last;                            // this work-group combines the query's key splits
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t hi_src, uint32_t lo_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);  // (lo16 of lo_src, lo16 of hi_src)
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t hi_src, uint32_t lo_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);  // (hi16 of lo_src, hi16 of hi_src)
}
__device__ __forceinline__ float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Device-coherent 32-bit store and load (relaxed atomics at device scope): written through
// to, and read from, the level every XCD shares.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes per lane from global memory straight into LDS: lane l's land at LDS byte address
// lds + 16l. The compiler does not see these loads, so completion is tracked by hand with
// s_waitcnt vmcnt (the kernel issues no other vector-memory load before its output).
__device__ __forceinline__ void to_lds16(const void* src, uint32_t lds) {
  // s_nop: an LDS-DMA load must not directly follow the write of M0 (one wait state)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
// Partial O of key splits: per (query, split) unit, [value wave][half][head group][i][lane]
// f32x4, so each buffer instruction of a wave moves 1 KB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const AttnArgs& a, int units) {
  return __builtin_amdgcn_make_buffer_rsrc(a.part_o, (short)0, (int)(units * kAttnPartBytesO), kRsrcWord3);
}
__device__ __forceinline__ uint32_t part_off(int unit, int vw, int hh, int h, int i) {   // lane 0's byte
  return (uint32_t)(((((unit * kVW + vw) * 2 + hh) * kHG + h) * 4 + i) * 64 * 16);
}

// One 1 KB latent row: lane l moves bytes 16l..16l+15.
__device__ __forceinline__ void row_to_lds(const uint16_t* row, uint32_t lds, int lane) {
  to_lds16(row + lane * 8, lds);
}
// 4 bytes per lane to LDS byte lds + 4 * lane (same rules as to_lds16)
__device__ __forceinline__ void to_lds4(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
// an e4m3 row (512 bytes): the first half-wave moves it into the first half of the slot
__device__ __forceinline__ void row8_to_lds(const uint16_t* row, uint32_t lds, int lane) {
  if (lane < 32) to_lds16(reinterpret_cast<const uint8_t*>(row) + 16 * lane, lds);
}
// e4m3 codes 2w, 2w+1 of a dword -> two bf16 (exact), packed (code 2w in the low half)
template <bool W>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, W));
}
// E2M1 elements 2b, 2b+1 of a dword (byte b) times an E8M0 scale -> two bf16 (exact)
template <int B>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t x, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, B));
}
// 8 e4m3 codes (two dwords) -> bf16x8
__device__ __forceinline__ bf16x8 e4m3x8(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(bf16x8, u32x4{e4m3_pair<false>(lo), e4m3_pair<true>(lo), e4m3_pair<false>(hi),
                                          e4m3_pair<true>(hi)});
}
// 8 E2M1 elements (one dword) with their block's scale -> bf16x8
__device__ __forceinline__ bf16x8 fp4x8(uint32_t x, float scale) {
  return __builtin_bit_cast(bf16x8, u32x4{fp4_pair<0>(x, scale), fp4_pair<1>(x, scale), fp4_pair<2>(x, scale),
                                          fp4_pair<3>(x, scale)});
}
// An E8M0 byte -> its fp32 scale 2^(e-127) (e = 0: the fp32 subnormal 2^-127; codes here
// are at most 254, the encoder's range)
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : e << 23);
}

// a 1.0 that the scale slots of MXFP4 rows (their scales are applied while widening) and
// of slots past the key list load
__device__ float g_unit_scale = 1.0f;

// KVM: 0 bf16 rows. 1: the latents and the window are e4m3 rows with one fp32 scale each
// (X_j = s_j code_j). 2: MXFP4 latents (256 bytes of E2M1 plus 16 E8M0 block scales per
// row) and an e4m3 window. Code rows travel and stay in LDS as they are stored (half or a
// quarter of a bf16 row's bytes) and are widened exactly to bf16 in registers as the MFMA
// operands are read (MXFP4 elements with their block scales); the raw score of key j is
// multiplied by its row scale s_j (1 for MXFP4), and so is P_j before the values (the
// normaliser sums the unscaled P). Score waves of code rows take dims 128g + 8s .. +7 of
// their key in k-step s (the query operands in the same order), so a lane's four k-steps
// 4t .. 4t+3 read 32 consecutive dims: one MXFP4 block, one scale.
template <int HS, int KVM>
__global__ __launch_bounds__(kAThreads, 1) void attn_kernel(AttnArgs a) {
  constexpr bool KV8 = KVM != 0, FP4L = KVM == 2;
  // HS = 2: the query's heads are split over two work-groups (32 each) that gather the same
  // rows (normally on one XCD, so the second reads them from L2); with key splits as well,
  // each (query, split) unit is two such work-groups, each owning its half of the heads
  static_assert(HS == 1 || HS == 2, "one or two head sets");
  constexpr int NJ = 2 / HS;          // head groups per score wave
  constexpr int NV = kHG / HS;        // head groups per value wave
  constexpr int kQPW = kHeads / HS / kAW;   // query heads each wave loads
  __shared__ __attribute__((aligned(16))) AttnShared sh;
  // work-group -> query: ids are dealt round-robin over the 8 XCDs, so XCD x gets the
  // contiguous query range x*Q8 .. x*Q8+Q8-1 (neighbouring queries share window rows).
  // With key splits the unit is (query, split), split fastest (after the head set), so the
  // work-groups of a query normally share an XCD.
  const int T = (int)a.m.T, S = a.splits, U = T * S * HS;
  const int u8 = (U + 7) >> 3;
  const int uw = (blockIdx.x & 7) * u8 + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= u8 || uw >= U) return;
  const int hs = HS == 2 ? (uw & 1) : 0;
  const int u = uw / HS;   // (query, split) unit
  const int t = u / S, split = u - t * S;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int c = lane & 15, g = lane >> 4;
  // waves 0-3 score (keys 16kh.., head groups 2hp, 2hp+1), waves 4-7 weigh the values
  // (dims 128vw..128vw+127); waves w and w+4 share a SIMD
  const bool sw = wave < kSW;
  const int kh = wave & 1, hp = (wave >> 1) & 1;
  const int vw = wave & 3;
  // head group of the score wave's j-th set; of the value wave's h-th
  auto sgrp = [&](int j) { return HS == 1 ? 2 * hp + j : 2 * hs + hp; };
  auto vgrp = [&](int h) { return hs * NV + h; };

  const int seq = a.m.seq_id[t], p = a.m.pos[t];
  const bool valid_q = seq >= 0 && seq < a.m.num_seqs && p >= 0;
  int64_t n = 0;
  if (valid_q) {
    n = ((int64_t)p + 1) / a.m.ratio;
    n = n < a.m.max_visible ? n : a.m.max_visible;
    n = n < a.m.compressed_cap ? n : a.m.compressed_cap;
  }

  // Key list order. bf16 rows with one work-group per query (large batches): the window
  // first, then the selected latents in topk order; the first steps then gather window
  // rows, which neighbouring queries share and the L2 mostly holds, so the pipeline fills
  // sooner (prefill chunk 475 -> 456 us). Otherwise the latents first: smaller batches
  // measured 1-4 % slower with the window first, and code rows' format switch and scale
  // loads assume latents first.
  const bool wf = !KV8 && HS == 1 && S == 1;
  const int u0 = p - kWindow + 1 > 0 ? p - kWindow + 1 : 0;
  const int nwin = valid_q ? p - u0 + 1 : 0;
  constexpr int LRB = FP4L ? kDim / 2 : (KV8 ? kDim : 2 * kDim);   // latent row bytes
  constexpr int WRB = KV8 ? kDim : 2 * kDim;                       // window row bytes
  auto window_row = [&](int i) {   // raw position u0 + i in ring row (u0 + i) % window_cap
    const int64_t wr = (int64_t)((u0 + i) % a.window_cap);
    return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.window) +
                                             (int64_t)seq * a.window_seq_stride * (KV8 ? 1 : 2) + wr * WRB);
  };

  // ---- the selection (2 KB) and the query (64 KB) by direct loads: the selection into its
  // own LDS array, the query's 64 heads into tiles 2 and 3 (one padded row per head) until
  // step 2's rows replace it. Every load the kernel makes before its output is one of these,
  // so all waits are explicit vmcnt counts. ----
  const uint32_t tile0 = (uint32_t)(uintptr_t)&sh.tile[0][0];
  const uint32_t qlds = tile0 + (uint32_t)(2 * kKT * kRow);
  static_assert(kBufs >= 4 && kHeads <= 2 * kKT, "the query needs two tiles");
  if (valid_q) {
    if (wave < 2) {   // 256 entries per wave
      const int32_t* src = a.topk + (int64_t)t * kTopK + 256 * wave + 4 * lane;
      to_lds16(src, (uint32_t)(uintptr_t)&sh.topk[256 * wave]);
    }
    const uint16_t* qt = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)t * kHeads * kDim;
#pragma unroll
    for (int i = 0; i < kQPW; ++i) {
      const int head = (kHeads / HS) * hs + kQPW * wave + i;
      to_lds16(qt + head * kDim + 8 * lane, qlds + head * kRow);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kQPW));   // the selection (query loads in flight)
  }
  __syncthreads();

  // ---- key list ----
  int m = 0, nlat = 0;   // keys; code rows: the first nlat of them are latents
  if (valid_q) {
    const int32_t j = sh.topk[tid];   // kAThreads == kTopK
    const bool v = j >= 0 && j < n;
    const int incl = wave_incl_scan((int)v);
    if (lane == 63) sh.wave_cnt[wave] = incl;
    __syncthreads();
    int nsel = 0, before = 0;
    for (int w = 0; w < kAW; ++w) {
      nsel += sh.wave_cnt[w];
      before += (w < wave) ? sh.wave_cnt[w] : 0;
    }
    // global row of each key (and, for code rows, where its scale is: an fp32, or the 16
    // E8M0 bytes of an MXFP4 row). Strides are in elements of the store: bf16, or bytes.
    const uint8_t* latb = reinterpret_cast<const uint8_t*>(a.latents);
    const int lat0 = wf ? nwin : 0;   // first latent slot
    if (v) {
      int64_t off, sidx;
      if (a.pages.table) {   // paged latents: the row of position j is in page table[seq][j / page]
        const int64_t r = pool_row(a.pages, page_of(a.pages, seq, j), j);
        off = r * LRB;
        sidx = r;
      } else {
        off = (int64_t)seq * a.latents_seq_stride * (KV8 ? 1 : 2) + (int64_t)j * LRB;
        sidx = FP4L ? -1 : (int64_t)seq * a.latent_scales_seq_stride + j;
      }
      sh.rows[lat0 + before + incl - 1] = reinterpret_cast<const uint16_t*>(latb + off);
      if constexpr (FP4L) {
        const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.latent_scales) +
                            (a.pages.table ? sidx * 16 : (int64_t)seq * a.latent_scales_seq_stride + (int64_t)j * 16);
        sh.sptr[before + incl - 1] = reinterpret_cast<const float*>(sb);
      } else if constexpr (KV8) {
        sh.sptr[before + incl - 1] = reinterpret_cast<const float*>(a.latent_scales) + sidx;
      }
    }
    if (tid < nwin) {
      const int ws = wf ? tid : nsel + tid;   // the window's slot
      sh.rows[ws] = window_row(tid);
      if (KV8) sh.sptr[ws] = a.window_scales + (int64_t)seq * a.window_scales_seq_stride + (u0 + tid) % a.window_cap;
    }
    m = nsel + nwin;
    nlat = nsel;
  }
  __syncthreads();

  if (m == 0) {  // invalid query (no load was issued): zero output, lse = -inf
    if (split != 0 || hs != 0) return;
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (int64_t)t * kHeads * kDim;
    for (int i = tid; i < kHeads * kDim / 8; i += kAThreads)
      *reinterpret_cast<u32x4*>(o + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    if (a.lse && tid < kHeads) a.lse[(int64_t)t * kHeads + tid] = neg_inf();
    return;
  }

  // ---- this work-group's steps of the key list: kb .. kb + mk - 1 ----
  const int ns_all = (m + kKT - 1) / kKT;
  const int st0 = split * ns_all / S, st1 = (split + 1) * ns_all / S;
  const int kb = st0 * kKT;
  const int mk = min(m, st1 * kKT) - kb;   // 0 for a split without a step

  // ---- tile loader: wave w moves rows 4w..4w+3 of a step. Rows past the key list repeat
  // the last real row (finite data; their scores are masked), so every wave issues exactly
  // kRowsPerWave loads per step and the wait counts are constants.
  auto issue = [&](int step) {
    const uint32_t base = tile0 + (uint32_t)((step % kBufs) * (kKT * kRow) + wave * kRowsPerWave * kRow);
    const uint16_t* r[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) r[i] = sh.rows[kb + min(step * kKT + wave * kRowsPerWave + i, mk - 1)];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int idx = kb + min(step * kKT + wave * kRowsPerWave + i, mk - 1);
      if (FP4L && idx < nlat) {   // 256 code bytes (lanes 0-15) and 16 scale bytes (lane 16)
        const uint8_t* src = lane < 16 ? reinterpret_cast<const uint8_t*>(r[i]) + 16 * lane
                                       : reinterpret_cast<const uint8_t*>(sh.sptr[idx]);
        if (lane <= 16) to_lds16(src, base + i * kRow);
      } else if constexpr (KV8) {
        row8_to_lds(r[i], base + i * kRow, lane);
      } else {
        row_to_lds(r[i], base + i * kRow, lane);
      }
    }
  };
  // code rows: the slots' scales by direct loads, issued before the first rows so the
  // rows' waits cover them
  if constexpr (KV8) {
    for (int i = wave; i < kMaxKeys / 64; i += kAW) {
      const int slot = 64 * i + lane;
      const float* src = (FP4L && slot < nlat) || slot >= m ? &g_unit_scale : sh.sptr[slot];
      to_lds4(src, (uint32_t)(uintptr_t)&sh.rscale[64 * i]);
    }
  }
  // ---- score waves: query heads 16(2hp + j) + c as B operands (k-step s: dims
  // (4s+g)*8 .. +8), from LDS; steps 0 and 1 are already on their way meanwhile ----
  if (mk > 0) {
    issue(0);
    issue(1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kRowsPerWave));   // the query (steps 0, 1 in flight)
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitAll);
  }
  __syncthreads();
  const float sc2 = a.scale * kLog2e;
  const int nsteps = (mk + kKT - 1) / kKT;
  const int npass = mk > 0 ? 2 : 0;

  if (sw) {
    // ==================================== score waves ====================================
    bf16x8 qb[NJ][16];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(&sh.tile[0][0]) + 2 * kKT * kRow +
                            (16 * sgrp(j) + c) * kRow;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        qb[j][s] = *reinterpret_cast<const bf16x8*>(qrow + (KV8 ? (128 * g + 8 * s) * 2 : (4 * s + g) * 16));
    }
    __syncthreads();   // every wave holds its query heads: tile 2 may take step 2's rows
    if (mk > 0) issue(2);

    float m_ref[NJ], m_max[NJ], l_run[NJ];   // per head 16 sgrp(j) + c: reference (log2 domain),
#pragma unroll                                // max over this wave's keys so far, this lane's
    for (int j = 0; j < NJ; ++j) {            // part of the normaliser
      m_ref[j] = neg_inf();
      m_max[j] = neg_inf();
      l_run[j] = 0.f;
    }
    // raw S^T of step `step`: keys 16kh + 4g + i (rows), heads 16(2hp + j) + c (columns)
    auto scores_raw = [&](int step, f32x4 (&acc)[NJ]) {
      const uint8_t* krow = sh.tile[step % kBufs] + (16 * kh + c) * kRow;
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto mma = [&](int s, const bf16x8& ka) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[j][s], acc[j], 0, 0, 0);
      };
      if constexpr (!KV8 && NJ == 2) {
        // six operand reads ahead of the MFMAs that use them (the compiler's own order
        // keeps two in flight)
        constexpr int kAhead = 6;
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 kr[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) kr[s] = *reinterpret_cast<const bf16x8*>(krow + (4 * s + g) * 16);
#pragma unroll
        for (int s = 0; s < 16; ++s) mma(s, kr[s]);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);   // LDS reads
#pragma unroll
        for (int i = 0; i < 16 - kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, NJ, 0);     // MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NJ * kAhead, 0);
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (!KV8) {
#pragma unroll
        for (int s = 0; s < 16; ++s) mma(s, *reinterpret_cast<const bf16x8*>(krow + (4 * s + g) * 16));
      } else {
        // code rows widened here: k-steps 4t .. 4t+3 take dims 128g + 32t .. +31 of the
        // lane's key. MXFP4 latents and e4m3 window rows share a step only where the latents
        // end; slots past the list repeat the last key, in its format.
        const int k0 = step * kKT + 16 * kh;
        const bool all8 = !FP4L || kb + min(k0, mk - 1) >= nlat;
        const bool all4 = FP4L && kb + min(k0 + 15, mk - 1) < nlat;
        auto e4m3_t = [&](int t) {   // 32 codes of dims 128g + 32t ..
          const u32x4 e0 = *reinterpret_cast<const u32x4*>(krow + 128 * g + 32 * t);
          const u32x4 e1 = *reinterpret_cast<const u32x4*>(krow + 128 * g + 32 * t + 16);
          return [=](int u) { return u < 2 ? e4m3x8(e0[2 * u], e0[2 * u + 1]) : e4m3x8(e1[2 * u - 4], e1[2 * u - 3]); };
        };
        auto fp4_t = [&](int t, uint32_t sc4) {   // block 4g + t: 16 code bytes and its scale
          const u32x4 f = *reinterpret_cast<const u32x4*>(krow + 64 * g + 16 * t);
          const float bs = e8m0_f32((sc4 >> (8 * t)) & 0xFFu);
          return [=](int u) { return fp4x8(f[u], bs); };
        };
        if (all8) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const auto k8 = e4m3_t(t);
#pragma unroll
            for (int u = 0; u < 4; ++u) mma(4 * t + u, k8(u));
          }
        } else {
          // scales of blocks 4g .. 4g+3 of the lane's key (after its 256 code bytes)
          const uint32_t sc4 = *reinterpret_cast<const uint32_t*>(krow + kDim / 2 + 4 * g);
          if (all4) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const auto k4 = fp4_t(t, sc4);
#pragma unroll
              for (int u = 0; u < 4; ++u) mma(4 * t + u, k4(u));
            }
          } else {
            const bool mine4 = kb + min(k0 + c, mk - 1) < nlat;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const auto k8 = e4m3_t(t);
              const auto k4 = fp4_t(t, sc4);
#pragma unroll
              for (int u = 0; u < 4; ++u) mma(4 * t + u, mine4 ? k4(u) : k8(u));
            }
          }
        }
      }
      if constexpr (KV8) {   // raw score of key j times s_j (slots past the list: any value, masked)
        const int k0 = min(kb + step * kKT + 16 * kh + 4 * g, kMaxKeys - 4);
        const f32x4 rs = *reinterpret_cast<const f32x4*>(&sh.rscale[k0]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] *= rs[i];
      }
    };
    // softmax of step `step`: P to LDS buffer step & 1 (keys past mk, and whole steps past
    // the last, come out with P = 0). k-slots 0..3 of a P^T operand hold key half 0, 4..7
    // key half 1.
    auto softmax = [&](int step, const f32x4 (&acc)[NJ]) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float x[4];
        float mt = neg_inf();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = step * kKT + 16 * kh + 4 * g + i;
          x[i] = k < mk ? acc[j][i] * sc2 : neg_inf();
          mt = fmaxf(mt, x[i]);
        }
        mt = max_xor32(max_xor16(mt));   // all four lane groups of head c agree
        m_max[j] = fmaxf(m_max[j], mt);
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(x[i] - m_ref[j]);
          l_run[j] += pv[i];
        }
        if constexpr (KV8) {   // the values are the codes: P_j s_j weighs them
          const int k0 = min(kb + step * kKT + 16 * kh + 4 * g, kMaxKeys - 4);
          const f32x4 rs = *reinterpret_cast<const f32x4*>(&sh.rscale[k0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] *= rs[i];
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(&sh.P[step & 1][sgrp(j)][lane]) + 2 * kh;
        dst[0] = pack_bf16x2(pv[0], pv[1]);
        dst[1] = pack_bf16x2(pv[2], pv[3]);
      }
    };

    for (int pass = 0; pass < npass; ++pass) {
      if (pass == 1) {   // (the first pass's rows went out with the query)
#pragma unroll
        for (int j = 0; j < kDepth; ++j) issue(j);
      }
      __builtin_amdgcn_s_waitcnt(kWaitLater);   // step 0's rows (steps 1, 2 in flight)
      __syncthreads();
      f32x4 acc[NJ];
      scores_raw(0, acc);
      if (pass == 0) {
        // reference: the max of step 0's keys of the head (step 0 always holds a real key),
        // over both key halves
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          float mt = neg_inf();
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * kh + 4 * g + i < mk) mt = fmaxf(mt, acc[j][i] * sc2);
          mt = max_xor32(max_xor16(mt));
          if (g == 0) sh.tmax[kh][16 * sgrp(j) + c] = mt;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int head = 16 * sgrp(j) + c;
        if (pass == 0) {
          m_ref[j] = fmaxf(sh.tmax[0][head], sh.tmax[1][head]);
        } else {
          m_ref[j] = m_max[j];   // second pass: the true max (both halves), so every P <= 1
          m_max[j] = neg_inf();
        }
        l_run[j] = 0.f;
      }
      softmax(0, acc);
      // one barrier per step makes visible the P of step s, the rows of step s+1 and frees
      // the buffer of step s-1; the value waves weigh step s meanwhile. Steps past the last
      // are not requested (their tiles' stale rows only meet masked scores): the last
      // kDepth steps run in a loop of their own without requests (a branch around the
      // request would split the step's code, which the compiler interleaves), and once no
      // later step is in flight the wait is for all.
      int step = 0;
      for (; step < nsteps - kDepth; ++step) {
        __builtin_amdgcn_s_waitcnt(kWaitNext);   // step s+1's rows (step s+2's in flight)
        __syncthreads();
        scores_raw(step + 1, acc);
        issue(step + kDepth);                    // (queues while the MFMAs run)
        softmax(step + 1, acc);
      }
      for (; step < nsteps; ++step) {
        if (step == 0 || step + 2 < nsteps) __builtin_amdgcn_s_waitcnt(kWaitNext);
        else __builtin_amdgcn_s_waitcnt(kWaitAll);
        __syncthreads();
        scores_raw(step + 1, acc);               // past the last step: P = 0, never read
        softmax(step + 1, acc);
      }
      __builtin_amdgcn_s_waitcnt(kWaitAll);   // no row load may outlive the pass (or the LDS)
      if (pass == 1) break;
      // a second pass only if some head saw a score more than kSafe above its reference
      bool over = false;
#pragma unroll
      for (int j = 0; j < NJ; ++j) over = over || m_max[j] > m_ref[j] + kSafe;
      const bool wave_redo = __ballot(over) != 0;
      if (lane == 0) sh.redo[wave] = wave_redo;
      __syncthreads();
      int redo = 0;
      for (int w = 0; w < kSW; ++w) redo |= sh.redo[w];
      if (!redo) break;
      // the second pass's reference: the max over both key halves
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (g == 0) sh.tmax[kh][16 * sgrp(j) + c] = m_max[j];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int head = 16 * sgrp(j) + c;
        m_max[j] = fmaxf(sh.tmax[0][head], sh.tmax[1][head]);
      }
      __syncthreads();   // every wave read the flags and maxima and is done with the tiles
    }

    // ---- normaliser of head 16(2hp+j) + c: both key halves, four lane groups each ----
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float L = add_xor32(add_xor16(l_run[j]));
      if (g == 0) sh.tmax[kh][16 * sgrp(j) + c] = L;
    }
    __syncthreads();
    if (kh == 0 && g == 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int head = 16 * sgrp(j) + c;
        const float Lh = sh.tmax[0][head] + sh.tmax[1][head];
        if (S == 1) {
          sh.norm[head] = Lh;
          if (a.lse) a.lse[(int64_t)t * kHeads + head] = (m_ref[j] + __log2f(Lh)) * kLn2;
        } else {
          float* ml = a.part_ml + ((int64_t)u * kHeads + head) * 2;
          store_dev(ml, m_ref[j]);
          store_dev(ml + 1, Lh);
        }
      }
    }
    __syncthreads();
    if (S == 1) return;
  } else {

    // ==================================== value waves ====================================
    __syncthreads();   // (the score waves read their query heads)
    if (mk > 0) issue(2);
    // O^T accumulators [half][head group][e4]: dims 128vw + 64hh + 4r + e4 (r = MFMA row) of
    // head 16h + c
    f32x4 O[2][NV][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int h = 0; h < NV; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) O[hh][h][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    // O^T += V^T P^T for step `step`: A = V^T from LDS rows by byte permutes (8 keys x 1 dim
    // per lane), B = P^T of each head group
    auto values = [&](int step) {
      const uint8_t* T8 = sh.tile[step % kBufs];
      bf16x8 pb[NV];
#pragma unroll
      for (int h = 0; h < NV; ++h) pb[h] = __builtin_bit_cast(bf16x8, sh.P[step & 1][vgrp(h)][lane]);
      // key slot j of half hh: dims 128vw + 64hh + 4c .. +3 (two dwords of bf16 pairs;
      // code rows are widened to them here)
      uint32_t R[2][8][2];
      auto key_of = [&](int j) { return (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4)); };
      auto bf16_R = [&](int hh, int j) {
        const uint2 v = *reinterpret_cast<const uint2*>(T8 + key_of(j) * kRow + (128 * vw + 64 * hh + 4 * c) * 2);
        R[hh][j][0] = v.x;
        R[hh][j][1] = v.y;
      };
      auto e4m3_R = [&](int hh, int j) {   // 4 codes
        const uint32_t x = *reinterpret_cast<const uint32_t*>(T8 + key_of(j) * kRow + 128 * vw + 64 * hh + 4 * c);
        return uint2{e4m3_pair<false>(x), e4m3_pair<true>(x)};
      };
      auto fp4_R = [&](int hh, int j) {    // 4 E2M1 elements (2 bytes) and their block's scale
        const uint8_t* row = T8 + key_of(j) * kRow;
        const uint32_t x = *reinterpret_cast<const uint16_t*>(row + 64 * vw + 32 * hh + 2 * c);
        const float bs = e8m0_f32(row[kDim / 2 + 4 * vw + 2 * hh + (c >> 3)]);
        return uint2{fp4_pair<0>(x, bs), fp4_pair<1>(x, bs)};
      };
      if constexpr (!KV8) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < 8; ++j) bf16_R(hh, j);
      } else {
        const int k0 = step * kKT;
        const bool all8 = !FP4L || kb + min(k0, mk - 1) >= nlat;
        const bool all4 = FP4L && kb + min(k0 + kKT - 1, mk - 1) < nlat;
        auto put = [&](int hh, int j, uint2 v) {
          R[hh][j][0] = v.x;
          R[hh][j][1] = v.y;
        };
        if (all8) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < 8; ++j) put(hh, j, e4m3_R(hh, j));
        } else if (all4) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < 8; ++j) put(hh, j, fp4_R(hh, j));
        } else {   // the step where the latents end: each key slot its own format
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const bool lat = kb + min(k0 + key_of(j), mk - 1) < nlat;
              const uint2 a = e4m3_R(hh, j), b = fp4_R(hh, j);
              put(hh, j, lat ? b : a);
            }
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int w = e4 >> 1;
          u32x4 va;
          if (e4 & 1) {
            va = u32x4{perm_hi(R[hh][1][w], R[hh][0][w]), perm_hi(R[hh][3][w], R[hh][2][w]),
                       perm_hi(R[hh][5][w], R[hh][4][w]), perm_hi(R[hh][7][w], R[hh][6][w])};
          } else {
            va = u32x4{perm_lo(R[hh][1][w], R[hh][0][w]), perm_lo(R[hh][3][w], R[hh][2][w]),
                       perm_lo(R[hh][5][w], R[hh][4][w]), perm_lo(R[hh][7][w], R[hh][6][w])};
          }
          const bf16x8 A = __builtin_bit_cast(bf16x8, va);
#pragma unroll
          for (int h = 0; h < NV; ++h)
            O[hh][h][e4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pb[h], O[hh][h][e4], 0, 0, 0);
        }
    };

    for (int pass = 0; pass < npass; ++pass) {
      if (pass == 1) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int h = 0; h < NV; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) O[hh][h][e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kDepth; ++j) issue(j);
      }
      __builtin_amdgcn_s_waitcnt(kWaitLater);
      __syncthreads();
      __syncthreads();   // (the score waves' step-0 maxima)
      int step = 0;
      for (; step < nsteps - kDepth; ++step) {
        __builtin_amdgcn_s_waitcnt(kWaitNext);
        __syncthreads();
        values(step);
        issue(step + kDepth);
      }
      for (; step < nsteps; ++step) {
        if (step == 0 || step + 2 < nsteps) __builtin_amdgcn_s_waitcnt(kWaitNext);
        else __builtin_amdgcn_s_waitcnt(kWaitAll);
        __syncthreads();
        values(step);
      }
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      if (pass == 1) break;
      if (lane == 0) sh.redo[wave] = 0;
      __syncthreads();
      int redo = 0;
      for (int w = 0; w < kSW; ++w) redo |= sh.redo[w];
      if (!redo) break;
      __syncthreads();
      __syncthreads();
    }

    __syncthreads();   // (the score waves' normalisers)
    __syncthreads();
    if (S == 1) {
      // ---- store: lane (c, g) holds dims 128vw + 64hh + 4(4g+i) + e4 of head 16h + c ----
#pragma unroll
      for (int h = 0; h < NV; ++h) {
        const float inv = 1.0f / sh.norm[16 * vgrp(h) + c];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)t * kHeads + 16 * vgrp(h) + c) * kDim +
                           128 * vw + 64 * hh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;  // row of the MFMA result = group of 4 dims
            uint2 o;
            o.x = pack_bf16x2(O[hh][h][0][i] * inv, O[hh][h][1][i] * inv);
            o.y = pack_bf16x2(O[hh][h][2][i] * inv, O[hh][h][3][i] * inv);
            *reinterpret_cast<uint2*>(orow + 4 * r) = o;
          }
        }
      }
      return;
    }
    // partial O of this split's head groups, in the lanes' own order (every instruction:
    // 1 KB of lines); a unit holds all 64 heads, each head set writes its own groups
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int h = 0; h < NV; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 v = __builtin_bit_cast(u32x4, f32x4{O[hh][h][0][i], O[hh][h][1][i], O[hh][h][2][i], O[hh][h][3][i]});
          __builtin_amdgcn_raw_buffer_store_b128(v, part_rsrc(a, T * S), part_off(u, vw, hh, vgrp(h), i) + lane * 16, 0,
                                                 kCoherent);
        }
  }
  {

  // ---- key splits: the last work-group of the query to finish combines the partials ----
  // The softmax of the whole key list from the splits' partial ones: with M the largest
  // reference, o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) L_s. Partials travel by
  // device-coherent stores and loads (written through to, and read from, the level all
  // XCDs share), so no cache-wide write-back or invalidation is needed; the count is
  // raised only after every store of the work-group has completed.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partial is device-visible
  __syncthreads();
  // one counter per (query, head set)
  if (tid == 0) sh.last = atomicAdd(&a.counters[t * HS + hs], 1u) == (uint32_t)(S - 1);
  __syncthreads();
  if (!sh.last) return;
  if (tid == 0) a.counters[t * HS + hs] = 0u;   // every split of this call has counted: ready for the next
  // every wave combines one slice: dims 128cv + 64chh .. +63 of the head set's heads
  const int cv = wave & 3, chh = wave >> 2;
  const int u0 = t * S;
  float wgt[NV][kMaxSplits], Lsum[NV], Mx[NV];
#pragma unroll
  for (int h = 0; h < NV; ++h) {
    const int head = 16 * vgrp(h) + c;
    float mref[kMaxSplits], lsp[kMaxSplits];
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
      const float* ml = a.part_ml + ((int64_t)(u0 + min(s2, S - 1)) * kHeads + head) * 2;
      mref[s2] = s2 < S ? load_dev(ml) : neg_inf();
      lsp[s2] = s2 < S ? load_dev(ml + 1) : 0.f;
    }
    float M = neg_inf();
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) M = fmaxf(M, mref[s2]);
    float L = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
      wgt[h][s2] = s2 < S ? __builtin_amdgcn_exp2f(mref[s2] - M) : 0.f;   // an empty split: 2^-inf = 0
      L += wgt[h][s2] * lsp[s2];
    }
    Lsum[h] = L;
    Mx[h] = M;
  }
  // sum over the splits in split order (the same bits whichever work-group combines)
  f32x4 acc[NV][4];
#pragma unroll
  for (int s2 = 0; s2 < kMaxSplits; ++s2) {
    if (s2 >= S) break;
    asm volatile("" ::: "memory");   // one split's loads in flight at a time (registers)
    f32x4 v[NV][4];
#pragma unroll
    for (int h = 0; h < NV; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[h][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
            part_rsrc(a, T * S), part_off(u0 + s2, cv, chh, vgrp(h), i) + lane * 16, 0, kCoherent));
#pragma unroll
    for (int h = 0; h < NV; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] = s2 == 0 ? wgt[h][0] * v[h][i] : acc[h][i] + wgt[h][s2] * v[h][i];
  }
#pragma unroll
  for (int h = 0; h < NV; ++h) {
    const int head = 16 * vgrp(h) + c;
    const float inv = 1.0f / Lsum[h];
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)t * kHeads + head) * kDim + 128 * cv + 64 * chh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 o;
      o.x = pack_bf16x2(acc[h][i][0] * inv, acc[h][i][1] * inv);
      o.y = pack_bf16x2(acc[h][i][2] * inv, acc[h][i][3] * inv);
      *reinterpret_cast<uint2*>(orow + 4 * (4 * g + i)) = o;
    }
    if (a.lse && wave == 0 && g == 0) a.lse[(int64_t)t * kHeads + head] = (Mx[h] + __log2f(Lsum[h])) * kLn2;
  }
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

// Work-groups per query for batches with fewer queries than CUs: up to 16 queries split each
// query's heads over two work-groups and its keys over four (8 per query), 17 to 32 split
// the keys over four, 33 to 128 only the heads over two (key splits as well measured no
// faster for 64 queries: 19.8 against 19.3 us); larger batches take one work-group per query.
int attn_head_sets(int64_t T, int splits) { return (T <= 16 && splits > 1) || (T > 32 && T <= 128) ? 2 : 1; }

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  const int hs = attn_head_sets(a.m.T, a.splits);
  const int64_t u8 = (a.m.T * a.splits * hs + 7) / 8;   // work units per XCD
  if (hs == 2)
    if (a.kv_mode == 2)
      hipLaunchKernelGGL((attn_kernel<2, 2>), dim3((unsigned)(8 * u8)), dim3(kAThreads), 0, stream, a);
    else if (a.kv_mode == 1)
      hipLaunchKernelGGL((attn_kernel<2, 1>), dim3((unsigned)(8 * u8)), dim3(kAThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_kernel<2, 0>), dim3((unsigned)(8 * u8)), dim3(kAThreads), 0, stream, a);
  else
    if (a.kv_mode == 2)
      hipLaunchKernelGGL((attn_kernel<1, 2>), dim3((unsigned)(8 * u8)), dim3(kAThreads), 0, stream, a);
    else if (a.kv_mode == 1)
      hipLaunchKernelGGL((attn_kernel<1, 1>), dim3((unsigned)(8 * u8)), dim3(kAThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_kernel<1, 0>), dim3((unsigned)(8 * u8)), dim3(kAThreads), 0, stream, a);
  return hipGetLastError();
}

// Small batches (at most 32 queries): a query's keys are spread over kMaxSplits work-groups
// (the last to finish for each head set reads the others' partials). With more queries the
// partial traffic costs about what the shorter key lists save.
int attn_splits(int64_t T) { return T <= 32 ? kMaxSplits : 1; }

int64_t attn_max_units(int64_t max_queries) {
  int64_t best = 0;
  const int64_t lim = max_queries < 32 ? max_queries : 32;
  for (int64_t T = 1; T <= lim; ++T) {
    const int s = attn_splits(T);
    if (s > 1 && T * s > best) best = T * s;
  }
  return best;
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace sa

// Key-split state for callers that cannot allocate (sparse_attn_fwd_noalloc): one fixed
// array per GPU instead of a workspace. Layout: [kScratchCounters u32 counters, padded to
// 512 B][kScratchUnits x 64 x 2 fp32 partial references and normalisers][kScratchUnits
// partial outputs of 128 KiB]. Host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (attn_scratch below).
namespace {
constexpr size_t kScratchMlOff = 512;
constexpr size_t kScratchOOff = kScratchMlOff + (size_t)sa::kScratchUnits * 64 * 2 * sizeof(float);
constexpr size_t kScratchBytes = kScratchOOff + (size_t)sa::kScratchUnits * 64 * 512 * sizeof(float);
static_assert(sa::kScratchCounters * sizeof(uint32_t) <= kScratchMlOff, "counters fit before the partials");
static_assert(kScratchOOff % 256 == 0, "partial outputs 256-byte aligned");
constexpr int kScratchDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace sa {

hipError_t attn_scratch(AttnScratch& s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  static std::atomic<uint8_t*> ptrs[kScratchDevices] = {};
  static std::mutex mu;
  uint8_t* base = ptrs[dev].load(std::memory_order_acquire);
  if (base == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    base = ptrs[dev].load(std::memory_order_relaxed);
    if (base == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // this device's copy of the array
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      base = static_cast<uint8_t*>(p);
      ptrs[dev].store(base, std::memory_order_release);
    }
  }
  s.counters = reinterpret_cast<uint32_t*>(base);
  s.part_ml = reinterpret_cast<float*>(base + kScratchMlOff);
  s.part_o = reinterpret_cast<float*>(base + kScratchOOff);
  s.bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace sa
