// S1 indexer scores on gfx950 MFMA.
//
// Score of compressed position j for a query: I(j) = s_j * sum_h w_h * max(0, <qI_h, k_j>)
// over 16 index heads x 128 dims, one key per position ("deepseek-ai/DeepSeek-V4.1-Flash"
// recipe, Overview, two-tier sparse attention bullet: a small side attention scores the
// compressed latents). s_j is the fp32 row scale of e4m3 keys (1 for bf16 keys). e4m3 keys
// are widened to bf16 exactly in registers; the index query stays bf16.
//
// Block maxima (blocks of 8 positions) are taken in registers with DPP.
//
// Decode (every query has its own key stream, HBM-bound): each wave streams 32 KB of keys
// (16 e4m3 or 8 bf16 tiles of 16 keys) from HBM straight into its own LDS ring (kDepth
// tiles in flight, no registers held; every load instruction moves 1 KB of whole rows).
// v_mfma_f32_16x16x32_bf16 then takes the 16 heads of the query as rows (A, in registers)
// and the tile's 16 keys as columns (B, from LDS). In the 16x16 result each lane holds
// heads 4g..4g+3 (g = lane/16) of key lane%16: ReLU and head weights in-lane, then two
// row-swap adds finish the 16-head sum. The k order inside an MFMA is free (A and B use the
// same one). Scores are staged in LDS and written at the end with their row scales and
// block maxima, 64 consecutive keys per store.
//
// Prefill (a chunk of queries shares one key stream, MFMA-bound): v_mfma_f32_32x32x16_bf16
// with two queries x 16 heads as rows and 32 keys as columns. Key tiles are staged once per
// work-group in padded LDS rows (prefetched two tiles ahead through registers) and read by
// every wave; each wave holds two query pairs. The A rows are ordered so that a lane's 16
// results are the 16 heads of one query for one key: the head sum finishes in-lane.
#include "sa_compress.h"
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

__device__ __forceinline__ int visible_of(int pos, int ratio) {
  return ratio == 2 ? (pos + 1) >> 1 : pos + 1;
}

// n of query t: visible compressed count, capped; 0 for invalid metadata.
__device__ __forceinline__ int query_n(const IndexerArgs& a, int t) {
  const int seq = a.seq_id[t], pos = a.pos[t];
  if (seq < 0 || seq >= a.num_seqs || pos < 0) return 0;
  int64_t n = visible_of(pos, a.ratio);
  n = n < a.max_visible ? n : a.max_visible;
  n = n < a.compressed_cap ? n : a.compressed_cap;
  return (int)n;
}

// ======================================================================================
// Decode
// ======================================================================================
#ifndef SA_IDX_DEPTH
#define SA_IDX_DEPTH 8
#endif
constexpr int kDWaves = 4;
constexpr int kDThreads = 64 * kDWaves;
constexpr int kTilesPerWave = 16;                  // most tiles of one wave (e4m3 keys)
constexpr int kRingBytes = SA_IDX_DEPTH * 16 * kIdxDim;   // per wave: kDepth e4m3 tiles

// Decode key tiles (16 keys) travel HBM -> LDS by direct loads (no registers): each load
// instruction moves 1 KB of whole key rows, so every request is full cache lines. Inside a
// row the 16-byte chunks are stored rotated (chunk q of row r at position q ^ f(r)), which
// the loads do for free by choosing each lane's source; the B-operand reads (16 rows, one
// chunk each per lane group) then hit 16 different bank groups.
template <bool FP8>
struct DecodeTile {
  static constexpr int RB = FP8 ? kIdxDim : 2 * kIdxDim;   // row bytes
  static constexpr int TB = 16 * RB;                       // tile bytes
  static constexpr int NK = TB / 1024;                     // loads per tile
  static constexpr int D = kRingBytes / TB;                // tiles in flight per wave
  static constexpr int CPR = RB / 16;                      // chunks per row
  // position of chunk q in row r
  static __device__ __forceinline__ int pos(int r, int q) {
    return FP8 ? (q ^ ((r & 7) ^ (r >> 3))) : (q ^ r);
  }
};

struct DecodeShared {
  uint8_t ring[kDWaves][kRingBytes];
  float stage[kDWaves][kTilesPerWave * 16];   // unscaled scores of the wave's keys
  uint16_t q[kIdxHeads * kIdxDim];
  float w[kIdxHeads];
  int32_t ids[kDWaves * kTilesPerWave * 2];   // candidate mode: the group's block ids
};

// Dims of k-step s (0..3) held by lane group g, in elements. bf16 keys: chunk 4s+g of
// 8 dims; e4m3 keys: ksteps (2i, 2i+1) share one 16-byte chunk, 4i+g.
__device__ __forceinline__ int kdim_bf16(int g, int s) { return (4 * s + g) * 8; }
__device__ __forceinline__ int kdim_fp8(int g, int s) { return ((s >> 1) * 4 + g) * 16 + (s & 1) * 8; }

template <bool FP8>
struct KeyRegs {
  u32x4 v[FP8 ? 2 : 4];
};

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t c0, uint32_t c1) {
  uint32_t u0, u1, u2, u3;
  e4m3x4_to_bf16x4(c0, u0, u1);
  e4m3x4_to_bf16x4(c1, u2, u3);
  u32x4 u = {u0, u1, u2, u3};
  return __builtin_bit_cast(bf16x8, u);
}

template <bool FP8>
__device__ __forceinline__ f32x4 tile_dots(const bf16x8 (&qa)[4], const KeyRegs<FP8>& K) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 b;
    if constexpr (FP8) b = e4m3x8_to_bf16x8(K.v[s >> 1][2 * (s & 1)], K.v[s >> 1][2 * (s & 1) + 1]);
    else b = __builtin_bit_cast(bf16x8, K.v[s]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], b, acc, 0, 0, 0);
  }
  return acc;
}

// 16 bytes per lane from global memory to LDS byte lds + 16 * lane. The compiler does not
// see these loads; completion is tracked with explicit vmcnt waits, and the kernel issues
// no other vector-memory operation between the first of them and the last wait. The key
// stream is read once, so the loads are non-temporal (nt): streamed through the caches
// without displacing other lines (measured 7 % faster than the default policy).
__device__ __forceinline__ void to_lds16(const void* src, uint32_t lds) {
  // s_nop: an LDS-DMA load must not directly follow the write of M0 (one wait state)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" :: "v"(src), "{m0}"(lds) : "memory");
}
// Same, after every LDS read of this wave has returned (the slot being refilled was just read).
__device__ __forceinline__ void to_lds16_after_reads(const void* src, uint32_t lds) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" :: "v"(src), "{m0}"(lds) : "memory");
}
// 4 bytes per lane to LDS byte lds + 4 * lane (same rules as to_lds16).
__device__ __forceinline__ void to_lds4(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// Register values loaded before a loop of direct loads: the compiler counts only its own
// loads, so a wait it places before a later use (in every unrolled tile whose guard it cannot
// resolve) would also hold for the direct loads in flight and drain the ring. Passing the
// values through an empty asm makes that asm their last definition: the compiler waits for
// their loads once, there, and never again.
template <class T>
__device__ __forceinline__ void settle(T& v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 16, "a dword or a 16-byte vector");
  if constexpr (sizeof(T) == 4) {
    asm volatile("" : "+v"(v));
  } else {
    u32x4 x = __builtin_bit_cast(u32x4, v);
    asm volatile("" : "+v"(x));
    v = __builtin_bit_cast(T, x);
  }
}

// A compressor job riding in an indexer launch: work-groups of the grid rows from
// a.cj_row0 on run it (all indexer kernels have the compressor's 256 threads) and return.
__device__ __forceinline__ bool run_compress_rows(const IndexerArgs& a) {
  if (a.cj.G == 0 || (int)blockIdx.y < a.cj_row0) return false;
  compress_blocks(a.cj, (int64_t)(blockIdx.y - a.cj_row0) * gridDim.x + blockIdx.x,
                  (int64_t)(gridDim.y - a.cj_row0) * gridDim.x);
  return true;
}

// Modes. kPlain: each query's keys are contiguous rows of its sequence. kCand (candidate-
// bounded re-scoring): the score row is in slot order, entry 8i + r belonging to position
// 8 cand[i] + r of the query's carried candidate blocks (ascending, -1 padded); a tile of 16
// entries is two candidate blocks, and the loads gather those blocks' rows. kPaged: the keys
// (and e4m3 scales) are page pools; a tile of 16 positions lies in one page (pages hold a
// multiple of 16 positions), whose id each wave reads from the block table up front.
enum DecodeMode { kPlain = 0, kCand = 1, kPaged = 2 };

// Tiles per wave: the same 32 KB of key rows per wave in either format (16 e4m3 tiles or 8
// bf16 tiles). Fewer, longer waves measured slower with e4m3 keys (8 or 32 tiles: 202-226
// against 180 us on 128 queries at 64K keys); with bf16 keys 8 tiles beat 16 (64 queries at
// 16K keys 45.7 -> 44.4 us, 4 queries at 1K keys 10.4 -> 9.0 us). Candidate mode keeps 16
// (a wave's two block ids per tile fill its 32 lanes).
template <bool FP8, int MODE>
constexpr int decode_tpw() { return FP8 || MODE == kCand ? kTilesPerWave : kTilesPerWave / 2; }

template <bool FP8, int MODE>
__global__ __launch_bounds__(kDThreads) void indexer_decode_kernel(IndexerArgs a) {
  if (run_compress_rows(a)) return;
  constexpr bool CAND = MODE == kCand, PAGED = MODE == kPaged;
  using DT = DecodeTile<FP8>;
  constexpr int RB = DT::RB, TB = DT::TB, NK = DT::NK, D = DT::D;
  constexpr int TPW = decode_tpw<FP8, MODE>();
  static_assert(TPW % 4 == 0 && TPW <= kTilesPerWave, "whole 64-key stores; shared arrays sized for the most");
  static_assert((D & (D - 1)) == 0 && D >= 2, "ring depth must be a power of two");
  static_assert(D * NK <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) DecodeShared sh;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int E = (int)a.E;
  const int chunk0 = blockIdx.x * (kDWaves * TPW * 16);
  const int key0 = chunk0 + wave * TPW * 16;   // the keys this wave stores
  const int n = query_n(a, t);
  const int ntiles = key0 < E ? min(TPW, (E - key0 + 15) >> 4) : 0;
  // tiles of the group's chunk below n, and this wave's share of them (candidate mode:
  // decided once the block ids are in)
  const int chunk_live = CAND ? (n > 0 ? 1 : 0)
                              : (chunk0 < n ? min(kDWaves * TPW, (n - chunk0 + 15) >> 4) : 0);
  int live = CAND ? 0 : min(max(chunk_live - wave * TPW, 0), TPW);
  auto tile_of = [&](int i) { return wave * TPW + i; };
  const bool wg_live = chunk_live > 0;

  float* srow = a.scores + (int64_t)t * a.ld_scores;
  float* brow = a.block_max ? a.block_max + (int64_t)t * a.ld_block_max : nullptr;
  const int seq = a.seq_id[t];
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) +
                        (PAGED ? 0 : (int64_t)seq * a.keys_seq_stride * (FP8 ? 1 : 2));

  // e4m3 row scales of the keys this lane stores at the end (issued first: the loads
  // complete in order, so the row waits below also cover them)
  float scv[TPW / 4] = {};
  if (FP8 && MODE == kPlain && key0 < n) {   // (a query without keys may have no valid sequence)
    const float* scales = a.scales + (int64_t)seq * a.scales_seq_stride;
#pragma unroll
    for (int j = 0; j < TPW / 4; ++j) scv[j] = scales[min(key0 + 64 * j + lane, n - 1)];
  }
  // paged mode: page id of the wave's tile `lane` (lanes past the last tile take its page),
  // read before any tile load since the tile addresses depend on it. The wave's tiles span
  // at most 16 consecutive table entries, read with uniform addresses ahead of every other
  // memory operation, so they come through the scalar cache (lgkmcnt, not vmcnt)
  int pgreg = 0;
  if constexpr (PAGED) {
    if (live > 0) {
      const int32_t* trow = a.pages.table + (int64_t)seq * a.pages.stride;
      const int lp = a.pages.log2_page;
      const int e0 = key0 >> lp, elast = (n - 1) >> lp;
      int ent[TPW];
#pragma unroll
      for (int j = 0; j < TPW; ++j) ent[j] = trow[min(e0 + j, elast)];
      const int mine = ((key0 + 16 * min(lane, TPW - 1)) >> lp) - e0;   // 0 .. 15
      int v = ent[0];
#pragma unroll
      for (int j = 1; j < TPW; ++j) v = mine == j ? ent[j] : v;
      pgreg = (int)min(max((int64_t)v, (int64_t)0), a.pages.num_pages - 1);
    }
  }
  const uint32_t lds_q = (uint32_t)(uintptr_t)&sh.q[0];
  const uint32_t lds_w = (uint32_t)(uintptr_t)&sh.w[0];
  if (wg_live) {
    // the query's 16 x 128 index heads (4 KB): wave w moves bytes 1024w .. 1024w + 1023
    static_assert(kDWaves * 1024 == kIdxHeads * kIdxDim * 2, "one KB of the query per wave");
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q_idx) + (int64_t)t * kIdxHeads * kIdxDim * 2;
    to_lds16(qb + 1024 * wave + 16 * lane, lds_q + 1024 * wave);
    if (wave == 0 && lane < kIdxHeads / 4) to_lds16(a.w + (int64_t)t * kIdxHeads + 4 * lane, lds_w);
    if (CAND && wave == 1 && lane < kDWaves * TPW * 2 / 4)   // the group's block ids
      to_lds16(a.cand + (int64_t)t * kCandBlocks + chunk0 / 8 + 4 * lane, (uint32_t)(uintptr_t)&sh.ids[0]);
  }
  // paged mode: the e4m3 scales, each lane's key in the page of its tile
  if constexpr (PAGED) {
    if (live > 0) {
      if constexpr (FP8) {
        const float* scales = a.scales;
#pragma unroll
        for (int j = 0; j < TPW / 4; ++j) {
          const int x = min(key0 + 64 * j + lane, n - 1);
          const int pg = __shfl(pgreg, (x - key0) >> 4);
          scv[j] = scales[pool_row(a.pages, pg, x)];
        }
      }
    }
  }
  // candidate mode: block id of the wave's slot `lane` (lane reads pick one per load). A
  // slot is valid when its block holds a visible position (0 <= id < ceil(n / 8), compared
  // without forming 8 id); the wave loads tiles up to its last valid slot, and invalid
  // slots among them read row n - 1 and are masked.
  static_assert(2 * TPW <= 64, "one slot per lane");
  constexpr int kSlots = 2 * TPW;   // candidate blocks per wave
  const int nbv = (n + 7) >> 3;
  auto valid_id = [&](int id) { return id >= 0 && id < nbv; };
  int idreg = -1;
  if constexpr (CAND) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("s_barrier" ::: "memory");
    if (wg_live && lane < kSlots) idreg = sh.ids[kSlots * wave + lane];
    const uint64_t vm = __ballot(valid_id(idreg));
    live = vm ? (64 - __builtin_clzll(vm) + 1) >> 1 : 0;
    if (FP8 && live > 0) {
      const float* scales = a.scales + (int64_t)seq * a.scales_seq_stride;
#pragma unroll
      for (int j = 0; j < TPW / 4; ++j) {
        const int id = sh.ids[kSlots * wave + 8 * j + (lane >> 3)];
        scv[j] = valid_id(id) ? scales[min(8 * id + (lane & 7), n - 1)] : 0.f;
      }
    }
  }

  // load j of a tile: lane -> row rr[j], chunk qq[j]; its 16 bytes land at position
  // pos(row, chunk) of that row in LDS
  int rr[NK], qq[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int r = j * (64 / DT::CPR) + lane / DT::CPR;
    const int p = lane % DT::CPR;
    rr[j] = r;
    qq[j] = DT::pos(r, p);   // pos is an involution in q for a fixed row
  }
  const uint32_t ring0 = (uint32_t)(uintptr_t)&sh.ring[wave][0];
  auto issue = [&](int i, bool after_reads) {
    const int k = chunk0 + 16 * tile_of(i);
    const uint8_t* tb = keys + (int64_t)k * RB;
    const int last = n - 1 - k;   // rows past n in the last live tile repeat row n - 1
    const uint32_t lds = ring0 + (uint32_t)((i & (D - 1)) * TB);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const uint8_t* src;
      if constexpr (CAND) {
        // load j covers rows of one slot: 2i + j (e4m3) or 2i + j/2 (bf16); slots past the
        // valid ones read row n - 1 (masked)
        const int id = __builtin_amdgcn_readlane(idreg, 2 * i + (j * (64 / DT::CPR)) / 8);
        const int row = valid_id(id) ? min(8 * id + (rr[j] & 7), n - 1) : n - 1;
        src = keys + (int64_t)row * RB + qq[j] * 16;
      } else if constexpr (PAGED) {
        const int64_t pg = __builtin_amdgcn_readlane(pgreg, i);
        src = keys + (pool_row(a.pages, pg, k) + min(rr[j], last)) * RB + qq[j] * 16;
      } else {
        src = tb + (min(rr[j], last) * RB + qq[j] * 16);
      }
      if (j == 0 && after_reads) to_lds16_after_reads(src, lds + 1024 * j);
      else to_lds16(src, lds + 1024 * j);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < live) issue(u, false);
  if constexpr (!CAND) {
    if (live >= D) __builtin_amdgcn_s_waitcnt(waitcnt_vm(D * NK));   // query, weights, scales
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    // every wave's part of the query is in LDS (its loads completed above); a bare barrier,
    // since a fence here would also wait for the row loads in flight
    asm volatile("s_barrier" ::: "memory");
  }

  if (live > 0) {
    bf16x8 qa[4];
    float wq[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[s] = *reinterpret_cast<const bf16x8*>(&sh.q[c * kIdxDim + (FP8 ? kdim_fp8(g, s) : kdim_bf16(g, s))]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wq[i] = sh.w[4 * g + i];
    // B-operand reads of lane (c, g): chunk g + 4i (e4m3) or 4i + g (bf16) of row c
    uint32_t roff[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int q = FP8 ? g + 4 * i : 4 * i + g;
      roff[i] = (uint32_t)(c * RB + DT::pos(c, q) * 16);
    }
    float* stage = sh.stage[wave];   // row stride: the most tiles of a wave
    for (int i = 0; i < live; ++i) {
      if (i + D - 1 < live) __builtin_amdgcn_s_waitcnt(waitcnt_vm((D - 1) * NK));   // tile i landed
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      const uint8_t* tile = sh.ring[wave] + (i & (D - 1)) * TB;
      KeyRegs<FP8> K;
#pragma unroll
      for (int j = 0; j < NK; ++j) K.v[j] = *reinterpret_cast<const u32x4*>(tile + roff[j]);
      const f32x4 acc = tile_dots<FP8>(qa, K);
      if (i + D < live) issue(i + D, true);
      float v = wq[0] * relu(acc[0]);
      v = fmaf(wq[1], relu(acc[1]), v);
      v = fmaf(wq[2], relu(acc[2]), v);
      v = fmaf(wq[3], relu(acc[3]), v);
      v = add_xor32(add_xor16(v));
      if (lane < 16) stage[16 * i + lane] = v;
    }
  }

  // ---- scores and block maxima of the wave's keys: 64 consecutive keys per store ----
  const float* stage = sh.stage[wave];
#pragma unroll
  for (int j = 0; j < TPW / 4; ++j) {
    const int k = key0 + 64 * j + lane;
    if (64 * j >= 16 * ntiles) break;
    float v = neg_inf();
    bool ok = k < n;
    if constexpr (CAND) {
      const int id = wg_live ? sh.ids[kSlots * wave + 8 * j + (lane >> 3)] : -1;
      ok = valid_id(id) && 8 * id + (lane & 7) < n;
    }
    if (ok) {
      v = stage[64 * j + lane];
      if constexpr (FP8) v *= scv[j];
    }
    const float m = max8_lanes(v);   // E is a multiple of 8: groups are all in or all out
    if (k < E) {
      srow[k] = v;
      if (brow && (lane & 7) == 0) brow[k >> 3] = m;
    }
  }
}

// ======================================================================================
// Decode, MXFP4 keys
// ======================================================================================
// MXFP4 keys (OCP MX: 128 FP4 E2M1 elements in 64 bytes, element 2i in the low nibble of
// byte i, and one E8M0 scale per block of 32 elements): the decode kernel's stream with
// 64-byte rows, so one load instruction moves a 16-key tile and the ring holds 16 of them.
// Lane group g of the MFMA takes block g of its key row: its k-steps s = 0..3 are dims
// 32g + 8s .. +7 (the query's A operand uses the same dims), so each lane reads one 16-byte
// chunk per tile and applies one block scale, while widening E2M1 x scale to bf16 exactly
// (v_cvt_scalef32_pk_bf16_fp4: two elements per instruction). The wave's block scales
// (4 bytes per key) arrive in LDS by direct loads ahead of the tiles. 32 tiles per wave
// and an 8 KiB ring (8 tiles in flight) leave room for three work-groups per CU: 99 us on
// 128 queries at 64K keys, against 118 us with 16 tiles and a 16 KiB ring (two per CU).
#ifndef SA_MX_TPW
#define SA_MX_TPW 32
#endif
#ifndef SA_MX_RING
#define SA_MX_RING 8192
#endif
constexpr int kMxRB = kIdxDim / 2;                     // row bytes
constexpr int kMxTPW = SA_MX_TPW;                      // tiles per wave
constexpr int kMxRing = SA_MX_RING;                    // ring bytes per wave
constexpr int kMxD = kMxRing / (16 * kMxRB);           // tiles in flight per wave
constexpr int kMxKeysPerWG = kDWaves * kMxTPW * 16;
static_assert(kMxD <= kMxTPW && (kMxD & (kMxD - 1)) == 0 && kMxD <= 63, "ring depth");
static_assert(kMxTPW % 4 == 0, "64 keys per store");

struct MxShared {
  uint8_t ring[kDWaves][kMxRing];
  uint8_t scale[kDWaves][kMxTPW * 16 * 4];   // E8M0 scales of the wave's keys
  float stage[kDWaves][kMxTPW * 16];
  uint16_t q[kIdxHeads * kIdxDim];
  float w[kIdxHeads];
  int32_t ids[kDWaves * kMxTPW * 2];         // candidate mode: the work-group's block ids
};

// Position of chunk q (block q) of row r in LDS: rotated by r/4 so that the 16 rows' reads
// of one block hit 16 different bank groups.
__device__ __forceinline__ int mx_pos(int r, int q) { return q ^ ((r >> 2) & 3); }
__device__ __forceinline__ int kdim_mx(int g, int s) { return 32 * g + 8 * s; }


// MODE kPaged: keys and block scales are page pools (pages of 16+ rows, so a 16-key tile
// lies in one page); the wave's page ids, one per lane and tile, are read before its other
// loads. MODE kCand: candidate-bounded re-scoring as in the decode kernel; a tile is two
// slots (blocks of 8 rows), each load instruction reads both, and the block scales of each
// slot's rows are loaded once the ids are in.
template <int MODE>
__global__ __launch_bounds__(kDThreads) void indexer_mx_kernel(IndexerArgs a) {
  if (run_compress_rows(a)) return;
  constexpr int RB = kMxRB, TB = 16 * kMxRB, D = kMxD;
  constexpr bool CAND = MODE == kCand, PAGED = MODE == kPaged;
  static_assert(kMxTPW * 2 <= 64, "one page id or one slot per lane");
  static_assert(TB == 1024, "one load instruction per tile");
  __shared__ __attribute__((aligned(16))) MxShared sh;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int E = (int)a.E;
  const int chunk0 = blockIdx.x * kMxKeysPerWG;
  const int key0 = chunk0 + wave * kMxTPW * 16;
  const int n = query_n(a, t);
  const int ntiles = key0 < E ? min(kMxTPW, (E - key0 + 15) >> 4) : 0;
  const int chunk_live = CAND ? (n > 0 ? 1 : 0) : (chunk0 < n ? min(kDWaves * kMxTPW, (n - chunk0 + 15) >> 4) : 0);
  int live = CAND ? 0 : min(max(chunk_live - wave * kMxTPW, 0), kMxTPW);
  float* srow = a.scores + (int64_t)t * a.ld_scores;
  float* brow = a.block_max ? a.block_max + (int64_t)t * a.ld_block_max : nullptr;
  const int seq = a.seq_id[t];
  const int sq = n > 0 ? seq : 0;   // n > 0 implies a valid sequence
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) + (PAGED ? 0 : (int64_t)sq * a.keys_seq_stride);
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(a.scales) + (PAGED ? 0 : (int64_t)sq * a.scales_seq_stride);
  // paged: page id of the wave's tile `lane` (lanes past the last live tile take its page)
  int pgreg = 0;
  if constexpr (PAGED) {
    if (live > 0) pgreg = (int)page_of(a.pages, sq, min(key0 + 16 * min(lane, kMxTPW - 1), n - 1));
  }
  // store row of key x (x < n) of this wave
  auto krow = [&](int x) -> int64_t {
    if constexpr (PAGED) return pool_row(a.pages, __shfl(pgreg, (x - key0) >> 4), x);
    else return x;
  };

  const uint32_t lds_q = (uint32_t)(uintptr_t)&sh.q[0];
  const uint32_t lds_w = (uint32_t)(uintptr_t)&sh.w[0];
  if (chunk_live > 0) {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q_idx) + (int64_t)t * kIdxHeads * kIdxDim * 2;
    to_lds16(qb + 1024 * wave + 16 * lane, lds_q + 1024 * wave);
    if (wave == 0 && lane < kIdxHeads / 4) to_lds16(a.w + (int64_t)t * kIdxHeads + 4 * lane, lds_w);
    if (CAND && wave == 1) {   // the work-group's 256 block ids (1 KB)
      static_assert(kDWaves * kMxTPW * 2 == 256, "one 16-byte load per lane");
      to_lds16(a.cand + (int64_t)t * kCandBlocks + chunk0 / 8 + 4 * lane, (uint32_t)(uintptr_t)&sh.ids[0]);
    }
  }
  // candidate mode: block id of the wave's slot `lane` (slot 2i + h is half h of tile i). A
  // slot is valid when its block holds a visible position; the wave loads tiles up to its
  // last valid slot, and invalid slots among them read row n - 1 and are masked.
  constexpr int kSlots = 2 * kMxTPW;
  const int nbv = (n + 7) >> 3;
  auto valid_id = [&](int id) { return id >= 0 && id < nbv; };
  int idreg = -1;
  if constexpr (CAND) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("s_barrier" ::: "memory");
    if (chunk_live > 0) idreg = sh.ids[kSlots * wave + lane];
    const uint64_t vm = __ballot(valid_id(idreg));
    live = vm ? (64 - __builtin_clzll(vm) + 1) >> 1 : 0;
  }
  // row of entry e (0 .. 16 kMxTPW - 1) of the wave in candidate mode
  auto cand_row = [&](int id, int e) { return valid_id(id) ? min(8 * id + (e & 7), n - 1) : n - 1; };
  // the wave's block scales, one key (4 bytes) per lane and load (rows past n repeat row n-1)
  if constexpr (CAND) {
    if (live > 0) {
#pragma unroll
      for (int j = 0; j < kMxTPW / 4; ++j) {
        const int id = sh.ids[kSlots * wave + 8 * j + (lane >> 3)];
        to_lds4(scales + (int64_t)cand_row(id, lane) * 4, (uint32_t)(uintptr_t)&sh.scale[wave][256 * j]);
      }
    }
  } else if (live > 0) {
#pragma unroll
    for (int j = 0; j < kMxTPW / 4; ++j)
      to_lds4(scales + krow(min(key0 + 64 * j + lane, n - 1)) * 4,
              (uint32_t)(uintptr_t)&sh.scale[wave][256 * j]);
  }

  // load of a tile: lane -> row r = lane / 4, position p = lane % 4 holds chunk mx_pos(r, p)
  const int rr = lane >> 2, qq = mx_pos(rr, lane & 3);
  const uint32_t ring0 = (uint32_t)(uintptr_t)&sh.ring[wave][0];
  auto issue = [&](int i, bool after_reads) {
    const int k = key0 + 16 * i;
    // rows past n repeat row n-1 (same page: a tile never crosses one)
    int64_t row;
    if constexpr (CAND) {   // lanes 0-31 load slot 2i, lanes 32-63 slot 2i + 1 (uniform lane reads)
      const int id0 = __builtin_amdgcn_readlane(idreg, 2 * i), id1 = __builtin_amdgcn_readlane(idreg, 2 * i + 1);
      row = cand_row(rr >= 8 ? id1 : id0, rr);
    }
    else if constexpr (PAGED) row = pool_row(a.pages, __builtin_amdgcn_readlane(pgreg, i), k) + min(rr, n - 1 - k);
    else row = min(k + rr, n - 1);
    const uint8_t* src = keys + row * RB + qq * 16;
    const uint32_t lds = ring0 + (uint32_t)((i & (D - 1)) * TB);
    if (after_reads) to_lds16_after_reads(src, lds);
    else to_lds16(src, lds);
  };
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < live) issue(u, false);
  if (live >= D) __builtin_amdgcn_s_waitcnt(waitcnt_vm(D));   // query, weights, scales
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  asm volatile("s_barrier" ::: "memory");

  if (live > 0) {
    bf16x8 qa[4];
    float wq[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) qa[s2] = *reinterpret_cast<const bf16x8*>(&sh.q[c * kIdxDim + kdim_mx(g, s2)]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wq[i] = sh.w[4 * g + i];
    const uint32_t roff = (uint32_t)(c * RB + mx_pos(c, g) * 16);
    float* stage = sh.stage[wave];
    for (int i = 0; i < live; ++i) {
      if (i + D - 1 < live) __builtin_amdgcn_s_waitcnt(waitcnt_vm(D - 1));   // tile i landed
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      const uint8_t* tile = sh.ring[wave] + (i & (D - 1)) * TB;
      const u32x4 K = *reinterpret_cast<const u32x4*>(tile + roff);
      const float sc = e8m0_scale(sh.scale[wave][(16 * i + c) * 4 + g]);
      if (i + D < live) issue(i + D, true);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const u32x4 u = {
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 0)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 1)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 2)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 3))};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2], __builtin_bit_cast(bf16x8, u), acc, 0, 0, 0);
      }
      float v = wq[0] * relu(acc[0]);
      v = fmaf(wq[1], relu(acc[1]), v);
      v = fmaf(wq[2], relu(acc[2]), v);
      v = fmaf(wq[3], relu(acc[3]), v);
      v = add_xor32(add_xor16(v));
      if (lane < 16) stage[16 * i + lane] = v;
    }
  }

  // ---- scores and block maxima of the wave's keys: 64 consecutive keys per store ----
  const float* stage = sh.stage[wave];
#pragma unroll
  for (int j = 0; j < kMxTPW / 4; ++j) {
    const int k = key0 + 64 * j + lane;
    if (64 * j >= 16 * ntiles) break;
    bool ok = k < n;
    if constexpr (CAND) {
      const int id = chunk_live > 0 ? sh.ids[kSlots * wave + 8 * j + (lane >> 3)] : -1;
      ok = valid_id(id) && 8 * id + (lane & 7) < n;   // valid slots all lie in the loaded tiles
    }
    const float v = ok ? stage[64 * j + lane] : neg_inf();
    const float m = max8_lanes(v);
    if (k < E) {
      srow[k] = v;
      if (brow && (lane & 7) == 0) brow[k >> 3] = m;
    }
  }
}

// ======================================================================================
// Grouped decode
// ======================================================================================
// Up to G consecutive queries that read one sequence (a multi-token decode step: a
// verified token and the drafted tokens after it) share one key stream. Same LDS ring and
// direct loads as the decode kernel, with every query's 16 heads in registers, so each
// 16-key tile feeds 4G MFMAs. The arithmetic of each query (MFMA k order, ReLU and head
// weights in-lane, the 16-head sum as (row 0 + row 1) + (row 2 + row 3)) is the decode
// kernel's, so a query's scores are the same bits whichever kernel runs it. The head sums
// of four queries finish together: a row-swap add within each pair of queries, then a
// half-swap add that leaves query j's totals in row j, so one store instruction writes the
// tile's 16 keys of four queries. Scores stay in registers until the wave's tiles are done:
// no store may sit between the ring loads and their explicit vmcnt waits.
// Tiles per wave: 32 while the results fit the registers (fewer work-groups, so fewer
// query reloads and start-ups; 6 % faster than 16 at 6 queries), 16 for 8 queries.
template <int G>
constexpr int group_tpw() { return G <= 6 ? 32 : 16; }
template <int G>
constexpr int group_keys_per_wg() { return kDWaves * group_tpw<G>() * 16; }

// PAGED: keys and e4m3 scales are page pools (pages of 16+ rows); each wave reads the page
// ids of its tiles (one per lane) ahead of its other loads.
template <bool FP8, int G, bool PAGED>
__global__ __launch_bounds__(kDThreads, 2) void indexer_group_kernel(IndexerArgs a) {
  if (run_compress_rows(a)) return;
  using DT = DecodeTile<FP8>;
  constexpr int RB = DT::RB, TB = DT::TB, NK = DT::NK, D = DT::D;
  constexpr int TPW = group_tpw<G>();
  constexpr int N4 = G / 4, N2 = (G % 4) / 2;   // four-query chunks, then one pair
  static_assert(G >= 2 && G <= 8 && G % 2 == 0, "groups of 2, 4, 6 or 8 queries");
  static_assert((D & (D - 1)) == 0 && D >= 2 && D <= TPW, "ring depth");
  static_assert(D * NK <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kDWaves][kRingBytes];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int E = (int)a.E, T = (int)a.T;
  const int t0 = blockIdx.y * a.group;
  const int gs = min(a.group, T - t0);   // queries of this group (a.group <= G)
  const int key0 = blockIdx.x * group_keys_per_wg<G>() + wave * TPW * 16;   // the wave's keys
  const int seq = a.seq_id[t0];

  // visible count of the group's j-th query; 0 past the group or for another sequence
  auto n_of = [&](int j) { return j < gs && a.seq_id[t0 + j] == seq ? query_n(a, t0 + j) : 0; };
  int nmax = 0;
  for (int j = 0; j < gs; ++j) nmax = max(nmax, n_of(j));
  const int ntiles = key0 < E ? min(TPW, (E - key0 + 15) >> 4) : 0;
  const int live = key0 < nmax ? min(TPW, (nmax - key0 + 15) >> 4) : 0;
  const int sq = nmax > 0 ? seq : 0;   // nmax > 0 implies a valid sequence
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) +
                        (PAGED ? 0 : (int64_t)sq * a.keys_seq_stride * (FP8 ? 1 : 2));
  // paged: page id of the wave's tile `lane` (lanes past the last live tile take its page)
  int pgreg = 0;
  if constexpr (PAGED) {
    static_assert(TPW <= 64, "one tile per lane");
    if (live > 0)
      pgreg = (int)page_of(a.pages, sq, min(key0 + 16 * min(lane, TPW - 1), nmax - 1));
  }

  int rr[NK], qq[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int r = j * (64 / DT::CPR) + lane / DT::CPR;
    rr[j] = r;
    qq[j] = DT::pos(r, lane % DT::CPR);
  }
  const uint32_t ring0 = (uint32_t)(uintptr_t)&ring[wave][0];
  auto issue = [&](int i, bool after_reads) {
    const int k = key0 + 16 * i;
    const uint8_t* tb = keys + (PAGED ? pool_row(a.pages, __builtin_amdgcn_readlane(pgreg, i), k) : (int64_t)k) * RB;
    const int last = nmax - 1 - k;   // rows past the group's last key repeat that row
    const uint32_t lds = ring0 + (uint32_t)((i & (D - 1)) * TB);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const uint8_t* src = tb + (min(rr[j], last) * RB + qq[j] * 16);
      if (j == 0 && after_reads) to_lds16_after_reads(src, lds + 1024 * j);
      else to_lds16(src, lds + 1024 * j);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < live) issue(u, false);

  // Head weights, e4m3 row scales (4 consecutive keys per lane per 256) and the A operands,
  // after the first D tiles' loads (their latencies overlap); waiting for them (settle)
  // then also covers those tiles, as loads complete in order.
  float wq[G][4];
  float sv[TPW / 16][4] = {};
  bf16x8 qa[G][4];
  if (live > 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int tq = t0 + min(j, gs - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[j][i] = a.w[(int64_t)tq * kIdxHeads + 4 * g + i];
    }
    if constexpr (FP8) {
      const float* scales = a.scales + (PAGED ? 0 : (int64_t)sq * a.scales_seq_stride);
#pragma unroll
      for (int k2 = 0; k2 < TPW / 16; ++k2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = min(key0 + 256 * k2 + 4 * lane + e, nmax - 1);
          if constexpr (PAGED) sv[k2][e] = scales[pool_row(a.pages, __shfl(pgreg, (x - key0) >> 4), x)];
          else sv[k2][e] = scales[x];
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int tq = t0 + min(j, gs - 1);
      const uint16_t* row = reinterpret_cast<const uint16_t*>(a.q_idx) + ((int64_t)tq * kIdxHeads + c) * kIdxDim;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        qa[j][s2] = *reinterpret_cast<const bf16x8*>(row + (FP8 ? kdim_fp8(g, s2) : kdim_bf16(g, s2)));
    }
  }

#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      settle(wq[j][i]);
      settle(qa[j][i]);
    }
  }
#pragma unroll
  for (int k2 = 0; k2 < TPW / 16; ++k2)
#pragma unroll
    for (int e = 0; e < 4; ++e) settle(sv[k2][e]);

  uint32_t roff[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int q = FP8 ? g + 4 * i : 4 * i + g;
    roff[i] = (uint32_t)(c * RB + DT::pos(c, q) * 16);
  }
  float r4[TPW][N4 > 0 ? N4 : 1];   // tile i, chunk h: query 4h + g's score of key c
  float r2[TPW];                    // tile i, pair: query 4 N4 + (g & 1)'s score of key c
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (i < live) {
      if (i + D - 1 < live) __builtin_amdgcn_s_waitcnt(waitcnt_vm((D - 1) * NK));   // tile i landed
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      const uint8_t* tile = ring[wave] + (i & (D - 1)) * TB;
      KeyRegs<FP8> K;
#pragma unroll
      for (int j = 0; j < NK; ++j) K.v[j] = *reinterpret_cast<const u32x4*>(tile + roff[j]);
      if (i + D < live) issue(i + D, true);
      bf16x8 b[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        if constexpr (FP8) b[s2] = e4m3x8_to_bf16x8(K.v[s2 >> 1][2 * (s2 & 1)], K.v[s2 >> 1][2 * (s2 & 1) + 1]);
        else b[s2] = __builtin_bit_cast(bf16x8, K.v[s2]);
      }
      float p[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j][s2], b[s2], acc, 0, 0, 0);
        float v = wq[j][0] * relu(acc[0]);
        v = fmaf(wq[j][1], relu(acc[1]), v);
        v = fmaf(wq[j][2], relu(acc[2]), v);
        p[j] = fmaf(wq[j][3], relu(acc[3]), v);
      }
      // row-swap adds: rows (0+1) and (2+3) of two queries side by side
      auto sw16 = [](float x, float y) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
      };
#pragma unroll
      for (int h = 0; h < N4; ++h) {
        const float ab = sw16(p[4 * h], p[4 * h + 1]);       // rows: a01 b01 a23 b23
        const float cd = sw16(p[4 * h + 2], p[4 * h + 3]);   // rows: c01 d01 c23 d23
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ab), __float_as_uint(cd), false, false);
        r4[i][h] = __uint_as_float(r[0]) + __uint_as_float(r[1]);   // row j: query 4h + j
      }
      if constexpr (N2 > 0) r2[i] = add_xor32(sw16(p[4 * N4], p[4 * N4 + 1]));   // rows 0, 2: e; 1, 3: f
    }
  }

  // ---- scores and block maxima: per tile, 16 keys of four queries per store ----
  float* sc_l = reinterpret_cast<float*>(&ring[wave][0]);   // the ring is idle now
  if constexpr (FP8) {
    if (live > 0) {
#pragma unroll
      for (int k2 = 0; k2 < TPW / 16; ++k2)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc_l[256 * k2 + 4 * lane + e] = sv[k2][e];
    }
  }
  int jq4[N4 > 0 ? N4 : 1], nl4[N4 > 0 ? N4 : 1];
#pragma unroll
  for (int h = 0; h < N4; ++h) {
    jq4[h] = 4 * h + g;
    nl4[h] = n_of(jq4[h]);
  }
  const int jq2 = 4 * N4 + (g & 1);
  const int nl2 = N2 > 0 ? n_of(jq2) : 0;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (i >= ntiles) break;
    const int k = key0 + 16 * i + c;
    const float sc = FP8 && i < live ? sc_l[16 * i + c] : 1.f;
    auto put = [&](float v, int jq, bool mine) {
      const float m = max8_lanes(v);   // E is a multiple of 8: groups are all in or all out
      if (mine && jq < gs && k < E) {
        const int64_t tq = t0 + jq;
        a.scores[tq * a.ld_scores + k] = v;
        if (a.block_max && (c & 7) == 0) a.block_max[tq * a.ld_block_max + (k >> 3)] = m;
      }
    };
#pragma unroll
    for (int h = 0; h < N4; ++h) {
      float v = neg_inf();
      if (i < live && k < nl4[h]) {
        v = r4[i][h];
        if constexpr (FP8) v *= sc;
      }
      put(v, jq4[h], true);
    }
    if constexpr (N2 > 0) {
      float v = neg_inf();
      if (i < live && k < nl2) {
        v = r2[i];
        if constexpr (FP8) v *= sc;
      }
      put(v, jq2, g < 2);
    }
  }
}

// Grouped decode with MXFP4 keys: the grouped kernel's key stream, head sums and stores
// with the MXFP4 kernel's tiles. A 16-key tile is one 1 KB load (64-byte rows); lane (c, g)
// takes 32-dim block g of key c (its chunk at mx_pos(c, g)) and widens it with that key's
// E8M0 block scale into the four B operands, so each query's arithmetic is the MXFP4
// kernel's and its scores are the same bits. The block scales of the wave's keys arrive in
// LDS by direct loads ahead of the A operands.
constexpr int kGMxD = 8;   // MXFP4 tiles in flight per wave
template <int G>
struct GroupMxShared {
  uint8_t ring[kDWaves][kGMxD * 16 * kMxRB];
  uint8_t scale[kDWaves][group_tpw<G>() * 16 * 4];
};

template <int G, bool PAGED>
__global__ __launch_bounds__(kDThreads, 2) void indexer_group_mx_kernel(IndexerArgs a) {
  if (run_compress_rows(a)) return;
  constexpr int RB = kMxRB, TB = 16 * kMxRB, D = kGMxD;
  constexpr int TPW = group_tpw<G>();
  constexpr int N4 = G / 4, N2 = (G % 4) / 2;
  static_assert(TB == 1024, "one load instruction per tile");
  static_assert(G >= 2 && G <= 8 && G % 2 == 0, "groups of 2, 4, 6 or 8 queries");
  static_assert((D & (D - 1)) == 0 && D <= TPW && D <= 63, "ring depth");
  static_assert(TPW % 4 == 0, "64 scales per load");
  __shared__ __attribute__((aligned(16))) GroupMxShared<G> sh;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int E = (int)a.E, T = (int)a.T;
  const int t0 = blockIdx.y * a.group;
  const int gs = min(a.group, T - t0);
  const int key0 = blockIdx.x * group_keys_per_wg<G>() + wave * TPW * 16;
  const int seq = a.seq_id[t0];
  auto n_of = [&](int j) { return j < gs && a.seq_id[t0 + j] == seq ? query_n(a, t0 + j) : 0; };
  int nmax = 0;
  for (int j = 0; j < gs; ++j) nmax = max(nmax, n_of(j));
  const int ntiles = key0 < E ? min(TPW, (E - key0 + 15) >> 4) : 0;
  const int live = key0 < nmax ? min(TPW, (nmax - key0 + 15) >> 4) : 0;
  const int sq = nmax > 0 ? seq : 0;
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) + (PAGED ? 0 : (int64_t)sq * a.keys_seq_stride);
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(a.scales) + (PAGED ? 0 : (int64_t)sq * a.scales_seq_stride);
  // paged: page id of the wave's tile `lane` (lanes past the last live tile take its page),
  // read before every other load
  int pgreg = 0;
  if constexpr (PAGED) {
    static_assert(TPW <= 64, "one page id per lane");
    if (live > 0) pgreg = (int)page_of(a.pages, sq, min(key0 + 16 * min(lane, TPW - 1), nmax - 1));
  }
  auto krow = [&](int x) -> int64_t {
    if constexpr (PAGED) return pool_row(a.pages, __shfl(pgreg, (x - key0) >> 4), x);
    else return x;
  };

  // the wave's block scales (direct loads, one key's 4 bytes per lane), then the first D
  // tiles, then the head weights and the A operands; waiting for those (settle) covers
  // everything before them, as loads complete in order
  if (live > 0) {
#pragma unroll
    for (int j = 0; j < TPW / 4; ++j)
      to_lds4(scales + krow(min(key0 + 64 * j + lane, nmax - 1)) * 4,
              (uint32_t)(uintptr_t)&sh.scale[wave][256 * j]);
  }
  // tile load: lane -> row lane / 4, position lane % 4 holds chunk mx_pos(row, position)
  const int rr = lane >> 2, qq = mx_pos(rr, lane & 3);
  const uint32_t ring0 = (uint32_t)(uintptr_t)&sh.ring[wave][0];
  auto issue = [&](int i, bool after_reads) {
    const int k = key0 + 16 * i;
    // rows past nmax repeat row nmax-1 (same page: a tile never crosses one)
    int64_t row;
    if constexpr (PAGED) row = pool_row(a.pages, __builtin_amdgcn_readlane(pgreg, i), k) + min(rr, nmax - 1 - k);
    else row = min(k + rr, nmax - 1);
    const uint8_t* src = keys + row * RB + qq * 16;
    const uint32_t lds = ring0 + (uint32_t)((i & (D - 1)) * TB);
    if (after_reads) to_lds16_after_reads(src, lds);
    else to_lds16(src, lds);
  };
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < live) issue(u, false);

  float wq[G][4];
  bf16x8 qa[G][4];
  if (live > 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int tq = t0 + min(j, gs - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[j][i] = a.w[(int64_t)tq * kIdxHeads + 4 * g + i];
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int tq = t0 + min(j, gs - 1);
      const uint16_t* row = reinterpret_cast<const uint16_t*>(a.q_idx) + ((int64_t)tq * kIdxHeads + c) * kIdxDim;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) qa[j][s2] = *reinterpret_cast<const bf16x8*>(row + kdim_mx(g, s2));
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      settle(wq[j][i]);
      settle(qa[j][i]);
    }
  }

  const uint32_t roff = (uint32_t)(c * RB + mx_pos(c, g) * 16);
  float r4[TPW][N4 > 0 ? N4 : 1];
  float r2[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (i < live) {
      if (i + D - 1 < live) __builtin_amdgcn_s_waitcnt(waitcnt_vm(D - 1));   // tile i landed
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      const uint8_t* tile = sh.ring[wave] + (i & (D - 1)) * TB;
      const u32x4 K = *reinterpret_cast<const u32x4*>(tile + roff);
      const float sc = e8m0_scale(sh.scale[wave][(16 * i + c) * 4 + g]);
      if (i + D < live) issue(i + D, true);
      bf16x8 b[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const u32x4 u = {
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 0)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 1)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 2)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(K[s2], sc, 3))};
        b[s2] = __builtin_bit_cast(bf16x8, u);
      }
      float p[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j][s2], b[s2], acc, 0, 0, 0);
        float v = wq[j][0] * relu(acc[0]);
        v = fmaf(wq[j][1], relu(acc[1]), v);
        v = fmaf(wq[j][2], relu(acc[2]), v);
        p[j] = fmaf(wq[j][3], relu(acc[3]), v);
      }
      auto sw16 = [](float x, float y) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
      };
#pragma unroll
      for (int h = 0; h < N4; ++h) {
        const float ab = sw16(p[4 * h], p[4 * h + 1]);
        const float cd = sw16(p[4 * h + 2], p[4 * h + 3]);
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ab), __float_as_uint(cd), false, false);
        r4[i][h] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
      if constexpr (N2 > 0) r2[i] = add_xor32(sw16(p[4 * N4], p[4 * N4 + 1]));
    }
  }

  // ---- scores and block maxima: per tile, 16 keys of four queries per store ----
  int jq4[N4 > 0 ? N4 : 1], nl4[N4 > 0 ? N4 : 1];
#pragma unroll
  for (int h = 0; h < N4; ++h) {
    jq4[h] = 4 * h + g;
    nl4[h] = n_of(jq4[h]);
  }
  const int jq2 = 4 * N4 + (g & 1);
  const int nl2 = N2 > 0 ? n_of(jq2) : 0;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (i >= ntiles) break;
    const int k = key0 + 16 * i + c;
    auto put = [&](float v, int jq, bool mine) {
      const float m = max8_lanes(v);
      if (mine && jq < gs && k < E) {
        const int64_t tq = t0 + jq;
        a.scores[tq * a.ld_scores + k] = v;
        if (a.block_max && (c & 7) == 0) a.block_max[tq * a.ld_block_max + (k >> 3)] = m;
      }
    };
#pragma unroll
    for (int h = 0; h < N4; ++h) put(i < live && k < nl4[h] ? r4[i][h] : neg_inf(), jq4[h], true);
    if constexpr (N2 > 0) put(i < live && k < nl2 ? r2[i] : neg_inf(), jq2, g < 2);
  }
}

// ======================================================================================
// Prefill
// ======================================================================================
#ifndef SA_P_WAVES
#define SA_P_WAVES 4
#endif
#ifndef SA_P_CHUNK
#define SA_P_CHUNK 4096
#endif
constexpr int kPWaves = SA_P_WAVES;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPairsPerWave = 2;
constexpr int kQPerWG = kPWaves * kPairsPerWave * 2;   // 16 queries
static_assert(kQPerWG == kChunkQueriesPerWG, "the host sizes the chunk grid with this");
constexpr int kPKT = 32;                                // keys per tile
constexpr int kPChunk = SA_P_CHUNK;                     // keys per work-group (4096: 3 % faster than 2048)
constexpr int kPST = 2 * kPKT;                          // keys per LDS stage (two tiles)
constexpr int kPBufs = 3;

// LDS key tile: 32 keys as bf16 rows (e4m3 keys are widened once, while staging), padded
// to 272 bytes so the B-operand reads of 32 rows are bank-conflict free.
constexpr int kPRS = 2 * kIdxDim + 16;
struct PrefillShared {
  uint8_t tile[kPBufs][kPST * kPRS];
  float scale[kPBufs][kPST];
};

// Dims of k-step s (0..7) for lane half hh: (2s + hh) * 8 .. +8 (32x32x16 operands).
__device__ __forceinline__ int pdim(int hh, int s) { return (2 * s + hh) * 8; }

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, 32-bit data (gfx9 family)
constexpr uint32_t kDrop = 0x80000000u;  // buffer offset past every extent: store dropped

// KF: key format, 0 bf16, 1 e4m3 (row scale applied to the score), 2 MXFP4 (each 16-byte
// chunk of a 64-byte row is one 32-element block: widened with its E8M0 scale while
// staging, so the tile holds exact bf16 values). PAGED: keys and scales (e4m3 or MXFP4) are
// page pools of at least kPST rows per page, so each stage of 64 keys lies in one page; the
// chunk's page ids (at most 64) are read once, one per lane.
template <int KF, bool PAGED>
__global__ __launch_bounds__(kPThreads, 8 / kPWaves) void indexer_prefill_kernel(IndexerArgs a) {
  if (run_compress_rows(a)) return;
  constexpr bool FP8 = KF == 1, MX = KF == 2;
  constexpr int RB = MX ? kIdxDim / 2 : (FP8 ? kIdxDim : 2 * kIdxDim);   // key row bytes in HBM
  __shared__ __attribute__((aligned(16))) PrefillShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r32 = lane & 31, hh = lane >> 5;
  const int E = (int)a.E;
  const int k0 = blockIdx.x * kPChunk;
  const int q0 = blockIdx.y * kQPerWG;
  if (k0 >= E) return;
  const int kend = min(k0 + kPChunk, E);
  const int T = (int)a.T;

  // queries of this wave: q0 + 4*wave + j, j = 0..3 (pair p = j/2); the WG's queries must
  // read one sequence (queries of another sequence, or invalid ones, get n = 0).
  const int seq = a.seq_id[q0];
  auto n_of = [&](int tq) { return tq < T && a.seq_id[tq] == seq ? query_n(a, tq) : 0; };
  int nmax_wg = 0;
  for (int j = 0; j < kQPerWG; ++j) nmax_wg = max(nmax_wg, n_of(q0 + j));
  const int klive = min(kend, nmax_wg);   // keys past every query's n are masked
  // tiles covering [k0, klive), rounded up to an even count (steps run in pairs); keys of
  // the extra tile are past klive, so they come out masked like the rest
  const int nsteps = klive > k0 ? ((klive - k0 + 2 * kPKT - 1) / (2 * kPKT)) * 2 : 0;

  // part of the chunk past the steps' tiles, for every valid query of the wave
  for (int j = 0; j < 4; ++j) {
    const int tq = q0 + 4 * wave + j;
    if (tq >= T) break;
    float* srow = a.scores + (int64_t)tq * a.ld_scores;
    float* brow = a.block_max ? a.block_max + (int64_t)tq * a.ld_block_max : nullptr;
    for (int k = k0 + nsteps * kPKT + lane; k < kend; k += 64) srow[k] = neg_inf();
    if (brow)
      for (int b = (k0 + nsteps * kPKT) / 8 + lane; b < kend / 8; b += 64) brow[b] = neg_inf();
  }
  if (nsteps == 0) return;

  // A operands and head weights of the wave's two query pairs. Row r of a pair's A operand
  // is head 4 (r / 8) + r % 4 of the pair's query (r / 4) % 2, so that in the 32x32 result
  // (lane (r32, hh) holds rows 8 (i / 4) + 4 hh + i % 4, i = 0..15) a lane's 16 values are
  // heads 0..15 of query hh of the pair for key r32, and each lane finishes its head sum.
  bf16x8 qa[kPairsPerWave][8];
  float wt[kPairsPerWave][16];
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p) {
    const int jq = 2 * p + ((r32 >> 2) & 1);
    const int head = 4 * (r32 >> 3) + (r32 & 3);
    const int tq = min(q0 + 4 * wave + jq, T - 1);
    const uint16_t* row = reinterpret_cast<const uint16_t*>(a.q_idx) + ((int64_t)tq * kIdxHeads + head) * kIdxDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[p][s] = *reinterpret_cast<const bf16x8*>(row + pdim(hh, s));
    const int tw = min(q0 + 4 * wave + 2 * p + hh, T - 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) wt[p][i] = a.w[(int64_t)tw * kIdxHeads + i];
  }

  // Outputs. After the head sum of pair p, lanes 0-31 hold query 2p's score of key r32 and
  // lanes 32-63 query 2p+1's. Each pair stores through buffer resources based at its first
  // query's rows, covering the pair's valid rows; a lane whose entry is not to be written
  // gets offset kDrop, which the hardware discards, so the epilogue needs no branches.
  __amdgpu_buffer_rsrc_t srs[kPairsPerWave], brs[kPairsPerWave];
  int nl[kPairsPerWave];
  const uint32_t soff_hh = (uint32_t)hh * (uint32_t)a.ld_scores * 4u;
  const uint32_t boff_hh = (uint32_t)hh * (uint32_t)a.ld_block_max * 4u;
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p) {
    const int tp = q0 + 4 * wave + 2 * p;
    const int rows = tp + 1 < T ? 2 : (tp < T ? 1 : 0);
    const int tpc = min(tp, T - 1);
    srs[p] = __builtin_amdgcn_make_buffer_rsrc(a.scores + (int64_t)tpc * a.ld_scores, (short)0,
                                               rows * (int)a.ld_scores * 4, kRsrcWord3);
    brs[p] = __builtin_amdgcn_make_buffer_rsrc(a.block_max ? a.block_max + (int64_t)tpc * a.ld_block_max : a.scores,
                                               (short)0, a.block_max ? rows * (int)a.ld_block_max * 4 : 0,
                                               kRsrcWord3);
    nl[p] = n_of(tp + hh);
  }

  // Keys and scales through buffer resources over rows [k0, klive) of the sequence: loads
  // past klive read zeros (their scores are masked), so the loads need no clamping. The
  // whole offset goes in the VGPR operand, which the range check covers.
  const int sq = (seq >= 0 && seq < a.num_seqs) ? seq : 0;
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) +
                        (int64_t)sq * a.keys_seq_stride * (KF == 0 ? 2 : 1) + (int64_t)k0 * RB;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(keys), (short)0, (klive - k0) * RB, kRsrcWord3);
  // scales: e4m3 fp32 per row; MXFP4 4 E8M0 bytes per row (one dword per row)
  const int64_t soff = MX ? (int64_t)sq * a.scales_seq_stride + (int64_t)k0 * 4   // bytes (stride in bytes)
                          : ((int64_t)sq * a.scales_seq_stride + k0) * 4;          // bytes (stride in floats)
  const float* scales = (FP8 || MX) ? reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.scales) + soff)
                                    : a.w;
  const __amdgpu_buffer_rsrc_t scrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scales), (short)0, (FP8 || MX) ? (klive - k0) * 4 : 0, kRsrcWord3);
  // paged: page id of table entry (k0 >> lp) + lane (entries past the live keys repeat the last)
  int pgl = 0;
  if constexpr (PAGED) {
    static_assert(kPChunk / kPST <= 64, "one page id per lane");
    const int lp = a.pages.log2_page;
    const int e = min((k0 >> lp) + lane, (klive - 1) >> lp);
    pgl = (int)min(max((int64_t)a.pages.table[(int64_t)sq * a.pages.stride + e], (int64_t)0), a.pages.num_pages - 1);
  }
  // buffer resources of stage S: the chunk's (contiguous) or the stage's page (paged); rows
  // past klive are outside the resource and read zeros
  auto stage_rsrc = [&](int S, __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& sr, uint32_t& skoff, uint32_t& ssoff) {
    if constexpr (PAGED) {
      const int lp = a.pages.log2_page;
      const int ks = k0 + S * kPST;
      const int rows = max(0, min(kPST, klive - ks));
      const int64_t pg = __builtin_amdgcn_readlane(pgl, min((ks >> lp) - (k0 >> lp), 63));
      const int64_t row0 = (pg << lp) + (ks & ((1 << lp) - 1));
      kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.keys) + row0 * RB),
                                             (short)0, rows * RB, kRsrcWord3);
      // one dword per row: the fp32 scale (e4m3) or the 4 E8M0 bytes (MXFP4)
      sr = __builtin_amdgcn_make_buffer_rsrc(
          (FP8 || MX) ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.scales) + row0 * 4)
                      : reinterpret_cast<uint8_t*>(const_cast<float*>(a.w)),
          (short)0, (FP8 || MX) ? rows * 4 : 0, kRsrcWord3);
      skoff = 0;
      ssoff = 0;
    } else {
      kr = krs;
      sr = scrs;
      skoff = (uint32_t)(S * kPST * RB);
      ssoff = (uint32_t)(S * kPST * 4);
    }
  };

  // staging, one stage (64 keys) at a time: 16-byte chunk q = tid + kPThreads*h of a stage
  // (h < CPT) is row q / CPR, chunk q % CPR: each wave loads whole rows (contiguous 1 KiB
  // per instruction) and each group of CPR lanes writes one padded LDS row contiguously
  // (e4m3 chunks are widened to 32 bytes of bf16 on the way).
  constexpr int CPR = RB / 16;                          // chunks per row: 16 (bf16) or 8 (e4m3)
  constexpr int CPT = kPST * CPR / kPThreads;           // chunks per thread: 4 or 2
  uint32_t kvoff[CPT], ldsoff[CPT];
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    const int q = tid + kPThreads * h;
    kvoff[h] = (uint32_t)((q / CPR) * RB + (q % CPR) * 16);
    ldsoff[h] = (uint32_t)((q / CPR) * kPRS + (q % CPR) * (MX ? 64 : FP8 ? 32 : 16));
  }
  // e4m3: thread t < 64 loads row t's scale; MXFP4: every thread the scale dword of its
  // chunk's row (its block's byte picked at commit)
  static_assert(!MX || CPT == 1, "one MXFP4 chunk per thread");
  const uint32_t scoff = MX ? (uint32_t)(tid / CPR) * 4u : (tid < kPST ? (uint32_t)tid * 4u : kDrop);
  struct Stage {
    u32x4 v[CPT];
    float scale;
  };
  auto fetch = [&](Stage& st, int S) {
    __amdgpu_buffer_rsrc_t kr, sr;
    uint32_t skoff, ssoff;
    stage_rsrc(S, kr, sr, skoff, ssoff);
#pragma unroll
    for (int h = 0; h < CPT; ++h)
      st.v[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, kvoff[h] + skoff, 0, 0));
    if (FP8 || MX) st.scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, scoff + ssoff, 0, 0));
  };
  auto commit = [&](const Stage& st, int buf) {
#pragma unroll
    for (int h = 0; h < CPT; ++h) {
      uint8_t* dst = &sh.tile[buf][ldsoff[h]];
      if constexpr (MX) {
        // 32 E2M1 elements of block (tid % 4) times its scale: 64 bytes of bf16
        const float bs = e8m0_scale((__float_as_uint(st.scale) >> (8 * (tid % CPR))) & 0xFFu);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 u = {
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(st.v[h][c], bs, 0)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(st.v[h][c], bs, 1)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(st.v[h][c], bs, 2)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(st.v[h][c], bs, 3))};
          *reinterpret_cast<u32x4*>(dst + 16 * c) = u;
        }
      } else if constexpr (FP8) {
        uint32_t u[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) e4m3x4_to_bf16x4(st.v[h][c], u[2 * c], u[2 * c + 1]);
        *reinterpret_cast<u32x4*>(dst) = u32x4{u[0], u[1], u[2], u[3]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{u[4], u[5], u[6], u[7]};
      } else {
        *reinterpret_cast<u32x4*>(dst) = st.v[h];
      }
    }
    if (FP8 && tid < kPST) sh.scale[buf][tid] = st.scale;
  };
  // B operands of tile i (stage i/2, half i%2): lane (r32, hh) reads key row r32, dims pdim(hh, s).
  auto load_b = [&](bf16x8 (&b)[8], float& sc, int i) {
    const int buf = (i >> 1) % kPBufs, row = (i & 1) * kPKT + r32;
    const uint8_t* T8 = sh.tile[buf] + row * kPRS;
#pragma unroll
    for (int s = 0; s < 8; ++s) b[s] = *reinterpret_cast<const bf16x8*>(T8 + 2 * pdim(hh, s));
    sc = FP8 ? sh.scale[buf][row] : 1.f;
  };

  // Epilogue of pair p for the tile at key k: ReLU and head weights in-lane over the lane's
  // 16 heads (heads in order), key scale, mask past the query's n, block max over 8 lanes,
  // two stores.
  // The tile's key offset goes in the stores' scalar offset; the lane-dependent parts
  // (row, key within the tile, the lanes that store block maxima) are fixed, and the
  // masks compare the tile's first key with per-lane limits computed once.
  const uint32_t sbase = soff_hh + (uint32_t)r32 * 4u;
  const uint32_t bbase = (lane & 7) == 0 ? boff_hh + (uint32_t)(r32 >> 3) * 4u : kDrop;
  const int kend_l = kend - r32;   // key k of lane r32 is this chunk's while k < kend_l
  int nvis_l[kPairsPerWave];       // ... and visible to the lane's query while k < nvis_l
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p) nvis_l[p] = nl[p] - r32;
  auto epilogue = [&](int p, const f32x16& acc, int k, float sc) {
    float v = wt[p][0] * relu(acc[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) v = fmaf(wt[p][i], relu(acc[i]), v);
    if (FP8) v *= sc;
    v = k < nvis_l[p] ? v : neg_inf();
    const float m = max8_lanes(v);
    const bool in = k < kend_l;                // keys of later chunks belong to other WGs
    // a dropped store's vector offset alone is past every extent
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), srs[p], in ? sbase : kDrop, k * 4, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), brs[p], in ? bbase : kDrop, (k >> 3) * 4, 0);
  };

  // One tile: B operands of the next tile are read from LDS while this one's MFMAs run.
  // Pair 1's epilogue of tile i-1 runs in step i (in step 0 on zeros, every store dropped).
  // After every second step (one stage) the next stages move up; staging, loads and barriers
  // are unconditional (past the last stage, loads read zeros and commits fill buffers
  // nobody reads), so the compiler's wait counts stay exact.
  // Issue order, fixed with scheduling barriers: pair 0's MFMA chain with pair 1's previous
  // epilogue, then pair 1's chain with pair 0's epilogue, each MFMA followed by a few VALU
  // ops so one wave keeps the matrix core and the VALU busy together.
  Stage st;
  f32x16 acc0, acc1 = {};
  int kprev = E;
  float scprev = 1.f;
  auto step = [&](int i, const bf16x8 (&bc)[8], float sc, bf16x8 (&bn)[8], float& scn, bool stage_end) {
    const int k = k0 + i * kPKT;
    load_b(bn, scn, i + 1);   // stale past the last tile, never used then
    __builtin_amdgcn_sched_barrier(0);
    acc0 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], bc[s], acc0, 0, 0, 0);
    epilogue(1, acc1, kprev, scprev);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    acc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], bc[s], acc1, 0, 0, 0);
    epilogue(0, acc0, k, sc);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    kprev = k;
    scprev = sc;
    if (stage_end) {
      // end of stage S = i/2: stage S+2 goes to buffer (S+2)%3, which held stage S-1, last
      // read in stage S-1 (before the previous barrier); stage S+3 starts loading
      const int S = i >> 1;
      commit(st, (S + 2) % kPBufs);
      fetch(st, S + 3);
      __syncthreads();
    }
  };

  fetch(st, 0);
  commit(st, 0);
  fetch(st, 1);
  commit(st, 1);
  // Nothing loaded so far is still in flight past here, so the waits the compiler places
  // inside the loop only cover the loop's own loads.
  __builtin_amdgcn_s_waitcnt(0);
  fetch(st, 2);
  __syncthreads();

  bf16x8 b0[8], b1[8];
  float sc0, sc1;
  load_b(b0, sc0, 0);
  for (int i = 0; i < nsteps; i += 2) {
    step(i, b0, sc0, b1, sc1, false);
    step(i + 1, b1, sc1, b0, sc0, true);
  }
  epilogue(1, acc1, kprev, scprev);
}

static_assert(kDThreads == kCThreads && kPThreads == kCThreads, "compressor jobs need 256-thread work-groups");

// The grid of an indexer launch with the compressor job's rows appended (b.cj_row0 set).
dim3 with_job_rows(dim3 g, IndexerArgs& b) {
  if (b.cj.G > 0) {
    b.cj_row0 = (int32_t)g.y;
    g.y += (unsigned)((compress_blocks_wanted(b.cj) + g.x - 1) / g.x);
  }
  return g;
}

template <int G>
void launch_group(IndexerArgs& b, hipStream_t stream) {
  constexpr int KW = group_keys_per_wg<G>();
  const dim3 grid = with_job_rows(dim3((unsigned)((b.E + KW - 1) / KW), (unsigned)((b.T + b.group - 1) / b.group)), b);
  if (b.mxfp4) {
    if (b.pages.table)
      hipLaunchKernelGGL((indexer_group_mx_kernel<G, true>), grid, dim3(kDThreads), 0, stream, b);
    else
      hipLaunchKernelGGL((indexer_group_mx_kernel<G, false>), grid, dim3(kDThreads), 0, stream, b);
    return;
  }
  if (b.pages.table) {
    if (b.fp8)
      hipLaunchKernelGGL((indexer_group_kernel<true, G, true>), grid, dim3(kDThreads), 0, stream, b);
    else
      hipLaunchKernelGGL((indexer_group_kernel<false, G, true>), grid, dim3(kDThreads), 0, stream, b);
  } else if (b.fp8) {
    hipLaunchKernelGGL((indexer_group_kernel<true, G, false>), grid, dim3(kDThreads), 0, stream, b);
  } else {
    hipLaunchKernelGGL((indexer_group_kernel<false, G, false>), grid, dim3(kDThreads), 0, stream, b);
  }
}

// Grid rows (y) the launch puts the queries in, before any job rows (the dispatch below).
unsigned query_rows(const IndexerArgs& a, bool prefill) {
  if (a.mxfp4 && !prefill && a.group <= 1) return (unsigned)a.T;
  if (a.group > 1 && !a.cand) return (unsigned)((a.T + a.group - 1) / a.group);
  if (!prefill) return (unsigned)a.T;
  return (unsigned)((a.T + kQPerWG - 1) / kQPerWG);
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool prefill, hipStream_t stream) {
  IndexerArgs b = a;
  if (b.cj.G > 0) {
    // the job's rows must fit the grid's y limit beside the queries' rows (the narrowest
    // grid of any kernel here has one work-group per row); otherwise it runs on its own,
    // first, on the same stream
    if ((int64_t)query_rows(a, prefill) + compress_blocks_wanted(b.cj) > 65535) {
      const hipError_t e = launch_compress(b.cj, stream);
      if (e != hipSuccess) return e;
      b.cj.G = 0;
    }
  }
  if (b.mxfp4 && !prefill && b.group <= 1) {
    // every query streams its own keys
    const dim3 grid = with_job_rows(dim3((unsigned)((b.E + kMxKeysPerWG - 1) / kMxKeysPerWG), (unsigned)b.T), b);
    if (b.cand)
      hipLaunchKernelGGL((indexer_mx_kernel<kCand>), grid, dim3(kDThreads), 0, stream, b);
    else if (b.pages.table)
      hipLaunchKernelGGL((indexer_mx_kernel<kPaged>), grid, dim3(kDThreads), 0, stream, b);
    else
      hipLaunchKernelGGL((indexer_mx_kernel<kPlain>), grid, dim3(kDThreads), 0, stream, b);
  } else if (b.group > 1 && !b.cand) {
    // the smallest even group size that holds b.group (extra queries are masked)
    if (b.group <= 2) launch_group<2>(b, stream);
    else if (b.group <= 4) launch_group<4>(b, stream);
    else if (b.group <= 6) launch_group<6>(b, stream);
    else launch_group<8>(b, stream);
  } else if (!prefill) {
    const int kpw = kDWaves * 16 * (b.cand ? decode_tpw<true, kCand>()
                                           : b.fp8 ? decode_tpw<true, kPlain>() : decode_tpw<false, kPlain>());
    const dim3 grid = with_job_rows(dim3((unsigned)((b.E + kpw - 1) / kpw), (unsigned)b.T), b);
    if (b.cand) {
      if (b.fp8)
        hipLaunchKernelGGL((indexer_decode_kernel<true, kCand>), grid, dim3(kDThreads), 0, stream, b);
      else
        hipLaunchKernelGGL((indexer_decode_kernel<false, kCand>), grid, dim3(kDThreads), 0, stream, b);
    } else if (b.pages.table) {
      if (b.fp8)
        hipLaunchKernelGGL((indexer_decode_kernel<true, kPaged>), grid, dim3(kDThreads), 0, stream, b);
      else
        hipLaunchKernelGGL((indexer_decode_kernel<false, kPaged>), grid, dim3(kDThreads), 0, stream, b);
    } else if (b.fp8) {
      hipLaunchKernelGGL((indexer_decode_kernel<true, kPlain>), grid, dim3(kDThreads), 0, stream, b);
    } else {
      hipLaunchKernelGGL((indexer_decode_kernel<false, kPlain>), grid, dim3(kDThreads), 0, stream, b);
    }
  } else {
    // blockIdx.x (key chunk) varies fastest, so with a multiple of 8 chunks every XCD
    // keeps the same chunks and their keys stay in its L2.
    const dim3 grid = with_job_rows(dim3((unsigned)((b.E + kPChunk - 1) / kPChunk), (unsigned)((b.T + kQPerWG - 1) / kQPerWG)), b);
    if (b.mxfp4) {
      if (b.pages.table)
        hipLaunchKernelGGL((indexer_prefill_kernel<2, true>), grid, dim3(kPThreads), 0, stream, b);
      else
        hipLaunchKernelGGL((indexer_prefill_kernel<2, false>), grid, dim3(kPThreads), 0, stream, b);
    } else if (b.pages.table) {
      if (b.fp8)
        hipLaunchKernelGGL((indexer_prefill_kernel<1, true>), grid, dim3(kPThreads), 0, stream, b);
      else
        hipLaunchKernelGGL((indexer_prefill_kernel<0, true>), grid, dim3(kPThreads), 0, stream, b);
    } else if (b.fp8) {
      hipLaunchKernelGGL((indexer_prefill_kernel<1, false>), grid, dim3(kPThreads), 0, stream, b);
    } else {
      hipLaunchKernelGGL((indexer_prefill_kernel<0, false>), grid, dim3(kPThreads), 0, stream, b);
    }
  }
  return hipGetLastError();
}

}  // namespace sa
