// S1 indexer scores on gfx950 MFMA.
//
// Score of compressed position j for a query: I(j) = s_j * sum_h w_h * max(0, <qI_h, k_j>)
// over 16 index heads x 128 dims, one key per position ("deepseek-ai/DeepSeek-V4.1-Flash"
// recipe, Overview, two-tier sparse attention bullet: a small side attention scores the
// compressed latents). s_j is the fp32 row scale of e4m3 keys (1 for bf16 keys). e4m3 keys
// are widened to bf16 exactly in registers; the index query stays bf16.
//
// Block maxima (blocks of 8 positions) are taken from the same registers with DPP.
//
// Decode (every query has its own key stream, HBM-bound): v_mfma_f32_16x16x32_bf16 with
// the 16 heads of one query as rows (A, in registers) and 16 keys as columns (B, streamed
// from HBM, kDepth tiles in flight per wave). In the 16x16 result each lane holds heads
// 4g..4g+3 (g = lane/16) of key lane%16: ReLU and head weights in-lane, then two row-swap
// adds finish the 16-head sum. The k order inside an MFMA is free (A and B use the same
// one), so each lane group reads 64 contiguous bytes of a key row.
//
// Prefill (a chunk of queries shares one key stream, MFMA-bound): v_mfma_f32_32x32x16_bf16
// with two queries x 16 heads as rows and 32 keys as columns. Key tiles are staged once per
// work-group in padded LDS rows (prefetched two tiles ahead through registers) and read by
// every wave; each wave holds two query pairs. A lane's 16 results are 8 heads of each of
// the two queries for one key, so the head sum is in-lane plus one 32-lane swap.
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
#ifndef SA_IDX_TPW
#define SA_IDX_TPW 16
#endif
#ifndef SA_IDX_DEPTH
#define SA_IDX_DEPTH 8
#endif
constexpr int kDWaves = 4;
constexpr int kDThreads = 64 * kDWaves;
constexpr int kTilesPerWave = SA_IDX_TPW;
constexpr int kKeysPerWG = kDWaves * kTilesPerWave * 16;
constexpr int kDepth = SA_IDX_DEPTH;

// Dims of k-step s (0..3) held by lane group g, in elements. bf16 keys: chunk 4s+g of
// 8 dims; e4m3 keys: ksteps (2i, 2i+1) share one 16-byte load at byte (4i+g)*16.
__device__ __forceinline__ int kdim_bf16(int g, int s) { return (4 * s + g) * 8; }
__device__ __forceinline__ int kdim_fp8(int g, int s) { return ((s >> 1) * 4 + g) * 16 + (s & 1) * 8; }

template <bool FP8>
struct KeyRegs {
  u32x4 v[FP8 ? 2 : 4];
  float scale;
};

template <bool FP8>
__device__ __forceinline__ void load_keys(KeyRegs<FP8>& K, const uint8_t* tile, const float* tscale,
                                          uint32_t lane_off, int c) {
  if constexpr (FP8) {
    K.v[0] = *reinterpret_cast<const u32x4*>(tile + lane_off);
    K.v[1] = *reinterpret_cast<const u32x4*>(tile + lane_off + 64);
    K.scale = tscale[c];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) K.v[s] = *reinterpret_cast<const u32x4*>(tile + lane_off + 64 * s);
    K.scale = 1.0f;
  }
}

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

template <bool FP8>
__global__ __launch_bounds__(kDThreads) void indexer_decode_kernel(IndexerArgs a) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int E = (int)a.E;
  const int key0 = blockIdx.x * kKeysPerWG + wave * kTilesPerWave * 16;
  if (key0 >= E) return;

  const int n = query_n(a, t);
  float* srow = a.scores + (int64_t)t * a.ld_scores;
  float* brow = a.block_max ? a.block_max + (int64_t)t * a.ld_block_max : nullptr;

  int ntiles = min(kTilesPerWave, (E - key0 + 15) >> 4);
  int live = key0 < n ? min(ntiles, (n - key0 + 15) >> 4) : 0;

  // Tiles past n: -inf scores and block maxima, no key reads.
  for (int i = live; i < ntiles; ++i) {
    const int k = key0 + 16 * i;
    if (lane < 16 && k + lane < E) srow[k + lane] = neg_inf();
    if (brow && lane < 2 && k + 8 * lane < E) brow[(k >> 3) + lane] = neg_inf();
  }
  if (live == 0) return;

  const int seq = a.seq_id[t];
  bf16x8 qa[4];
  float wq[4];
  {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(a.q_idx) + ((int64_t)t * kIdxHeads + c) * kIdxDim;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[s] = *reinterpret_cast<const bf16x8*>(row + (FP8 ? kdim_fp8(g, s) : kdim_bf16(g, s)));
#pragma unroll
    for (int i = 0; i < 4; ++i) wq[i] = a.w[(int64_t)t * kIdxHeads + 4 * g + i];
  }
  constexpr int RB = FP8 ? kIdxDim : 2 * kIdxDim;  // key row bytes
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) + (int64_t)seq * a.keys_seq_stride * (FP8 ? 1 : 2);
  const float* scales = FP8 ? a.scales + (int64_t)seq * a.scales_seq_stride : nullptr;
  // A lane reads row c of a tile: 64 contiguous bytes at 16g (bf16) or 16 at 16g (+64) (e4m3).
  const uint32_t lane_off = (uint32_t)(c * RB + 16 * g);

  // Rows past n inside the last live tile are clamped to row n-1 (read, then masked).
  auto tile_ptr = [&](int i, const uint8_t*& tp, const float*& sp, uint32_t& off) {
    const int k = key0 + 16 * i;
    if (k + 16 <= n) {
      tp = keys + (int64_t)k * RB;
      sp = FP8 ? scales + k : nullptr;
      off = lane_off;
    } else {
      const int row = min(k + c, n - 1);
      tp = keys;
      sp = FP8 ? scales + row - c : nullptr;
      off = (uint32_t)(row * RB + 16 * g);
    }
  };

  KeyRegs<FP8> buf[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    if (u < live) {
      const uint8_t* tp; const float* sp; uint32_t off;
      tile_ptr(u, tp, sp, off);
      load_keys<FP8>(buf[u], tp, sp, off, c);
    }
  }
  for (int i0 = 0; i0 < live; i0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int i = i0 + u;
      if (i < live) {
        const f32x4 acc = tile_dots<FP8>(qa, buf[u]);
        const float sc = buf[u].scale;
        if (i + kDepth < live) {
          const uint8_t* tp; const float* sp; uint32_t off;
          tile_ptr(i + kDepth, tp, sp, off);
          load_keys<FP8>(buf[u], tp, sp, off, c);
        }
        float v = wq[0] * relu(acc[0]);
        v = fmaf(wq[1], relu(acc[1]), v);
        v = fmaf(wq[2], relu(acc[2]), v);
        v = fmaf(wq[3], relu(acc[3]), v);
        v = add_xor32(add_xor16(v));
        if (FP8) v *= sc;
        const int k = key0 + 16 * i;
        if (k + 16 <= n) {  // whole tile visible
          const float m = max8_lanes(v);
          if (lane < 16) srow[k + lane] = v;
          if (brow && (lane == 0 || lane == 8)) brow[(k >> 3) + (lane >> 3)] = m;
        } else {
          if (k + c >= n) v = neg_inf();
          const float m = max8_lanes(v);
          if (lane < 16 && k + lane < E) srow[k + lane] = v;
          if (brow && (lane == 0 || lane == 8) && k + lane < E) brow[(k >> 3) + (lane >> 3)] = m;
        }
      }
    }
  }
}

// ======================================================================================
// Prefill
// ======================================================================================
constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPairsPerWave = 2;
constexpr int kQPerWG = kPWaves * kPairsPerWave * 2;   // 16 queries
constexpr int kPKT = 32;                                // keys per tile
constexpr int kPChunk = 2048;                           // keys per work-group
constexpr int kPBufs = 3;

template <bool FP8>
struct PrefillShared {
  static constexpr int RB = FP8 ? kIdxDim : 2 * kIdxDim;
  static constexpr int RS = RB + 16;                   // padded row stride
  uint8_t tile[kPBufs][kPKT * RS];
  float scale[kPBufs][kPKT];
};

// Dims of k-step s (0..7) for lane half hh: (2s + hh) * 8 .. +8 (32x32x16 operands).
__device__ __forceinline__ int pdim(int hh, int s) { return (2 * s + hh) * 8; }

template <bool FP8>
__global__ __launch_bounds__(kPThreads, 2) void indexer_prefill_kernel(IndexerArgs a) {
  using SH = PrefillShared<FP8>;
  constexpr int RB = SH::RB, RS = SH::RS;
  __shared__ __attribute__((aligned(16))) SH sh;
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
  int nq[4];
  int nmax_wg = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) nq[j] = 0;
  for (int j = 0; j < kQPerWG; ++j) {
    const int tq = q0 + j;
    int nj = 0;
    if (tq < T && a.seq_id[tq] == seq) nj = query_n(a, tq);
    nmax_wg = max(nmax_wg, nj);
    if ((j >> 2) == wave) nq[j & 3] = nj;
  }
  int nmin_w = INT32_MAX;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (q0 + 4 * wave + j < T) nmin_w = min(nmin_w, nq[j]);
  const int klive = min(kend, nmax_wg);   // keys past every query's n are masked
  const int ntiles = klive > k0 ? (klive - k0 + kPKT - 1) / kPKT : 0;

  // masked part of the chunk (tiles past klive), for every valid query of the wave
  for (int j = 0; j < 4; ++j) {
    const int tq = q0 + 4 * wave + j;
    if (tq >= T) break;
    float* srow = a.scores + (int64_t)tq * a.ld_scores;
    float* brow = a.block_max ? a.block_max + (int64_t)tq * a.ld_block_max : nullptr;
    for (int k = k0 + ntiles * kPKT + lane; k < kend; k += 64) srow[k] = neg_inf();
    if (brow)
      for (int b = (k0 + ntiles * kPKT) / 8 + lane; b < kend / 8; b += 64) brow[b] = neg_inf();
  }
  if (ntiles == 0) return;

  // A operands and head weights of the wave's two query pairs.
  bf16x8 qa[kPairsPerWave][8];
  float wt[kPairsPerWave][2][8];
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p) {
    const int jq = 2 * p + (r32 >> 4);
    const int tq = min(q0 + 4 * wave + jq, T - 1);
    const uint16_t* row = reinterpret_cast<const uint16_t*>(a.q_idx) + ((int64_t)tq * kIdxHeads + (r32 & 15)) * kIdxDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[p][s] = *reinterpret_cast<const bf16x8*>(row + pdim(hh, s));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tw = min(q0 + 4 * wave + 2 * p + j, T - 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) wt[p][j][i] = a.w[(int64_t)tw * kIdxHeads + 8 * (i >> 2) + 4 * hh + (i & 3)];
    }
  }

  const int sq = (seq >= 0 && seq < a.num_seqs) ? seq : 0;
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) + (int64_t)sq * a.keys_seq_stride * (FP8 ? 1 : 2);
  const float* scales = FP8 ? a.scales + (int64_t)sq * a.scales_seq_stride : nullptr;

  // staging: 16-byte chunk q = tid + kPThreads*h of the tile (h < CPT) is row q / CPR,
  // chunk q % CPR: each wave loads whole rows (contiguous 1 KiB per instruction) and
  // each group of CPR lanes writes one padded LDS row contiguously.
  constexpr int CPR = RB / 16;                          // chunks per row: 16 (bf16) or 8 (e4m3)
  constexpr int CPT = kPKT * CPR / kPThreads;           // chunks per thread: 2 or 1
  u32x4 stg[CPT];
  float stg_scale = 1.f;
  auto fetch = [&](int i) {
#pragma unroll
    for (int h = 0; h < CPT; ++h) {
      const int q = tid + kPThreads * h;
      const int row = min(k0 + i * kPKT + q / CPR, klive - 1);
      stg[h] = *reinterpret_cast<const u32x4*>(keys + (int64_t)row * RB + (q % CPR) * 16);
    }
    if (FP8 && tid < kPKT) stg_scale = scales[min(k0 + i * kPKT + tid, klive - 1)];
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int h = 0; h < CPT; ++h) {
      const int q = tid + kPThreads * h;
      *reinterpret_cast<u32x4*>(&sh.tile[buf][(q / CPR) * RS + (q % CPR) * 16]) = stg[h];
    }
    if (FP8 && tid < kPKT) sh.scale[buf][tid] = stg_scale;
  };

  fetch(0);
  commit(0);
  if (ntiles > 1) {
    fetch(1);
    commit(1);
  }
  if (ntiles > 2) fetch(2);
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    const int buf = i % kPBufs;
    const int k = k0 + i * kPKT;
    const uint8_t* T8 = sh.tile[buf] + r32 * RS;
    bf16x8 b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if constexpr (FP8) {
        const uint2 v = *reinterpret_cast<const uint2*>(T8 + pdim(hh, s));
        b[s] = e4m3x8_to_bf16x8(v.x, v.y);
      } else {
        b[s] = *reinterpret_cast<const bf16x8*>(T8 + 2 * pdim(hh, s));
      }
    }
    const float sc = FP8 ? sh.scale[buf][r32] : 1.f;
    const bool full = k + kPKT <= nmin_w;   // every key of the tile visible to all 4 queries
    // both pairs' MFMA chains first (independent accumulators), then the epilogues, so
    // the second chain runs under the first epilogue
    f32x16 acc[kPairsPerWave];
#pragma unroll
    for (int p = 0; p < kPairsPerWave; ++p) {
      acc[p] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[p][s], b[s], acc[p], 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < kPairsPerWave; ++p) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int jq = 2 * p + j;
        const int tq = q0 + 4 * wave + jq;
        float v = wt[p][j][0] * relu(acc[p][8 * j + 0]);
#pragma unroll
        for (int ii = 1; ii < 8; ++ii) v = fmaf(wt[p][j][ii], relu(acc[p][8 * j + ii]), v);
        v = add_xor32(v);
        if (FP8) v *= sc;
        if (tq < T) {
          float* srow = a.scores + (int64_t)tq * a.ld_scores;
          float* brow = a.block_max ? a.block_max + (int64_t)tq * a.ld_block_max : nullptr;
          if (full) {
            const float m = max8_lanes(v);
            if (lane < 32) srow[k + lane] = v;
            if (brow && lane < 32 && (lane & 7) == 0) brow[(k >> 3) + (lane >> 3)] = m;
          } else {
            if (k + r32 >= nq[jq]) v = neg_inf();
            const float m = max8_lanes(v);
            if (lane < 32 && k + lane < E) srow[k + lane] = v;
            if (brow && lane < 32 && (lane & 7) == 0 && k + lane < E) brow[(k >> 3) + (lane >> 3)] = m;
          }
        }
      }
    }
    if (i + 1 < ntiles) {
      // buffer (i+2)%3 was last read in step i-1, which every wave finished before the
      // barrier at the end of step i-1
      if (i + 2 < ntiles) {
        commit((i + 2) % kPBufs);
        if (i + 3 < ntiles) fetch(i + 3);
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool prefill, hipStream_t stream) {
  if (!prefill) {
    dim3 grid((unsigned)((a.E + kKeysPerWG - 1) / kKeysPerWG), (unsigned)a.T);
    if (a.fp8)
      hipLaunchKernelGGL(indexer_decode_kernel<true>, grid, dim3(kDThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(indexer_decode_kernel<false>, grid, dim3(kDThreads), 0, stream, a);
  } else {
    // blockIdx.x (key chunk) varies fastest, so with a multiple of 8 chunks every XCD
    // keeps the same chunks and their keys stay in its L2.
    dim3 grid((unsigned)((a.E + kPChunk - 1) / kPChunk), (unsigned)((a.T + kQPerWG - 1) / kQPerWG));
    if (a.fp8)
      hipLaunchKernelGGL(indexer_prefill_kernel<true>, grid, dim3(kPThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(indexer_prefill_kernel<false>, grid, dim3(kPThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sa
