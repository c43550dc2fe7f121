// S1 indexer scores on gfx950 MFMA.
//
// Score of compressed position j for a query: I(j) = s_j * sum_h w_h * max(0, <qI_h, k_j>)
// over 16 index heads x 128 dims, one key per position ("deepseek-ai/DeepSeek-V4.1-Flash"
// recipe, Overview, two-tier sparse attention bullet: a small side attention scores the
// compressed latents). s_j is the fp32 row scale of e4m3 keys (1 for bf16 keys).
//
// Contraction layout: one v_mfma_f32_16x16x32_bf16 tile has the 16 index heads of one
// query as rows (A operand, kept in registers) and 16 keys as columns (B operand, streamed
// from HBM); four MFMAs cover the 128 dims. In the 16x16 fp32 result each lane holds heads
// 4g..4g+3 (g = lane/16) of key lane%16, so the ReLU and head weights are applied
// in-lane and two cross-lane adds finish the 16-head sum. The k order inside an MFMA is
// free (A and B use the same one), so each lane group reads 64 contiguous bytes of every
// key row, which keeps the key stream in whole cache lines.
//
// Block maxima (blocks of 8 positions) fall out of the same registers: a max over 8 lanes.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Dims of k-step s (0..3) held by lane group g, in elements. bf16 keys: chunk 4s+g of
// 8 dims; e4m3 keys: ksteps (2i, 2i+1) share one 16-byte load at byte (4i+g)*16.
__device__ __forceinline__ int kdim_bf16(int g, int s) { return (4 * s + g) * 8; }
__device__ __forceinline__ int kdim_fp8(int g, int s) { return ((s >> 1) * 4 + g) * 16 + (s & 1) * 8; }

struct QueryRegs {
  bf16x8 a[4];   // A operand: head = lane%16, 4 k-steps
  float w[4];    // weights of heads 4g..4g+3
};

template <bool FP8>
__device__ __forceinline__ void load_query(QueryRegs& Q, const uint16_t* qI, const float* w, int lane) {
  const int c = lane & 15, g = lane >> 4;
  const uint16_t* row = qI + c * kIdxDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int d = FP8 ? kdim_fp8(g, s) : kdim_bf16(g, s);
    Q.a[s] = *reinterpret_cast<const bf16x8*>(row + d);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) Q.w[i] = w[4 * g + i];
}

// Raw key data of one 16-key tile for one lane: 4 x 16 bytes (bf16) or 2 x 16 bytes (e4m3).
template <bool FP8>
struct KeyRegs {
  u32x4 v[FP8 ? 2 : 4];
  float scale;
};

template <bool FP8>
__device__ __forceinline__ void load_keys(KeyRegs<FP8>& K, const uint8_t* keys, const float* scales,
                                          int64_t row, int lane) {
  const int g = lane >> 4;
  if constexpr (FP8) {
    const uint8_t* r = keys + row * kIdxDim;
    K.v[0] = *reinterpret_cast<const u32x4*>(r + (0 * 4 + g) * 16);
    K.v[1] = *reinterpret_cast<const u32x4*>(r + (1 * 4 + g) * 16);
    K.scale = scales[row];
  } else {
    const uint8_t* r = keys + row * (kIdxDim * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) K.v[s] = *reinterpret_cast<const u32x4*>(r + (4 * s + g) * 16);
    K.scale = 1.0f;
  }
}

template <bool FP8>
__device__ __forceinline__ f32x4 tile_dots(const QueryRegs& Q, const KeyRegs<FP8>& K) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 b;
    if constexpr (FP8) {
      // 8 e4m3 codes of k-step s: dwords 2*(s&1), 2*(s&1)+1 of load s>>1.
      uint32_t c0 = K.v[s >> 1][2 * (s & 1)], c1 = K.v[s >> 1][2 * (s & 1) + 1];
      uint32_t u0, u1, u2, u3;
      e4m3x4_to_bf16x4(c0, u0, u1);
      e4m3x4_to_bf16x4(c1, u2, u3);
      u32x4 u = {u0, u1, u2, u3};
      b = __builtin_bit_cast(bf16x8, u);
    } else {
      b = __builtin_bit_cast(bf16x8, K.v[s]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.a[s], b, acc, 0, 0, 0);
  }
  return acc;
}

// Weighted-ReLU head sum of one tile. Returns the score of key lane%16 (in every lane).
__device__ __forceinline__ float head_sum(const QueryRegs& Q, f32x4 acc) {
  float v = Q.w[0] * fmaxf(acc[0], 0.f);
  v = fmaf(Q.w[1], fmaxf(acc[1], 0.f), v);
  v = fmaf(Q.w[2], fmaxf(acc[2], 0.f), v);
  v = fmaf(Q.w[3], fmaxf(acc[3], 0.f), v);
  return add_xor32(add_xor16(v));
}

// Store a tile's 16 scores and its two block maxima. `valid` = number of visible keys in
// the tile (<= 16); masked keys score -inf. `lim` = entries of the row that may be written
// from the tile start (the row ends at E, a multiple of 8).
__device__ __forceinline__ void store_tile(float v, int valid, int64_t lim, int lane, float* srow,
                                           float* brow) {
  const int c = lane & 15;
  if (c >= valid) v = neg_inf();
  const float m = max8_lanes(v);
  if (lane < 16 && c < lim) srow[c] = v;
  if (brow != nullptr && (lane == 0 || lane == 8) && lane < lim) brow[lane >> 3] = m;
}

// ---------------------------------------------------------------------------------------
// Decode: every query has its own key stream. Grid (key chunks, T); each wave owns a run
// of TPW consecutive 16-key tiles and keeps kDepth tiles of loads in flight.
// ---------------------------------------------------------------------------------------
constexpr int kTilesPerWave = 16;
constexpr int kKeysPerWG = kWaves * kTilesPerWave * 16;  // 1024
constexpr int kDepth = 4;

template <bool FP8>
__global__ __launch_bounds__(kThreads) void indexer_decode_kernel(IndexerArgs a) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t key0 = (int64_t)blockIdx.x * kKeysPerWG + (int64_t)wave * kTilesPerWave * 16;
  if (key0 >= a.E) return;

  const int seq = a.seq_id[t];
  const int pos = a.pos[t];
  int64_t n = 0;
  if (seq >= 0 && seq < a.num_seqs && pos >= 0) {
    n = ((int64_t)pos + 1) / a.ratio;
    n = n < a.max_visible ? n : a.max_visible;
    n = n < a.compressed_cap ? n : a.compressed_cap;
  }
  float* srow = a.scores + (int64_t)t * a.ld_scores;
  float* brow = a.block_max ? a.block_max + (int64_t)t * a.ld_block_max : nullptr;

  int ntiles = kTilesPerWave;
  if (key0 + ntiles * 16 > a.E) ntiles = (int)((a.E - key0 + 15) / 16);
  int live = 0;  // tiles with at least one visible key
  if (key0 < n) live = (int)min<int64_t>(ntiles, (n - key0 + 15) / 16);

  // Tiles past n: -inf scores and block maxima, no key reads.
  for (int i = live; i < ntiles; ++i) {
    int64_t k = key0 + (int64_t)i * 16;
    if (lane < 16 && k + lane < a.E) srow[k + lane] = neg_inf();
    if (brow && lane < 2 && k + 8 * lane < a.E) brow[(k >> 3) + lane] = neg_inf();
  }
  if (live == 0) return;

  QueryRegs Q;
  load_query<FP8>(Q, reinterpret_cast<const uint16_t*>(a.q_idx) + (int64_t)t * kIdxHeads * kIdxDim,
                  a.w + (int64_t)t * kIdxHeads, lane);
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) +
                        (int64_t)seq * a.keys_seq_stride * (FP8 ? 1 : 2);
  const float* scales = FP8 ? a.scales + (int64_t)seq * a.scales_seq_stride : nullptr;
  const int c = lane & 15;

  KeyRegs<FP8> buf[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    int64_t row = key0 + (int64_t)u * 16 + c;
    row = row < n ? row : n - 1;  // clamp inside the visible rows
    if (u < live) load_keys<FP8>(buf[u], keys, scales, row, lane);
  }
  for (int i0 = 0; i0 < live; i0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int i = i0 + u;
      if (i < live) {
        f32x4 acc = tile_dots<FP8>(Q, buf[u]);
        float sc = buf[u].scale;
        int nxt = i + kDepth;
        if (nxt < live) {
          int64_t row = key0 + (int64_t)nxt * 16 + c;
          row = row < n ? row : n - 1;
          load_keys<FP8>(buf[u], keys, scales, row, lane);
        }
        float v = head_sum(Q, acc);
        if (FP8) v *= sc;
        const int64_t k = key0 + (int64_t)i * 16;
        int valid = (int)min<int64_t>(16, n - k);
        store_tile(v, valid, a.E - k, lane, srow + k, brow ? brow + (k >> 3) : nullptr);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Prefill: many queries share one sequence's keys. Each wave keeps the A operands of
// kQPW queries in registers and streams 16-key tiles; every tile feeds 4*kQPW MFMAs.
// Grid (key chunks of kPKeys, query groups of kWaves*kQPW).
// ---------------------------------------------------------------------------------------
constexpr int kQPW = 4;
constexpr int kPKeys = 1024;

template <bool FP8>
__global__ __launch_bounds__(kThreads) void indexer_prefill_kernel(IndexerArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int64_t k0 = (int64_t)blockIdx.x * kPKeys;
  const int64_t tq0 = ((int64_t)blockIdx.y * kWaves + wave) * kQPW;
  if (tq0 >= a.T || k0 >= a.E) return;
  const int nq = (int)min<int64_t>(kQPW, a.T - tq0);

  // All queries of a wave must read one sequence; queries of another sequence (or
  // invalid ones) are handled with n = 0.
  const int seq = a.seq_id[tq0];
  int64_t n[kQPW];
  int64_t nmax = 0;
#pragma unroll
  for (int j = 0; j < kQPW; ++j) {
    n[j] = 0;
    if (j < nq) {
      int s = a.seq_id[tq0 + j], p = a.pos[tq0 + j];
      if (s == seq && s >= 0 && s < a.num_seqs && p >= 0) {
        int64_t v = ((int64_t)p + 1) / a.ratio;
        v = v < a.max_visible ? v : a.max_visible;
        v = v < a.compressed_cap ? v : a.compressed_cap;
        n[j] = v;
      }
      nmax = n[j] > nmax ? n[j] : nmax;
    }
  }
  const int64_t kend = min<int64_t>(k0 + kPKeys, a.E);
  const int64_t klive = min<int64_t>(kend, nmax);  // keys past every query's n are masked

  // Masked tail of the chunk for all queries.
  for (int64_t k = (klive > k0 ? ((klive - k0 + 15) / 16) * 16 + k0 : k0); k < kend; k += 16) {
    for (int j = 0; j < nq; ++j) {
      float* srow = a.scores + (tq0 + j) * a.ld_scores;
      if (lane < 16 && k + lane < a.E) srow[k + lane] = neg_inf();
      if (a.block_max && lane < 2 && k + 8 * lane < a.E)
        a.block_max[(tq0 + j) * a.ld_block_max + (k >> 3) + lane] = neg_inf();
    }
  }
  if (klive <= k0) return;

  QueryRegs Q[kQPW];
#pragma unroll
  for (int j = 0; j < kQPW; ++j) {
    int64_t tj = tq0 + (j < nq ? j : 0);
    load_query<FP8>(Q[j], reinterpret_cast<const uint16_t*>(a.q_idx) + tj * kIdxHeads * kIdxDim,
                    a.w + tj * kIdxHeads, lane);
  }
  const int sq = (seq >= 0 && seq < a.num_seqs) ? seq : 0;
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys) +
                        (int64_t)sq * a.keys_seq_stride * (FP8 ? 1 : 2);
  const float* scales = FP8 ? a.scales + (int64_t)sq * a.scales_seq_stride : nullptr;

  const int ntiles = (int)((klive - k0 + 15) / 16);
  KeyRegs<FP8> cur, nxt;
  {
    int64_t row = min<int64_t>(k0 + c, nmax - 1);
    load_keys<FP8>(cur, keys, scales, row, lane);
  }
  for (int i = 0; i < ntiles; ++i) {
    const int64_t k = k0 + (int64_t)i * 16;
    if (i + 1 < ntiles) {
      int64_t row = min<int64_t>(k + 16 + c, nmax - 1);
      load_keys<FP8>(nxt, keys, scales, row, lane);
    }
#pragma unroll
    for (int j = 0; j < kQPW; ++j) {
      if (j < nq) {
        f32x4 acc = tile_dots<FP8>(Q[j], cur);
        float v = head_sum(Q[j], acc);
        if (FP8) v *= cur.scale;
        int valid = (int)max<int64_t>(0, min<int64_t>(16, n[j] - k));
        float* srow = a.scores + (tq0 + j) * a.ld_scores;
        float* brow = a.block_max ? a.block_max + (tq0 + j) * a.ld_block_max : nullptr;
        store_tile(v, valid, a.E - k, lane, srow + k, brow ? brow + (k >> 3) : nullptr);
      }
    }
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool prefill, hipStream_t stream) {
  if (!prefill) {
    dim3 grid((unsigned)((a.E + kKeysPerWG - 1) / kKeysPerWG), (unsigned)a.T);
    if (a.fp8)
      hipLaunchKernelGGL(indexer_decode_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(indexer_decode_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  } else {
    dim3 grid((unsigned)((a.E + kPKeys - 1) / kPKeys),
              (unsigned)((a.T + kWaves * kQPW - 1) / (kWaves * kQPW)));
    if (a.fp8)
      hipLaunchKernelGGL(indexer_prefill_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(indexer_prefill_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sa
