// Kernel argument blocks and launchers (host <-> device boundary inside the library).
// Every launcher assumes the host-side checks in api.cpp have passed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Paged compressed stores: position j of sequence s is pool row
// table[s * stride + (j >> log2_page)] * page + (j & (page - 1)); table == null: the stores
// are contiguous per sequence. Page ids are clamped into [0, num_pages).
struct PageTable {
  const int32_t* table;
  int64_t stride;
  int32_t log2_page;
  int64_t num_pages;
};

struct QueryMeta {
  const int32_t* seq_id;
  const int32_t* pos;
  int64_t T;
  int64_t max_visible;     // host hint, caps n
  int64_t num_seqs;
  int64_t compressed_cap;  // caps n
  int32_t ratio;
};

struct CompressArgs {
  const void* raw;
  int64_t raw_stride;
  const void* gate;
  int64_t gate_stride;
  const float* bias;        // [ratio][512]
  void* out;
  int64_t out_stride;
  int64_t G;
  int32_t ratio;
  // code rows (kv_mode 1: e4m3 + fp32 row scale, 2: MXFP4 + 16 E8M0 bytes); out_stride and
  // scales_stride in bytes then
  int32_t kv_mode;
  void* scales;
  int64_t scales_stride;
};
struct IndexerArgs {
  const int32_t* seq_id;
  const int32_t* pos;
  int64_t T;
  int64_t max_visible;
  int64_t num_seqs;
  int64_t compressed_cap;
  int32_t ratio;
  bool fp8;
  bool mxfp4;               // MXFP4 keys: [seq][cap][64] bytes, E8M0 scales [seq][cap][4]
  const void* q_idx;        // bf16 [T][16][128]
  const float* w;           // [T][16]
  const void* keys;         // bf16 / e4m3 [seq][cap][128]
  int64_t keys_seq_stride;  // elements
  const float* scales;      // e4m3: fp32 per row; MXFP4: the E8M0 bytes (cast back in the kernel)
  int64_t scales_seq_stride;
  float* scores;            // [T][ld_scores]
  int64_t ld_scores;
  float* block_max;         // [T][ld_block_max] or null
  int64_t ld_block_max;
  int64_t E;                // score row extent: max_visible rounded up to 8 (candidate mode: 8 * 2048)
  const int32_t* cand;      // candidate mode: [T][2048] carried block ids, else null
  int32_t group;            // > 1: queries g*group .. g*group+group-1 share a sequence (<= 8)
  PageTable pages;          // keys and scales are page pools when pages.table is set
  // A compressor job (cj.G > 0) that rides in the launch: work-groups in grid rows from
  // cj_row0 on (set by the launcher) run it instead of indexer work.
  CompressArgs cj{};
  int32_t cj_row0 = 0;
};
hipError_t launch_indexer(const IndexerArgs& a, bool prefill, hipStream_t stream);
// Queries per work-group of the chunk kernel (its grid holds ceil(T / this) in y).
constexpr int kChunkQueriesPerWG = 16;

constexpr int kPartBlocks = 8192;   // blocks per part of the two-level candidate stage (rows of
                                    // up to 8 parts; longer rows use parts of twice that)
constexpr int kMaxParts = 8;        // part lists the second level holds (8 x 2048 block ids)

struct SelectArgs {
  QueryMeta m;
  const float* scores;
  int64_t ld_scores;
  const float* block_max;   // may be null
  int64_t ld_block_max;
  int32_t* cand;            // [T][2048]
  int32_t* topk;            // [T][512]
  int32_t* part_ids;        // [T][parts][2048] workspace, used when parts > 1
  uint32_t* part_keys;      // [T][parts][2048] order-preserving block maxima of part_ids
  int parts;                // select_parts(m.max_visible)
  int part_blocks;          // blocks per part (kPartBlocks or 2 * kPartBlocks)
};
// Parts of the candidate stage for queries of up to max_visible positions (parts 1: one
// level), and their size in blocks.
struct PartSplit {
  int parts, part_blocks;
};
PartSplit select_parts(int64_t max_visible);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
// Candidate mode: top-512 positions inside carried candidate blocks (a.cand is the input,
// scores / block_max in slot order as the candidate-mode indexer writes them).
hipError_t launch_select_cand(const SelectArgs& a, hipStream_t stream);

struct AttnArgs {
  QueryMeta m;
  const void* q;            // bf16 [T][64][512]
  const int32_t* topk;      // [T][512]
  const void* latents;      // bf16 [seq][cap][512]
  int64_t latents_seq_stride;
  const void* window;       // bf16 [seq][wcap][512]
  int64_t window_seq_stride;
  int32_t window_cap;
  float scale;
  void* out;                // bf16 [T][64][512]
  float* lse;               // [T][64] or null
  // key splits: splits > 1 spreads each query's keys over that many work-groups, which
  // leave partial results in part_o / part_ml; the last one of a query to finish (counted
  // in counters[t], zero before and after the call) combines them
  int splits;
  float* part_o;            // [T * splits][64][512] unnormalised outputs
  float* part_ml;           // [T * splits][64][2] reference (log2 domain) and normaliser
  uint32_t* counters;       // [T]
  PageTable pages;          // latents are a page pool when pages.table is set
  // kv_mode 1: e4m3 latents and window, rows of 512 codes (strides above in bytes then),
  // one fp32 scale per row ([seq][cap] / [seq][wcap], or the pool's rows when paged).
  // kv_mode 2: MXFP4 latents (256 code bytes per row, latent_scales 16 E8M0 bytes per row,
  // its stride in bytes) and an e4m3 window.
  int kv_mode;
  const void* latent_scales;
  int64_t latent_scales_seq_stride;
  const float* window_scales;
  int64_t window_scales_seq_stride;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);
// Key splits used for T queries, and the partial slots (T * splits) the largest of them
// needs for any T up to max_queries. Split batches keep one counter per (query, head set):
// 2 * T at most.
int attn_splits(int64_t T);
int64_t attn_max_units(int64_t max_queries);
// Zero n 32-bit words (a kernel, so the call may be captured in a graph).
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t stream);
// Key-split state in a fixed per-GPU array (for callers that cannot allocate): counters,
// partial references / normalisers and partial outputs of every batch that splits its keys
// (at most kScratchQueries queries, at most kScratchUnits (query, split) units), on the
// current device.
constexpr int kScratchQueries = 32;
constexpr int kMaxAttnSplits = 4;
constexpr int64_t kScratchUnits = 128;
constexpr int kScratchCounters = 2 * kScratchQueries;   // one per (query, head set)
struct AttnScratch {
  uint32_t* counters;       // [kScratchCounters]
  float* part_ml;           // [kScratchUnits][64][2]
  float* part_o;            // [kScratchUnits][64][512]
  size_t bytes;
};
hipError_t attn_scratch(AttnScratch& s);

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);

}  // namespace sa
