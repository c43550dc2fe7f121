/*
 * sparse_attn.h -- C ABI of the two-tier sparse-attention hot path of a
 * DeepSeek-V4.1 Flash layer, for AMD MI355X (gfx950).
 *
 * What is computed (per query t of sequence b at raw position p):
 *   S0  compressor: a group of r raw latents is pooled into one compressed
 *       latent by a learned softmax gate ("deepseek-ai/DeepSeek-V4.1-Flash"
 *       vLLM recipe, Overview, two-tier sparse attention bullet: latents
 *       "pooled by a learned softmax gate"; "DeepSeek-V4.1 Flash" Miles docs,
 *       section 1: 2 positions into 1, or 1-to-1).
 *   S1  indexer: every visible compressed latent j < n = (p+1)/r gets the score
 *       I(j) = s_j * sum_h w_h * max(0, <qI_h, kI_j>) over 16 index heads of
 *       128 dims (recipe Overview: an indexer scores the latents).
 *   S2  candidate stage: the 2048 blocks of 8 consecutive positions with the
 *       highest block score (max of the block's visible scores) are kept
 *       (recipe Overview: "a candidate stage that selects 2048 blocks of 8").
 *   S3  top-512: the 512 best positions inside the candidates (recipe
 *       Overview: keeps the best 512 per query; Miles docs section 1).
 *   S4  attention: 64 query heads, one softmax over the selected latents plus
 *       the 128-position window [p-127, p]; each 512-wide latent is both key
 *       and value (Miles docs section 1).
 * Ties at S2 and S3 are broken by the lower position / block id.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are GPU memory owned by the caller; the library
 *     never allocates, frees or synchronises inside these calls, so each call
 *     only enqueues kernels on `stream` (a hipStream_t, or NULL for the null
 *     stream) and may be captured in a HIP graph. Outputs are valid once the
 *     stream reaches the enqueued work.
 *   - bf16 is bfloat16 (upper half of IEEE binary32). e4m3 is OCP FP8 E4M3
 *     ("e4m3fn": bias 7, max 448, no infinities).
 *   - Strides are in elements. Rows (the last dimension) are contiguous.
 *   - Every device pointer must be 16-byte aligned, and every stride a
 *     multiple of 8 elements (16 for e4m3 keys).
 *   - Return value: SA_OK, or an error code with a message available from
 *     sparse_attn_last_error() on the calling thread. All argument checks run
 *     on the host before any HIP call; an invalid call enqueues nothing.
 *     Device faults are asynchronous and surface at the caller's next sync.
 *   - Device metadata (seq_id, pos, topk entries) is not read on the host.
 *     Kernels clamp it so that memory stays in bounds: a query with seq_id
 *     outside [0, num_seqs) or pos < 0 gets n = 0; n is capped at
 *     max_visible and compressed_cap; attention skips topk entries outside
 *     [0, n). Results for such queries are unspecified but memory-safe.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_EINVAL = 1,        /* null pointer, misalignment, size or shape mismatch */
  SA_EUNSUPPORTED = 2,  /* dimensions other than the ones the kernels are built for */
  SA_EWORKSPACE = 3,    /* workspace missing or smaller than the plan requires */
  SA_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} sa_status;

typedef enum sa_key_dtype {
  SA_KEY_BF16 = 0,      /* index keys bf16 [.][128] */
  SA_KEY_FP8_E4M3 = 1,  /* index keys e4m3 [.][128] plus one fp32 scale per key */
  SA_KEY_MXFP4 = 2      /* index keys OCP MXFP4: the FP4 indexer cache ("SGLang and Miles Add
                           Day-0 Support for DeepSeek-V4.1", SGLang Features table,
                           Quantization row), set as indexer_kv_dtype mxfp4 in the
                           "deepseek-ai/DeepSeek-V4.1-Flash" recipe's Blackwell TP and DEP
                           section:
                           [.][64] bytes of FP4 E2M1, element 2i in the low nibble of
                           byte i, plus [.][4] E8M0 scales, scale b for elements
                           32b .. 32b+31. Key = 2^(scale-127) * element. indexer_score
                           runs the chunk kernel (one-sequence chunks, ragged runs), the
                           group kernel (groups, runs of 2 to 8 queries) or one key stream
                           per query for these keys, on contiguous or paged stores;
                           indexer_score_cand takes them on contiguous stores */
} sa_key_dtype;

/* Fixed at plan time. The kernels support exactly num_heads 64, latent_dim 512,
 * window 128, topk 512, idx_heads 16, idx_dim 128, block 8, cand_blocks 2048,
 * ratio 1 or 2, and max_compressed up to 1,048,576 (the pages' 1M-token context on a
 * 1-to-1 layer: "deepseek-ai/DeepSeek-V4.1-Flash" recipe, Context length; "DeepSeek-V4.1
 * Flash" Miles docs, section 1: 1-to-1 from layer 20 on); anything else returns
 * SA_EUNSUPPORTED. */
/* Latent and window store element type. The pages name an FP8 window cache and FP4
 * compressed state ("SGLang and Miles Add Day-0 Support for DeepSeek-V4.1", Miles Day-0
 * Support table, Quantization row), latents trained for FP4 storage ("deepseek-ai/
 * DeepSeek-V4.1-Flash" recipe, Memory) and --kv-cache-dtype fp8 (same recipe, Blackwell TP
 * and DEP). bf16 is the precision the layer configurations fix. */
typedef enum sa_kv_dtype {
  SA_KV_BF16 = 0,       /* rows of 512 bf16 */
  SA_KV_FP8_E4M3 = 1,   /* rows of 512 OCP E4M3 codes plus one fp32 scale per row:
                           X = scale * code. Read by sparse_attn_fwd (decoded exactly where
                           the MFMA operands are built) and written by
                           sparse_attn_compress_codes; sparse_attn_compress writes bf16
                           rows and returns SA_EUNSUPPORTED for these plans */
  SA_KV_MXFP4 = 2       /* FP4 compressed state beside an FP8 window (the Miles Day-0 Support
                           table cited above): latent rows of OCP MXFP4, 256 bytes
                           of E2M1 (element 2i in the low nibble of byte i) plus 16 E8M0
                           block scales (scale b for elements 32b .. 32b+31, X = 2^(scale-127)
                           * element); window rows e4m3 as for SA_KV_FP8_E4M3. Same calls
                           and limits as SA_KV_FP8_E4M3 */
} sa_kv_dtype;

typedef struct sa_params {
  int32_t num_heads;
  int32_t latent_dim;
  int32_t window;
  int32_t topk;
  int32_t idx_heads;
  int32_t idx_dim;
  int32_t block;
  int32_t cand_blocks;
  int32_t ratio;
  int32_t idx_key_dtype;   /* sa_key_dtype */
  float softmax_scale;     /* multiplies <q_h, x>; 1/sqrt(512) for this layer */
  int64_t max_queries;     /* largest T of any call made with this plan */
  int64_t max_compressed;  /* largest visible compressed count of any query */
  int32_t kv_dtype;        /* sa_kv_dtype of the latents and the window (0: bf16) */
} sa_params;

typedef struct sa_plan sa_plan;

/* A batch of T queries. */
typedef struct sa_queries {
  int64_t T;               /* 1 <= T <= plan max_queries */
  const int32_t* seq_id;   /* device [T]: sequence of query t */
  const int32_t* pos;      /* device [T]: raw position p of query t */
  int64_t max_visible;     /* host: >= (pos[t]+1)/ratio for every t, <= plan max_compressed.
                              Sizes the grids and the score rows. */
  int32_t group;           /* host, 0..8. 0 or 1: no grouping. G > 1: queries
                              gG .. gG+G-1 (the last group may be shorter) read one
                              sequence, as the tokens of a multi-token decode step do (a
                              verified token and the drafted tokens after it); indexer_score
                              then streams each group's keys once for all its queries. A
                              query whose seq_id differs from its group's first query gets
                              -inf scores. sparse_attn_fwd uses it only to check
                              window_cap (see sa_cache); the other calls ignore it. */
  const int32_t* runs;     /* host, optional (NULL: none): a ragged batch as num_runs runs of
                              consecutive queries, runs[i] >= 1 queries each, summing to T;
                              the queries of a run read one sequence (a prefill chunk, a
                              decode step with drafted tokens, or one decode query).
                              indexer_score then launches the chunk kernel for runs of 9 or
                              more queries, the group kernel for neighbouring runs of one
                              length in 2..8, and one key stream per query for the rest
                              (and "group" is ignored). sparse_attn_fwd uses it only to
                              check window_cap; the other calls ignore it. */
  int32_t num_runs;
} sa_queries;

/* Per-sequence stores, all device memory. */
typedef struct sa_cache {
  int64_t num_seqs;
  int64_t compressed_cap;        /* rows per sequence in latents / idx_keys / idx_scales */
  const void* latents;           /* bf16 [num_seqs][compressed_cap][512] compressed latents */
  int64_t latents_seq_stride;    /* >= compressed_cap * 512 */
  const void* window;            /* bf16 [num_seqs][window_cap][512]; raw position u is row u % window_cap */
  int64_t window_seq_stride;     /* >= window_cap * 512 */
  int32_t window_cap;            /* >= 128, and >= 127 + s where s is the span of raw
                                    positions (max - min + 1) of the queries of one
                                    sequence in a call: a later position's row would
                                    otherwise overwrite a row an earlier query reads.
                                    sparse_attn_fwd refuses (SA_EINVAL) what the host can
                                    see: s >= the longest run, the group size, or T when
                                    num_seqs is 1 (queries of one sequence in one call
                                    are at distinct positions) */
  const void* idx_keys;          /* bf16 or e4m3 [num_seqs][compressed_cap][128], or MXFP4
                                    bytes [num_seqs][compressed_cap][64]; 16-byte aligned */
  int64_t idx_keys_seq_stride;   /* in elements of the store (bf16, bytes, bytes):
                                    >= compressed_cap * 128 (64 for MXFP4) */
  const void* idx_scales;        /* fp32 [num_seqs][compressed_cap] for e4m3 keys (16-byte
                                    aligned), E8M0 bytes [num_seqs][compressed_cap][4] for
                                    MXFP4 keys (4-byte aligned), NULL for bf16 */
  int64_t idx_scales_seq_stride; /* in scale elements: >= compressed_cap (e4m3) or
                                    >= 4 * compressed_cap and a multiple of 4 (MXFP4) */
  /* Paged stores (the layout serving engines keep caches in). NULL block_table: the
   * stores above are contiguous per sequence. Otherwise latents, idx_keys and idx_scales
   * are page pools of num_pages pages of page_size rows each (pool row r = page r /
   * page_size, row r % page_size; the *_seq_stride fields are ignored), and compressed
   * position j of sequence s is pool row block_table[s * block_table_stride + j /
   * page_size] * page_size + j % page_size. The window stays per sequence. Page ids
   * outside [0, num_pages) are clamped. Supported by indexer_score (bf16, e4m3 and MXFP4
   * keys, every kernel; a chunk runs on the chunk kernel only when pages hold at least 64
   * rows, else one key stream per query) and sparse_attn_fwd; indexer_score_cand returns
   * SA_EUNSUPPORTED. MXFP4 key pools: idx_keys [num_pages * page_size][64] bytes and
   * idx_scales [num_pages * page_size][4] bytes. */
  const int32_t* block_table;    /* device int32 [num_seqs][block_table_stride] or NULL */
  int64_t block_table_stride;    /* >= ceil(compressed_cap / page_size) */
  int32_t page_size;             /* power of two in [16, 2^20] */
  int64_t num_pages;             /* pages in each pool, 1 .. 2^31 - 1 */
  /* e4m3 latents and window (plan kv_dtype SA_KV_FP8_E4M3): latents and window hold 512
   * codes per row and their *_seq_stride fields count bytes (multiples of 16); the fp32
   * row scales are latent_scales [num_seqs][compressed_cap] (or one per pool row when
   * paged) and window_scales [num_seqs][window_cap].
   * MXFP4 latents (SA_KV_MXFP4): latents hold 256 bytes per row (latents_seq_stride in
   * bytes, >= 256 * compressed_cap, a multiple of 16) and latent_scales 16 E8M0 bytes per
   * row, [num_seqs][compressed_cap][16] or per pool row when paged (16-byte aligned,
   * latent_scales_seq_stride in bytes); the window is e4m3 as above. */
  const void* latent_scales;
  int64_t latent_scales_seq_stride;  /* >= compressed_cap, or >= 16 * compressed_cap and a
                                        multiple of 16 for MXFP4 (ignored when paged) */
  const float* window_scales;
  int64_t window_scales_seq_stride;  /* >= window_cap */
} sa_cache;

/* Validate `params` and create a plan (host memory owned by the library,
 * immutable, shareable across threads and streams). `*workspace_bytes`
 * receives the device workspace size that select_topk and sparse_attn_fwd
 * need for T = max_queries; concurrent calls need separate workspaces.
 * A workspace holds a select area (scratch between calls) and an attention
 * area (used by batches of at most 32 queries) whose counters must
 * be zero before a call: zero them once with sparse_attn_workspace_init after
 * allocating; every sparse_attn_fwd call leaves them zero again. */
sa_status sparse_attn_plan(const sa_params* params, sa_plan** plan, size_t* workspace_bytes);

void sparse_attn_plan_destroy(sa_plan* plan);

/* Zero the attention counters of a workspace of at least the plan's size (a
 * kernel on `stream`, so the call may be captured in a graph). Needed once per
 * allocation, before its first use by sparse_attn_fwd. Not a step of the
 * method: the library's own bookkeeping for sparse_attn_fwd's key splits. */
sa_status sparse_attn_workspace_init(const sa_plan* plan, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* sparse_attn_last_error(void);

/* S1. Indexer scores and block maxima.
 *   q_idx      device bf16 [T][16][128]   index query of each query
 *   w          device fp32 [T][16]        index head weights
 *   scores     device fp32 [T][ld_scores] out: scores[t][j] = I(j) for j < n_t,
 *              -inf for n_t <= j < E, with E = max_visible rounded up to 8;
 *              entries at j >= E are not written.  ld_scores >= E.
 *   block_max  device fp32 [T][ld_block_max] or NULL. out: the max of block
 *              b's visible scores for b < ceil(n_t/8), -inf for the rest of
 *              the first E/8 entries. ld_block_max >= E/8, a multiple of 4.
 *   ld_scores and ld_block_max must be multiples of 4 (rows start 16-byte
 *   aligned) and at most 2^26.
 * Launch limits (SA_EUNSUPPORTED beyond them, nothing enqueued): at most 65535
 * independent queries or groups per call, and at most 65535 * 16 queries in one
 * one-sequence batch or one run. */
sa_status indexer_score(const sa_plan* plan, const sa_queries* queries, const sa_cache* cache,
                        const void* q_idx, const float* w, float* scores, int64_t ld_scores,
                        float* block_max, int64_t ld_block_max, void* stream);

/* S0 + S1 in one launch (a decode step compresses the group each query completes, the
 * softmax-gate pooling of "deepseek-ai/DeepSeek-V4.1-Flash" recipe, Overview, two-tier
 * sparse attention bullet, and scores the index keys of that same bullet's indexer).
 * The compressor's work-groups ride in the indexer's grid (extra rows after the queries'),
 * so the step needs one launch fewer. A job holds the arguments of sparse_attn_compress
 * (bf16 plans) or of sparse_attn_compress_codes (e4m3 and MXFP4 plans), with their meaning
 * and rules; out_scales and scales_group_stride are read for code-row plans only. */
typedef struct sa_compress_job {
  const void* raw;
  int64_t raw_group_stride;
  const void* gate;
  int64_t gate_group_stride;
  const float* slot_bias;
  void* out;
  int64_t out_group_stride;
  void* out_scales;
  int64_t scales_group_stride;
  int64_t G;
} sa_compress_job;

/* Results: those of the compressor with *job's arguments followed by indexer_score with
 * the others, on `stream`, with the same checks and errors (nothing is enqueued when any
 * check fails). The job's outputs must not overlap anything the indexer reads or writes.
 * job NULL or job->G = 0: indexer_score. Ragged batches (sa_queries.runs) take the job in
 * their first launch; a job whose rows would not fit the grid, or a batch with no visible
 * keys, runs it in a launch of its own, first. */
sa_status indexer_score_compress(const sa_plan* plan, const sa_queries* queries, const sa_cache* cache,
                                 const void* q_idx, const float* w, float* scores, int64_t ld_scores,
                                 float* block_max, int64_t ld_block_max, const sa_compress_job* job,
                                 void* stream);

/* S2 + S3. Candidate blocks, then the top-512 positions inside them.
 *   scores, ld_scores      as written by indexer_score (same limits on the strides)
 *   block_max              as written by indexer_score, or NULL (then the block
 *                          maxima are recomputed from scores)
 *   cand       device int32 [T][2048] or NULL: out, the kept block ids of each
 *              query in ascending order, -1 after the last one (ceil(n_t/8)
 *              blocks are kept when there are at most 2048). NULL keeps them
 *              in the workspace only.
 *   topk       device int32 [T][512]: out, the selected positions in ascending
 *              order, -1 after the last one (min(512, n_t) are selected).
 *   workspace  device, >= the size reported by sparse_attn_plan; used for the
 *              candidate blocks when cand is NULL and, for queries longer than
 *              65536 positions, for per-part candidate lists (the candidate stage then
 *              runs in two levels over parts of 8192 blocks, 16384 past 524288
 *              positions). Such long rows allow at most 65535 queries per call
 *              (SA_EUNSUPPORTED beyond, nothing enqueued). */
sa_status select_topk(const sa_plan* plan, const sa_queries* queries, const float* scores,
                      int64_t ld_scores, const float* block_max, int64_t ld_block_max,
                      int32_t* cand, int32_t* topk, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Candidate-bounded re-scoring (layers that only index re-score the candidate blocks an
 * earlier layer's candidate stage kept; the pages' candidate stage selecting 2048 blocks of
 * 8, "deepseek-ai/DeepSeek-V4.1-Flash" recipe, Overview, two-tier sparse attention bullet).
 * S1 over the visible positions of the carried blocks only, with this query's own index
 * heads and weights; one stream of 2 KB (bf16), 1 KB (e4m3) or 512-byte (MXFP4) blocks per
 * query.
 *   cand       device int32 [T][2048]: carried block ids, ascending, -1 after the last
 *              (the layout select_topk writes); 16-byte aligned. An entry outside
 *              [0, ceil(n_t / 8)) is an empty slot (its entries are -inf).
 *   scores     device fp32 [T][ld_scores] out, slot order: scores[t][8i + r] = I(8 cand[t][i] + r)
 *              when cand[t][i] >= 0 and that position is visible, -inf otherwise, for
 *              every i < 2048 (entries past 16384 are not written). ld_scores >= 16384.
 *   block_max  device fp32 [T][ld_block_max] out: the max of slot i's 8 entries.
 *              ld_block_max >= 2048. Both strides multiples of 4, at most 2^26.
 * Other arguments as for indexer_score; T <= 65535. */
sa_status indexer_score_cand(const sa_plan* plan, const sa_queries* queries, const sa_cache* cache,
                             const void* q_idx, const float* w, const int32_t* cand, float* scores,
                             int64_t ld_scores, float* block_max, int64_t ld_block_max, void* stream);

/* S3 inside carried candidates: the min(512, m) best of the m re-scored visible positions by
 * (score desc, position asc), written ascending to topk[t][0..), -1 after the last. The
 * 512 best slots by (slot max desc, block id asc) are found first and only their positions
 * are ranked (they hold the 512 best positions).
 *   cand, scores, block_max  as passed to / written by indexer_score_cand. */
sa_status select_topk_cand(const sa_plan* plan, const sa_queries* queries, const int32_t* cand,
                           const float* scores, int64_t ld_scores, const float* block_max,
                           int64_t ld_block_max, int32_t* topk, void* stream);

/* S4. Joint-softmax attention over the selected latents and the window.
 *   q      device bf16 [T][64][512]
 *   topk   device int32 [T][512]: positions into the sequence's compressed store;
 *          entries outside [0, n_t) are skipped
 *   out    device bf16 [T][64][512]: out, per-head attention output
 *   lse    device fp32 [T][64] or NULL: out, natural-log sum of exp of the
 *          scaled logits (max + log of the normaliser)
 *   workspace  device or NULL. With T <= 32 and a workspace of the plan's
 *          size (counters zeroed, see sparse_attn_workspace_init), each query's
 *          key list is split over 4 work-groups per head set (two head sets for
 *          T <= 16) whose
 *          partial softmax results are combined at the end (the probabilities are
 *          rounded to bf16 against each part's own reference, so the output may
 *          differ from the unsplit one by that rounding; it is the same for every
 *          call); otherwise the query's heads are taken by one work-group, or by
 *          two (33 to 128 queries). */
sa_status sparse_attn_fwd(const sa_plan* plan, const sa_queries* queries, const sa_cache* cache,
                          const void* q, const int32_t* topk, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* sparse_attn_fwd for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, serving loops that forbid allocation). Same arguments,
 * checks, results and limits as sparse_attn_fwd with a workspace of the plan's size;
 * batches of at most 32 queries keep their key-split state in a fixed array of
 * 16.1 MiB that the library holds on each GPU it runs on until the process ends,
 * instead of a workspace (larger batches use no scratch memory). The call allocates and
 * frees nothing: it enqueues a kernel that zeroes the array's per-query counters and the
 * attention kernel on `stream`. Calls that overlap on one GPU (other streams, other
 * threads) share the array and race; serialise them. The first call on each GPU looks up
 * that GPU's copy of the array (hipGetSymbolAddress) and must not run under graph capture.
 * SA_EUNSUPPORTED if a batch's key splits would not fit the array; SA_EHIP if the lookup
 * or a launch fails. */
sa_status sparse_attn_fwd_noalloc(const sa_plan* plan, const sa_queries* queries, const sa_cache* cache,
                                  const void* q, const int32_t* topk, void* out, float* lse,
                                  void* stream);

/* S0. Softmax-gate compressor over G groups of `ratio` raw latents.
 * Group g reads raw rows raw + g*raw_group_stride + k*512 and gate logits
 * gate + g*gate_group_stride + k*512 (k < ratio, bf16), and writes
 * out + g*out_group_stride (bf16, round to nearest even):
 *   out[c] = sum_k softmax_k(gate[k][c] + slot_bias[k][c]) * raw[k][c].
 * slot_bias: device fp32 [ratio][512]. For ratio 1 the output is the raw row.
 * Output rows must not overlap input rows. */
sa_status sparse_attn_compress(const sa_plan* plan, const void* raw, int64_t raw_group_stride,
                               const void* gate, int64_t gate_group_stride,
                               const float* slot_bias, void* out, int64_t out_group_stride,
                               int64_t G, void* stream);

/* S0 into code rows: the compressor above, its fp32 result quantised into the e4m3 or MXFP4
 * latent store of the plan's kv_dtype (the FP8 and FP4 caches named in the Miles Day-0
 * Support table of "SGLang and Miles Add Day-0 Support for DeepSeek-V4.1"; bf16 plans return
 * SA_EUNSUPPORTED). raw, gate, slot_bias and their
 * strides as for sparse_attn_compress. Group g writes its code row at out + g*out_group_stride
 * and its scales at out_scales + g*scales_group_stride (both strides in bytes):
 *   SA_KV_FP8_E4M3: 512 e4m3 codes and one fp32 scale s = amax / 448 over the row (1 if the
 *     row is zero); code = nearest e4m3 of x / s, ties to the even code.
 *   SA_KV_MXFP4: 256 bytes of E2M1 (element 2i in the low nibble of byte i) and 16 E8M0
 *     bytes; block b (elements 32b .. 32b+31) has exponent X = floor(log2 amax_b) - 2
 *     (-127 if the block is zero, clamped to [-127, 127]), stored as X + 127; element =
 *     nearest E2M1 of x * 2^-X, ties to the even code, saturating at 6.
 * x is the compressor's fp32 value; divisions are IEEE fp32. out must be 16-byte aligned,
 * out_group_stride >= the row bytes (512 or 256) and a multiple of 16; out_scales 4-byte
 * aligned, scales_group_stride >= 4 (e4m3) or 16 (MXFP4) and a multiple of 4. Outputs must
 * not overlap inputs. */
sa_status sparse_attn_compress_codes(const sa_plan* plan, const void* raw, int64_t raw_group_stride,
                                     const void* gate, int64_t gate_group_stride,
                                     const float* slot_bias, void* out, int64_t out_group_stride,
                                     void* out_scales, int64_t scales_group_stride, int64_t G,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
