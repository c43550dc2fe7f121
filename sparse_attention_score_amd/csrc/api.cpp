// C ABI of the sparse-attention library: argument checks, plan and workspace sizing,
// kernel dispatch. Every check runs on the host before any HIP call, no C++ exception
// leaves this file, and nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <new>

#include "../../include/sparse_attn.h"
#include "sa_launch.h"

struct sa_plan {
  sa_params p;
  size_t workspace;
};

namespace {

thread_local char g_err[512] = "";

sa_status fail(sa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sa_status ok() {
  g_err[0] = '\0';
  return SA_OK;
}

// SPARSE_ATTN_LOG=1 in the environment: one line on stderr per accepted call, naming the
// kernel path and launch shape it takes (read once; host only, nothing on the device).
bool log_on() {
  static const bool on = [] {
    const char* e = std::getenv("SPARSE_ATTN_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

void log_call(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[384];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[sparse_attn] %s\n", buf);
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

constexpr int64_t kMaxVisible = 1LL << 20;        // 1,048,576 positions: 131072 blocks, 8 parts
                                                   // of 16384 for the two-level candidate stage
constexpr int kMaxGroup = 8;                        // queries per group sharing one key stream
constexpr int64_t kMaxGridY = 65535;               // grid y holds queries, groups or query tiles
constexpr int64_t kMaxLd = 1LL << 26;              // row strides of scores / block maxima: two rows
                                                   // stay addressable by 32-bit buffer offsets

size_t cand_bytes(int64_t T) { return (size_t)T * 2048 * sizeof(int32_t); }
// Part lists of the two-level candidate stage (queries longer than 8192 blocks).
size_t part_bytes(int64_t T, int64_t max_visible) {
  const int parts = sa::select_parts(max_visible).parts;
  return parts > 1 ? (size_t)T * parts * 2048 * (sizeof(int32_t) + sizeof(uint32_t)) : 0;   // ids, keys
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace layout: [select area][attention area]. The select area holds the candidate
// blocks (when cand is NULL) and the part lists; the attention area holds one counter per
// query (zero between calls) and the partial results of key splits.
struct WsLayout {
  size_t select_bytes, counters_off, ml_off, o_off, total;
  int64_t units;
};
WsLayout ws_layout(const sa_params& p) {
  WsLayout w;
  w.select_bytes = cand_bytes(p.max_queries) + part_bytes(p.max_queries, p.max_compressed);
  w.units = sa::attn_max_units(p.max_queries);
  w.counters_off = align256(w.select_bytes);
  w.ml_off = w.counters_off + align256((size_t)p.max_queries * 2 * sizeof(uint32_t));   // per (query, head set)
  w.o_off = w.ml_off + align256((size_t)w.units * 64 * 2 * sizeof(float));
  w.total = w.units > 0 ? w.o_off + (size_t)w.units * 64 * 512 * sizeof(float) : w.select_bytes;
  return w;
}

sa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define SA_REQUIRE(cond, st, ...)              \
  do {                                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

sa_status check_plan(const sa_plan* plan) {
  SA_REQUIRE(plan != nullptr, SA_EINVAL, "plan is NULL");
  return SA_OK;
}

sa_status check_queries(const sa_plan* plan, const sa_queries* q) {
  SA_REQUIRE(q != nullptr, SA_EINVAL, "queries is NULL");
  SA_REQUIRE(q->T >= 1 && q->T <= plan->p.max_queries, SA_EINVAL,
             "queries->T = %lld outside [1, max_queries = %lld]", (long long)q->T,
             (long long)plan->p.max_queries);
  SA_REQUIRE(q->T <= 65535LL * 1024, SA_EUNSUPPORTED, "T = %lld too large", (long long)q->T);
  SA_REQUIRE(q->seq_id != nullptr && q->pos != nullptr, SA_EINVAL, "queries seq_id/pos is NULL");
  SA_REQUIRE(q->max_visible >= 0 && q->max_visible <= plan->p.max_compressed, SA_EINVAL,
             "queries->max_visible = %lld outside [0, max_compressed = %lld]",
             (long long)q->max_visible, (long long)plan->p.max_compressed);
  SA_REQUIRE(q->group >= 0 && q->group <= kMaxGroup, SA_EUNSUPPORTED,
             "queries->group = %d outside [0, %d]", (int)q->group, kMaxGroup);
  if (q->runs) {
    SA_REQUIRE(q->num_runs >= 1, SA_EINVAL, "queries->num_runs = %d < 1", (int)q->num_runs);
    int64_t sum = 0;
    for (int32_t i = 0; i < q->num_runs; ++i) {
      SA_REQUIRE(q->runs[i] >= 1, SA_EINVAL, "queries->runs[%d] = %d < 1", (int)i, (int)q->runs[i]);
      sum += q->runs[i];
    }
    SA_REQUIRE(sum == q->T, SA_EINVAL, "queries->runs sum to %lld, not T = %lld", (long long)sum,
               (long long)q->T);
  }
  return SA_OK;
}

sa::PageTable page_table(const sa_cache* c) {
  sa::PageTable pt;
  pt.table = c->block_table;
  pt.stride = c->block_table_stride;
  pt.log2_page = 0;
  while (c->block_table && (1 << pt.log2_page) < c->page_size) ++pt.log2_page;
  pt.num_pages = c->num_pages;
  return pt;
}

sa_status check_cache(const sa_plan* plan, const sa_queries* q, const sa_cache* c, bool keys,
                      bool latents) {
  SA_REQUIRE(c != nullptr, SA_EINVAL, "cache is NULL");
  SA_REQUIRE(c->num_seqs >= 1, SA_EINVAL, "cache->num_seqs must be >= 1");
  SA_REQUIRE(c->compressed_cap >= 0, SA_EINVAL, "cache->compressed_cap < 0");
  SA_REQUIRE(q->max_visible <= c->compressed_cap, SA_EINVAL,
             "queries->max_visible = %lld exceeds cache->compressed_cap = %lld",
             (long long)q->max_visible, (long long)c->compressed_cap);
  const bool paged = c->block_table != nullptr;
  if (paged) {
    SA_REQUIRE(reinterpret_cast<uintptr_t>(c->block_table) % 4 == 0, SA_EINVAL,
               "cache->block_table not 4-byte aligned");
    SA_REQUIRE(c->page_size >= 16 && c->page_size <= (1 << 20) && (c->page_size & (c->page_size - 1)) == 0,
               SA_EINVAL, "cache->page_size = %d must be a power of two in [16, 2^20]", (int)c->page_size);
    SA_REQUIRE(c->num_pages >= 1 && c->num_pages <= INT32_MAX, SA_EINVAL,
               "cache->num_pages = %lld invalid", (long long)c->num_pages);
    SA_REQUIRE(c->block_table_stride >= (c->compressed_cap + c->page_size - 1) / c->page_size, SA_EINVAL,
               "cache->block_table_stride = %lld < pages of compressed_cap", (long long)c->block_table_stride);
  }
  if (keys) {
    SA_REQUIRE(c->idx_keys != nullptr && aligned16(c->idx_keys), SA_EINVAL,
               "cache->idx_keys is NULL or not 16-byte aligned");
    // stride unit: bf16 elements, e4m3 bytes, or MXFP4 bytes (64 per row); 16-byte rows
    const bool mx = plan->p.idx_key_dtype == SA_KEY_MXFP4;
    const int64_t rowmul = plan->p.idx_key_dtype == SA_KEY_BF16 ? 8 : 16;
    const int64_t rowunits = mx ? 64 : 128;
    SA_REQUIRE(paged || (c->idx_keys_seq_stride >= c->compressed_cap * rowunits && c->idx_keys_seq_stride % rowmul == 0),
               SA_EINVAL, "cache->idx_keys_seq_stride = %lld invalid", (long long)c->idx_keys_seq_stride);
    if (mx) {
      SA_REQUIRE(c->idx_scales != nullptr && reinterpret_cast<uintptr_t>(c->idx_scales) % 4 == 0, SA_EINVAL,
                 "cache->idx_scales is NULL or not 4-byte aligned (required for MXFP4 keys)");
      SA_REQUIRE(paged || (c->idx_scales_seq_stride >= c->compressed_cap * 4 && c->idx_scales_seq_stride % 4 == 0),
                 SA_EINVAL, "cache->idx_scales_seq_stride = %lld must be >= 4 * compressed_cap and a multiple of 4",
                 (long long)c->idx_scales_seq_stride);
    }
    if (plan->p.idx_key_dtype == SA_KEY_FP8_E4M3) {
      SA_REQUIRE(c->idx_scales != nullptr && aligned16(c->idx_scales), SA_EINVAL,
                 "cache->idx_scales is NULL or misaligned (required for e4m3 keys)");
      SA_REQUIRE(paged || c->idx_scales_seq_stride >= c->compressed_cap, SA_EINVAL,
                 "cache->idx_scales_seq_stride = %lld < compressed_cap",
                 (long long)c->idx_scales_seq_stride);
    }
  }
  if (latents) {
    SA_REQUIRE(c->latents != nullptr && aligned16(c->latents), SA_EINVAL,
               "cache->latents is NULL or not 16-byte aligned");
    // strides: bf16 elements, or bytes for code rows (16-byte rows either way): latent rows
    // of 512 elements (256 bytes for MXFP4), window rows of 512
    const bool kv8 = plan->p.kv_dtype != SA_KV_BF16, fp4l = plan->p.kv_dtype == SA_KV_MXFP4;
    const int64_t smul = kv8 ? 16 : 8, lrow = fp4l ? 256 : 512;
    SA_REQUIRE(paged || (c->latents_seq_stride >= c->compressed_cap * lrow && c->latents_seq_stride % smul == 0),
               SA_EINVAL, "cache->latents_seq_stride = %lld invalid", (long long)c->latents_seq_stride);
    if (kv8) {
      SA_REQUIRE(c->latent_scales != nullptr && c->window_scales != nullptr, SA_EINVAL,
                 "cache->latent_scales / window_scales NULL (required for e4m3 and MXFP4 latents)");
      if (fp4l) {
        SA_REQUIRE(aligned16(c->latent_scales), SA_EINVAL, "cache->latent_scales not 16-byte aligned (MXFP4 latents)");
        SA_REQUIRE(paged || (c->latent_scales_seq_stride >= 16 * c->compressed_cap &&
                             c->latent_scales_seq_stride % 16 == 0),
                   SA_EINVAL, "cache->latent_scales_seq_stride = %lld must be >= 16 * compressed_cap and a multiple of 16",
                   (long long)c->latent_scales_seq_stride);
      } else {
        SA_REQUIRE(paged || c->latent_scales_seq_stride >= c->compressed_cap, SA_EINVAL,
                   "cache->latent_scales_seq_stride = %lld < compressed_cap", (long long)c->latent_scales_seq_stride);
      }
      SA_REQUIRE(c->window_scales_seq_stride >= c->window_cap, SA_EINVAL,
                 "cache->window_scales_seq_stride = %lld < window_cap", (long long)c->window_scales_seq_stride);
    }
    SA_REQUIRE(c->window != nullptr && aligned16(c->window), SA_EINVAL,
               "cache->window is NULL or not 16-byte aligned");
    SA_REQUIRE(c->window_cap >= plan->p.window, SA_EINVAL, "cache->window_cap = %d < window %d",
               c->window_cap, plan->p.window);
    SA_REQUIRE(c->window_seq_stride >= (int64_t)c->window_cap * 512 && c->window_seq_stride % smul == 0,
               SA_EINVAL, "cache->window_seq_stride = %lld invalid", (long long)c->window_seq_stride);
  }
  return SA_OK;
}

sa::QueryMeta meta(const sa_plan* plan, const sa_queries* q, int64_t num_seqs, int64_t cap) {
  sa::QueryMeta m;
  m.seq_id = q->seq_id;
  m.pos = q->pos;
  m.T = q->T;
  m.max_visible = q->max_visible;
  m.num_seqs = num_seqs;
  m.compressed_cap = cap;
  m.ratio = plan->p.ratio;
  return m;
}

int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

// Fewest distinct positions the queries of one sequence in this call can span, as far as
// the host knows it: a run's length, a group's size, T for a batch over one sequence.
int64_t min_window_span(const sa_queries* q, const sa_cache* c) {
  int64_t span = 1;
  if (q->runs) {
    for (int32_t i = 0; i < q->num_runs; ++i) span = q->runs[i] > span ? q->runs[i] : span;
  } else if (q->group > 1) {
    span = q->group < q->T ? q->group : q->T;
  }
  if (c->num_seqs == 1) span = q->T;
  return span;
}

// A ragged batch (sa_queries.runs): one launch per class of run over each contiguous
// query range of that class. Runs of 9+ queries go to the chunk kernel (one launch per
// run), neighbouring runs of one length in 2..8 to the group kernel, single queries (and
// runs the store layout keeps off those kernels) to the per-query kernel. The cursor walks
// the runs without allocating.
struct RunLaunch {
  int64_t t0, len;
  int kind;       // 0 per query, 1 group, 2 chunk
  int32_t group;  // queries per group (kind 1)
};

struct RunCursor {
  const sa_queries* q;
  bool chunk_ok, group_ok;
  int32_t i = 0;
  int64_t t0 = 0;
  int cls(int32_t len) const {
    return len >= 9 && chunk_ok ? 2 : (len >= 2 && len <= 8 && group_ok ? 1 : 0);
  }
  bool next(RunLaunch& r) {
    if (i >= q->num_runs) return false;
    const int k = cls(q->runs[i]);
    int32_t j = i + 1;
    int64_t len = q->runs[i];
    if (k != 2)
      while (j < q->num_runs && cls(q->runs[j]) == k && (k != 1 || q->runs[j] == q->runs[i])) len += q->runs[j++];
    r = RunLaunch{t0, len, k, k == 1 ? q->runs[i] : 1};
    t0 += len;
    i = j;
    return true;
  }
};

sa_status indexer_runs(const sa::IndexerArgs& a, const sa_queries* q, const sa_cache* c, const void* q_idx,
                       const float* w, hipStream_t stream) {
  const bool chunk_ok = !a.pages.table || c->page_size >= 64, group_ok = true;
  RunLaunch r;
  // per-query and group launches index queries in grid y
  for (RunCursor cur{q, chunk_ok, group_ok}; cur.next(r);) {
    SA_REQUIRE(r.kind == 2 || r.len / r.group <= kMaxGridY, SA_EUNSUPPORTED,
               "a range of %lld queries on the per-query or group kernel: at most 65535 per launch",
               (long long)r.len);
    SA_REQUIRE(r.kind != 2 || (r.len + sa::kChunkQueriesPerWG - 1) / sa::kChunkQueriesPerWG <= kMaxGridY,
               SA_EUNSUPPORTED, "a run of %lld queries: at most %lld per run", (long long)r.len,
               (long long)(kMaxGridY * sa::kChunkQueriesPerWG));
  }
  for (RunCursor cur{q, chunk_ok, group_ok}; cur.next(r);) {
    sa::IndexerArgs b = a;
    if (r.t0 > 0) b.cj.G = 0;   // a compressor job rides in the first launch only
    b.seq_id = a.seq_id + r.t0;
    b.pos = a.pos + r.t0;
    b.T = r.len;
    b.q_idx = static_cast<const uint16_t*>(q_idx) + r.t0 * 16 * 128;
    b.w = w + r.t0 * 16;
    b.scores = a.scores + r.t0 * a.ld_scores;
    b.block_max = a.block_max ? a.block_max + r.t0 * a.ld_block_max : nullptr;
    b.group = r.group;
    log_call("indexer_score run: queries %lld..%lld on the %s kernel%s", (long long)r.t0,
             (long long)(r.t0 + r.len - 1), r.kind == 2 ? "chunk" : r.kind == 1 ? "group" : "per-query",
             r.kind == 1 ? " (one key stream per group)" : "");
    const hipError_t e = sa::launch_indexer(b, r.kind == 2, stream);
    if (e != hipSuccess) return hip_status(e, "indexer_score launch");
  }
  return ok();
}

// Checks shared by the attention entry points; fills every field but the key-split state.
sa_status attn_args(const sa_plan* plan, const sa_queries* q, const sa_cache* c, const void* qv,
                    const int32_t* topk, void* out, float* lse, sa::AttnArgs& a) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  if ((st = check_queries(plan, q)) != SA_OK) return st;
  if ((st = check_cache(plan, q, c, false, true)) != SA_OK) return st;
  SA_REQUIRE(qv && aligned16(qv), SA_EINVAL, "q NULL or not 16-byte aligned");
  SA_REQUIRE(topk && aligned16(topk), SA_EINVAL, "topk NULL or not 16-byte aligned");
  SA_REQUIRE(out && aligned16(out), SA_EINVAL, "out NULL or not 16-byte aligned");
  SA_REQUIRE(lse == nullptr || aligned16(lse), SA_EINVAL, "lse not 16-byte aligned");
  // The window store is a ring (raw position u in row u % window_cap): the queries of one
  // sequence in one call need window_cap >= 127 + the positions they span. Checked where
  // the host knows a lower bound of that span: groups, runs, a one-sequence batch.
  const int64_t span = min_window_span(q, c);
  SA_REQUIRE(c->window_cap >= plan->p.window - 1 + span, SA_EINVAL,
             "cache->window_cap = %d: queries of one sequence spanning %lld positions need >= %lld "
             "(the window ring would overwrite rows they read)",
             c->window_cap, (long long)span, (long long)(plan->p.window - 1 + span));
  a.m = meta(plan, q, c->num_seqs, c->compressed_cap);
  a.pages = page_table(c);
  a.kv_mode = plan->p.kv_dtype;
  a.latent_scales = c->latent_scales;
  a.latent_scales_seq_stride = c->latent_scales_seq_stride;
  a.window_scales = c->window_scales;
  a.window_scales_seq_stride = c->window_scales_seq_stride;
  a.q = qv;
  a.topk = topk;
  a.latents = c->latents;
  a.latents_seq_stride = c->latents_seq_stride;
  a.window = c->window;
  a.window_seq_stride = c->window_seq_stride;
  a.window_cap = c->window_cap;
  a.scale = plan->p.softmax_scale;
  a.out = out;
  a.lse = lse;
  a.splits = 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.counters = nullptr;
  return ok();
}

// Checks of a compressor job (the arguments of sparse_attn_compress for bf16 plans, of
// sparse_attn_compress_codes for code-row plans); fills a.
sa_status compress_args(const sa_plan* plan, const void* raw, int64_t raw_group_stride, const void* gate,
                        int64_t gate_group_stride, const float* slot_bias, void* out, int64_t out_group_stride,
                        void* out_scales, int64_t scales_group_stride, int64_t G, sa::CompressArgs& a) {
  const int r = plan->p.ratio;
  const int kv = plan->p.kv_dtype;
  SA_REQUIRE(G >= 0 && G <= ((int64_t)1 << 31) - 1, SA_EINVAL, "G = %lld out of range", (long long)G);
  SA_REQUIRE(raw && aligned16(raw) && out && aligned16(out), SA_EINVAL,
             "raw / out NULL or not 16-byte aligned");
  SA_REQUIRE(raw_group_stride >= (int64_t)r * 512 && raw_group_stride % 8 == 0, SA_EINVAL,
             "raw_group_stride = %lld invalid", (long long)raw_group_stride);
  if (kv == SA_KV_BF16) {
    SA_REQUIRE(out_group_stride >= 512 && out_group_stride % 8 == 0, SA_EINVAL,
               "out_group_stride = %lld invalid", (long long)out_group_stride);
  } else {
    const int64_t row = kv == SA_KV_MXFP4 ? 256 : 512, srow = kv == SA_KV_MXFP4 ? 16 : 4;
    SA_REQUIRE(out_group_stride >= row && out_group_stride % 16 == 0, SA_EINVAL,
               "out_group_stride = %lld bytes must be >= %lld and a multiple of 16", (long long)out_group_stride,
               (long long)row);
    SA_REQUIRE(out_scales && reinterpret_cast<uintptr_t>(out_scales) % 4 == 0, SA_EINVAL,
               "out_scales NULL or not 4-byte aligned");
    SA_REQUIRE(scales_group_stride >= srow && scales_group_stride % 4 == 0, SA_EINVAL,
               "scales_group_stride = %lld bytes must be >= %lld and a multiple of 4",
               (long long)scales_group_stride, (long long)srow);
  }
  if (r == 2) {
    SA_REQUIRE(gate && aligned16(gate) && slot_bias && aligned16(slot_bias), SA_EINVAL,
               "gate / slot_bias NULL or not 16-byte aligned");
    SA_REQUIRE(gate_group_stride >= 1024 && gate_group_stride % 8 == 0, SA_EINVAL,
               "gate_group_stride = %lld invalid", (long long)gate_group_stride);
  }
  if (G > 0)
    log_call("compressor: %lld groups of %d rows into %s rows", (long long)G, r,
             kv == SA_KV_MXFP4 ? "mxfp4" : kv == SA_KV_FP8_E4M3 ? "e4m3" : "bf16");
  a.raw = raw;
  a.raw_stride = raw_group_stride;
  a.gate = gate;
  a.gate_stride = gate_group_stride;
  a.bias = slot_bias;
  a.out = out;
  a.out_stride = out_group_stride;
  a.G = G;
  a.ratio = r;
  a.kv_mode = kv;
  a.scales = kv == SA_KV_BF16 ? nullptr : out_scales;
  a.scales_stride = kv == SA_KV_BF16 ? 0 : scales_group_stride;
  return ok();
}

// indexer_score, with an optional compressor job (already checked) riding in its launch.
sa_status indexer_common(const sa_plan* plan, const sa_queries* q, const sa_cache* c, const void* q_idx,
                         const float* w, float* scores, int64_t ld_scores, float* block_max,
                         int64_t ld_block_max, const sa::CompressArgs* cj, void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  if ((st = check_queries(plan, q)) != SA_OK) return st;
  if ((st = check_cache(plan, q, c, true, false)) != SA_OK) return st;
  SA_REQUIRE(q_idx && aligned16(q_idx) && w && aligned16(w), SA_EINVAL,
             "q_idx / w NULL or not 16-byte aligned");
  SA_REQUIRE(scores && aligned16(scores), SA_EINVAL, "scores NULL or not 16-byte aligned");
  const int64_t E = round8(q->max_visible);
  SA_REQUIRE(ld_scores >= E && ld_scores % 4 == 0 && ld_scores <= kMaxLd, SA_EINVAL,
             "ld_scores = %lld must be >= %lld (max_visible rounded up to 8), <= %lld and a multiple of 4",
             (long long)ld_scores, (long long)E, (long long)kMaxLd);
  if (block_max) {
    SA_REQUIRE(aligned16(block_max), SA_EINVAL, "block_max not 16-byte aligned");
    SA_REQUIRE(ld_block_max >= E / 8 && ld_block_max % 4 == 0 && ld_block_max <= kMaxLd, SA_EINVAL,
               "ld_block_max = %lld must be >= %lld, <= %lld and a multiple of 4",
               (long long)ld_block_max, (long long)(E / 8), (long long)kMaxLd);
  }
  if (E == 0) {
    if (!cj) return ok();
    return hip_status(sa::launch_compress(*cj, (hipStream_t)stream), "indexer_score_compress launch");
  }
  sa::IndexerArgs a;
  a.seq_id = q->seq_id;
  a.pos = q->pos;
  a.T = q->T;
  a.max_visible = q->max_visible;
  a.num_seqs = c->num_seqs;
  a.compressed_cap = c->compressed_cap;
  a.ratio = plan->p.ratio;
  a.fp8 = plan->p.idx_key_dtype == SA_KEY_FP8_E4M3;
  a.mxfp4 = plan->p.idx_key_dtype == SA_KEY_MXFP4;
  a.q_idx = q_idx;
  a.w = w;
  a.keys = c->idx_keys;
  a.keys_seq_stride = c->idx_keys_seq_stride;
  a.scales = static_cast<const float*>(c->idx_scales);
  a.scales_seq_stride = c->idx_scales_seq_stride;
  a.scores = scores;
  a.ld_scores = ld_scores;
  a.block_max = block_max;
  a.ld_block_max = ld_block_max;
  a.E = E;
  a.cand = nullptr;
  a.group = q->group > 1 ? q->group : 1;
  a.pages = page_table(c);
  if (cj) a.cj = *cj;   // its work-groups join the (first) indexer launch
  // paged stores: the chunk kernel needs pages of at least one 64-key stage
  // Queries that share a sequence in one call (a prefill chunk) reuse each key tile
  // across many queries; groups of a multi-token decode step share one key stream per
  // group; independent decode queries each stream their own keys.
  if (q->runs) return indexer_runs(a, q, c, q_idx, w, (hipStream_t)stream);
  const bool prefill = (!a.pages.table || c->page_size >= 64) && a.group == 1 && c->num_seqs == 1 && q->T > 1;
  SA_REQUIRE(prefill || (q->T + a.group - 1) / a.group <= kMaxGridY, SA_EUNSUPPORTED,
             "T = %lld queries in groups of %d over several sequences: at most 65535 groups per call",
             (long long)q->T, (int)a.group);
  SA_REQUIRE(!prefill || (q->T + sa::kChunkQueriesPerWG - 1) / sa::kChunkQueriesPerWG <= kMaxGridY,
             SA_EUNSUPPORTED, "T = %lld queries of one sequence: at most %lld per call", (long long)q->T,
             (long long)(kMaxGridY * sa::kChunkQueriesPerWG));
  log_call("indexer_score: T=%lld max_visible=%lld E=%lld keys=%s %s%s kernel, group %d", (long long)q->T,
           (long long)q->max_visible, (long long)E, a.mxfp4 ? "mxfp4" : a.fp8 ? "e4m3" : "bf16",
           a.pages.table ? "paged " : "", prefill ? "chunk" : a.group > 1 ? "group" : "per-query", (int)a.group);
  return hip_status(sa::launch_indexer(a, prefill, (hipStream_t)stream), "indexer_score launch");
}

}  // namespace

extern "C" {

const char* sparse_attn_last_error(void) { return g_err; }

sa_status sparse_attn_plan(const sa_params* p, sa_plan** plan, size_t* workspace_bytes) {
  SA_REQUIRE(p != nullptr && plan != nullptr, SA_EINVAL, "params or plan is NULL");
  *plan = nullptr;
  SA_REQUIRE(p->num_heads == 64 && p->latent_dim == 512 && p->window == 128 && p->topk == 512 &&
                 p->idx_heads == 16 && p->idx_dim == 128 && p->block == 8 && p->cand_blocks == 2048,
             SA_EUNSUPPORTED,
             "unsupported dims (need heads 64, latent 512, window 128, topk 512, idx 16x128, "
             "block 8, cand_blocks 2048)");
  SA_REQUIRE(p->ratio == 1 || p->ratio == 2, SA_EUNSUPPORTED, "ratio %d not in {1, 2}", p->ratio);
  SA_REQUIRE(p->idx_key_dtype == SA_KEY_BF16 || p->idx_key_dtype == SA_KEY_FP8_E4M3 ||
                 p->idx_key_dtype == SA_KEY_MXFP4,
             SA_EUNSUPPORTED, "idx_key_dtype %d unknown", p->idx_key_dtype);
  SA_REQUIRE(p->kv_dtype == SA_KV_BF16 || p->kv_dtype == SA_KV_FP8_E4M3 || p->kv_dtype == SA_KV_MXFP4,
             SA_EUNSUPPORTED,
             "kv_dtype %d unknown", p->kv_dtype);
  SA_REQUIRE(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f, SA_EINVAL,
             "softmax_scale must be finite and > 0");
  SA_REQUIRE(p->max_queries >= 1, SA_EINVAL, "max_queries must be >= 1");
  SA_REQUIRE(p->max_compressed >= 0, SA_EINVAL, "max_compressed must be >= 0");
  SA_REQUIRE(p->max_compressed <= kMaxVisible, SA_EUNSUPPORTED,
             "max_compressed %lld above the supported %lld", (long long)p->max_compressed,
             (long long)kMaxVisible);
  sa_plan* pl = new (std::nothrow) sa_plan;
  SA_REQUIRE(pl != nullptr, SA_EINVAL, "out of host memory");
  pl->p = *p;
  pl->workspace = ws_layout(*p).total;
  *plan = pl;
  if (workspace_bytes) *workspace_bytes = pl->workspace;
  return ok();
}

void sparse_attn_plan_destroy(sa_plan* plan) { delete plan; }

sa_status indexer_score(const sa_plan* plan, const sa_queries* q, const sa_cache* c,
                        const void* q_idx, const float* w, float* scores, int64_t ld_scores,
                        float* block_max, int64_t ld_block_max, void* stream) {
  return indexer_common(plan, q, c, q_idx, w, scores, ld_scores, block_max, ld_block_max, nullptr, stream);
}

sa_status indexer_score_cand(const sa_plan* plan, const sa_queries* q, const sa_cache* c,
                             const void* q_idx, const float* w, const int32_t* cand, float* scores,
                             int64_t ld_scores, float* block_max, int64_t ld_block_max, void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  if ((st = check_queries(plan, q)) != SA_OK) return st;
  if ((st = check_cache(plan, q, c, true, false)) != SA_OK) return st;
  SA_REQUIRE(c->block_table == nullptr, SA_EUNSUPPORTED,
             "candidate-bounded re-scoring reads contiguous stores only");
  SA_REQUIRE(q_idx && aligned16(q_idx) && w && aligned16(w), SA_EINVAL,
             "q_idx / w NULL or not 16-byte aligned");
  SA_REQUIRE(cand && aligned16(cand), SA_EINVAL, "cand NULL or not 16-byte aligned");
  SA_REQUIRE(scores && aligned16(scores), SA_EINVAL, "scores NULL or not 16-byte aligned");
  SA_REQUIRE(block_max && aligned16(block_max), SA_EINVAL, "block_max NULL or not 16-byte aligned");
  constexpr int64_t E = 2048LL * 8;
  SA_REQUIRE(ld_scores >= E && ld_scores % 4 == 0 && ld_scores <= kMaxLd, SA_EINVAL,
             "ld_scores = %lld must be >= %lld, <= %lld and a multiple of 4", (long long)ld_scores,
             (long long)E, (long long)kMaxLd);
  SA_REQUIRE(ld_block_max >= 2048 && ld_block_max % 4 == 0 && ld_block_max <= kMaxLd, SA_EINVAL,
             "ld_block_max = %lld must be >= 2048, <= %lld and a multiple of 4", (long long)ld_block_max,
             (long long)kMaxLd);
  SA_REQUIRE(q->T <= kMaxGridY, SA_EUNSUPPORTED, "T = %lld: at most 65535 queries per call", (long long)q->T);
  sa::IndexerArgs a;
  a.seq_id = q->seq_id;
  a.pos = q->pos;
  a.T = q->T;
  a.max_visible = q->max_visible;
  a.num_seqs = c->num_seqs;
  a.compressed_cap = c->compressed_cap;
  a.ratio = plan->p.ratio;
  a.fp8 = plan->p.idx_key_dtype == SA_KEY_FP8_E4M3;
  a.mxfp4 = plan->p.idx_key_dtype == SA_KEY_MXFP4;
  a.q_idx = q_idx;
  a.w = w;
  a.keys = c->idx_keys;
  a.keys_seq_stride = c->idx_keys_seq_stride;
  a.scales = static_cast<const float*>(c->idx_scales);
  a.scales_seq_stride = c->idx_scales_seq_stride;
  a.scores = scores;
  a.ld_scores = ld_scores;
  a.block_max = block_max;
  a.ld_block_max = ld_block_max;
  a.E = E;
  a.cand = cand;
  a.group = 1;
  a.pages = sa::PageTable{nullptr, 0, 0, 0};
  log_call("indexer_score_cand: T=%lld, 2048 carried blocks per query, keys=%s", (long long)q->T,
           a.mxfp4 ? "mxfp4" : a.fp8 ? "e4m3" : "bf16");
  return hip_status(sa::launch_indexer(a, false, (hipStream_t)stream), "indexer_score_cand launch");
}

sa_status select_topk_cand(const sa_plan* plan, const sa_queries* q, const int32_t* cand,
                           const float* scores, int64_t ld_scores, const float* block_max,
                           int64_t ld_block_max, int32_t* topk, void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  if ((st = check_queries(plan, q)) != SA_OK) return st;
  SA_REQUIRE(cand && aligned16(cand), SA_EINVAL, "cand NULL or not 16-byte aligned");
  SA_REQUIRE(scores && aligned16(scores), SA_EINVAL, "scores NULL or not 16-byte aligned");
  SA_REQUIRE(block_max && aligned16(block_max), SA_EINVAL, "block_max NULL or not 16-byte aligned");
  SA_REQUIRE(topk && aligned16(topk), SA_EINVAL, "topk NULL or not 16-byte aligned");
  SA_REQUIRE(ld_scores >= 2048LL * 8 && ld_scores % 4 == 0 && ld_scores <= kMaxLd, SA_EINVAL,
             "ld_scores = %lld must be >= 16384, <= %lld and a multiple of 4", (long long)ld_scores,
             (long long)kMaxLd);
  SA_REQUIRE(ld_block_max >= 2048 && ld_block_max % 4 == 0 && ld_block_max <= kMaxLd, SA_EINVAL,
             "ld_block_max = %lld must be >= 2048, <= %lld and a multiple of 4", (long long)ld_block_max,
             (long long)kMaxLd);
  sa::SelectArgs a;
  a.m = meta(plan, q, INT32_MAX, q->max_visible);
  a.scores = scores;
  a.ld_scores = ld_scores;
  a.block_max = block_max;
  a.ld_block_max = ld_block_max;
  a.cand = const_cast<int32_t*>(cand);   // read only in this mode
  a.topk = topk;
  a.part_ids = nullptr;
  a.part_keys = nullptr;
  a.parts = 1;
  a.part_blocks = sa::kPartBlocks;
  log_call("select_topk_cand: T=%lld", (long long)q->T);
  return hip_status(sa::launch_select_cand(a, (hipStream_t)stream), "select_topk_cand launch");
}

sa_status select_topk(const sa_plan* plan, const sa_queries* q, const float* scores,
                      int64_t ld_scores, const float* block_max, int64_t ld_block_max,
                      int32_t* cand, int32_t* topk, void* workspace, size_t workspace_bytes,
                      void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  if ((st = check_queries(plan, q)) != SA_OK) return st;
  const int64_t E = round8(q->max_visible);
  SA_REQUIRE(scores && aligned16(scores), SA_EINVAL, "scores NULL or not 16-byte aligned");
  SA_REQUIRE(ld_scores >= E && ld_scores % 4 == 0 && ld_scores <= kMaxLd, SA_EINVAL,
             "ld_scores = %lld must be >= %lld, <= %lld and a multiple of 4", (long long)ld_scores,
             (long long)E, (long long)kMaxLd);
  if (block_max) {
    SA_REQUIRE(aligned16(block_max), SA_EINVAL, "block_max not 16-byte aligned");
    SA_REQUIRE(ld_block_max >= E / 8 && ld_block_max % 4 == 0 && ld_block_max <= kMaxLd, SA_EINVAL,
               "ld_block_max = %lld must be >= %lld, <= %lld and a multiple of 4",
               (long long)ld_block_max, (long long)(E / 8), (long long)kMaxLd);
  }
  SA_REQUIRE(topk && aligned16(topk), SA_EINVAL, "topk NULL or not 16-byte aligned");
  if (cand) SA_REQUIRE(aligned16(cand), SA_EINVAL, "cand not 16-byte aligned");
  // workspace: [cand_bytes(T)] candidate blocks when cand is NULL, then the part lists
  const size_t parts_need = part_bytes(q->T, q->max_visible);
  if (!cand || parts_need) {
    const size_t need = cand_bytes(q->T) + parts_need;
    SA_REQUIRE(workspace != nullptr && aligned16(workspace), SA_EWORKSPACE,
               "workspace NULL or misaligned (needed when cand is NULL or max_visible > %d)",
               sa::kPartBlocks * 8);
    SA_REQUIRE(workspace_bytes >= need, SA_EWORKSPACE, "workspace_bytes = %zu < %zu", workspace_bytes, need);
  }
  const sa::PartSplit ps = sa::select_parts(q->max_visible);
  SA_REQUIRE(ps.parts <= 1 || q->T <= kMaxGridY, SA_EUNSUPPORTED,
             "T = %lld queries longer than %d positions: at most 65535 per call", (long long)q->T,
             sa::kPartBlocks * 8);
  if (!cand) cand = static_cast<int32_t*>(workspace);
  sa::SelectArgs a;
  // num_seqs / compressed_cap are not known here: the per-query n is capped by max_visible.
  a.m = meta(plan, q, INT32_MAX, q->max_visible);
  a.scores = scores;
  a.ld_scores = ld_scores;
  a.block_max = block_max;
  a.ld_block_max = ld_block_max;
  a.cand = cand;
  a.topk = topk;
  a.parts = ps.parts;
  a.part_blocks = ps.part_blocks;
  log_call("select_topk: T=%lld max_visible=%lld, candidate stage in %d part(s) of %d blocks%s", (long long)q->T,
           (long long)q->max_visible, ps.parts, ps.part_blocks, cand == workspace ? ", candidates in the workspace" : "");
  a.part_ids = a.parts > 1 ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cand_bytes(q->T)) : nullptr;
  a.part_keys = a.parts > 1 ? reinterpret_cast<uint32_t*>(a.part_ids + (size_t)q->T * a.parts * 2048) : nullptr;
  return hip_status(sa::launch_select(a, (hipStream_t)stream), "select_topk launch");
}

sa_status sparse_attn_fwd(const sa_plan* plan, const sa_queries* q, const sa_cache* c,
                          const void* qv, const int32_t* topk, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  sa::AttnArgs a;
  sa_status st;
  if ((st = attn_args(plan, q, c, qv, topk, out, lse, a)) != SA_OK) return st;
  // key splits need the plan's whole workspace (its counters zeroed once by
  // sparse_attn_workspace_init); without it every query runs in one work-group
  const WsLayout wl = ws_layout(plan->p);
  a.splits = sa::attn_splits(q->T);
  if (a.splits > 1 && workspace != nullptr && aligned16(workspace) && workspace_bytes >= wl.total &&
      q->T * a.splits <= wl.units) {
    char* ws = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<uint32_t*>(ws + wl.counters_off);
    a.part_ml = reinterpret_cast<float*>(ws + wl.ml_off);
    a.part_o = reinterpret_cast<float*>(ws + wl.o_off);
  } else {
    a.splits = 1;
  }
  log_call("sparse_attn_fwd: T=%lld kv=%s, key list split over %d work-group(s)%s", (long long)q->T,
           a.kv_mode == 2 ? "mxfp4+e4m3" : a.kv_mode == 1 ? "e4m3" : "bf16", a.splits,
           a.pages.table ? ", paged latents" : "");
  return hip_status(sa::launch_attn(a, (hipStream_t)stream), "sparse_attn_fwd launch");
}

sa_status sparse_attn_fwd_noalloc(const sa_plan* plan, const sa_queries* q, const sa_cache* c,
                                  const void* qv, const int32_t* topk, void* out, float* lse,
                                  void* stream) {
  sa::AttnArgs a;
  sa_status st;
  if ((st = attn_args(plan, q, c, qv, topk, out, lse, a)) != SA_OK) return st;
  a.splits = sa::attn_splits(q->T);
  if (a.splits > 1) {
    SA_REQUIRE(q->T * a.splits <= sa::kScratchUnits && q->T <= sa::kScratchQueries, SA_EUNSUPPORTED,
               "sparse_attn_fwd_noalloc: %lld queries in %d key splits exceed the fixed scratch "
               "(%lld partial slots)", (long long)q->T, a.splits, (long long)sa::kScratchUnits);
    sa::AttnScratch s;
    hipError_t e = sa::attn_scratch(s);
    if (e != hipSuccess) return hip_status(e, "sparse_attn_fwd_noalloc scratch address");
    a.counters = s.counters;
    a.part_ml = s.part_ml;
    a.part_o = s.part_o;
    // the counters must start at zero: cleared by a kernel on the caller's stream
    e = sa::launch_zero_u32(s.counters, 2 * q->T, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "sparse_attn_fwd_noalloc counter reset launch");
  }
  log_call("sparse_attn_fwd_noalloc: T=%lld kv=%s, key list split over %d work-group(s)%s", (long long)q->T,
           a.kv_mode == 2 ? "mxfp4+e4m3" : a.kv_mode == 1 ? "e4m3" : "bf16", a.splits,
           a.splits > 1 ? " (fixed scratch)" : "");
  return hip_status(sa::launch_attn(a, (hipStream_t)stream), "sparse_attn_fwd_noalloc launch");
}

sa_status sparse_attn_workspace_init(const sa_plan* plan, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  SA_REQUIRE(workspace != nullptr && aligned16(workspace), SA_EWORKSPACE, "workspace NULL or misaligned");
  SA_REQUIRE(workspace_bytes >= plan->workspace, SA_EWORKSPACE, "workspace_bytes = %zu < %zu",
             workspace_bytes, plan->workspace);
  const WsLayout wl = ws_layout(plan->p);
  if (wl.units == 0) return ok();
  uint32_t* counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + wl.counters_off);
  return hip_status(sa::launch_zero_u32(counters, 2 * plan->p.max_queries, (hipStream_t)stream),
                    "sparse_attn_workspace_init launch");
}

sa_status sparse_attn_compress(const sa_plan* plan, const void* raw, int64_t raw_group_stride,
                               const void* gate, int64_t gate_group_stride,
                               const float* slot_bias, void* out, int64_t out_group_stride,
                               int64_t G, void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  SA_REQUIRE(plan->p.kv_dtype == SA_KV_BF16, SA_EUNSUPPORTED,
             "sparse_attn_compress writes bf16 rows (plan kv_dtype is e4m3 or MXFP4: use "
             "sparse_attn_compress_codes)");
  sa::CompressArgs a;
  if ((st = compress_args(plan, raw, raw_group_stride, gate, gate_group_stride, slot_bias, out, out_group_stride,
                          nullptr, 0, G, a)) != SA_OK)
    return st;
  if (G == 0) return ok();
  return hip_status(sa::launch_compress(a, (hipStream_t)stream), "sparse_attn_compress launch");
}

sa_status sparse_attn_compress_codes(const sa_plan* plan, const void* raw, int64_t raw_group_stride,
                                     const void* gate, int64_t gate_group_stride,
                                     const float* slot_bias, void* out, int64_t out_group_stride,
                                     void* out_scales, int64_t scales_group_stride, int64_t G,
                                     void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  SA_REQUIRE(plan->p.kv_dtype == SA_KV_FP8_E4M3 || plan->p.kv_dtype == SA_KV_MXFP4, SA_EUNSUPPORTED,
             "sparse_attn_compress_codes needs a plan with e4m3 or MXFP4 latents (plan kv_dtype is bf16)");
  sa::CompressArgs a;
  if ((st = compress_args(plan, raw, raw_group_stride, gate, gate_group_stride, slot_bias, out, out_group_stride,
                          out_scales, scales_group_stride, G, a)) != SA_OK)
    return st;
  if (G == 0) return ok();
  return hip_status(sa::launch_compress(a, (hipStream_t)stream), "sparse_attn_compress_codes launch");
}

sa_status indexer_score_compress(const sa_plan* plan, const sa_queries* q, const sa_cache* c,
                                 const void* q_idx, const float* w, float* scores, int64_t ld_scores,
                                 float* block_max, int64_t ld_block_max, const sa_compress_job* job,
                                 void* stream) {
  sa_status st;
  if ((st = check_plan(plan)) != SA_OK) return st;
  if (job == nullptr || job->G == 0)
    return indexer_common(plan, q, c, q_idx, w, scores, ld_scores, block_max, ld_block_max, nullptr, stream);
  sa::CompressArgs cj;
  if ((st = compress_args(plan, job->raw, job->raw_group_stride, job->gate, job->gate_group_stride, job->slot_bias,
                          job->out, job->out_group_stride, job->out_scales, job->scales_group_stride, job->G,
                          cj)) != SA_OK)
    return st;
  return indexer_common(plan, q, c, q_idx, w, scores, ld_scores, block_max, ld_block_max, &cj, stream);
}

}  // extern "C"
