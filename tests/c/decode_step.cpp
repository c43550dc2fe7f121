// The decode path from a plain host program: HIP runtime calls for memory, the library's C
// entry points for the work (indexer_score, select_topk, sparse_attn_fwd), no Python.
//   decode_step DIR   reads DIR/meta.txt ("B cap wcap T max_visible ratio") and the raw
//                     little-endian inputs seq.bin pos.bin (int32 [T]), q.bin (bf16
//                     [T][64][512]), qi.bin (bf16 [T][16][128]), w.bin (fp32 [T][16]),
//                     lat.bin (bf16 [B][cap][512]), win.bin (bf16 [B][wcap][512]),
//                     keys.bin (bf16 [B][cap][128]); writes topk.bin (int32 [T][512]),
//                     out.bin (bf16 [T][64][512]) and lse.bin (fp32 [T][64]).
// Exit status 0 on success; every failing call is reported with its message.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "sparse_attn.h"

namespace {

std::string g_dir;

bool slurp(const char* name, std::vector<char>& buf, size_t bytes) {
  FILE* f = std::fopen((g_dir + "/" + name).c_str(), "rb");
  if (!f) return false;
  buf.resize(bytes);
  const size_t got = std::fread(buf.data(), 1, bytes, f);
  std::fclose(f);
  return got == bytes;
}

bool spill(const char* name, const void* data, size_t bytes) {
  FILE* f = std::fopen((g_dir + "/" + name).c_str(), "wb");
  if (!f) return false;
  const size_t put = std::fwrite(data, 1, bytes, f);
  std::fclose(f);
  return put == bytes;
}

struct Dev {
  void* p = nullptr;
  ~Dev() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      return 1;                                                                   \
    }                                                                             \
  } while (0)
#define SA_OK_(call)                                                              \
  do {                                                                            \
    sa_status s_ = (call);                                                        \
    if (s_ != SA_OK) {                                                            \
      std::fprintf(stderr, "%s -> %d: %s\n", #call, (int)s_, sparse_attn_last_error()); \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: decode_step DIR\n");
    return 2;
  }
  g_dir = argv[1];
  long long B, cap, wcap, T, maxvis, ratio;
  {
    FILE* f = std::fopen((g_dir + "/meta.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%lld %lld %lld %lld %lld %lld", &B, &cap, &wcap, &T, &maxvis, &ratio) != 6) {
      std::fprintf(stderr, "cannot read meta.txt\n");
      return 2;
    }
    std::fclose(f);
  }
  const size_t nq = T * 64 * 512 * 2, nqi = T * 16 * 128 * 2, nw = T * 16 * 4, nlat = B * cap * 512 * 2,
               nwin = B * wcap * 512 * 2, nkeys = B * cap * 128 * 2, nidx = T * 4;
  std::vector<char> seq, pos, q, qi, w, lat, win, keys;
  if (!slurp("seq.bin", seq, nidx) || !slurp("pos.bin", pos, nidx) || !slurp("q.bin", q, nq) ||
      !slurp("qi.bin", qi, nqi) || !slurp("w.bin", w, nw) || !slurp("lat.bin", lat, nlat) ||
      !slurp("win.bin", win, nwin) || !slurp("keys.bin", keys, nkeys)) {
    std::fprintf(stderr, "cannot read the inputs\n");
    return 2;
  }

  sa_params p;
  std::memset(&p, 0, sizeof p);
  p.num_heads = 64;
  p.latent_dim = 512;
  p.window = 128;
  p.topk = 512;
  p.idx_heads = 16;
  p.idx_dim = 128;
  p.block = 8;
  p.cand_blocks = 2048;
  p.ratio = (int32_t)ratio;
  p.idx_key_dtype = SA_KEY_BF16;
  p.softmax_scale = 1.0f / std::sqrt(512.0f);
  p.max_queries = T;
  p.max_compressed = cap;
  p.kv_dtype = SA_KV_BF16;
  sa_plan* plan = nullptr;
  size_t ws_bytes = 0;
  SA_OK_(sparse_attn_plan(&p, &plan, &ws_bytes));

  // score rows: E = max_visible rounded up to 8 entries, rows padded to multiples of 4
  const long long E = (maxvis + 7) / 8 * 8;
  const long long ld = E > 4 ? (E + 3) / 4 * 4 : 4, ldb = E / 8 > 4 ? (E / 8 + 3) / 4 * 4 : 4;
  Dev d_seq, d_pos, d_q, d_qi, d_w, d_lat, d_win, d_keys, d_sc, d_bm, d_cand, d_topk, d_out, d_lse, d_ws;
  HIP_OK(hipMalloc(&d_seq.p, nidx));
  HIP_OK(hipMalloc(&d_pos.p, nidx));
  HIP_OK(hipMalloc(&d_q.p, nq));
  HIP_OK(hipMalloc(&d_qi.p, nqi));
  HIP_OK(hipMalloc(&d_w.p, nw));
  HIP_OK(hipMalloc(&d_lat.p, nlat));
  HIP_OK(hipMalloc(&d_win.p, nwin));
  HIP_OK(hipMalloc(&d_keys.p, nkeys));
  HIP_OK(hipMalloc(&d_sc.p, T * ld * 4));
  HIP_OK(hipMalloc(&d_bm.p, T * ldb * 4));
  HIP_OK(hipMalloc(&d_cand.p, T * 2048 * 4));
  HIP_OK(hipMalloc(&d_topk.p, T * 512 * 4));
  HIP_OK(hipMalloc(&d_out.p, nq));
  HIP_OK(hipMalloc(&d_lse.p, T * 64 * 4));
  HIP_OK(hipMalloc(&d_ws.p, ws_bytes > 16 ? ws_bytes : 16));
  HIP_OK(hipMemcpy(d_seq.p, seq.data(), nidx, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_pos.p, pos.data(), nidx, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_q.p, q.data(), nq, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_qi.p, qi.data(), nqi, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w.p, w.data(), nw, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_lat.p, lat.data(), nlat, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_win.p, win.data(), nwin, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_keys.p, keys.data(), nkeys, hipMemcpyHostToDevice));
  SA_OK_(sparse_attn_workspace_init(plan, d_ws.p, ws_bytes, nullptr));

  sa_queries qs;
  std::memset(&qs, 0, sizeof qs);
  qs.T = T;
  qs.seq_id = static_cast<const int32_t*>(d_seq.p);
  qs.pos = static_cast<const int32_t*>(d_pos.p);
  qs.max_visible = maxvis;
  sa_cache c;
  std::memset(&c, 0, sizeof c);
  c.num_seqs = B;
  c.compressed_cap = cap;
  c.latents = d_lat.p;
  c.latents_seq_stride = cap * 512;
  c.window = d_win.p;
  c.window_seq_stride = wcap * 512;
  c.window_cap = (int32_t)wcap;
  c.idx_keys = d_keys.p;
  c.idx_keys_seq_stride = cap * 128;

  float* sc = static_cast<float*>(d_sc.p);
  float* bm = static_cast<float*>(d_bm.p);
  int32_t* topk = static_cast<int32_t*>(d_topk.p);
  SA_OK_(indexer_score(plan, &qs, &c, d_qi.p, static_cast<const float*>(d_w.p), sc, ld, bm, ldb, nullptr));
  SA_OK_(select_topk(plan, &qs, sc, ld, bm, ldb, static_cast<int32_t*>(d_cand.p), topk, d_ws.p, ws_bytes,
                     nullptr));
  SA_OK_(sparse_attn_fwd(plan, &qs, &c, d_q.p, topk, d_out.p, static_cast<float*>(d_lse.p), d_ws.p, ws_bytes,
                         nullptr));
  HIP_OK(hipDeviceSynchronize());

  std::vector<char> h_topk(T * 512 * 4), h_out(nq), h_lse(T * 64 * 4);
  HIP_OK(hipMemcpy(h_topk.data(), d_topk.p, h_topk.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_out.data(), d_out.p, h_out.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_lse.data(), d_lse.p, h_lse.size(), hipMemcpyDeviceToHost));
  sparse_attn_plan_destroy(plan);
  if (!spill("topk.bin", h_topk.data(), h_topk.size()) || !spill("out.bin", h_out.data(), h_out.size()) ||
      !spill("lse.bin", h_lse.data(), h_lse.size())) {
    std::fprintf(stderr, "cannot write the outputs\n");
    return 2;
  }
  std::printf("decode_step ok: %lld queries\n", T);
  return 0;
}
