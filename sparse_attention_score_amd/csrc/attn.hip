// S4 joint-softmax gather attention on gfx950 MFMA.
//
// For query t (sequence b, raw position p) and each of its 64 heads h:
//   X = [latents[b][j] for j in topk[t] (those in [0, n))] ++ [window rows of u = max(0,p-127)..p]
//   s_i = scale * <q_h, X_i>,  o_h = sum_i softmax(s)_i * X_i,  lse_h = log sum_i exp(s_i)
// Every 512-wide latent is both key and value and all 64 heads share it ("DeepSeek-V4.1
// Flash" Miles docs, section 1 Model Introduction; one softmax over both tiers, recipe
// Overview, two-tier sparse attention bullet).
//
// One work-group per query; wave w owns heads 16w..16w+15. Keys are gathered 32 at a time
// into an LDS tile (double-buffered through registers) that all four waves share.
//   S^T = K Q^T : v_mfma_f32_16x16x32_bf16, A = 16 keys from LDS, B = the wave's 16 heads
//                 (kept in registers), 16 k-steps over the 512 dims.
//   O^T += V^T P^T : A = V^T, built from LDS rows with byte permutes (8 keys x 1 dim per
//                 lane), B = P^T taken straight from the S^T accumulators.
// In both results a lane's column is its head, so the online-softmax max, sum and
// rescale are per lane; only the tile max needs two cross-lane steps.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kAW = 4;              // waves, 16 heads each
constexpr int kAThreads = 64 * kAW;
constexpr int kKT = 32;             // keys per step
constexpr int kRow = kDim * 2 + 16; // padded LDS row bytes
constexpr int kMaxKeys = kTopK + kWindow;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnShared {
  uint8_t tile[2][kKT * kRow];
  const uint16_t* rows[kMaxKeys];
  int wave_cnt[kAW];
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t hi_src, uint32_t lo_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);  // (lo16 of lo_src, lo16 of hi_src)
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t hi_src, uint32_t lo_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);  // (hi16 of lo_src, hi16 of hi_src)
}

__global__ __launch_bounds__(kAThreads) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnShared sh;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  const int seq = a.m.seq_id[t], p = a.m.pos[t];
  const bool valid_q = seq >= 0 && seq < a.m.num_seqs && p >= 0;
  int64_t n = 0;
  if (valid_q) {
    n = ((int64_t)p + 1) / a.m.ratio;
    n = n < a.m.max_visible ? n : a.m.max_visible;
    n = n < a.m.compressed_cap ? n : a.m.compressed_cap;
  }

  // ---- key list: selected latents in topk order, then the window ----
  int nsel = 0, m = 0;
  if (valid_q) {
    const int32_t* tk = a.topk + (int64_t)t * kTopK;
    const int j0 = tk[2 * tid], j1 = tk[2 * tid + 1];
    const bool v0 = j0 >= 0 && j0 < n, v1 = j1 >= 0 && j1 < n;
    int cnt = (int)v0 + (int)v1;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) sh.wave_cnt[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < kAW; ++w) {
      nsel += sh.wave_cnt[w];
      before += (w < wave) ? sh.wave_cnt[w] : 0;
    }
    int off = before + incl - cnt;
    const uint16_t* lat = reinterpret_cast<const uint16_t*>(a.latents) + (int64_t)seq * a.latents_seq_stride;
    if (v0) sh.rows[off++] = lat + (int64_t)j0 * kDim;
    if (v1) sh.rows[off] = lat + (int64_t)j1 * kDim;
    const int u0 = p - kWindow + 1 > 0 ? p - kWindow + 1 : 0;
    const int nwin = p - u0 + 1;
    const uint16_t* win = reinterpret_cast<const uint16_t*>(a.window) + (int64_t)seq * a.window_seq_stride;
    if (tid < nwin) sh.rows[nsel + tid] = win + (int64_t)((u0 + tid) % a.window_cap) * kDim;
    m = nsel + nwin;
  }
  __syncthreads();

  const int head = wave * 16 + c;
  uint16_t* outp = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)t * kHeads + head) * kDim;
  if (m == 0) {  // invalid query: zero output, lse = -inf
    for (int i = g; i < kDim / 8; i += 4)
      *reinterpret_cast<u32x4*>(outp + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    if (a.lse && g == 0) a.lse[(int64_t)t * kHeads + head] = neg_inf();
    return;
  }

  // ---- the wave's 16 query heads as the B operand (k-step s: dims (4s+g)*8 .. +8) ----
  bf16x8 qb[16];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)t * kHeads + head) * kDim;
#pragma unroll
    for (int s = 0; s < 16; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + (4 * s + g) * 8);
  }

  // ---- tile loader: thread (wave w, lane l) moves 16 bytes of rows w*8 .. w*8+7 ----
  u32x4 stage[8];
  auto fetch = [&](int step) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = step * kKT + wave * 8 + i;
      if (k < m) stage[i] = *reinterpret_cast<const u32x4*>(sh.rows[k] + lane * 8);
      else stage[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&sh.tile[buf][(wave * 8 + i) * kRow + lane * 16]) = stage[i];
  };

  f32x4 O[4][8];
#pragma unroll
  for (int bk = 0; bk < 4; ++bk)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[bk][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = neg_inf(), l_run = 0.f;
  const float sc2 = a.scale * kLog2e;

  const int nsteps = (m + kKT - 1) / kKT;
  fetch(0);
  commit(0);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) fetch(step + 1);
    const uint8_t* T = sh.tile[buf];

    // S^T for keys 16st + 4g + i of this step, head c.
    f32x4 sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = T + (16 * st + c) * kRow;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + (4 * s + g) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[s], acc, 0, 0, 0);
      }
      sacc[st] = acc;
    }

    // Online softmax in the log2 domain.
    float x[8];
    float mt = neg_inf();
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = step * kKT + 16 * st + 4 * g + i;
        float v = k < m ? sacc[st][i] * sc2 : neg_inf();
        x[4 * st + i] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = __builtin_amdgcn_exp2f(x[j] - m_new);
      psum += pv[j];
    }
    if (__ballot(m_new > m_run) != 0) {
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[bk][e] *= alpha;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // P^T as the B operand: k-slots 0..3 = keys 4g+i, 4..7 = keys 16+4g+i.
    u32x4 pu = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pu);

    // O^T[dim 128bk + 8(4g+i) + e][head c] += V^T P^T.
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      u32x4 R[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4));
        R[j] = *reinterpret_cast<const u32x4*>(T + key * kRow + (128 * bk + 8 * c) * 2);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        u32x4 va;
        if (e & 1) {
          va = u32x4{perm_hi(R[1][w], R[0][w]), perm_hi(R[3][w], R[2][w]),
                     perm_hi(R[5][w], R[4][w]), perm_hi(R[7][w], R[6][w])};
        } else {
          va = u32x4{perm_lo(R[1][w], R[0][w]), perm_lo(R[3][w], R[2][w]),
                     perm_lo(R[5][w], R[4][w]), perm_lo(R[7][w], R[6][w])};
        }
        O[bk][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb,
                                                            O[bk][e], 0, 0, 0);
      }
    }

    if (step + 1 < nsteps) {
      commit(buf ^ 1);  // the other buffer was last read in the previous step
      __syncthreads();
    }
  }

  // ---- normalise and store ----
  float l = l_run + shfl_xor_f(l_run, 16);
  l = l + shfl_xor_f(l, 32);
  const float inv = 1.0f / l;
#pragma unroll
  for (int bk = 0; bk < 4; ++bk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 128 * bk + 8 * (4 * g + i);
      u32x4 o = {pack_bf16x2(O[bk][0][i] * inv, O[bk][1][i] * inv),
                 pack_bf16x2(O[bk][2][i] * inv, O[bk][3][i] * inv),
                 pack_bf16x2(O[bk][4][i] * inv, O[bk][5][i] * inv),
                 pack_bf16x2(O[bk][6][i] * inv, O[bk][7][i] * inv)};
      *reinterpret_cast<u32x4*>(outp + d0) = o;
    }
  if (a.lse && g == 0) a.lse[(int64_t)t * kHeads + head] = (m_run + __log2f(l)) * kLn2;
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)a.m.T), dim3(kAThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
