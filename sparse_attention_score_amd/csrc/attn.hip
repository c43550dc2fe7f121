// S4 joint-softmax gather attention on gfx950 MFMA.
//
// For query t (sequence b, raw position p) and each of its 64 heads h:
//   X = [latents[b][j] for j in topk[t] (those in [0, n))] ++ [window rows of u = max(0,p-127)..p]
//   s_i = scale * <q_h, X_i>,  o_h = sum_i softmax(s)_i * X_i,  lse_h = log sum_i exp(s_i)
// Every 512-wide latent is both key and value and all 64 heads share it ("DeepSeek-V4.1
// Flash" Miles docs, section 1 Model Introduction; one softmax over both tiers, recipe
// Overview, two-tier sparse attention bullet).
//
// One work-group (4 waves) per (query, half of the heads); the two halves of a query are
// placed on the same XCD so the second gather of each row hits that XCD's L2, and two
// work-groups fit on a CU. Keys are gathered 32 per step into an LDS tile (rows staged
// through registers one step ahead, two LDS buffers).
//   scores: wave (hg, kh) computes S^T for keys 16kh..16kh+15 of the step and the 16 heads of
//           head group hg with v_mfma_f32_16x16x32_bf16 (A = keys from LDS, B = the wave's
//           query heads held in registers, 16 k-steps over the 512 dims).
//   softmax: per head, online in the log2 domain with a lazy running max; the two key halves
//           exchange their tile maxima through LDS; P (bf16) and the rescale factors go to LDS.
//   values: wave w owns output dims 128w..128w+127 of the 32 heads: O^T += V^T P^T with
//           A = V^T built from LDS rows by byte permutes (8 keys x 1 dim per lane) and
//           B = P^T read from LDS. Each value element is read from LDS once per step.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {
namespace {

constexpr int kAW = 4;              // waves
constexpr int kAThreads = 64 * kAW;
constexpr int kHH = 32;             // heads per work-group
constexpr int kKT = 32;             // keys per step
constexpr int kRow = kDim * 2 + 32; // padded LDS row bytes (+32: conflict-free 16-row reads)
constexpr int kMaxKeys = kTopK + kWindow;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;       // running-max slack, log2 units

struct AttnShared {
  uint8_t tile[2][kKT * kRow];         // 66,560 B
  u32x4 P[2][64];                      // P^T B operands: [head group][lane], 8 bf16 each
  float tmax[2][kHH];                  // per key half: tile max of each head
  float alpha[kHH];                    // rescale factor of each head this step
  const uint16_t* rows[kMaxKeys];      // global row of every key slot
  int wave_cnt[kAW];
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

__global__ __launch_bounds__(kAThreads, 2) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnShared sh;
  // work-group -> (query, head half): 16 consecutive ids hold 8 queries x 2 halves with both
  // halves of a query on the same XCD (ids are dealt round-robin over 8 XCDs).
  const int bid = blockIdx.x;
  const int t = (bid >> 4) * 8 + (bid & 7);
  const int hh = (bid >> 3) & 1;
  if (t >= a.m.T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
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
  int m = 0;
  if (valid_q) {
    const int32_t* tk = a.topk + (int64_t)t * kTopK;
    const int2 jj = *reinterpret_cast<const int2*>(tk + 2 * tid);
    const bool v0 = jj.x >= 0 && jj.x < n, v1 = jj.y >= 0 && jj.y < n;
    const int cnt = (int)v0 + (int)v1;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) sh.wave_cnt[wave] = incl;
    __syncthreads();
    int nsel = 0, before = 0;
    for (int w = 0; w < kAW; ++w) {
      nsel += sh.wave_cnt[w];
      before += (w < wave) ? sh.wave_cnt[w] : 0;
    }
    const uint16_t* lat = reinterpret_cast<const uint16_t*>(a.latents) + (int64_t)seq * a.latents_seq_stride;
    int off = before + incl - cnt;
    if (v0) sh.rows[off++] = lat + (int64_t)jj.x * kDim;
    if (v1) sh.rows[off] = lat + (int64_t)jj.y * kDim;
    const int u0 = p - kWindow + 1 > 0 ? p - kWindow + 1 : 0;
    const int nwin = p - u0 + 1;
    const uint16_t* win = reinterpret_cast<const uint16_t*>(a.window) + (int64_t)seq * a.window_seq_stride;
    if (tid < nwin) sh.rows[nsel + tid] = win + (int64_t)((u0 + tid) % a.window_cap) * kDim;
    m = nsel + nwin;
  }
  __syncthreads();

  const int head0 = kHH * hh;
  if (m == 0) {  // invalid query: zero output, lse = -inf
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)t * kHeads + head0) * kDim;
    for (int i = tid; i < kHH * kDim / 8; i += kAThreads)
      *reinterpret_cast<u32x4*>(o + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    if (a.lse && tid < kHH) a.lse[(int64_t)t * kHeads + head0 + tid] = neg_inf();
    return;
  }

  // roles
  const int hg = wave & 1, kh = wave >> 1;   // scores: head group, key half
  const int d0 = wave * 128;                  // values: output dims d0..d0+127

  // ---- query heads head0 + 16hg + c as the B operand (k-step s: dims (4s+g)*8 .. +8) ----
  bf16x8 qb[16];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)t * kHeads + head0 + 16 * hg + c) * kDim;
#pragma unroll
    for (int s = 0; s < 16; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + (4 * s + g) * 8);
  }

  // ---- tile loader: wave w moves rows 8w..8w+7 of a step, 16 bytes per lane ----
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

  // O^T accumulators: [e][head group]: dims d0 + 8r + e (r = MFMA row), heads 16h + c'
  f32x4 O[8][2];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int h = 0; h < 2; ++h) O[e][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = neg_inf();   // running max of head 16hg + c (log2 domain), scores role
  float l_run = 0.f;         // partial normaliser of that head over this wave's keys
  const float sc2 = a.scale * kLog2e;
  const int nsteps = (m + kKT - 1) / kKT;

  fetch(0);
  commit(0);
  if (nsteps > 1) fetch(1);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const uint8_t* T = sh.tile[buf];

    // -- scores: S^T[keys 16kh + 4g + i][head 16hg + c]
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* krow = T + (16 * kh + c) * kRow;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + (4 * s + g) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[s], acc, 0, 0, 0);
      }
    }
    float x[4];
    float mt = neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = step * kKT + 16 * kh + 4 * g + i;
      x[i] = k < m ? acc[i] * sc2 : neg_inf();
      mt = fmaxf(mt, x[i]);
    }
    mt = max_xor32(max_xor16(mt));
    if (g == 0) sh.tmax[kh][16 * hg + c] = mt;
    __syncthreads();  // (1) tile maxima visible; every wave is done with the previous step

    if (step + 1 < nsteps) commit(buf ^ 1);   // buffer last read in the previous step
    // Lazy running max: it only moves when the tile max exceeds it by more than kLazy
    // (log2 units), so most steps need no rescale; P stays below 2^kLazy. Both key halves
    // read the same maxima and take the same decision for a head.
    const float mt2 = fmaxf(sh.tmax[0][16 * hg + c], sh.tmax[1][16 * hg + c]);
    const float m_new = mt2 > m_run + kLazy ? mt2 : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pv[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
      psum += pv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P^T operand of head group hg: k-slots 0..3 from key half 0, 4..7 from key half 1.
    {
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sh.P[hg][lane]) + 2 * kh;
      dst[0] = pack_bf16x2(pv[0], pv[1]);
      dst[1] = pack_bf16x2(pv[2], pv[3]);
    }
    if (kh == 0 && g == 0) sh.alpha[16 * hg + c] = alpha;
    if (step + 2 < nsteps) fetch(step + 2);
    __syncthreads();  // (2) P, alpha and the next tile visible

    // -- values: O^T[dims d0 + 8r + e][heads 16h + c'] += V^T P^T
    float al[2];
    bool any = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      al[h] = sh.alpha[16 * h + c];
      any |= al[h] != 1.0f;
    }
    if (__ballot(any) != 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h) O[e][h] *= al[h];
    }
    bf16x8 pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) pb[h] = __builtin_bit_cast(bf16x8, sh.P[h][lane]);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // key slot j: dims d0 + 8c + 4*half .. +3 (two dwords)
      uint32_t R[8][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4));
        const uint2 v = *reinterpret_cast<const uint2*>(T + key * kRow + (d0 + 8 * c + 4 * half) * 2);
        R[j][0] = v.x;
        R[j][1] = v.y;
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int w = e4 >> 1;
        u32x4 va;
        if (e4 & 1) {
          va = u32x4{perm_hi(R[1][w], R[0][w]), perm_hi(R[3][w], R[2][w]),
                     perm_hi(R[5][w], R[4][w]), perm_hi(R[7][w], R[6][w])};
        } else {
          va = u32x4{perm_lo(R[1][w], R[0][w]), perm_lo(R[3][w], R[2][w]),
                     perm_lo(R[5][w], R[4][w]), perm_lo(R[7][w], R[6][w])};
        }
        const bf16x8 A = __builtin_bit_cast(bf16x8, va);
        const int e = 4 * half + e4;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          O[e][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pb[h], O[e][h], 0, 0, 0);
      }
    }
  }

  // ---- normaliser per head: sum of the partial sums of both key halves ----
  {
    float l = add_xor32(add_xor16(l_run));
    if (g == 0) sh.tmax[kh][16 * hg + c] = l;   // reuse: partial normaliser
    __syncthreads();
    if (kh == 0 && g == 0) {
      const float L = sh.tmax[0][16 * hg + c] + sh.tmax[1][16 * hg + c];
      sh.alpha[16 * hg + c] = L;
      if (a.lse) a.lse[(int64_t)t * kHeads + head0 + 16 * hg + c] = (m_run + __log2f(L)) * kLn2;
    }
    __syncthreads();
  }
  // ---- normalise and store: lane (c', g) holds dims d0 + 8(4g+i) + e of heads 16h + c' ----
  uint16_t* outp = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)t * kHeads + head0) * kDim;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float inv = 1.0f / sh.alpha[16 * h + c];
    uint16_t* orow = outp + (int64_t)(16 * h + c) * kDim + d0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;  // row of the MFMA result = group of 8 dims
      u32x4 o;
      o[0] = pack_bf16x2(O[0][h][i] * inv, O[1][h][i] * inv);
      o[1] = pack_bf16x2(O[2][h][i] * inv, O[3][h][i] * inv);
      o[2] = pack_bf16x2(O[4][h][i] * inv, O[5][h][i] * inv);
      o[3] = pack_bf16x2(O[6][h][i] * inv, O[7][h][i] * inv);
      *reinterpret_cast<u32x4*>(orow + 8 * r) = o;
    }
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  const int64_t groups = (a.m.T + 7) / 8;  // 8 queries x 2 head halves per 16 ids
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)(groups * 16)), dim3(kAThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
