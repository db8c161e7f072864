// Block scoring, GQA-group aggregation and top-k selection (gfx950), decode.
//
// COBS (gist.science explainer, Technisches Resuemee 2.1-2.3; skill card
// "Method"): a block's attention mass is estimated from its query-independent
// summary by the truncated cumulant expansion
//     s_{h,b} = ln n_b + scale q_h.mu_b + alpha/2 scale^2 q_h^T Sigma_b q_h
// and the top-k blocks are kept.  A GQA group ranks blocks by
//     shat_b = ln sum_h exp(s_{h,b} - LSE_b' s_{h,b'})
// (each head's estimated share of its attention mass), ties to the lower index.
//
// Phase 1 (every workgroup): scores for a slice of 16-block tiles.  The score is
// a small contraction of [16 blocks x summary] with [summary x 16 heads]; it runs
// on the fp32 MFMA (v_mfma_f32_16x16x4_f32) so that selection keeps fp32
// accuracy.  Summaries are streamed once with 16-byte loads.  Each workgroup also
// leaves a per-head (max, sum exp) partial for the log-sum-exp.
// Phase 2 (the last workgroup of a (sequence, kv-head), found with an atomic
// counter): per-head LSE, group scores, an MSB-first 8-bit radix select of the
// k-th largest key in LDS, and an ordered compaction into ascending block order.
// Phase 2 is latency-bound, so each of its global reads is a single round.
#include "cobs_device.h"
#include "cobs_launch.h"
#include "score_common.h"

namespace cobs {

constexpr int kSelThreads = 256;
constexpr int kSelMaxPerThread = 16;           // up to 4096 blocks per sequence
constexpr int kSelMaxSplits = 64;              // scoring workgroups per (sequence, kv-head)

struct SelParams {
  int tokens, hkv, group, max_len, nb_max, nb_pad, top_k, rank, q_pos0, splits, tiles_per_wave;
  float alpha, scale;
  const int32_t* seq_lens;
  const void* Q;
  const float *mu, *so;
  int32_t* sel;
  float* sel_score;
  uint32_t* counters;
  float* scores;                               // [unit][nb_pad][16] block-major
  float* lse_part;
};


// Exclusive prefix sum over the 256 threads of a workgroup, in thread order.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_inclusive_sum(v);
  if (lane == 63) lds_w[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    const int c = lds_w[i];
    base += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}


// KIND 0: diagonal channel; KIND 1: rank-r scaled eigenvectors.
// HV = number of float4 holding the group's heads (G <= 4HV).
template <typename E, int D, int KIND, int HV>
__global__ __launch_bounds__(kSelThreads) void k_select(SelParams p) {
  constexpr int NU = D / 16;                    // 16-column slices of a summary row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int head = blockIdx.y;
  const int seq = blockIdx.z / p.tokens, tok = blockIdx.z % p.tokens;
  const int unit = blockIdx.z * p.hkv + head;
  const int L = p.seq_lens[seq];
  const int t = (p.q_pos0 < 0) ? L - 1 : p.q_pos0 + tok;
  const int ncand = candidate_blocks(L, t);
  const int G = p.group;

  __shared__ float red_m[4][16], red_s[4][16];
  __shared__ __align__(16) uint32_t hist2[2][4][256];
  __shared__ int scan_w[4];
  __shared__ int bcast[4];
  __shared__ float lse_sh[16];
  __shared__ float red_part[kSelMaxSplits * 32];
  extern __shared__ uint32_t s_dyn[];              // [nb_pad] keys, then [nb_pad] group scores
  uint32_t* s_key = s_dyn;
  float* s_shat = reinterpret_cast<float*>(s_dyn + p.nb_pad);

  const Coherent sc(p.scores + (size_t)unit * 16 * p.nb_pad, (uint32_t)(16 * p.nb_pad * 4));
  const Coherent lp(p.lse_part + (size_t)unit * p.splits * 32, (uint32_t)(p.splits * 32 * 4));

  // ---- phase 1: scores of this workgroup's tiles -------------------------
  // B operand (weights): lane (head n, k-group g) holds, for slice u and
  // component c, the weight of summary column 16u + 4g + c.
  float wlin[NU][4], wquad[NU][4];
  score_weights<E, D, KIND>(p.Q, ((size_t)blockIdx.z * (size_t)(p.hkv * G) + (size_t)head * G) * D, n, g, G,
                            p.scale, p.alpha, wlin, wquad);
  const bool use_quad = p.alpha != 0.f;
  float run_m = -INFINITY, run_s = 0.f;      // LSE partial of head n over this lane's blocks
  const size_t sum_base = (size_t)(seq * p.hkv + head) * p.nb_max;
  const int tiles_total = (ncand + 15) / 16;
  for (int j = 0; j < p.tiles_per_wave; ++j) {
    const int tile = (blockIdx.x * 4 + wave) * p.tiles_per_wave + j;
    if (tile >= tiles_total) break;
    const int brow = min(tile * 16 + n, ncand - 1);     // A-operand row (block) of this lane
    const f32x4 sc2 = score_tile<D, KIND>(p.mu + (sum_base + brow) * D,
                                          KIND == 0 ? p.so + (sum_base + brow) * D
                                                    : p.so + (sum_base + brow) * (size_t)(p.rank * D),
                                          p.rank, g, use_quad, p.alpha, wlin, wquad);
    // sc2[i]: score (without ln n_b) of block tile*16 + 4g + i for head n
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = tile * 16 + 4 * g + i;
      const int nbk = min(kBlock, L - b * kBlock);
      const float s = (b < ncand) ? sc2[i] + __logf((float)nbk) : -INFINITY;
      const float mx = fmaxf(run_m, s);
      if (mx != -INFINITY) {
        run_s = run_s * __expf(run_m - mx) + __expf(s - mx);
        run_m = mx;
      }
      if (n < G) sc.st1((uint32_t)((b * 16 + n) * 4), s);
    }
  }
  // combine the LSE partial over the four lane groups, then over the waves
#pragma unroll
  for (int m = 16; m < 64; m <<= 1) {
    const float om = shfl_xor_f(run_m, m), os = shfl_xor_f(run_s, m);
    const float mx = fmaxf(run_m, om);
    if (mx != -INFINITY) {
      run_s = run_s * __expf(run_m - mx) + os * __expf(om - mx);
      run_m = mx;
    }
  }
  if (g == 0) { red_m[wave][n] = run_m; red_s[wave][n] = run_s; }
  __syncthreads();
  if (threadIdx.x < 16) {
    float M = -INFINITY, S = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float om = red_m[w][threadIdx.x], os = red_s[w][threadIdx.x];
      const float mx = fmaxf(M, om);
      if (mx != -INFINITY) { S = S * __expf(M - mx) + os * __expf(om - mx); M = mx; }
    }
    const uint32_t o = (uint32_t)(((blockIdx.x * 16) + threadIdx.x) * 2 * 4);
    lp.st1(o, M);
    lp.st1(o + 4, S);
  }

  // ---- hand-off: the last workgroup of this unit selects -----------------
  if (!arrive_last(p.counters + unit, (uint32_t)p.splits, &bcast[0])) return;

  // ---- phase 2: LSE per head ------------------------------------------------
  for (int i = threadIdx.x; i < p.splits * 16; i += kSelThreads) {
    red_part[2 * i] = lp.ld1((uint32_t)(i * 8));
    red_part[2 * i + 1] = lp.ld1((uint32_t)(i * 8 + 4));
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float M = -INFINITY, S = 0.f;
    for (int x = 0; x < p.splits; ++x) {
      const float om = red_part[2 * (x * 16 + threadIdx.x)], os = red_part[2 * (x * 16 + threadIdx.x) + 1];
      const float mx = fmaxf(M, om);
      if (mx != -INFINITY) { S = S * __expf(M - mx) + os * __expf(om - mx); M = mx; }
    }
    lse_sh[threadIdx.x] = (M == -INFINITY) ? -INFINITY : M + __logf(S);
  }
  __syncthreads();

  // ---- group scores: thread owns blocks [tid*per, tid*per + per) ------------
  // Keys and scores live in LDS (s_key, s_shat) so the loops below stay compact.
  const int per = (p.nb_max + kSelThreads - 1) / kSelThreads;   // <= kSelMaxPerThread
  const int b0 = threadIdx.x * per;
  constexpr int kRound = 8 / HV;                                 // blocks per load round (8 float4)
  float lse_r[4 * HV];
#pragma unroll
  for (int h = 0; h < 4 * HV; ++h) lse_r[h] = (h < G) ? lse_sh[h] : 0.f;
#pragma unroll 1
  for (int e0 = 0; e0 < per; e0 += kRound) {
    f32x4 raw[kRound][HV];
#pragma unroll
    for (int e = 0; e < kRound; ++e) {
      const int b = b0 + e0 + e;
      const bool ok = e0 + e < per && b < ncand;
#pragma unroll
      for (int v = 0; v < HV; ++v)
        raw[e][v] = ok ? sc.ld4((uint32_t)((b * 16 + 4 * v) * 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int e = 0; e < kRound; ++e) {
      const int b = b0 + e0 + e;
      if (e0 + e < per && b < ncand) {
        float M = -INFINITY;
#pragma unroll
        for (int h = 0; h < 4 * HV; ++h)
          if (h < G) M = fmaxf(M, raw[e][h >> 2][h & 3] - lse_r[h]);
        float S = 0.f;
#pragma unroll
        for (int h = 0; h < 4 * HV; ++h)
          if (h < G) S += __expf(raw[e][h >> 2][h & 3] - lse_r[h] - M);
        const float sh = M + __logf(S);
        s_shat[b] = sh;
        s_key[b] = orderable(sh);
      }
    }
  }

  __syncthreads();                                 // s_key / s_shat complete
  if (p.sel_score) {
    float* ss = p.sel_score + (size_t)unit * p.nb_max;
    for (int b = threadIdx.x; b < p.nb_max; b += kSelThreads) ss[b] = (b < ncand) ? s_shat[b] : -INFINITY;
  }

  // ---- radix select of the k-th largest key --------------------------------
  // Each wave fills a private 256-bin histogram (double-buffered across passes);
  // after one barrier every wave sums the four and finds the digit itself.
  const int e_end = max(0, min(per, ncand - b0));   // this thread's candidates [b0, b0 + e_end)
  const int kk = min(p.top_k, ncand);
  uint32_t prefix = 0u, hi_mask = 0u;
  int need = kk;                                  // how many still to take at or below the prefix
  int eq_bin = 0;                                 // keys equal to the k-th largest
#pragma unroll 1
  for (int pass = 0; pass < 4 && kk > 0; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* mine = hist2[pass & 1][wave];
    *reinterpret_cast<u32x4*>(&mine[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int e = 0; e < per; ++e) {               // uniform trip count: wave-wide ballots inside
      const uint32_t key = (e < e_end) ? s_key[b0 + e] : 0u;
      wave_histogram_add(mine, e < e_end && (key & hi_mask) == prefix, (key >> shift) & 255u);
    }
    __syncthreads();
    u32x4 hb = *reinterpret_cast<const u32x4*>(&hist2[pass & 1][0][4 * lane]);
#pragma unroll
    for (int w = 1; w < 4; ++w) hb += *reinterpret_cast<const u32x4*>(&hist2[pass & 1][w][4 * lane]);
    prefix |= radix_digit(hb, need, eq_bin) << shift;
    hi_mask |= 255u << shift;
  }
  // `prefix` is the k-th largest key; `need` of the `eq_bin` keys equal to it are
  // taken, lowest block index first
  int eq_rank = 0;
  if (kk > 0 && need < eq_bin) {                  // a tie straddles the cut: rank the equal keys
    int eq_count = 0;
#pragma unroll 1
    for (int e = 0; e < e_end; ++e) eq_count += (s_key[b0 + e] == prefix) ? 1 : 0;
    int eq_total;
    eq_rank = block_exclusive_scan(eq_count, scan_w, &eq_total);
  }
  int take_count = 0;
  if (kk > 0) {
    int r = eq_rank;
#pragma unroll 1
    for (int e = 0; e < e_end; ++e) {
      const uint32_t key = s_key[b0 + e];
      if (key > prefix) ++take_count;
      else if (key == prefix) { take_count += (r < need) ? 1 : 0; ++r; }
    }
  }
  int sel_total;
  int pos = block_exclusive_scan(take_count, scan_w, &sel_total);
  int32_t* sel_u = p.sel + (size_t)unit * p.top_k;
  if (kk > 0) {
    int r = eq_rank;
#pragma unroll 1
    for (int e = 0; e < e_end; ++e) {
      const uint32_t key = s_key[b0 + e];
      bool tk = key > prefix;
      if (key == prefix) { tk = r < need; ++r; }
      if (tk) sel_u[pos++] = b0 + e;
    }
  }
  for (int i = sel_total + (int)threadIdx.x; i < p.top_k; i += kSelThreads) sel_u[i] = -1;
  if (threadIdx.x == 0) reset_counter(p.counters + unit);   // zero for the next call
}

template <typename E, int D, int KIND>
static hipError_t launch_sel_hv(const SelectArgs& a, const SelParams& sp, dim3 grid) {
  const size_t lds = (size_t)sp.nb_pad * 8;
  if (a.group <= 4) {
    hipLaunchKernelGGL((k_select<E, D, KIND, 1>), grid, dim3(kSelThreads), lds, a.stream, sp);
  } else if (a.group <= 8) {
    hipLaunchKernelGGL((k_select<E, D, KIND, 2>), grid, dim3(kSelThreads), lds, a.stream, sp);
  } else {
    hipLaunchKernelGGL((k_select<E, D, KIND, 4>), grid, dim3(kSelThreads), lds, a.stream, sp);
  }
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_sel_t(const SelectArgs& a, const SelParams& sp) {
  dim3 grid(a.splits, a.hkv, a.batch * a.tokens);
  return a.so_kind == 0 ? launch_sel_hv<E, D, 0>(a, sp, grid) : launch_sel_hv<E, D, 1>(a, sp, grid);
}

hipError_t launch_select(const SelectArgs& a) {
  SelParams sp;
  sp.tokens = a.tokens; sp.hkv = a.hkv; sp.group = a.group; sp.max_len = a.max_len;
  sp.nb_max = a.nb_max; sp.nb_pad = (a.nb_max + 15) / 16 * 16; sp.top_k = a.top_k; sp.rank = a.rank;
  sp.q_pos0 = a.q_pos0; sp.splits = a.splits; sp.tiles_per_wave = a.tiles_per_wave;
  sp.alpha = a.alpha; sp.scale = a.scale; sp.seq_lens = a.seq_lens; sp.Q = a.Q; sp.mu = a.mu;
  sp.so = a.so; sp.sel = a.sel; sp.sel_score = a.sel_score; sp.counters = a.counters;
  sp.scores = a.scores; sp.lse_part = a.lse_part;
  if (a.bf16) return a.head_dim == 128 ? launch_sel_t<EltBF16, 128>(a, sp) : launch_sel_t<EltBF16, 64>(a, sp);
  return a.head_dim == 128 ? launch_sel_t<EltF32, 128>(a, sp) : launch_sel_t<EltF32, 64>(a, sp);
}

}  // namespace cobs
