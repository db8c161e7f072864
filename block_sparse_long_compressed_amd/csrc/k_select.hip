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
#include "cobs_device.h"
#include "cobs_launch.h"

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
  float* scores;
  float* lse_part;
};

// Number of candidate blocks (a prefix [0, n)) for a query at position t of a
// sequence of length L: blocks whose keys all lie at positions <= t.
__device__ __forceinline__ int candidate_blocks(int L, int t) {
  return (t >= L - 1) ? (L + kBlock - 1) / kBlock : (t + 1) / kBlock;
}

// Exclusive prefix sum over the 256 threads of a workgroup, in thread order.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
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

template <typename E>
__device__ __forceinline__ void load_q4(const void* Q, size_t off, float* out4) {
  if constexpr (E::kBytes == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(Q) + off);
    out4[0] = __uint_as_float(w.x << 16);
    out4[1] = __uint_as_float(w.x & 0xFFFF0000u);
    out4[2] = __uint_as_float(w.y << 16);
    out4[3] = __uint_as_float(w.y & 0xFFFF0000u);
  } else {
    const f32x4 v = ld_f32x4(reinterpret_cast<const float*>(Q) + off);
    out4[0] = v[0]; out4[1] = v[1]; out4[2] = v[2]; out4[3] = v[3];
  }
}

// KIND 0: diagonal channel; KIND 1: rank-R scaled eigenvectors.
template <typename E, int D, int KIND, int R>
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
  __shared__ uint32_t hist[256];
  __shared__ int scan_w[4];
  __shared__ int bcast[4];
  __shared__ float lse_sh[16];
  __shared__ float red_part[kSelMaxSplits * 32];

  // ---- phase 1: scores of this workgroup's tiles -------------------------
  // B operand (weights): lane (head n, k-group g) holds, for slice u and
  // component c, the weight of summary column 16u + 4g + c.
  float wlin[NU][4], wquad[NU][4];
  {
    const bool hv = n < G;
    const size_t qoff = ((size_t)blockIdx.z * (size_t)(p.hkv * G) + (size_t)head * G + (hv ? n : 0)) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float q4[4];
      load_q4<E>(p.Q, qoff + 16 * u + 4 * g, q4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float qv = hv ? q4[c] : 0.f;
        wlin[u][c] = p.scale * qv;
        wquad[u][c] = (KIND == 0) ? 0.5f * p.alpha * p.scale * p.scale * qv * qv : 0.f;
      }
    }
  }
  const bool use_quad = p.alpha != 0.f;
  float run_m = -INFINITY, run_s = 0.f;      // LSE partial of head n over this lane's blocks
  const Coherent sc(p.scores + (size_t)unit * 16 * p.nb_pad, (uint32_t)(16 * p.nb_pad * 4));
  const Coherent lp(p.lse_part + (size_t)unit * p.splits * 32, (uint32_t)(p.splits * 32 * 4));
  const size_t sum_base = (size_t)(seq * p.hkv + head) * p.nb_max;
  const int tiles_total = (ncand + 15) / 16;
  for (int j = 0; j < p.tiles_per_wave; ++j) {
    const int tile = (blockIdx.x * 4 + wave) * p.tiles_per_wave + j;
    if (tile >= tiles_total) break;
    const int brow = min(tile * 16 + n, ncand - 1);     // A-operand row (block) of this lane
    const float* mrow = p.mu + (sum_base + brow) * D;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND == 0) {
      const float* vrow = p.so + (sum_base + brow) * D;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const f32x4 m4 = ld_f32x4(mrow + 16 * u + 4 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma_f32_16x16x4(m4[c], wlin[u][c], acc);
      }
      if (use_quad) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const f32x4 v4 = ld_f32x4(vrow + 16 * u + 4 * g);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc = mfma_f32_16x16x4(v4[c], wquad[u][c], acc);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const f32x4 m4 = ld_f32x4(mrow + 16 * u + 4 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma_f32_16x16x4(m4[c], wlin[u][c], acc);
      }
      if (use_quad) {
        const float* vbase = p.so + (sum_base + brow) * (size_t)(R * D);
        f32x4 quad = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          f32x4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const f32x4 v4 = ld_f32x4(vbase + r * D + 16 * u + 4 * g);
#pragma unroll
            for (int c = 0; c < 4; ++c) pr = mfma_f32_16x16x4(v4[c], wlin[u][c], pr);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) quad[i] += pr[i] * pr[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += 0.5f * p.alpha * quad[i];
      }
    }
    // acc[i]: score partial of block tile*16 + 4g + i for head n
    f32x4 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = tile * 16 + 4 * g + i;
      const int nbk = min(kBlock, L - b * kBlock);
      s[i] = (b < ncand) ? acc[i] + __logf((float)nbk) : -INFINITY;
      const float mx = fmaxf(run_m, s[i]);
      if (mx != -INFINITY) {
        run_s = run_s * __expf(run_m - mx) + __expf(s[i] - mx);
        run_m = mx;
      }
    }
    if (n < G) sc.st4((uint32_t)((n * p.nb_pad + tile * 16 + 4 * g) * 4), s);
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

  // ---- phase 2: LSE per head, group scores, radix select ------------------
  // every partial (max, sum) is fetched at once, then reduced from LDS
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

  const int per = (p.nb_max + kSelThreads - 1) / kSelThreads;   // <= kSelMaxPerThread
  uint32_t key[kSelMaxPerThread];
  float shat[kSelMaxPerThread];
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e) {
    key[e] = 0u;
    shat[e] = -INFINITY;
    const int b = threadIdx.x * per + e;
    if (e < per && b < ncand) {
      float v[16];
      float M = -INFINITY;
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        v[h] = (h < G) ? sc.ld1((uint32_t)((h * p.nb_pad + b) * 4)) - lse_sh[h] : -INFINITY;
        M = fmaxf(M, v[h]);
      }
      float S = 0.f;
#pragma unroll
      for (int h = 0; h < 16; ++h) S += (h < G) ? __expf(v[h] - M) : 0.f;
      shat[e] = M + __logf(S);
      key[e] = orderable(shat[e]);
    }
  }
  const int kk = min(p.top_k, ncand);
  uint32_t prefix = 0u, hi_mask = 0u;
  int need = kk;                                  // how many still to take at or below the prefix
  for (int pass = 0; pass < 4 && kk > 0; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[threadIdx.x] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      const int b = threadIdx.x * per + e;
      if (e < per && b < ncand && (key[e] & hi_mask) == prefix)
        atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int tot = (int)(h0 + h1 + h2 + h3);
      int incl = tot;                             // sum over lanes >= this lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += y;
      }
      int above = incl - tot;                     // elements in higher bins than this lane's
      const uint32_t hs[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < need && need <= above + (int)hs[j]) {
          bcast[1] = 4 * lane + j;
          bcast[2] = need - above;
        }
        above += (int)hs[j];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[1] << shift;
    hi_mask |= 255u << shift;
    need = bcast[2];
    __syncthreads();
  }
  // `prefix` is the k-th largest key; `need` keys equal to it are taken, lowest index first
  int eq_count = 0;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e) {
    const int b = threadIdx.x * per + e;
    eq_count += (e < per && b < ncand && kk > 0 && key[e] == prefix) ? 1 : 0;
  }
  int eq_total;
  int eq_rank = block_exclusive_scan(eq_count, scan_w, &eq_total);
  bool take[kSelMaxPerThread];
  int take_count = 0;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e) {
    const int b = threadIdx.x * per + e;
    const bool valid = e < per && b < ncand && kk > 0;
    bool tk = valid && key[e] > prefix;
    if (valid && key[e] == prefix) { tk = eq_rank < need; ++eq_rank; }
    take[e] = tk;
    take_count += tk ? 1 : 0;
  }
  int sel_total;
  int pos = block_exclusive_scan(take_count, scan_w, &sel_total);
  int32_t* sel_u = p.sel + (size_t)unit * p.top_k;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e) {
    if (take[e]) sel_u[pos++] = threadIdx.x * per + e;
  }
  for (int i = sel_total + (int)threadIdx.x; i < p.top_k; i += kSelThreads) sel_u[i] = -1;
  if (p.sel_score) {
    float* ss = p.sel_score + (size_t)unit * p.nb_max;
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      const int b = threadIdx.x * per + e;
      if (e < per && b < p.nb_max) ss[b] = shat[e];
    }
  }
  if (threadIdx.x == 0) reset_counter(p.counters + unit);   // zero for the next call
}

template <typename E, int D>
static hipError_t launch_sel_t(const SelectArgs& a, const SelParams& sp) {
  dim3 grid(a.splits, a.hkv, a.batch * a.tokens);
  if (a.so_kind == 0) {
    hipLaunchKernelGGL((k_select<E, D, 0, 1>), grid, dim3(kSelThreads), 0, a.stream, sp);
  } else {
    switch (a.rank) {
#define COBS_R(r) case r: hipLaunchKernelGGL((k_select<E, D, 1, r>), grid, dim3(kSelThreads), 0, a.stream, sp); break;
      COBS_R(1) COBS_R(2) COBS_R(3) COBS_R(4) COBS_R(5) COBS_R(6) COBS_R(7) COBS_R(8)
#undef COBS_R
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
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
