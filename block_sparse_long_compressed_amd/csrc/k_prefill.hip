// Chunked causal prefill (gfx950): per-token block selection, and the per-token
// attention path for fp32 inputs, for queries at positions t = q_pos0 .. q_pos0+T-1
// of a sequence whose block summaries were built once over the whole prefix.
//
// Selection (COBS explainer, Technisches Resuemee 2.1-2.3; skill card "Method")
// is the decode rule applied to each token's causal candidate set (blocks whose
// keys all lie at positions <= t).  Three kernels, by kind and context length:
//   k_prefill_select_pair  diagonal summaries, up to 512 blocks: two tokens per
//                          workgroup share each summary tile load; scores stay in
//                          registers and the group score is a DPP row reduction;
//   k_prefill_select_wg    other kinds, up to 2048 blocks: one workgroup per
//                          (token, group), per-head scores staged in LDS;
//   k_prefill_select       longer contexts: one wave per (token, group) scoring
//                          twice (online log-sum-exp, then the group scores) and a
//                          single-wave radix select (DPP scans, ballots, no barriers).
// All keep the top-k with ties to the lower block index.
//
// Attention for fp32 inputs (NSA branches, Janus issue #181): one workgroup per
// (token, group); wave 0 runs the selected blocks, wave 1 the window [t-W+1, t],
// waves 2-3 the two halves of the visible pooled tokens, each with the shared
// 64-key tile routine; the waves' (max, sum, O) are merged in LDS and the gated
// sum is written directly.  bf16 inputs use the token-blocked kernel in
// k_prefill_attn.hip.
#include "attn_tile.h"
#include "cobs_device.h"
#include "cobs_launch.h"
#include "score_common.h"

#include <algorithm>

namespace cobs {

struct PsParams {
  int tokens, hkv, group, max_len, nb_max, nb_pad, top_k, rank, q_pos0, L_fixed;
  float alpha, scale;
  const int32_t* seq_lens;          // null: every sequence has length L_fixed
  const void* Q;
  const void *mu, *so;
  const float* P;                   // query subspaces [hkv][sub_s][d] (subspace score kinds)
  int sub_s, vlen;                  // subspace dimension; length of a rank-r vector
  int32_t* sel;
  float* sel_score;
};

template <typename E, int D, int KIND>
__global__ __launch_bounds__(256) void k_prefill_select(PsParams p) {
  constexpr int NU = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int tok = blockIdx.x * 4 + wave;
  const int head = blockIdx.y, seq = blockIdx.z;
  __shared__ __align__(16) uint32_t hist[4][256];
  extern __shared__ uint32_t s_keys_all[];        // [4][nb_pad]
  if (tok >= p.tokens) return;                    // waves are independent: no barriers below
  uint32_t* s_key = s_keys_all + (size_t)wave * p.nb_pad;
  uint32_t* h = hist[wave];

  const int L = p.seq_lens ? p.seq_lens[seq] : p.L_fixed;
  const int t = p.q_pos0 + tok;
  const int ncand = candidate_blocks(L, t);
  const int G = p.group;
  const size_t unit = ((size_t)seq * p.tokens + tok) * p.hkv + head;
  const size_t sum_base = ((size_t)seq * p.hkv + head) * p.nb_max;
  const int tiles = (ncand + 15) / 16;

  ScoreW<D> W;
  prepare_weights<E, D, KIND>(p.Q, (((size_t)seq * p.tokens + tok) * (size_t)(p.hkv * G) + (size_t)head * G) * D,
                              n, g, G, p.scale, W);
  if constexpr (Kind<KIND>::kSub) {
    subspace_weights_part<D>(p.P + (size_t)head * p.sub_s * D, p.sub_s, p.vlen, 0, 1, n, g, W.lin, nullptr, W.quad);
    finish_subspace_weights<E, D, KIND>(W);
  }
  const bool use_quad = p.alpha != 0.f;
  auto scores = [&](int tile) -> f32x4 {
    const int brow = min(tile * 16 + n, ncand - 1);
    const void *mr, *vr;
    summary_rows<D, KIND>(p.mu, p.so, sum_base + brow, p.rank, p.vlen, mr, vr);
    f32x4 s = score_tile<E, D, KIND>(mr, vr, p.rank, p.vlen, g, use_quad, p.alpha, p.scale, W);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = tile * 16 + 4 * g + i;
      s[i] = (b < ncand && n < G) ? s[i] + __logf((float)min(kBlock, L - b * kBlock)) : -INFINITY;
    }
    return s;
  };

  // pass 1: per-head log-sum-exp over the candidates
  float run_m = -INFINITY, run_s = 0.f;
#pragma unroll 1
  for (int tile = 0; tile < tiles; ++tile) {
    const f32x4 s = scores(tile);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mx = fmaxf(run_m, s[i]);
      if (mx != -INFINITY) { run_s = run_s * __expf(run_m - mx) + __expf(s[i] - mx); run_m = mx; }
    }
  }
#pragma unroll
  for (int m = 16; m < 64; m <<= 1) {
    const float om = shfl_xor_f(run_m, m), os = shfl_xor_f(run_s, m);
    const float mx = fmaxf(run_m, om);
    if (mx != -INFINITY) { run_s = run_s * __expf(run_m - mx) + os * __expf(om - mx); run_m = mx; }
  }
  const float lse = (run_m == -INFINITY) ? 0.f : run_m + __logf(run_s);

  // pass 2: group score shat_b = ln sum_h exp(s_hb - LSE_h), reduced over the 16 lanes of a row
#pragma unroll 1
  for (int tile = 0; tile < tiles; ++tile) {
    const f32x4 s = scores(tile);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = s[i] - lse;                 // -inf for heads >= G and non-candidates
      float M = v;
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) M = fmaxf(M, shfl_xor_f(M, m));
      float S = (M == -INFINITY) ? 0.f : __expf(v - M);
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) S += shfl_xor_f(S, m);
      const int b = tile * 16 + 4 * g + i;
      if (n == 0 && b < ncand) s_key[b] = orderable(M + __logf(S));
      if (n == 0 && b < ncand && p.sel_score) p.sel_score[unit * p.nb_max + b] = M + __logf(S);
    }
  }
  if (p.sel_score) {
    for (int b = ncand + lane; b < p.nb_max; b += 64) p.sel_score[unit * p.nb_max + b] = -INFINITY;
  }

  // single-wave radix select over s_key[0, ncand); lane owns [lb0, lb1)
  const int per_l = (ncand + 63) / 64;
  const int lb0 = min(lane * per_l, ncand), lb1 = min(lb0 + per_l, ncand);
  const int kk = min(p.top_k, ncand);
  uint32_t prefix = 0u, hi_mask = 0u;
  int need = kk, eq_bin = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4 && kk > 0; ++pass) {
    const int shift = 24 - 8 * pass;
    *reinterpret_cast<u32x4*>(&h[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int e = 0; e < per_l; ++e) {
      const int b = lb0 + e;
      const uint32_t key = (b < lb1) ? s_key[b] : 0u;
      wave_histogram_add(h, b < lb1 && (key & hi_mask) == prefix, (key >> shift) & 255u);
    }
    const u32x4 hb = *reinterpret_cast<const u32x4*>(&h[4 * lane]);
    prefix |= radix_digit(hb, need, eq_bin) << shift;
    hi_mask |= 255u << shift;
  }
  int eq_rank = 0;
  if (kk > 0 && need < eq_bin) {
    int c = 0;
#pragma unroll 1
    for (int b = lb0; b < lb1; ++b) c += (s_key[b] == prefix) ? 1 : 0;
    eq_rank = wave_inclusive_sum(c) - c;
  }
  int take = 0;
  if (kk > 0) {
    int r = eq_rank;
#pragma unroll 1
    for (int b = lb0; b < lb1; ++b) {
      const uint32_t key = s_key[b];
      if (key > prefix) ++take;
      else if (key == prefix) { take += (r < need) ? 1 : 0; ++r; }
    }
  }
  const int tincl = wave_inclusive_sum(take);
  const int total = __builtin_amdgcn_readlane(tincl, 63);
  int pos = tincl - take;
  int32_t* sel_u = p.sel + unit * p.top_k;
  if (kk > 0) {
    int r = eq_rank;
#pragma unroll 1
    for (int b = lb0; b < lb1; ++b) {
      const uint32_t key = s_key[b];
      bool tk = key > prefix;
      if (key == prefix) { tk = r < need; ++r; }
      if (tk) sel_u[pos++] = b;
    }
  }
  for (int i = total + lane; i < p.top_k; i += 64) sel_u[i] = -1;
}

// One workgroup per (token, kv-head group) for contexts up to kPsWgMaxBlocks
// blocks: the four waves score interleaved 16-block tiles once, keep the per-head scores block-major in LDS, combine their
// per-head log-sum-exp partials, form the group scores from LDS and run the
// workgroup radix select.  Longer contexts use the one-wave kernel above, which
// scores twice instead of storing.
constexpr int kPsWgMaxBlocks = 2048;

struct PsWgLds {
  float red_m[4][16], red_s[4][16];
  uint32_t hist2[2][4][256];
  int scan_w[4];
  float lse_sh[16];
  // followed by [nb_pad][16] scores and [nb_pad] keys
};

template <typename E, int D, int KIND>
__global__ __launch_bounds__(256, (KIND == 1 || KIND == 4) ? 2 : 3) void k_prefill_select_wg(PsParams p) {
  constexpr int NU = D / 16;
  constexpr int RING = 1;        // one tile in flight per wave; three waves per SIMD hide the rest
  extern __shared__ __align__(16) unsigned char smem[];
  PsWgLds& sl = *reinterpret_cast<PsWgLds*>(smem);
  float* s_sc = reinterpret_cast<float*>(smem + sizeof(PsWgLds));
  uint32_t* s_key = reinterpret_cast<uint32_t*>(s_sc + (size_t)p.nb_pad * 16);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int tok = blockIdx.x, head = blockIdx.y, seq = blockIdx.z;
  const int L = p.seq_lens ? p.seq_lens[seq] : p.L_fixed;
  const int t = p.q_pos0 + tok;
  const int ncand = candidate_blocks(L, t);
  const int G = p.group;
  const size_t unit = ((size_t)seq * p.tokens + tok) * p.hkv + head;
  const size_t sum_base = ((size_t)seq * p.hkv + head) * p.nb_max;
  const int tiles = (ncand + 15) / 16;
  const bool use_quad = p.alpha != 0.f;
  auto rows_of = [&](int tile, const void*& mr, const void*& vr) {
    const int brow = min(tile * 16 + n, ncand - 1);
    summary_rows<D, KIND>(p.mu, p.so, sum_base + brow, p.rank, p.vlen, mr, vr);
  };

  // ---- scores of tiles wave, wave+4, ... (summary rows requested before the query)
  SumTile<D, KIND> st[RING];
  const void* vrow[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) {
    vrow[r] = nullptr;
    const int tile = wave + 4 * r;
    if (tile < tiles) {
      const void* mrow;
      rows_of(tile, mrow, vrow[r]);
      sum_tile_load<D, KIND>(mrow, vrow[r], p.rank, p.vlen, g, use_quad, st[r]);
    }
  }
  ScoreW<D> W;
  prepare_weights<E, D, KIND>(p.Q, (((size_t)seq * p.tokens + tok) * (size_t)(p.hkv * G) + (size_t)head * G) * D,
                              n, g, G, p.scale, W);
  if constexpr (Kind<KIND>::kSub) {
    // scale * P q: the four waves each contract a quarter of the column tiles (exchange
    // area after the keys)
    f32x4* xch = reinterpret_cast<f32x4*>(s_key + p.nb_pad);
    subspace_weights_part<D>(p.P + (size_t)head * p.sub_s * D, p.sub_s, p.vlen, wave, 4, n, g, W.lin, xch, W.quad);
    __syncthreads();
    subspace_weights_gather<D>(p.vlen, wave, 4, n, g, xch, W.quad);
    finish_subspace_weights<E, D, KIND>(W);
  }
  float run_m = -INFINITY, run_s = 0.f;
#pragma unroll 1
  for (int j0 = 0; wave + 4 * j0 < tiles; j0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int tile = wave + 4 * (j0 + r);
      if (tile < tiles) {
        const f32x4 s4 = tile_score<E, D, KIND>(st[r], vrow[r], p.rank, p.vlen, g, use_quad, p.alpha, p.scale, W);
        if (tile + 4 * RING < tiles) {
          const void* mrow;
          rows_of(tile + 4 * RING, mrow, vrow[r]);
          sum_tile_load<D, KIND>(mrow, vrow[r], p.rank, p.vlen, g, use_quad, st[r]);
        }
        float sv[4];
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = tile * 16 + 4 * g + i;
          const int nbk = min(kBlock, L - b * kBlock);
          sv[i] = (b < ncand) ? s4[i] + (nbk == kBlock ? kLnBlock : __logf((float)nbk)) : -INFINITY;
          mt = fmaxf(mt, sv[i]);
          s_sc[b * 16 + n] = sv[i];
        }
        const float mx = fmaxf(run_m, mt);      // one rescale per tile
        if (mx != -INFINITY) {
          run_s *= __expf(run_m - mx);
#pragma unroll
          for (int i = 0; i < 4; ++i) run_s += __expf(sv[i] - mx);
          run_m = mx;
        }
      }
    }
  }
#pragma unroll
  for (int m = 16; m < 64; m <<= 1) {
    const float om = shfl_xor_f(run_m, m), os = shfl_xor_f(run_s, m);
    const float mx = fmaxf(run_m, om);
    if (mx != -INFINITY) { run_s = run_s * __expf(run_m - mx) + os * __expf(om - mx); run_m = mx; }
  }
  if (g == 0) { sl.red_m[wave][n] = run_m; sl.red_s[wave][n] = run_s; }
  __syncthreads();
  if (threadIdx.x < 16) {
    float M = -INFINITY, S = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float om = sl.red_m[w][threadIdx.x], os = sl.red_s[w][threadIdx.x];
      const float mx = fmaxf(M, om);
      if (mx != -INFINITY) { S = S * __expf(M - mx) + os * __expf(om - mx); M = mx; }
    }
    sl.lse_sh[threadIdx.x] = (M == -INFINITY) ? -INFINITY : M + __logf(S);
  }
  __syncthreads();

  // ---- group scores shat_b = ln sum_h exp(s_hb - LSE_h); thread owns [tid*per, +per)
  const int per = (ncand + 255) / 256;
  float lse_r[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) lse_r[h] = sl.lse_sh[h];
  const int b0 = threadIdx.x * per;
#pragma unroll 1
  for (int e = 0; e < per; ++e) {
    const int b = b0 + e;
    if (b >= ncand) break;
    f32x4 raw[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) raw[v] = *reinterpret_cast<const f32x4*>(&s_sc[b * 16 + 4 * v]);
    float M = -INFINITY;
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if (h < G) M = fmaxf(M, raw[h >> 2][h & 3] - lse_r[h]);
    float S = 0.f;
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if (h < G) S += __expf(raw[h >> 2][h & 3] - lse_r[h] - M);
    const float sh = M + __logf(S);
    s_key[b] = orderable(sh);
    if (p.sel_score) p.sel_score[unit * p.nb_max + b] = sh;
  }
  if (p.sel_score) {
    for (int b = ncand + threadIdx.x; b < p.nb_max; b += 256) p.sel_score[unit * p.nb_max + b] = -INFINITY;
  }
  __syncthreads();

  int32_t* sel_u = p.sel + unit * p.top_k;
  const int total = wg_select_topk(s_key, ncand, per, p.top_k, &sl.hist2[0][0][0], sl.scan_w,
                                   [&](int pos, int b) { sel_u[pos] = b; });
  for (int i = total + (int)threadIdx.x; i < p.top_k; i += 256) sel_u[i] = -1;
}

// Diagonal summaries, up to kPairMaxBlocks candidate blocks: one workgroup per T
// consecutive tokens of a kv-head group.  Each summary tile is loaded once and
// scored for all T tokens (their query weights sit in LDS in the B-operand layout,
// read 16 bytes at a time), so a tile's load serves T times the MFMA work.  Every
// lane keeps its tiles' scores in registers; the group score of a block is formed
// across the 16 lanes of a row (one head each) with DPP row rotations, so no
// per-head score array is staged.  Then the workgroup radix select, per token.
constexpr int kPairTiles = 8;                         // tiles per wave (4 waves)
constexpr int kPairMaxBlocks = 4 * kPairTiles * 16;   // 512
constexpr int kPairTMax = 4;                          // tokens per workgroup, at most
constexpr int kPairTokens = 2;   // measured: 4 tokens (two waves per SIMD, four serial selects) is slower

template <typename E, int D>
constexpr size_t pair_weight_bytes(int T) {       // query weights of a workgroup's tokens in LDS
  return E::kBytes == 2 ? (size_t)T * 3 * (D / 32) * 64 * 16 : (size_t)T * (D / 8) * 64 * 16;
}

struct PsPairLds {
  float red_m[kPairTMax][4][16], red_s[kPairTMax][4][16];
  float lse_sh[kPairTMax][16];
  uint32_t hist2[2][4][256];
  int scan_w[4];
  int ncand[kPairTMax];
  // followed by the weights [T][2D/16][64][4] floats and the keys [T][kPairMaxBlocks]
};

// Full reduction over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false)));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
  return x;
}

template <typename E, int D, int T>
__global__ __launch_bounds__(256, (T <= 2 && E::kBytes == 4) ? 3 : 2) void k_prefill_select_pair(PsParams p) {
  constexpr int NU = D / 16, NJ = D / 32;
  constexpr int NQ = 2 * NU;                          // fp32: 16-byte weight groups per token, lin then quad
  constexpr bool kSplit = E::kBytes == 2;             // bf16 queries: split-bf16 contraction
  extern __shared__ __align__(16) unsigned char smem[];
  PsPairLds& sl = *reinterpret_cast<PsPairLds*>(smem);
  float* wB = reinterpret_cast<float*>(smem + sizeof(PsPairLds));        // fp32: [T][NQ][64][4]
  u32x4* wS = reinterpret_cast<u32x4*>(wB);                              // bf16: [T][3][NJ][64]
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem + sizeof(PsPairLds) + pair_weight_bytes<E, D>(T));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int tok0 = T * blockIdx.x, head = blockIdx.y, seq = blockIdx.z;
  const int L = p.seq_lens ? p.seq_lens[seq] : p.L_fixed;
  const int G = p.group;
  bool live[T];
  int ncand[T], nmax = 0;
#pragma unroll
  for (int u = 0; u < T; ++u) {
    live[u] = tok0 + u < p.tokens;
    ncand[u] = live[u] ? candidate_blocks(L, p.q_pos0 + tok0 + u) : 0;
    nmax = max(nmax, ncand[u]);
  }
  if (threadIdx.x < T) sl.ncand[threadIdx.x] = candidate_blocks(L, p.q_pos0 + tok0 + threadIdx.x);
  const int tiles = (nmax + 15) / 16;
  const size_t sum_base = ((size_t)seq * p.hkv + head) * p.nb_max;
  const bool use_quad = p.alpha != 0.f;

  // the first tile's summary rows go out before the weights are formed
  SumTile<D, 0> st;
  auto load_tile = [&](int tile) {
    const int brow = min(tile * 16 + n, nmax - 1);
    const void *mrow, *vrow;
    summary_rows<D, 0>(p.mu, p.so, sum_base + brow, 0, D, mrow, vrow);
    sum_tile_load<D, 0>(mrow, vrow, 0, D, g, use_quad, st);
  };
  if (wave < tiles) load_tile(wave);

  if constexpr (kSplit) {
    // bf16 queries: the contraction runs on v_mfma_f32_16x16x32_bf16 with exact
    // products.  Lane (n, g)'s eight k-slots of chunk j are features 16u + 4g + c for
    // u = 2j, 2j+1 (the order its fp32 summary loads hold); per token and chunk: q
    // (bf16, exact), and q^2 (exact in fp32, 16 significant bits) as hi + lo bf16 parts
    // whose sum is exact.  Zero for columns n >= G.
    for (int idx = threadIdx.x; idx < T * NJ * 64; idx += 256) {
      const int u = idx / (NJ * 64), r = idx % (NJ * 64), j = r / 64, l = r % 64;
      const int ln = l & 15, lg = l >> 4;
      u32x4 qw = {0u, 0u, 0u, 0u};
      if (ln < G && live[u]) {
        const uint16_t* qh = static_cast<const uint16_t*>(p.Q) +
            (((size_t)seq * p.tokens + tok0 + u) * (size_t)(p.hkv * G) + (size_t)head * G + ln) * D;
        const uint2 x0 = *reinterpret_cast<const uint2*>(qh + 32 * j + 4 * lg);
        const uint2 x1 = *reinterpret_cast<const uint2*>(qh + 32 * j + 16 + 4 * lg);
        qw = u32x4{x0.x, x0.y, x1.x, x1.y};
      }
      u32x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __uint_as_float(qw[e] << 16), b = __uint_as_float(qw[e] & 0xFFFF0000u);
        const float a2 = a * a, b2 = b * b;
        hi[e] = pack_bf16x2(a2, b2);
        lo[e] = pack_bf16x2(a2 - __uint_as_float(hi[e] << 16), b2 - __uint_as_float(hi[e] & 0xFFFF0000u));
      }
      wS[(((size_t)u * 3 + 0) * NJ + j) * 64 + l] = qw;
      wS[(((size_t)u * 3 + 1) * NJ + j) * 64 + l] = hi;
      wS[(((size_t)u * 3 + 2) * NJ + j) * 64 + l] = lo;
    }
  } else {
    // weights of the T tokens: lane (n, g) of 16-byte group j holds feature 16(j % NU) + 4g + c,
    // c = 0..3: scale q (j < NU), then alpha/2 (scale q)^2; zero for columns n >= G
    for (int idx = threadIdx.x; idx < T * NU * 64; idx += 256) {
      const int u = idx / (NU * 64), r = idx % (NU * 64), j = r / 64, l = r % 64;
      const int ln = l & 15, lg = l >> 4;
      float q4[4] = {0.f, 0.f, 0.f, 0.f};
      if (ln < G && live[u])
        load_q4<E>(p.Q, (((size_t)seq * p.tokens + tok0 + u) * (size_t)(p.hkv * G) + (size_t)head * G + ln) * D +
                            16 * j + 4 * lg, q4);
      f32x4 wl, wq;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        wl[c] = p.scale * q4[c];
        wq[c] = 0.5f * p.alpha * wl[c] * wl[c];
      }
      *reinterpret_cast<f32x4*>(&wB[(((size_t)u * NQ + j) * 64 + l) * 4]) = wl;
      *reinterpret_cast<f32x4*>(&wB[(((size_t)u * NQ + NU + j) * 64 + l) * 4]) = wq;
    }
  }
  __syncthreads();

  // ---- scores of tiles wave, wave + 4, ... for the T tokens, kept in registers
  f32x4 sreg[T][kPairTiles];
  float run_m[T], run_s[T];
#pragma unroll
  for (int u = 0; u < T; ++u) { run_m[u] = -INFINITY; run_s[u] = 0.f; }
#pragma unroll
  for (int i = 0; i < kPairTiles; ++i) {
    const int tile = wave + 4 * i;
#pragma unroll
    for (int u = 0; u < T; ++u) sreg[u][i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (tile < tiles) {
      f32x4 acc[T], acc2[T];
#pragma unroll
      for (int u = 0; u < T; ++u) {
        acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (kSplit) {
        // the tile's fp32 means and variances as hi + lo bf16 parts (16 of their 24
        // significand bits), in the chunk order of the weights
        u32x4 mh[NJ], ml[NJ], vh[NJ], vl[NJ];
        auto split8 = [&](const f32x4& x, const f32x4& y, u32x4& h, u32x4& lw) {
          h = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          const float xs[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lw[e] = pack_bf16x2(xs[2 * e] - __uint_as_float(h[e] << 16), xs[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u));
        };
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          split8(st.m4[2 * j], st.m4[2 * j + 1], mh[j], ml[j]);
          if (use_quad) split8(st.v4[0][2 * j], st.v4[0][2 * j + 1], vh[j], vl[j]);
        }
#pragma unroll
        for (int u = 0; u < T; ++u) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const u32x4 qw = wS[(((size_t)u * 3 + 0) * NJ + j) * 64 + lane];
            acc[u] = mfma_bf16_16x16x32(mh[j], qw, acc[u]);
            acc[u] = mfma_bf16_16x16x32(ml[j], qw, acc[u]);
          }
          if (use_quad) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              const u32x4 q2h = wS[(((size_t)u * 3 + 1) * NJ + j) * 64 + lane];
              const u32x4 q2l = wS[(((size_t)u * 3 + 2) * NJ + j) * 64 + lane];
              acc2[u] = mfma_bf16_16x16x32(vh[j], q2h, acc2[u]);
              acc2[u] = mfma_bf16_16x16x32(vh[j], q2l, acc2[u]);
              acc2[u] = mfma_bf16_16x16x32(vl[j], q2h, acc2[u]);
              acc2[u] = mfma_bf16_16x16x32(vl[j], q2l, acc2[u]);
            }
          }
          acc[u] = p.scale * acc[u] + (0.5f * p.alpha * p.scale * p.scale) * acc2[u];
          acc2[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      } else {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
#pragma unroll
          for (int u = 0; u < T; ++u) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(&wB[(((size_t)u * NQ + j) * 64 + lane) * 4]);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[u] = mfma_f32_16x16x4(st.m4[j][c], w[c], acc[u]);
          }
        }
        if (use_quad) {
#pragma unroll
          for (int j = 0; j < NU; ++j) {
#pragma unroll
            for (int u = 0; u < T; ++u) {
              const f32x4 w = *reinterpret_cast<const f32x4*>(&wB[(((size_t)u * NQ + NU + j) * 64 + lane) * 4]);
#pragma unroll
              for (int c = 0; c < 4; ++c) acc2[u] = mfma_f32_16x16x4(st.v4[0][j][c], w[c], acc2[u]);
            }
          }
        }
      }
      if (tile + 4 < tiles) load_tile(tile + 4);
#pragma unroll
      for (int u = 0; u < T; ++u) {
        const f32x4 s4 = acc[u] + acc2[u];
        float mt = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int b = tile * 16 + 4 * g + k;
          const int nbk = min(kBlock, L - b * kBlock);
          const float sv = (b < ncand[u]) ? s4[k] + (nbk == kBlock ? kLnBlock : __logf((float)nbk)) : -INFINITY;
          sreg[u][i][k] = sv;
          mt = fmaxf(mt, sv);
        }
        const float mx = fmaxf(run_m[u], mt);
        if (mx != -INFINITY) {
          run_s[u] *= __expf(run_m[u] - mx);
#pragma unroll
          for (int k = 0; k < 4; ++k) run_s[u] += __expf(sreg[u][i][k] - mx);
          run_m[u] = mx;
        }
      }
    }
  }
  // per-head log-sum-exp over the candidates, per token
#pragma unroll
  for (int u = 0; u < T; ++u) {
#pragma unroll
    for (int m = 16; m < 64; m <<= 1) {
      const float om = shfl_xor_f(run_m[u], m), os = shfl_xor_f(run_s[u], m);
      const float mx = fmaxf(run_m[u], om);
      if (mx != -INFINITY) {
        run_s[u] = run_s[u] * __expf(run_m[u] - mx) + os * __expf(om - mx);
        run_m[u] = mx;
      }
    }
    if (g == 0) { sl.red_m[u][wave][n] = run_m[u]; sl.red_s[u][wave][n] = run_s[u]; }
  }
  __syncthreads();
  if (threadIdx.x < 16 * T) {
    const int u = threadIdx.x >> 4, h = threadIdx.x & 15;
    float M = -INFINITY, S = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float om = sl.red_m[u][w][h], os = sl.red_s[u][w][h];
      const float mx = fmaxf(M, om);
      if (mx != -INFINITY) { S = S * __expf(M - mx) + os * __expf(om - mx); M = mx; }
    }
    sl.lse_sh[u][h] = (M == -INFINITY) ? -INFINITY : M + __logf(S);
  }
  __syncthreads();

  // ---- group scores shat_b = ln sum_h exp(s_hb - LSE_h): the 16 lanes of a row hold
  // the 16 heads of blocks 4g + k; lane n = k of the row writes block 4g + k's key
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const float lse_n = sl.lse_sh[u][n];
    const bool head_ok = n < G && lse_n != -INFINITY;
#pragma unroll
    for (int i = 0; i < kPairTiles; ++i) {
      const int tile = wave + 4 * i;
      if (tile < tiles) {
        float sh_mine = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = head_ok ? sreg[u][i][k] - lse_n : -INFINITY;
          const float M = row_max16(x);
          const float S = row_sum16(M == -INFINITY ? 0.f : __expf(x - M));
          const float sh = M + __logf(S);
          if (n == k) sh_mine = sh;
        }
        const int b = tile * 16 + 4 * g + n;
        if (n < 4 && b < ncand[u]) {
          keys[u * kPairMaxBlocks + b] = orderable(sh_mine);
          if (p.sel_score) p.sel_score[(((size_t)seq * p.tokens + tok0 + u) * p.hkv + head) * p.nb_max + b] = sh_mine;
        }
      }
    }
  }
  if (p.sel_score) {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      if (!live[u]) continue;
      float* ss = p.sel_score + (((size_t)seq * p.tokens + tok0 + u) * p.hkv + head) * p.nb_max;
      for (int b = ncand[u] + threadIdx.x; b < p.nb_max; b += 256) ss[b] = -INFINITY;
    }
  }
  __syncthreads();

#pragma unroll 1
  for (int u = 0; u < T; ++u) {
    if (tok0 + u >= p.tokens) break;
    const int nc = sl.ncand[u];
    int32_t* sel_u = p.sel + (((size_t)seq * p.tokens + tok0 + u) * p.hkv + head) * p.top_k;
    const int per = (nc + 255) / 256;
    const int total = wg_select_topk(keys + u * kPairMaxBlocks, nc, per, p.top_k, &sl.hist2[0][0][0],
                                     sl.scan_w, [&](int pos, int b) { sel_u[pos] = b; });
    for (int i = total + (int)threadIdx.x; i < p.top_k; i += 256) sel_u[i] = -1;
    __syncthreads();                                  // histograms reused by the next token
  }
}

struct AuParams {
  int tokens, hkv, group, seq_len, nc_max, top_k, window, cmp_on, q_pos0;
  float scale_log2;
  const void *Q, *K, *V, *kc, *vc;
  const float* gates;
  const int32_t* sel;
  float* out;
};

template <typename E, int D>
__global__ __launch_bounds__(256) void k_attn_unit(AuParams p) {
  using T = AttnTiling<E, D>;
  constexpr int NCH = T::kChunks, EPL = T::kEpl, NDT = T::kDt;
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int tok = blockIdx.x, head = blockIdx.y;
  const int G = p.group, L = p.seq_len;
  const int t = p.q_pos0 + tok;
  const size_t unit = (size_t)tok * p.hkv + head;

  u32x4 qf[NCH];
  {
    const typename E::storage* Qh = reinterpret_cast<const typename E::storage*>(p.Q) +
                                    ((size_t)tok * p.hkv * G + (size_t)head * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qf[c] = ld16(Qh + (4 * c + g) * EPL);
      if (n >= G) qf[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)head * L * D;
  const typename E::storage* Vu = reinterpret_cast<const typename E::storage*>(p.V) + (size_t)head * L * D;
  const int nc = (p.cmp_on && t >= 31) ? (t - 31) / 16 + 1 : 0;          // pooled tokens with 16j+31 <= t
  const int win_len = p.window > 0 ? min(p.window, t + 1) : 0;
  const int win_start = t + 1 - win_len;
  const int ntc = (nc + kBlock - 1) / kBlock, half = (ntc + 1) / 2;

  typename E::storage* lds = reinterpret_cast<typename E::storage*>(smem) + (size_t)wave * kBlock * T::kRowStride;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int count = wave == 0 ? p.top_k : wave == 1 ? (win_len + kBlock - 1) / kBlock : wave == 2 ? half : ntc - half;
  for (int j = 0; j < count; ++j) {
    const typename E::storage *Kt = nullptr, *Vt = nullptr;
    int nvalid = 0;
    if (wave == 0) {
      const int b = p.sel[unit * p.top_k + j];
      if (b >= 0) { nvalid = min(kBlock, L - b * kBlock); Kt = Ku + (size_t)b * kBlock * D; Vt = Vu + (size_t)b * kBlock * D; }
    } else if (wave == 1) {
      const int start = win_start + j * kBlock;
      nvalid = min(kBlock, t + 1 - start);
      Kt = Ku + (size_t)start * D; Vt = Vu + (size_t)start * D;
    } else {
      const int start = (j + (wave == 3 ? half : 0)) * kBlock;
      nvalid = min(kBlock, nc - start);
      const size_t cu = (size_t)head * p.nc_max;
      Kt = reinterpret_cast<const typename E::storage*>(p.kc) + (cu + start) * D;
      Vt = reinterpret_cast<const typename E::storage*>(p.vc) + (cu + start) * D;
    }
    if (nvalid <= 0) continue;
    attend_tile<E, D>(Kt, Vt, nvalid, qf, p.scale_log2, lds, m_run, l_run, acc_o);
  }

  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);        // [4][16][D]
  float* mml = mo + 4 * 16 * D;                      // [4][16][2]
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mo[((size_t)wave * 16 + n) * D + 16 * dt + 4 * g + i] = acc_o[dt][i];
  }
  if (g == 0) { mml[(wave * 16 + n) * 2] = m_run; mml[(wave * 16 + n) * 2 + 1] = l_run; }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += blockDim.x) {
    const int hh = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
    const int hq = head * G + hh;
    float gt[3] = {0.f, 1.f, 0.f};                   // (cmp, slc, win)
    if (p.gates) {
      const float* gp = p.gates + ((size_t)tok * p.hkv * G + hq) * 3;
      gt[0] = gp[0]; gt[1] = gp[1]; gt[2] = gp[2];
    }
    auto wave_o = [&](int w) -> f32x4 { return ld_f32x4(mo + ((size_t)w * 16 + hh) * D + d4); };
    auto wm = [&](int w) { return mml[(w * 16 + hh) * 2]; };
    auto wl = [&](int w) { return mml[(w * 16 + hh) * 2 + 1]; };
    f32x4 res = {0.f, 0.f, 0.f, 0.f};
    if (wl(0) > 0.f) res += (gt[1] / wl(0)) * wave_o(0);
    if (wl(1) > 0.f) res += (gt[2] / wl(1)) * wave_o(1);
    const float M = fmaxf(wl(2) > 0.f ? wm(2) : -INFINITY, wl(3) > 0.f ? wm(3) : -INFINITY);
    if (M != -INFINITY) {
      const float f2 = wl(2) > 0.f ? fast_exp2(wm(2) - M) : 0.f, f3 = wl(3) > 0.f ? fast_exp2(wm(3) - M) : 0.f;
      const float Ls = f2 * wl(2) + f3 * wl(3);
      res += (gt[0] / Ls) * (f2 * wave_o(2) + f3 * wave_o(3));
    }
    st_f32x4(p.out + ((size_t)tok * p.hkv * G + hq) * D + d4, res);
  }
}

template <typename E, int D, int KIND>
static hipError_t launch_ps(const PrefillArgs& a, const PsParams& sp) {
  if (KIND == 0 && sp.nb_pad <= kPairMaxBlocks) {
    constexpr int T = kPairTokens;
    dim3 grid((a.tokens + T - 1) / T, a.hkv, a.batch);
    const size_t lds = sizeof(PsPairLds) + pair_weight_bytes<E, D>(T) + (size_t)T * kPairMaxBlocks * sizeof(uint32_t);
    hipLaunchKernelGGL((k_prefill_select_pair<E, D, T>), grid, dim3(256), lds, a.stream, sp);
    return hipGetLastError();
  }
  if (sp.nb_pad <= kPsWgMaxBlocks) {
    dim3 grid(a.tokens, a.hkv, a.batch);
    const size_t lds = sizeof(PsWgLds) + (size_t)sp.nb_pad * 17 * sizeof(float) +
                       (Kind<KIND>::kSub ? (size_t)(D / 16) * 64 * sizeof(f32x4) : 0);
    hipLaunchKernelGGL((k_prefill_select_wg<E, D, KIND>), grid, dim3(256), lds, a.stream, sp);
    return hipGetLastError();
  }
  dim3 grid((a.tokens + 3) / 4, a.hkv, a.batch);
  const size_t lds = (size_t)4 * sp.nb_pad * sizeof(uint32_t);
  hipLaunchKernelGGL((k_prefill_select<E, D, KIND>), grid, dim3(256), lds, a.stream, sp);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_ps_e(const PrefillArgs& a, const PsParams& sp) {
  if (a.so_kind == 0) return launch_ps<E, D, 0>(a, sp);
  if (a.so_kind == 3) return launch_ps<E, D, 3>(a, sp);
  if (a.so_kind == 4) return launch_ps<E, D, 4>(a, sp);
  if (a.so_kind == 5) return launch_ps<E, D, 5>(a, sp);
  return launch_ps<E, D, 1>(a, sp);
}

hipError_t launch_prefill_select(const PrefillArgs& a) {
  PsParams sp;
  sp.tokens = a.tokens; sp.hkv = a.hkv; sp.group = a.group; sp.max_len = a.max_len; sp.nb_max = a.nb_max;
  sp.nb_pad = (a.nb_max + 15) / 16 * 16; sp.top_k = a.top_k; sp.rank = a.rank; sp.q_pos0 = a.q_pos0;
  sp.L_fixed = a.max_len; sp.alpha = a.alpha; sp.scale = a.scale; sp.seq_lens = a.seq_lens; sp.Q = a.Q;
  sp.mu = a.mu; sp.so = a.so; sp.P = a.P; sp.sub_s = a.sub_s; sp.vlen = a.vlen; sp.sel = a.sel; sp.sel_score = a.sel_score;
  if (a.bf16) return a.head_dim == 128 ? launch_ps_e<EltBF16, 128>(a, sp) : launch_ps_e<EltBF16, 64>(a, sp);
  return a.head_dim == 128 ? launch_ps_e<EltF32, 128>(a, sp) : launch_ps_e<EltF32, 64>(a, sp);
}

template <typename E, int D>
static hipError_t launch_au(const PrefillArgs& a, const AuParams& ap) {
  dim3 grid(a.tokens, a.hkv, 1);
  const size_t lds = std::max(attn_lds_bytes<E, D>(4), (size_t)4 * 16 * (D + 2) * sizeof(float));
  hipLaunchKernelGGL((k_attn_unit<E, D>), grid, dim3(256), lds, a.stream, ap);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillArgs& a) {
  if (a.bf16) return launch_prefill_attn_bf16(a);      // token-blocked kernel (k_prefill_attn.hip)
  AuParams ap;
  ap.tokens = a.tokens; ap.hkv = a.hkv; ap.group = a.group; ap.seq_len = a.max_len; ap.nc_max = a.nc_max;
  ap.top_k = a.top_k; ap.window = a.window; ap.cmp_on = a.cmp_on; ap.q_pos0 = a.q_pos0;
  ap.scale_log2 = a.scale * kLog2e; ap.Q = a.Q; ap.K = a.K; ap.V = a.V; ap.kc = a.kc; ap.vc = a.vc;
  ap.gates = a.gates; ap.sel = a.sel; ap.out = a.out;
  return a.head_dim == 128 ? launch_au<EltF32, 128>(a, ap) : launch_au<EltF32, 64>(a, ap);
}

}  // namespace cobs
