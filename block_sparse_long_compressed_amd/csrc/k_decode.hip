// One decode step in one launch (gfx950): block scoring and top-k selection,
// then exact softmax over the selected blocks, the sliding window and the pooled
// tokens, with the gated combine.
//
// Method: COBS (gist.science explainer, Technisches Resuemee 2.1-2.3; skill card
// "Method"): the attention mass of a block is estimated from its query-independent
// summary by the truncated cumulant expansion
//     s_{h,b} = ln n_b + scale q_h.mu_b + alpha/2 scale^2 q_h^T Sigma_b q_h,
// a GQA group ranks blocks by shat_b = ln sum_h exp(s_{h,b} - LSE_b' s_{h,b'})
// and keeps the top-k (ties to the lower index).  NSA (Janus issue #181): three
// paths, each an exact softmax over its own keys, combined with gates:
// out = g_cmp o_cmp + g_slc o_slc + g_win o_win.
//
// Workgroups take one of three roles, in linear index order:
//   [0, S)          scoring: 16-block tiles on the fp32 MFMA, per-head LSE partials;
//                   the last scoring workgroup of a (sequence, kv-head) runs the
//                   radix select and publishes each entry of the selection as a
//                   code (0 = not yet, 1 = no block, b + 2 = block b);
//   [S, S+WC)       window and pooled-token attention: independent of the
//                   selection, so they overlap scoring;
//   [S+WC, total)   selected-block attention: each wave polls (bounded) the codes
//                   of its own tiles, so it starts as soon as they are published.
// Workgroups are dispatched in index order on each XCD, so every scoring
// workgroup is resident before any waiter behind it and the wait cannot deadlock;
// the wait is capped regardless, and every address a waiter derives from the
// selection is bounds-checked.  The last attention workgroup of a unit merges the
// per-workgroup partials of each branch by log-sum-exp rescaling, applies the
// gates and resets the unit's counters and codes for the next call.
//
// Data one workgroup leaves for another travels with sc1 (device-coherent)
// stores and loads; see the hand-off helpers in cobs_device.h.
#include "attn_tile.h"
#include "cobs_device.h"
#include "cobs_launch.h"
#include "score_common.h"

#include <algorithm>

namespace cobs {

constexpr int kThreads = 256;
constexpr int kSelMaxSplits = 64;              // scoring workgroups per (sequence, kv-head)
constexpr uint32_t kSpinCap = 1u << 21;        // ~0.1 s of polling before a waiter gives up

struct DecodeParams {
  int hkv, group, max_len, nb_max, nb_pad, top_k;
  const int32_t* seq_lens;
  const void* Q;
  // scoring / selection
  int sel_wgs, splits, sel_tpw, rank;
  float alpha, scale;
  const void *mu, *so;
  const float* P;               // query subspaces [hkv][sub_s][d] (subspace score kinds)
  int sub_s, vlen;              // subspace dimension; length of a rank-r vector
  int32_t* sel;                 // selection written by the scoring role
  float* sel_score;
  uint32_t* sel_counters;
  float* scores;                // [unit][nb_pad][16]
  float* lse_part;              // [unit][splits][16][2]
  uint32_t* pub;                // [unit][top_k] published selection codes (null: nobody waits)
  // attention
  int wc_wgs, slc_wgs, nc_max, window, cmp_on, tpw, tpw_slc, wg_slc, wg_win, wg_cmp;
  float scale_log2;
  const void *K, *V, *kc, *vc;
  const float* gates;
  const int32_t* sel_attn;      // selection the attention reads (sel or the caller's)
  int wait_ready;
  float* out;
  uint32_t* attn_counters;
  float* part_ml;               // [unit][P][16][2]
  float* part_o;                // [unit][P][G][d]
};

// LDS of the scoring role (inside the launch's dynamic buffer).
struct SelLds {
  float red_m[4][16], red_s[4][16];
  uint32_t hist2[2][4][256];
  int scan_w[4];
  int bcast[4];
  float lse_sh[16];
  float red_part[kSelMaxSplits * 32];
  f32x4 wsub_x[8 * 64];          // subspace weights exchanged between the waves
  // followed by [nb_pad] keys and [nb_pad] group scores
};

template <typename E, int D, int KIND, int HV>
__device__ void select_role(const DecodeParams& p, int unit, int split, unsigned char* smem) {
  constexpr int NU = D / 16;
  SelLds& sl = *reinterpret_cast<SelLds*>(smem);
  uint32_t* s_key = reinterpret_cast<uint32_t*>(smem + sizeof(SelLds));
  float* s_shat = reinterpret_cast<float*>(s_key + p.nb_pad);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int seq = unit / p.hkv, head = unit % p.hkv;
  const int L = p.seq_lens[seq];
  const int ncand = candidate_blocks(L, L - 1);
  const int G = p.group;
  const Coherent sc(p.scores + (size_t)unit * 16 * p.nb_pad, (uint32_t)(16 * p.nb_pad * 4));
  const Coherent lp(p.lse_part + (size_t)unit * p.splits * 32, (uint32_t)(p.splits * 32 * 4));

  // ---- phase 1: scores of this workgroup's tiles -------------------------
  const int tiles_total = (ncand + 15) / 16;
  const int tile0 = (split * 4 + wave) * p.sel_tpw;
  float run_m = -INFINITY, run_s = 0.f;        // LSE partial of head n over this lane's blocks
  // scores s4[i] of blocks tile*16 + 4g + i for head n: running LSE and block-major hand-off
  auto post = [&](int tile, const f32x4& s4, bool add_ln_n) {
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = tile * 16 + 4 * g + i;
      const int nbk = min(kBlock, L - b * kBlock);
      const float ln_n = !add_ln_n ? 0.f : (nbk == kBlock ? kLnBlock : __logf((float)nbk));
      sv[i] = (b < ncand) ? s4[i] + ln_n : -INFINITY;
      mt = fmaxf(mt, sv[i]);
      if (n < G) sc.st1((uint32_t)((b * 16 + n) * 4), sv[i]);
    }
    const float mx = fmaxf(run_m, mt);          // one rescale per tile
    if (mx != -INFINITY) {
      run_s *= __expf(run_m - mx);
#pragma unroll
      for (int i = 0; i < 4; ++i) run_s += __expf(sv[i] - mx);
      run_m = mx;
    }
  };
  if constexpr (KIND == 2) {
    // Exact masses (the selection oracle of COBS 2.1, a diagnostic that reads every
    // key): ln m_b = ln sum_r exp(scale q_h . k_r) over the block's keys, from the
    // 64-key MFMA tile S = K Q^T with a log-sum-exp over the keys of each column.
    using T = AttnTiling<E, D>;
    u32x4 qf[T::kChunks];
    {
      const typename E::storage* Qh = reinterpret_cast<const typename E::storage*>(p.Q) +
                                      ((size_t)seq * p.hkv * G + (size_t)head * G + min(n, G - 1)) * D;
#pragma unroll
      for (int c = 0; c < T::kChunks; ++c) qf[c] = ld16(Qh + (4 * c + g) * T::kEpl);
    }
    const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)unit * p.max_len * D;
    const float scale_log2 = p.scale * kLog2e;
#pragma unroll 1
    for (int j = 0; j < p.sel_tpw; ++j) {
      const int tile = tile0 + j;
      if (tile >= tiles_total) break;
      f32x4 s4 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll 1
      for (int jb = 0; jb < 16; ++jb) {
        const int b = tile * 16 + jb;
        if (b >= ncand) break;
        const int nvalid = min(kBlock, L - b * kBlock);
        TileRegs<E, D> tr;
        tile_load_k<E, D>(Ku + (size_t)b * kBlock * D, nvalid, tr);
        f32x4 sk[4];
        tile_scores<E, D>(tr, qf, sk);
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = (16 * t + 4 * g + i < nvalid) ? sk[t][i] * scale_log2 : -INFINITY;
            sk[t][i] = x;
            mt = fmaxf(mt, x);
          }
        mt = fmaxf(mt, shfl_xor_f(mt, 16));
        mt = fmaxf(mt, shfl_xor_f(mt, 32));
        float ss = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) ss += fast_exp2(sk[t][i] - mt);
        ss += shfl_xor_f(ss, 16);
        ss += shfl_xor_f(ss, 32);
        const float lm = (mt + fast_log2(ss)) * kLn2;          // ln m_b for head n
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = (g == jb / 4 && i == jb % 4) ? lm : s4[i];
      }
      post(tile, s4, false);
    }
  } else {
    // Summary rows are requested before the query so that both arrive in one
    // round trip, and the wave keeps RING tiles in flight: each tile's slot is
    // refilled with the tile RING ahead as soon as it is scored.  (A rank-r tile
    // is already several times larger than a diagonal one.)
    constexpr int RING = KIND == 0 ? 2 : 1;
    const bool use_quad = p.alpha != 0.f;
    const size_t sum_base = (size_t)unit * p.nb_max;
    auto rows_of = [&](int tile, const void*& mr, const void*& vr) {
      const int brow = min(tile * 16 + n, ncand - 1);      // A-operand row (block) of this lane
      summary_rows<D, KIND>(p.mu, p.so, sum_base + brow, p.rank, p.vlen, mr, vr);
    };
    SumTile<D, KIND> st[RING];
    const void* vrow[RING];
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      vrow[r] = nullptr;
      if (r < p.sel_tpw && tile0 + r < tiles_total) {
        const void* mrow;
        rows_of(tile0 + r, mrow, vrow[r]);
        sum_tile_load<D, KIND>(mrow, vrow[r], p.rank, p.vlen, g, use_quad, st[r]);
      }
    }
    ScoreW<D> W;
    prepare_weights<E, D, KIND>(p.Q, ((size_t)seq * (size_t)(p.hkv * G) + (size_t)head * G) * D, n, g, G, p.scale,
                                W);
    if constexpr (Kind<KIND>::kSub) {
      // scale * P q: the four waves each contract a quarter of the column tiles
      const float* Ph = p.P + (size_t)head * p.sub_s * D;
      subspace_weights_part<D>(Ph, p.sub_s, p.vlen, wave, 4, n, g, W.lin, sl.wsub_x, W.quad);
      __syncthreads();
      subspace_weights_gather<D>(p.vlen, wave, 4, n, g, sl.wsub_x, W.quad);
      finish_subspace_weights<E, D, KIND>(W);
    }
    for (int j0 = 0; j0 < p.sel_tpw; j0 += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        const int j = j0 + r, tile = tile0 + j0 + r;
        if (j < p.sel_tpw && tile < tiles_total) {
          const f32x4 s4 = tile_score<E, D, KIND>(st[r], vrow[r], p.rank, p.vlen, g, use_quad, p.alpha, p.scale, W);
          if (j + RING < p.sel_tpw && tile + RING < tiles_total) {
            const void* mrow;
            rows_of(tile + RING, mrow, vrow[r]);
            sum_tile_load<D, KIND>(mrow, vrow[r], p.rank, p.vlen, g, use_quad, st[r]);
          }
          post(tile, s4, true);
        }
      }
    }
  }
#pragma unroll
  for (int m = 16; m < 64; m <<= 1) {
    const float om = shfl_xor_f(run_m, m), os = shfl_xor_f(run_s, m);
    const float mx = fmaxf(run_m, om);
    if (mx != -INFINITY) {
      run_s = run_s * __expf(run_m - mx) + os * __expf(om - mx);
      run_m = mx;
    }
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
    const uint32_t o = (uint32_t)((split * 16 + threadIdx.x) * 2 * 4);
    lp.st1(o, M);
    lp.st1(o + 4, S);
  }

  // ---- hand-off: the last scoring workgroup of this unit selects ----------
  if (!arrive_last(p.sel_counters + unit, (uint32_t)p.splits, &sl.bcast[0])) return;

  // phase 2 is latency-bound: the first round of this thread's block scores and the
  // LSE partials are fetched together, so both cost one memory round trip
  const int per = (p.nb_max + kThreads - 1) / kThreads;
  const int b0 = threadIdx.x * per;
  constexpr int kRound = 8 / HV;                                 // blocks per load round (8 float4)
  f32x4 raw[kRound][HV];
  auto load_round = [&](int e0) {
#pragma unroll
    for (int e = 0; e < kRound; ++e) {
      const int b = b0 + e0 + e;
      const bool ok = e0 + e < per && b < ncand;
#pragma unroll
      for (int v = 0; v < HV; ++v)
        raw[e][v] = ok ? sc.ld4((uint32_t)((b * 16 + 4 * v) * 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_round(0);
  for (int i = threadIdx.x; i < p.splits * 16; i += kThreads) {
    sl.red_part[2 * i] = lp.ld1((uint32_t)(i * 8));
    sl.red_part[2 * i + 1] = lp.ld1((uint32_t)(i * 8 + 4));
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float M = -INFINITY, S = 0.f;
    for (int x = 0; x < p.splits; ++x) {
      const float om = sl.red_part[2 * (x * 16 + threadIdx.x)], os = sl.red_part[2 * (x * 16 + threadIdx.x) + 1];
      const float mx = fmaxf(M, om);
      if (mx != -INFINITY) { S = S * __expf(M - mx) + os * __expf(om - mx); M = mx; }
    }
    sl.lse_sh[threadIdx.x] = (M == -INFINITY) ? -INFINITY : M + __logf(S);
  }
  __syncthreads();

  // ---- group scores: thread owns blocks [tid*per, tid*per + per) ------------
  float lse_r[4 * HV];
#pragma unroll
  for (int h = 0; h < 4 * HV; ++h) lse_r[h] = (h < G) ? sl.lse_sh[h] : 0.f;
#pragma unroll 1
  for (int e0 = 0; e0 < per; e0 += kRound) {
    if (e0 > 0) load_round(e0);
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
  __syncthreads();
  if (p.sel_score) {
    float* ss = p.sel_score + (size_t)unit * p.nb_max;
    for (int b = threadIdx.x; b < p.nb_max; b += kThreads) ss[b] = (b < ncand) ? s_shat[b] : -INFINITY;
  }

  // ---- radix select; the selection (ascending, -1 padded) and, for waiting
  // attention waves, its codes
  const Coherent so(p.sel + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
  const Coherent pc(p.pub ? static_cast<const void*>(p.pub + (size_t)unit * p.top_k) : static_cast<const void*>(p.sel),
                    (uint32_t)(p.top_k * 4));
  const int sel_total = wg_select_topk(s_key, ncand, per, p.top_k, &sl.hist2[0][0][0], sl.scan_w,
                                       [&](int pos, int b) {
                                         so.st1((uint32_t)(pos * 4), __int_as_float(b));
                                         if (p.pub) pc.st1((uint32_t)(pos * 4), __uint_as_float((uint32_t)(b + 2)));
                                       });
  for (int i = sel_total + (int)threadIdx.x; i < p.top_k; i += kThreads) {
    so.st1((uint32_t)(i * 4), __int_as_float(-1));
    if (p.pub) pc.st1((uint32_t)(i * 4), __uint_as_float(1u));
  }
  if (threadIdx.x == 0) reset_counter(p.sel_counters + unit);
}

// branch: 0 = SLC, 1 = WIN, 2 = CMP; slot = the workgroup's partial index in its unit.
template <typename E, int D>
__device__ void attn_role(const DecodeParams& p, int unit, int branch, int local, int slot,
                          unsigned char* smem, int* flag) {
  using T = AttnTiling<E, D>;
  constexpr int NCH = T::kChunks, EPL = T::kEpl, NDT = T::kDt;
  constexpr int nw = kThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int seq = unit / p.hkv, head = unit % p.hkv;
  const int G = p.group;
  const int L = p.seq_lens[seq];
  const int P = p.wg_slc + p.wg_win + p.wg_cmp;

  const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)unit * p.max_len * D;
  const typename E::storage* Vu = reinterpret_cast<const typename E::storage*>(p.V) + (size_t)unit * p.max_len * D;
  const typename E::storage* kcu = p.cmp_on ? reinterpret_cast<const typename E::storage*>(p.kc) + (size_t)unit * p.nc_max * D : nullptr;
  const typename E::storage* vcu = p.cmp_on ? reinterpret_cast<const typename E::storage*>(p.vc) + (size_t)unit * p.nc_max * D : nullptr;
  const int nb = (L + kBlock - 1) / kBlock;
  const int nc = (p.cmp_on && L >= 32) ? (L - 32) / 16 + 1 : 0;
  const int win_len = min(p.window, L);
  const int win_start = L - win_len;

  // Source rows of this wave's j-th tile; returns the number of valid keys (0:
  // none).  Selected blocks come from the published codes (polled, bounded) or
  // the caller's selection; every block index is bounds-checked.
  auto tile_src = [&](int j, const typename E::storage*& Kt, const typename E::storage*& Vt) -> int {
    const int tpw = branch == 0 ? p.tpw_slc : p.tpw;       // tiles per wave of this branch
    if (j >= tpw) return 0;
    const int tile = (local * nw + wave) * tpw + j;
    if (branch == 0) {
      if (tile >= p.top_k) return 0;
      int b = -1;
      if (p.wait_ready) {
        const Coherent pc(p.pub + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
        uint32_t code = 0;
        for (uint32_t it = 0; it < kSpinCap; ++it) {
          code = __float_as_uint(pc.ld1((uint32_t)(tile * 4)));
          if (code != 0u) break;
          __builtin_amdgcn_s_sleep(1);
        }
        b = (code >= 2u) ? (int)(code - 2u) : -1;
      } else {
        const Coherent si(p.sel_attn + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
        b = __float_as_int(si.ld1((uint32_t)(tile * 4)));
      }
      if (b < 0 || b >= nb) return 0;
      Kt = Ku + (size_t)b * kBlock * D;
      Vt = Vu + (size_t)b * kBlock * D;
      return min(kBlock, L - b * kBlock);
    }
    if (branch == 1) {
      const int start = win_start + tile * kBlock;
      if (start >= L) return 0;
      Kt = Ku + (size_t)start * D;
      Vt = Vu + (size_t)start * D;
      return min(kBlock, L - start);
    }
    const int start = tile * kBlock;
    if (start >= nc) return 0;
    Kt = kcu + (size_t)start * D;
    Vt = vcu + (size_t)start * D;
    return min(kBlock, nc - start);
  };

  typename E::storage* lds = reinterpret_cast<typename E::storage*>(smem) + (size_t)wave * kBlock * T::kRowStride;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over the wave's tiles (valid tiles form a prefix): the next
  // tile's K loads go out once this tile's scores are formed (overlapping the
  // softmax and P V), its V loads after P V (overlapping the next scores).
  TileRegs<E, D> tr;
  const typename E::storage *Kt = nullptr, *Vt = nullptr;
  int nv = tile_src(0, Kt, Vt);
  if (nv > 0) {
    tile_load_k<E, D>(Kt, nv, tr);
    tile_load_v<E, D>(Vt, nv, tr);
  }
  // The group's queries as the B operand of S = K Q^T, requested after the first
  // tile so that no round trip precedes the tile loads.  Columns n >= G repeat
  // head G-1: their scores and outputs stay in their own columns and are never
  // merged or written.
  u32x4 qf[NCH];
  {
    const typename E::storage* Qh = reinterpret_cast<const typename E::storage*>(p.Q) +
                                    ((size_t)seq * p.hkv * G + (size_t)head * G + min(n, G - 1)) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[c] = ld16(Qh + (4 * c + g) * EPL);
  }
  for (int j = 0; nv > 0; ++j) {
    f32x4 sc4[4];
    tile_scores<E, D>(tr, qf, sc4);
    const typename E::storage *Kn = nullptr, *Vn = nullptr;
    const int nv_next = tile_src(j + 1, Kn, Vn);
    if (nv_next > 0) tile_load_k<E, D>(Kn, nv_next, tr);
    tile_stage_v<E, D>(tr, lds);
    tile_softmax_pv<E, D>(sc4, nv, p.scale_log2, lds, m_run, l_run, acc_o);
    if (nv_next > 0) tile_load_v<E, D>(Vn, nv_next, tr);
    nv = nv_next;
  }

  // ---- merge the waves of this workgroup in LDS ----------------------------
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);        // [nw][16][D] then [nw][16][2]
  float* mml = mo + (size_t)nw * 16 * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mo[((size_t)wave * 16 + n) * D + 16 * dt + 4 * g + i] = acc_o[dt][i];
  }
  if (g == 0) { mml[(wave * 16 + n) * 2] = m_run; mml[(wave * 16 + n) * 2 + 1] = l_run; }
  __syncthreads();
  const Coherent po(p.part_o + (size_t)unit * P * G * D, (uint32_t)(P * G * D * 4));
  const Coherent pm(p.part_ml + (size_t)unit * P * 32, (uint32_t)(P * 32 * 4));
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += kThreads) {
    const int h = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
    float M = -INFINITY;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, mml[(w * 16 + h) * 2]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float Ls = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < nw; ++w) {
        const float mw = mml[(w * 16 + h) * 2];
        if (mw == -INFINITY) continue;
        const float f = fast_exp2(mw - M);
        Ls += f * mml[(w * 16 + h) * 2 + 1];
        const float* src = mo + ((size_t)w * 16 + h) * D + d4;
        o[0] += f * src[0]; o[1] += f * src[1]; o[2] += f * src[2]; o[3] += f * src[3];
      }
    }
    po.st4((uint32_t)(((slot * G + h) * D + d4) * 4), o);
    if (d4 == 0) {
      pm.st1((uint32_t)(((slot * 16 + h) * 2) * 4), M);
      pm.st1((uint32_t)(((slot * 16 + h) * 2 + 1) * 4), Ls);
    }
  }

  // ---- the last attention workgroup of this unit combines -----------------
  if (!arrive_last(p.attn_counters + unit, (uint32_t)P, flag)) return;

  // this thread's two outputs (G*d/4 <= 512 float4): the first 16 partials of each
  // are fetched in the same round as every partial's (max, sum)
  const int items = G * (D / 4);
  const int i0 = threadIdx.x, i1 = threadIdx.x + kThreads;
  const bool has0 = i0 < items, has1 = i1 < items;
  const int h0 = has0 ? i0 / (D / 4) : 0, d0 = has0 ? (i0 % (D / 4)) * 4 : 0;
  const int h1 = has1 ? i1 / (D / 4) : h0, d1 = has1 ? (i1 % (D / 4)) * 4 : d0;
  f32x4 o0[16], o1[16];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = min(c0 + j, P - 1);
      o0[j] = po.ld4((uint32_t)(((q * G + h0) * D + d0) * 4));
      o1[j] = po.ld4((uint32_t)(((q * G + h1) * D + d1) * 4));
    }
  };
  load_chunk(0);
  float* sm = reinterpret_cast<float*>(smem);          // [P][16][2]
  float* fac = sm + (size_t)P * 32;                    // [P][16]
  for (int i = threadIdx.x; i < P * G; i += kThreads) {
    const int q = i / G, h = i % G;
    sm[(q * 16 + h) * 2] = pm.ld1((uint32_t)(((q * 16 + h) * 2) * 4));
    sm[(q * 16 + h) * 2 + 1] = pm.ld1((uint32_t)(((q * 16 + h) * 2 + 1) * 4));
  }
  __syncthreads();
  const int pb[4] = {0, p.wg_slc, p.wg_slc + p.wg_win, P};   // SLC, WIN, CMP partial ranges
  // merge factor of partial q for head h: gate / L_branch * 2^(m_q - M_branch)
  for (int i = threadIdx.x; i < 3 * G; i += kThreads) {
    const int br = i / G, h = i % G;
    const int hq = head * G + h;
    float gate = (br == 0) ? 1.f : 0.f;                 // gates absent: slc only
    if (p.gates) gate = p.gates[((size_t)seq * p.hkv * G + hq) * 3 + (br == 0 ? 1 : br == 1 ? 2 : 0)];
    const int q0 = pb[br], q1 = pb[br + 1];
    float M = -INFINITY, Ls = 0.f;
    for (int c0 = q0; c0 < q1; c0 += 16) {            // all reads of a chunk in flight together
      float mv[16], lv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool ok = c0 + j < q1;
        mv[j] = ok ? sm[((c0 + j) * 16 + h) * 2] : -INFINITY;
        lv[j] = ok ? sm[((c0 + j) * 16 + h) * 2 + 1] : 0.f;
      }
      float Mc = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) if (lv[j] > 0.f) Mc = fmaxf(Mc, mv[j]);
      if (Mc == -INFINITY) continue;
      const float Mn = fmaxf(M, Mc);
      Ls = (M == -INFINITY) ? 0.f : Ls * fast_exp2(M - Mn);
#pragma unroll
      for (int j = 0; j < 16; ++j) if (lv[j] > 0.f) Ls += fast_exp2(mv[j] - Mn) * lv[j];
      M = Mn;
    }
    const float inv = (Ls > 0.f) ? gate / Ls : 0.f;
    for (int q = q0; q < q1; ++q) {
      const float lq = sm[(q * 16 + h) * 2 + 1];
      fac[q * 16 + h] = (lq > 0.f) ? inv * fast_exp2(sm[(q * 16 + h) * 2] - M) : 0.f;
    }
  }
  __syncthreads();
  // out[h][d] = sum_q fac[q][h] O_q[h][d]
  f32x4 r0 = {0.f, 0.f, 0.f, 0.f}, r1 = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < P; c0 += 16) {
    if (c0 > 0) load_chunk(c0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (c0 + j < P) {
        r0 += fac[(c0 + j) * 16 + h0] * o0[j];
        r1 += fac[(c0 + j) * 16 + h1] * o1[j];
      }
    }
  }
  if (has0) st_f32x4(p.out + ((size_t)seq * p.hkv * G + head * G + h0) * D + d0, r0);
  if (has1) st_f32x4(p.out + ((size_t)seq * p.hkv * G + head * G + h1) * D + d1, r1);
  if (threadIdx.x == 0) reset_counter(p.attn_counters + unit);
  if (p.wait_ready) {                               // codes back to "not yet" for the next call
    const Coherent pc(p.pub + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
    for (int i = threadIdx.x; i < p.top_k; i += kThreads) pc.st1((uint32_t)(i * 4), 0.f);
  }
}

template <typename E, int D, int KIND, int HV>
__global__ __launch_bounds__(kThreads, E::kBytes * D <= 256 ? 2 : 1) void k_decode(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int flag;
  const int i = blockIdx.x;
  if (i < p.sel_wgs) {
    select_role<E, D, KIND, HV>(p, i / p.splits, i % p.splits, smem);
    return;
  }
  const int j = i - p.sel_wgs;
  int unit, branch, local, slot;
  if (j < p.wc_wgs) {
    const int per_unit = p.wg_win + p.wg_cmp;
    unit = j / per_unit;
    const int l = j % per_unit;
    branch = l < p.wg_win ? 1 : 2;
    local = l < p.wg_win ? l : l - p.wg_win;
    slot = p.wg_slc + l;
  } else {
    const int k = j - p.wc_wgs;
    unit = k / p.wg_slc;
    branch = 0;
    local = slot = k % p.wg_slc;
  }
  attn_role<E, D>(p, unit, branch, local, slot, smem, &flag);
}

size_t select_lds_bytes(int nb_pad) { return sizeof(SelLds) + (size_t)nb_pad * 8; }

template <typename E, int D>
size_t attn_role_lds_bytes(int P) {
  return std::max(attn_lds_bytes<E, D>(kThreads / 64), (size_t)P * 48 * sizeof(float));
}

template <typename E, int D, int KIND, int HV>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodeParams& dp) {
  const int total = dp.sel_wgs + dp.wc_wgs + dp.slc_wgs;
  size_t lds = 0;
  if (dp.sel_wgs) lds = std::max(lds, select_lds_bytes(dp.nb_pad));
  if (dp.wc_wgs + dp.slc_wgs) lds = std::max(lds, attn_role_lds_bytes<E, D>(dp.wg_slc + dp.wg_win + dp.wg_cmp));
  hipLaunchKernelGGL((k_decode<E, D, KIND, HV>), dim3(total), dim3(kThreads), lds, a.stream, dp);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_decode_ed(const DecodeArgs& a, const DecodeParams& dp) {
  const int hv = a.group <= 4 ? 1 : a.group <= 8 ? 2 : 4;
  if (a.so_kind == 2) {                       // exact masses: scoring roles only
    if (hv == 1) return launch_decode_t<E, D, 2, 1>(a, dp);
    if (hv == 2) return launch_decode_t<E, D, 2, 2>(a, dp);
    return launch_decode_t<E, D, 2, 4>(a, dp);
  }
  if (a.so_kind == 0) {
    if (hv == 1) return launch_decode_t<E, D, 0, 1>(a, dp);
    if (hv == 2) return launch_decode_t<E, D, 0, 2>(a, dp);
    return launch_decode_t<E, D, 0, 4>(a, dp);
  }
  if (a.so_kind == 3) {                       // compressed storage
    if (hv == 1) return launch_decode_t<E, D, 3, 1>(a, dp);
    if (hv == 2) return launch_decode_t<E, D, 3, 2>(a, dp);
    return launch_decode_t<E, D, 3, 4>(a, dp);
  }
  if (a.so_kind == 4) {                       // rank-r fp32 in a query subspace
    if (hv == 1) return launch_decode_t<E, D, 4, 1>(a, dp);
    if (hv == 2) return launch_decode_t<E, D, 4, 2>(a, dp);
    return launch_decode_t<E, D, 4, 4>(a, dp);
  }
  if (a.so_kind == 5) {                       // compressed storage in a query subspace
    if (hv == 1) return launch_decode_t<E, D, 5, 1>(a, dp);
    if (hv == 2) return launch_decode_t<E, D, 5, 2>(a, dp);
    return launch_decode_t<E, D, 5, 4>(a, dp);
  }
  if (hv == 1) return launch_decode_t<E, D, 1, 1>(a, dp);
  if (hv == 2) return launch_decode_t<E, D, 1, 2>(a, dp);
  return launch_decode_t<E, D, 1, 4>(a, dp);
}

hipError_t launch_decode(const DecodeArgs& a) {
  DecodeParams p;
  const int units = a.batch * a.hkv;
  p.hkv = a.hkv; p.group = a.group; p.max_len = a.max_len; p.nb_max = a.nb_max;
  p.nb_pad = (a.nb_max + 15) / 16 * 16; p.top_k = a.top_k; p.seq_lens = a.seq_lens; p.Q = a.Q;
  p.sel_wgs = a.do_select ? units * a.splits : 0;
  p.splits = a.splits; p.sel_tpw = a.sel_tpw; p.rank = a.rank; p.alpha = a.alpha; p.scale = a.scale;
  p.mu = a.mu; p.so = a.so; p.P = a.P; p.sub_s = a.sub_s; p.vlen = a.vlen; p.sel = a.sel; p.sel_score = a.sel_score; p.sel_counters = a.sel_counters;
  p.scores = a.scores; p.lse_part = a.lse_part;
  p.pub = (a.do_select && a.do_attn) ? a.ready : nullptr;
  p.wc_wgs = a.do_attn ? units * (a.wg_win + a.wg_cmp) : 0;
  p.slc_wgs = a.do_attn ? units * a.wg_slc : 0;
  p.nc_max = a.nc_max; p.window = a.window; p.cmp_on = a.cmp_on; p.tpw = a.tpw_wc; p.tpw_slc = a.tpw_slc;
  p.wg_slc = a.wg_slc; p.wg_win = a.wg_win; p.wg_cmp = a.wg_cmp; p.scale_log2 = a.scale * kLog2e;
  p.K = a.K; p.V = a.V; p.kc = a.kc; p.vc = a.vc; p.gates = a.gates;
  p.sel_attn = a.do_select ? a.sel : a.sel_in;
  p.wait_ready = (a.do_select && a.do_attn) ? 1 : 0;
  p.out = a.out; p.attn_counters = a.attn_counters; p.part_ml = a.part_ml; p.part_o = a.part_o;
  if (a.bf16) return a.head_dim == 128 ? launch_decode_ed<EltBF16, 128>(a, p) : launch_decode_ed<EltBF16, 64>(a, p);
  return a.head_dim == 128 ? launch_decode_ed<EltF32, 128>(a, p) : launch_decode_ed<EltF32, 64>(a, p);
}

}  // namespace cobs
