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
// A unit is one (sequence, kv-head).  Workgroups of NW waves take one of three
// roles, in linear index order:
//   scoring   `splits` per unit.  Each scores a share of the unit's 16-block summary
//             tiles.  With one scoring workgroup per unit the raw block scores stay in
//             LDS; otherwise they travel block-major through the workspace and the
//             last workgroup to arrive collects them.  The workgroup that holds all
//             the scores (the lead) forms shat, runs the radix select, writes the
//             selection and then attends to the first `lead_tiles` selected blocks
//             itself, straight from the selection in LDS.  The remaining selected
//             blocks are published as codes (0 = not yet, 1 = no block, b + 2 = block
//             b) for the selected-branch workgroups.
//   window /  `wg_wc` per unit; their waves split the unit's window tiles and pooled
//   pooled    tiles evenly (independent of the selection, so they overlap scoring).
//   selected  `wg_slc` per unit: the selected blocks beyond the lead's share.  Each
//             wave polls (bounded) the codes of its own tiles; with the caller's
//             selection they read it directly.
// Window/pooled and selected workgroups are numbered round-robin over the units
// (every unit's l-th workgroup before any (l+1)-th), so that when the grid exceeds
// what the chip holds at once, the shares dispatched as earlier workgroups retire
// are spread over all units.
// Workgroups are dispatched in index order on each XCD, so a unit's lead is resident
// before any workgroup that waits on it.  The wait is capped regardless: a wave that
// gives up treats the tile as empty and sets bit 0 of the workspace status word,
// which the host reads with cobs_decode_status.  Every address derived from a
// selection is bounds-checked.  Each attention workgroup merges its waves per branch
// into one partial per branch slot; the last one of a unit merges the partials of
// each branch by log-sum-exp rescaling, applies the gates and resets the unit's
// counters and codes for the next call.  The lead arrives there too, so the codes are
// reset only after they were published.
//
// Data one workgroup leaves for another travels with sc1 (device-coherent)
// stores and loads; see the hand-off helpers in cobs_device.h.
#include "attn_tile.h"
#include "cobs_device.h"
#include "cobs_launch.h"
#include "score_common.h"

#include <algorithm>
#include <type_traits>

namespace cobs {

constexpr int kSelMaxSplits = 64;              // scoring workgroups per unit

struct DecodeParams {
  int units, hkv, group, max_len, nb_max, nb_pad, top_k;
  const int32_t* seq_lens;
  const void* Q;
  // scoring / selection
  int sel_wgs, splits, sel_tpw, rank;
  const void *mu, *so;
  const float* P;               // query subspaces [hkv][sub_s][d] (subspace score kinds)
  int sub_s, vlen;              // subspace dimension; length of a rank-r vector
  float alpha, scale;
  int32_t* sel;                 // selection written by the lead
  float* sel_score;
  uint32_t* sel_counters;
  float* scores;                // [unit][nb_pad][16] (splits > 1)
  float* lse_part;              // [unit][splits][16][2] (splits > 1)
  uint32_t* pub;                // [unit][top_k] published selection codes (null: nobody waits)
  // attention
  int do_attn, has_lead, lead_tiles;
  int wc_wgs, slc_wgs, nc_max, window, cmp_on, wg_wc, wg_slc, tpw_slc;
  float scale_log2;
  const void *K, *V, *kc, *vc;
  const float* gates;
  const int32_t* sel_in;        // the caller's selection (no lead)
  float* out;
  uint32_t* attn_counters;
  float* part_ml;               // [unit][P][16][2]
  float* part_o;                // [unit][P][G][d]
  uint32_t* status;             // bit 0: a selected-branch wait gave up
  uint32_t poll_cap;            // polls of one code before a wave gives up
};

// Partial slots of a unit: selected [0, ns), window [ns, ns + wg_wc), pooled
// [ns + wg_wc, ns + 2 wg_wc), with ns = has_lead + wg_slc.
__device__ __forceinline__ int slc_slots(const DecodeParams& p) { return p.has_lead + p.wg_slc; }
__device__ __forceinline__ int n_slots(const DecodeParams& p) { return slc_slots(p) + 2 * p.wg_wc; }

// LDS of the scoring role (inside the launch's dynamic buffer).
template <int NW>
struct SelLds {
  float red_m[NW][16], red_s[NW][16];
  uint32_t hist2[2][NW][256];
  int scan_w[NW];
  int bcast[4];
  float lse_sh[16];
  float red_part[kSelMaxSplits * 32];
  f32x4 wsub_x[8 * 64];          // subspace weights exchanged between the waves
  // followed by [nb_pad] keys, [nb_pad] group scores and, with one scoring
  // workgroup per unit, [nb_pad][16] raw scores
};

template <int NW>
__host__ __device__ constexpr size_t select_lds_bytes(int nb_pad, bool raw_in_lds) {
  return sizeof(SelLds<NW>) + (size_t)nb_pad * 8 + (raw_in_lds ? (size_t)nb_pad * 64 : 0);
}

// ---------------------------------------------------------------------------
// One wave's run over its 64-key tiles.  src(j, Kt, Vt) returns the number of valid
// keys of the wave's j-th tile (0: no more tiles; valid tiles form a prefix).  The
// next tile's K loads go out once this tile's scores are formed (overlapping the
// softmax and P V), its V loads after P V (overlapping the next scores).  The
// group's queries (the B operand of S = K Q^T; cached, they were read by the
// scoring) are requested just before the first tile: loads return in order, so
// the first scores then wait for Q and K only, not for V; columns n >= G repeat
// head G-1, whose scores and outputs stay in their own columns and are never
// merged or written.
// ---------------------------------------------------------------------------
template <typename E, int D, typename Src>
__device__ __forceinline__ void wave_tiles(Src&& src, const typename E::storage* Qg, int G, float scale_log2,
                                           typename E::storage* lds, float& m_run, float& l_run,
                                           f32x4 (&acc_o)[AttnTiling<E, D>::kDt]) {
  using T = AttnTiling<E, D>;
  constexpr int NCH = T::kChunks, EPL = T::kEpl, NDT = T::kDt;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  TileRegs<E, D> tr;
  const typename E::storage *Kt = nullptr, *Vt = nullptr;
  int nv = src(0, Kt, Vt);
  if (nv <= 0) return;
  u32x4 qf[NCH];
  {
    const typename E::storage* Qh = Qg + (size_t)min(n, G - 1) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[c] = ld16(Qh + (4 * c + g) * EPL);
  }
  tile_load_k<E, D>(Kt, nv, tr);
  tile_load_v<E, D>(Vt, nv, tr);
  for (int j = 0; nv > 0; ++j) {
    f32x4 sc4[4];
    tile_scores<E, D>(tr, qf, sc4);
    const typename E::storage *Kn = nullptr, *Vn = nullptr;
    const int nv_next = src(j + 1, Kn, Vn);
    if (nv_next > 0) tile_load_k<E, D>(Kn, nv_next, tr);
    tile_stage_v<E, D>(tr, lds);
    tile_softmax_pv<E, D>(sc4, nv, scale_log2, lds, m_run, l_run, acc_o);
    if (nv_next > 0) tile_load_v<E, D>(Vn, nv_next, tr);
    nv = nv_next;
  }
}

// The same for a wave with at most two tiles (the selecting workgroup's share of
// the selected blocks): Q, then both tiles' K loads and the first tile's V go out
// at once, so the second tile's scores need no round trip of their own; its V
// loads follow once V of the first tile is staged.
template <typename E, int D, typename Src>
__device__ __forceinline__ void wave_tiles_pair(Src&& src, const typename E::storage* Qg, int G, float scale_log2,
                                                typename E::storage* lds, float& m_run, float& l_run,
                                                f32x4 (&acc_o)[AttnTiling<E, D>::kDt]) {
  using T = AttnTiling<E, D>;
  constexpr int NCH = T::kChunks, EPL = T::kEpl, NDT = T::kDt;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const typename E::storage *K0 = nullptr, *V0 = nullptr, *K1 = nullptr, *V1 = nullptr;
  const int n0 = src(0, K0, V0);
  if (n0 <= 0) return;
  const int n1 = src(1, K1, V1);
  TileRegs<E, D> t0, t1;
  u32x4 qf[NCH];
  {
    const typename E::storage* Qh = Qg + (size_t)min(n, G - 1) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[c] = ld16(Qh + (4 * c + g) * EPL);
  }
  tile_load_k<E, D>(K0, n0, t0);
  tile_load_v<E, D>(V0, n0, t0);
  if (n1 > 0) tile_load_k<E, D>(K1, n1, t1);
  f32x4 sc4[4];
  tile_scores<E, D>(t0, qf, sc4);
  tile_stage_v<E, D>(t0, lds);
  if (n1 > 0) tile_load_v<E, D>(V1, n1, t1);
  tile_softmax_pv<E, D>(sc4, n0, scale_log2, lds, m_run, l_run, acc_o);
  if (n1 <= 0) return;
  tile_scores<E, D>(t1, qf, sc4);
  tile_stage_v<E, D>(t1, lds);
  tile_softmax_pv<E, D>(sc4, n1, scale_log2, lds, m_run, l_run, acc_o);
}

template <typename E, int D, int NW>
__host__ __device__ constexpr size_t attn_stage_bytes() {
  return (size_t)NW * kBlock * AttnTiling<E, D>::kRowStride * E::kBytes;
}

// ---------------------------------------------------------------------------
// Merge the workgroup's waves per branch slot in LDS and store one partial
// (max, sum, O) per slot with sc1 stores; then the unit's last attention
// workgroup combines every slot and writes the output.  wave_slot: the partial
// slot this wave contributes to (-1: none).  my_slots[0..nmine): the slots this
// workgroup owns (each is written, empty when no wave contributed).
// ---------------------------------------------------------------------------
template <typename E, int D, int NW>
__device__ __forceinline__ void merge_and_finish(const DecodeParams& p, int unit, int wave_slot, const int (&my_slots)[2], int nmine,
                                 float m_run, float l_run, const f32x4 (&acc_o)[D / 16], unsigned char* smem,
                                 int* flag, const float* spare = nullptr, const int* spare_used = nullptr) {
  constexpr int NT = 64 * NW, NDT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int seq = unit / p.hkv, head = unit % p.hkv;
  const int G = p.group;
  const int P = n_slots(p);

  constexpr int MS = D + 4;                          // padded row: the 16 rows of a wave hit distinct banks
  __syncthreads();                                   // every wave is done with its LDS slice
  float* mo = reinterpret_cast<float*>(smem);        // [NW][16][MS] then [NW][16][2], [NW] slots
  float* mml = mo + (size_t)NW * 16 * MS;
  int* wslot = reinterpret_cast<int*>(mml + NW * 32);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *reinterpret_cast<f32x4*>(mo + ((size_t)wave * 16 + n) * MS + 16 * dt + 4 * g) = acc_o[dt];
  if (g == 0) { mml[(wave * 16 + n) * 2] = m_run; mml[(wave * 16 + n) * 2 + 1] = l_run; }
  if (lane == 0) wslot[wave] = wave_slot;
  __syncthreads();
  // a parked window partial (see wc_attention) joins the window slot my_slots[0]
  const bool use_spare = spare_used && *spare_used;
  const Coherent po(p.part_o + (size_t)unit * P * G * D, (uint32_t)(P * G * D * 4));
  const Coherent pm(p.part_ml + (size_t)unit * P * 32, (uint32_t)(P * 32 * 4));
  const int items = G * (D / 4);
  for (int idx = threadIdx.x; idx < nmine * items; idx += NT) {
    const int which = idx / items, r = idx % items;
    const int slot = which == 0 ? my_slots[0] : my_slots[1];   // (no dynamically indexed array)
    const int h = r / (D / 4), d4 = (r % (D / 4)) * 4;
    const bool sp = use_spare && which == 0;
    // every wave's (max, sum, O) of head h are read at once (one LDS round trip),
    // those of other slots then drop out
    float mw[NW], lw[NW];
    f32x4 ow[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const bool in = wslot[w] == slot;
      mw[w] = in ? mml[(w * 16 + h) * 2] : -INFINITY;
      lw[w] = mml[(w * 16 + h) * 2 + 1];
      ow[w] = *reinterpret_cast<const f32x4*>(mo + ((size_t)w * 16 + h) * MS + d4);
    }
    float M = sp ? spare[16 * D + 2 * h] : -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (mw[w] == -INFINITY) continue;
        const float f = fast_exp2(mw[w] - M);
        Ls += f * lw[w];
        o += f * ow[w];
      }
      if (sp && spare[16 * D + 2 * h] != -INFINITY) {
        const float f = fast_exp2(spare[16 * D + 2 * h] - M);
        Ls += f * spare[16 * D + 2 * h + 1];
        const float* src = spare + h * D + d4;
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
  if (!arrive_last(p.attn_counters + unit, (uint32_t)(p.has_lead + p.wg_slc + p.wg_wc), flag)) return;

  // this thread's outputs (G*d/4 <= 512 float4, at most two per thread): the first
  // 16 partials of each are fetched in the same round as every partial's (max, sum)
  const int i0 = threadIdx.x, i1 = threadIdx.x + NT;
  const bool has0 = i0 < items, has1 = NT < items && i1 < items;
  const int h0 = has0 ? i0 / (D / 4) : 0, d0 = has0 ? (i0 % (D / 4)) * 4 : 0;
  const int h1 = has1 ? i1 / (D / 4) : h0, d1 = has1 ? (i1 % (D / 4)) * 4 : d0;
  f32x4 o0[16], o1[16];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = min(c0 + j, P - 1);
      o0[j] = po.ld4((uint32_t)(((q * G + h0) * D + d0) * 4));
      if (NT < 512) o1[j] = po.ld4((uint32_t)(((q * G + h1) * D + d1) * 4));
    }
  };
  load_chunk(0);
  float* sm = reinterpret_cast<float*>(smem);          // [P][16][2]
  float* fac = sm + (size_t)P * 32;                    // [P][16]
  for (int i = threadIdx.x; i < P * G; i += NT) {
    const int q = i / G, h = i % G;
    sm[(q * 16 + h) * 2] = pm.ld1((uint32_t)(((q * 16 + h) * 2) * 4));
    sm[(q * 16 + h) * 2 + 1] = pm.ld1((uint32_t)(((q * 16 + h) * 2 + 1) * 4));
  }
  __syncthreads();
  const int ns = slc_slots(p);
  // merge factor of partial q for head h: gate / L_branch * 2^(m_q - M_branch)
  for (int i = threadIdx.x; i < 3 * G; i += NT) {
    const int br = i / G, h = i % G;
    const int hq = head * G + h;
    float gate = (br == 0) ? 1.f : 0.f;                 // gates absent: slc only
    if (p.gates) gate = p.gates[((size_t)seq * p.hkv * G + hq) * 3 + (br == 0 ? 1 : br == 1 ? 2 : 0)];
    // partial ranges: SLC [0, ns), WIN [ns, ns + wg_wc), CMP [ns + wg_wc, P)
    const int q0 = br == 0 ? 0 : br == 1 ? ns : ns + p.wg_wc;
    const int q1 = br == 0 ? ns : br == 1 ? ns + p.wg_wc : P;
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
        if (NT < 512) r1 += fac[(c0 + j) * 16 + h1] * o1[j];
      }
    }
  }
  if (has0) st_f32x4(p.out + ((size_t)seq * p.hkv * G + head * G + h0) * D + d0, r0);
  if (has1) st_f32x4(p.out + ((size_t)seq * p.hkv * G + head * G + h1) * D + d1, r1);
  if (threadIdx.x == 0) reset_counter(p.attn_counters + unit);
  if (p.pub) {                                      // codes back to "not yet" for the next call
    const Coherent pc(p.pub + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
    for (int i = threadIdx.x; i < p.top_k; i += NT) pc.st1((uint32_t)(i * 4), 0.f);
  }
}

// Group scores shat_b = ln sum_h exp(s_{h,b} - LSE_h) of this thread's blocks
// [b0, b0 + per) from the raw scores (LDS or workspace, [nb_pad][16] block-major),
// as keys for the radix select.  HV float4s of head scores per block; rounds of 32
// float4 per thread; ready() runs after the first round's loads are issued and
// leaves the heads' LSE in lse_sh.
template <int HV, typename Ready>
__device__ __forceinline__ void group_scores(bool in_lds, const Coherent& sc, const float* s_raw,
                                             const float* lse_sh, int b0, int per, int ncand, int G, float* s_shat,
                                             uint32_t* s_key, Ready&& ready) {
  constexpr int KR = HV == 4 ? 2 : 16 / HV;       // blocks per round
  f32x4 raw[KR][HV];
  auto load_round = [&](int e0) {
#pragma unroll
    for (int e = 0; e < KR; ++e) {
      const int b = b0 + e0 + e;
      const bool ok = e0 + e < per && b < ncand;
#pragma unroll
      for (int v = 0; v < HV; ++v) {
        if (in_lds) raw[e][v] = ok ? *reinterpret_cast<const f32x4*>(s_raw + b * 16 + 4 * v) : f32x4{0.f, 0.f, 0.f, 0.f};
        else raw[e][v] = ok ? sc.ld4((uint32_t)((b * 16 + 4 * v) * 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  load_round(0);
  ready();
  float lse_r[4 * HV];
#pragma unroll
  for (int h = 0; h < 4 * HV; ++h) lse_r[h] = (h < G) ? lse_sh[h] : 0.f;
#pragma unroll 1
  for (int e0 = 0; e0 < per; e0 += KR) {
    if (e0 > 0) load_round(e0);
#pragma unroll
    for (int e = 0; e < KR; ++e) {
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
}

// ---------------------------------------------------------------------------
// Scoring role.  Returns true in the lead (every thread), with the selection of
// this unit in s_sel[0..top_k) (ascending, -1 padded) and the count in *n_sel.
// ---------------------------------------------------------------------------
template <typename E, int D, int KIND, int NW>
__device__ __forceinline__ bool select_role(const DecodeParams& p, int unit, int split, unsigned char* smem, int* s_sel,
                            int* n_sel) {
  constexpr int NT = 64 * NW;
  SelLds<NW>& sl = *reinterpret_cast<SelLds<NW>*>(smem);
  uint32_t* s_key = reinterpret_cast<uint32_t*>(smem + sizeof(SelLds<NW>));
  float* s_shat = reinterpret_cast<float*>(s_key + p.nb_pad);
  float* s_raw = s_shat + p.nb_pad;                  // [nb_pad][16] when splits == 1
  const bool in_lds = p.splits == 1;
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
  // the unit's tiles are dealt round-robin over its scoring waves, so a sequence
  // shorter than max_len still keeps every wave busy
  const int tile0 = split * NW + wave, tstride = p.splits * NW;
  float run_m = -INFINITY, run_s = 0.f;        // LSE partial of head n over this lane's blocks
  // scores s4[i] of blocks tile*16 + 4g + i for head n: running LSE and the block-major
  // raw scores (LDS with one scoring workgroup, the workspace otherwise)
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
      if (n < G) {
        if (in_lds) s_raw[b * 16 + n] = sv[i];
        else sc.st1((uint32_t)((b * 16 + n) * 4), sv[i]);
      }
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
      const int tile = tile0 + j * tstride;
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
    // refilled with the tile RING ahead as soon as it is scored.  (A fp32 rank-r
    // tile takes 160 registers, so it has one slot; deeper rings for the
    // compressed tiles measured no faster.)
    // Every slot is refilled with the same loads whether or not its next tile exists
    // (rows past the unit's candidates repeat the last one and are never posted),
    // and use_quad is a compile-time constant of the loop: the compiler then knows
    // how many loads were issued after each tile's, so a tile's scores wait for that
    // tile only and not also for the tile requested behind it.  Only the last round
    // requests nothing.
    constexpr int RING = (KIND == 0 || Kind<KIND>::kFp4) ? 2 : 1;
    const size_t sum_base = (size_t)unit * p.nb_max;
    auto rows_of = [&](int tile, const void*& mr, const void*& vr) {
      const int brow = max(0, min(tile * 16 + n, ncand - 1));   // A-operand row (block) of this lane
      summary_rows<D, KIND>(p.mu, p.so, sum_base + brow, p.rank, p.vlen, mr, vr);
    };
    // the subspace kinds request P's rows and the query first: scale * P q is formed
    // (and exchanged between the waves) while the summary tiles are in flight
    ScoreW<D> W;
    SubspaceRows<D> prow;
    const size_t q_base = ((size_t)seq * (size_t)(p.hkv * G) + (size_t)head * G) * D;
    if constexpr (Kind<KIND>::kSub) {
      subspace_rows_load<D>(p.P + (size_t)head * p.sub_s * D, p.sub_s, p.vlen, wave, NW, n, g, prow);
      prepare_weights<E, D, KIND>(p.Q, q_base, n, g, G, p.scale, W);
    }
    auto ring = [&](auto quad_c) {
      constexpr bool Q = decltype(quad_c)::value;
      SumTile<D, KIND> st[RING];
      const void* vrow[RING];
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        const void* mrow;
        rows_of(tile0 + r * tstride, mrow, vrow[r]);
        sum_tile_load<D, KIND>(mrow, vrow[r], p.rank, p.vlen, g, Q, st[r]);
      }
      if constexpr (Kind<KIND>::kSub) {
        subspace_rows_project<D>(prow, p.vlen, wave, NW, n, g, W.lin, sl.wsub_x);
        __syncthreads();
        subspace_weights_gather<D>(p.vlen, -1, NW, n, g, sl.wsub_x, W.quad);
        finish_subspace_weights<E, D, KIND>(W);
      } else {
        prepare_weights<E, D, KIND>(p.Q, q_base, n, g, G, p.scale, W);
      }
      int j0 = 0;
      for (; j0 + RING < p.sel_tpw; j0 += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
          const int tile = tile0 + (j0 + r) * tstride;
          const f32x4 s4 = tile_score<E, D, KIND>(st[r], vrow[r], p.rank, p.vlen, g, Q, p.alpha, p.scale, W);
          const void* mrow;
          rows_of(tile + RING * tstride, mrow, vrow[r]);
          sum_tile_load<D, KIND>(mrow, vrow[r], p.rank, p.vlen, g, Q, st[r]);
          if (tile < tiles_total) post(tile, s4, true);
        }
      }
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        const int j = j0 + r, tile = tile0 + j * tstride;
        if (j < p.sel_tpw && tile < tiles_total) {
          const f32x4 s4 = tile_score<E, D, KIND>(st[r], vrow[r], p.rank, p.vlen, g, Q, p.alpha, p.scale, W);
          post(tile, s4, true);
        }
      }
    };
    if (p.alpha != 0.f) ring(std::true_type{});
    else ring(std::false_type{});
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
    for (int w = 0; w < NW; ++w) {
      const float om = sl.red_m[w][threadIdx.x], os = sl.red_s[w][threadIdx.x];
      const float mx = fmaxf(M, om);
      if (mx != -INFINITY) { S = S * __expf(M - mx) + os * __expf(om - mx); M = mx; }
    }
    if (in_lds) {
      sl.lse_sh[threadIdx.x] = (M == -INFINITY) ? -INFINITY : M + __logf(S);
    } else {
      const uint32_t o = (uint32_t)((split * 16 + threadIdx.x) * 2 * 4);
      lp.st1(o, M);
      lp.st1(o + 4, S);
    }
  }

  // ---- hand-off: the last scoring workgroup of this unit selects ----------
  if (!in_lds && !arrive_last(p.sel_counters + unit, (uint32_t)p.splits, &sl.bcast[0])) return false;

  // phase 2 is latency-bound: with the scores in the workspace, the first round of
  // this thread's block scores and the LSE partials are fetched together, so both
  // cost one memory round trip (a round is 32 float4 per thread, the whole share
  // of a thread unless the context is long and the group large)
  const int per = (p.nb_max + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  if (in_lds) __syncthreads();                    // raw scores and the LSE are in LDS
  auto lse_ready = [&]() {
    if (in_lds) return;
    for (int i = threadIdx.x; i < p.splits * 16; i += NT) {
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
  };
  const int hv = (G + 3) / 4;                     // float4s of head scores a block needs
  if (hv == 1) group_scores<1>(in_lds, sc, s_raw, sl.lse_sh, b0, per, ncand, G, s_shat, s_key, lse_ready);
  else if (hv == 2) group_scores<2>(in_lds, sc, s_raw, sl.lse_sh, b0, per, ncand, G, s_shat, s_key, lse_ready);
  else group_scores<4>(in_lds, sc, s_raw, sl.lse_sh, b0, per, ncand, G, s_shat, s_key, lse_ready);
  __syncthreads();
  if (p.sel_score) {
    float* ss = p.sel_score + (size_t)unit * p.nb_max;
    for (int b = threadIdx.x; b < p.nb_max; b += NT) ss[b] = (b < ncand) ? s_shat[b] : -INFINITY;
  }

  // ---- radix select: the selection (ascending, -1 padded) to the caller, into LDS
  // for the lead's own tiles, and as codes for the waiting selected-branch waves
  int32_t* so = p.sel + (size_t)unit * p.top_k;
  const Coherent pc(p.pub ? static_cast<const void*>(p.pub + (size_t)unit * p.top_k) : static_cast<const void*>(so),
                    (uint32_t)(p.top_k * 4));
  const int sel_total = wg_select_topk<NW>(s_key, ncand, per, p.top_k, &sl.hist2[0][0][0], sl.scan_w,
                                           [&](int pos, int b) {
                                             so[pos] = b;
                                             s_sel[pos] = b;
                                             if (p.pub && pos >= p.lead_tiles)
                                               pc.st1((uint32_t)(pos * 4), __uint_as_float((uint32_t)(b + 2)));
                                           });
  for (int i = sel_total + (int)threadIdx.x; i < p.top_k; i += NT) {
    so[i] = -1;
    s_sel[i] = -1;
    if (p.pub && i >= p.lead_tiles) pc.st1((uint32_t)(i * 4), __uint_as_float(1u));
  }
  if (!in_lds && threadIdx.x == 0) reset_counter(p.sel_counters + unit);
  if (threadIdx.x == 0) *n_sel = sel_total;
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------
// The lead's share of the selected branch: tiles [0, lead_tiles) of the
// selection in LDS, strided over the waves.
// ---------------------------------------------------------------------------
template <typename E, int D, int NW>
__device__ __forceinline__ void lead_attention(const DecodeParams& p, int unit, const int* s_sel, int n_sel, unsigned char* smem,
                               int* flag) {
  using T = AttnTiling<E, D>;
  const int wave = threadIdx.x >> 6;
  const int seq = unit / p.hkv, head = unit % p.hkv;
  const int G = p.group;
  const int L = p.seq_lens[seq];
  const int nb = (L + kBlock - 1) / kBlock;
  const int ntiles = min(p.lead_tiles, n_sel);
  const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)unit * p.max_len * D;
  const typename E::storage* Vu = reinterpret_cast<const typename E::storage*>(p.V) + (size_t)unit * p.max_len * D;
  auto src = [&](int j, const typename E::storage*& Kt, const typename E::storage*& Vt) -> int {
    const int t = wave + j * NW;
    if (t >= ntiles) return 0;
    const int b = s_sel[t];
    if (b < 0 || b >= nb) return 0;
    Kt = Ku + (size_t)b * kBlock * D;
    Vt = Vu + (size_t)b * kBlock * D;
    return min(kBlock, L - b * kBlock);
  };
  const typename E::storage* Qg = reinterpret_cast<const typename E::storage*>(p.Q) + ((size_t)seq * p.hkv * G + (size_t)head * G) * D;
  typename E::storage* lds = reinterpret_cast<typename E::storage*>(smem) + (size_t)wave * kBlock * T::kRowStride;
  float m_run, l_run;
  f32x4 acc_o[T::kDt];
  if (p.lead_tiles <= 2 * NW) wave_tiles_pair<E, D>(src, Qg, G, p.scale_log2, lds, m_run, l_run, acc_o);
  else wave_tiles<E, D>(src, Qg, G, p.scale_log2, lds, m_run, l_run, acc_o);
  const int mine[2] = {0, 0};
  merge_and_finish<E, D, NW>(p, unit, 0, mine, 1, m_run, l_run, acc_o, smem, flag);
}

// ---------------------------------------------------------------------------
// Window and pooled-token workgroups (`local` of wg_wc per unit): the unit's window
// tiles followed by its pooled tiles form one list, split evenly over the unit's
// waves.  The one wave of a workgroup whose share crosses from window to pooled
// tiles parks its window partial in a spare LDS slot beyond the V staging area, and
// the workgroup merge counts it with the window waves.
// ---------------------------------------------------------------------------
template <typename E, int D, int NW>
__device__ __forceinline__ void wc_attention(const DecodeParams& p, int unit, int local, unsigned char* smem, int* flag) {
  using T = AttnTiling<E, D>;
  constexpr int NCH = T::kChunks, EPL = T::kEpl, NDT = T::kDt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int seq = unit / p.hkv, head = unit % p.hkv;
  const int G = p.group;
  const int L = p.seq_lens[seq];
  const int nc = (p.cmp_on && L >= 32) ? (L - 32) / 16 + 1 : 0;
  const int win_len = min(p.window, L);
  const int win_start = L - win_len;
  const int t_win = (win_len + kBlock - 1) / kBlock, t_cmp = (nc + kBlock - 1) / kBlock;
  const int Tt = t_win + t_cmp, waves = p.wg_wc * NW;
  const int gw = local * NW + wave;
  int j0, j1;                                  // this wave's share of the list
  if constexpr (NW == 8) {                     // even split; at most one wave per workgroup straddles
    j0 = (int)((int64_t)gw * Tt / waves);
    j1 = (int)((int64_t)(gw + 1) * Tt / waves);
  } else {                                     // no spare LDS slot: each wave stays in one branch,
    int nw_win = 0;                            // the split that makes the longest share shortest
    if (t_win > 0 && t_cmp == 0) {
      nw_win = waves;
    } else if (t_win > 0) {
      int best = 1 << 30;
      for (int a = 1; a < waves; ++a) {
        const int c = max((t_win + a - 1) / a, (t_cmp + waves - a - 1) / (waves - a));
        if (c < best) { best = c; nw_win = a; }
      }
    }
    const bool is_win = gw < nw_win;
    const int nwb = max(is_win ? nw_win : waves - nw_win, 1), idx = is_win ? gw : gw - nw_win;
    const int tb = is_win ? t_win : t_cmp, base = is_win ? 0 : t_win;
    j0 = base + (int)((int64_t)idx * tb / nwb);
    j1 = base + (int)((int64_t)(idx + 1) * tb / nwb);
  }
  const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)unit * p.max_len * D;
  const typename E::storage* Vu = reinterpret_cast<const typename E::storage*>(p.V) + (size_t)unit * p.max_len * D;
  const typename E::storage* kcu = p.cmp_on ? reinterpret_cast<const typename E::storage*>(p.kc) + (size_t)unit * p.nc_max * D : nullptr;
  const typename E::storage* vcu = p.cmp_on ? reinterpret_cast<const typename E::storage*>(p.vc) + (size_t)unit * p.nc_max * D : nullptr;
  auto src = [&](int t, const typename E::storage*& Kt, const typename E::storage*& Vt) -> int {
    if (t < t_win) {
      const int start = win_start + t * kBlock;
      Kt = Ku + (size_t)start * D;
      Vt = Vu + (size_t)start * D;
      return min(kBlock, L - start);
    }
    const int start = (t - t_win) * kBlock;
    Kt = kcu + (size_t)start * D;
    Vt = vcu + (size_t)start * D;
    return min(kBlock, nc - start);
  };
  typename E::storage* lds = reinterpret_cast<typename E::storage*>(smem) + (size_t)wave * kBlock * T::kRowStride;
  float* spare = reinterpret_cast<float*>(smem + attn_stage_bytes<E, D, NW>());   // [16][D] then [16][2]
  __shared__ int s_straddle;
  if (threadIdx.x == 0) s_straddle = 0;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  if (j0 < j1) {
    TileRegs<E, D> tr;
    const typename E::storage *Kt = nullptr, *Vt = nullptr;
    int nv = src(j0, Kt, Vt);
    u32x4 qf[NCH];                                // Q first: the first scores wait for Q and K only
    {
      const typename E::storage* Qh = reinterpret_cast<const typename E::storage*>(p.Q) +
                                      ((size_t)seq * p.hkv * G + (size_t)head * G + min(n, G - 1)) * D;
#pragma unroll
      for (int c = 0; c < NCH; ++c) qf[c] = ld16(Qh + (4 * c + g) * EPL);
    }
    tile_load_k<E, D>(Kt, nv, tr);
    tile_load_v<E, D>(Vt, nv, tr);
    // Every tile but the last requests the next one unconditionally (K after the
    // scores, V as soon as this tile's V is staged, before P V), so the compiler's
    // load counts are exact: staging waits for this tile's V only, not for the K
    // just requested behind it.  The last tile is peeled off and requests nothing.
    int t = j0;
    for (; t + 1 < j1; ++t) {
      f32x4 sc4[4];
      tile_scores<E, D>(tr, qf, sc4);
      const typename E::storage *Kn = nullptr, *Vn = nullptr;
      const int nv_next = src(t + 1, Kn, Vn);
      tile_load_k<E, D>(Kn, nv_next, tr);
      tile_stage_v<E, D>(tr, lds);
      tile_load_v<E, D>(Vn, nv_next, tr);
      tile_softmax_pv<E, D>(sc4, nv, p.scale_log2, lds, m_run, l_run, acc_o);
      if (t + 1 == t_win) {                        // window part done, pooled tiles follow
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) spare[n * D + 16 * dt + 4 * g + i] = acc_o[dt][i];
          acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (g == 0) { spare[16 * D + 2 * n] = m_run; spare[16 * D + 2 * n + 1] = l_run; }
        if (lane == 0) s_straddle = 1;
        m_run = -INFINITY;
        l_run = 0.f;
      }
      nv = nv_next;
    }
    f32x4 sc4[4];
    tile_scores<E, D>(tr, qf, sc4);
    tile_stage_v<E, D>(tr, lds);
    tile_softmax_pv<E, D>(sc4, nv, p.scale_log2, lds, m_run, l_run, acc_o);
  }
  const int ns = slc_slots(p);
  const int mine[2] = {ns + local, ns + p.wg_wc + local};
  const int wslot = j1 > j0 ? ((j1 - 1) < t_win ? mine[0] : mine[1]) : -1;
  merge_and_finish<E, D, NW>(p, unit, wslot, mine, 2, m_run, l_run, acc_o, smem, flag, spare, &s_straddle);
}

// ---------------------------------------------------------------------------
// Selected-branch workgroups beyond the lead's share (`local` of wg_slc): tile
// t = lead_tiles + local * NW * tpw_slc + j * NW + wave.  With a lead the block
// comes from its published code (polled, bounded); otherwise from the caller's
// selection.
// ---------------------------------------------------------------------------
template <typename E, int D, int NW>
__device__ __forceinline__ void slc_attention(const DecodeParams& p, int unit, int local, unsigned char* smem, int* flag) {
  using T = AttnTiling<E, D>;
  const int wave = threadIdx.x >> 6;
  const int seq = unit / p.hkv, head = unit % p.hkv;
  const int G = p.group;
  const int L = p.seq_lens[seq];
  const int nb = (L + kBlock - 1) / kBlock;
  const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)unit * p.max_len * D;
  const typename E::storage* Vu = reinterpret_cast<const typename E::storage*>(p.V) + (size_t)unit * p.max_len * D;
  bool gave_up = false;
  auto src = [&](int j, const typename E::storage*& Kt, const typename E::storage*& Vt) -> int {
    if (j >= p.tpw_slc) return 0;
    const int t = p.lead_tiles + local * NW * p.tpw_slc + j * NW + wave;
    if (t >= p.top_k) return 0;
    int b = -1;
    if (p.pub) {
      const Coherent pc(p.pub + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
      uint32_t code = 0;
      for (uint32_t it = 0; it < p.poll_cap; ++it) {
        code = pc.poll1((uint32_t)(t * 4));
        if (code != 0u) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (code == 0u) gave_up = true;
      b = (code >= 2u) ? (int)(code - 2u) : -1;
    } else {
      const Coherent si(p.sel_in + (size_t)unit * p.top_k, (uint32_t)(p.top_k * 4));
      b = __float_as_int(si.ld1((uint32_t)(t * 4)));
    }
    if (b < 0 || b >= nb) return 0;
    Kt = Ku + (size_t)b * kBlock * D;
    Vt = Vu + (size_t)b * kBlock * D;
    return min(kBlock, L - b * kBlock);
  };
  const typename E::storage* Qg = reinterpret_cast<const typename E::storage*>(p.Q) + ((size_t)seq * p.hkv * G + (size_t)head * G) * D;
  typename E::storage* lds = reinterpret_cast<typename E::storage*>(smem) + (size_t)wave * kBlock * T::kRowStride;
  float m_run, l_run;
  f32x4 acc_o[T::kDt];
  wave_tiles<E, D>(src, Qg, G, p.scale_log2, lds, m_run, l_run, acc_o);
  if (gave_up && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(p.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int mine[2] = {p.has_lead + local, 0};
  merge_and_finish<E, D, NW>(p, unit, mine[0], mine, 1, m_run, l_run, acc_o, smem, flag);
}

// Waves per workgroup: 8 (one workgroup per CU: the selecting workgroup holds a whole
// unit's scores) or 4 (two per CU, finer work for few units or long contexts); fp32
// keys at d = 128 take 4 (their attention tile needs a SIMD's whole register file).
template <typename E, int D, int NW>
struct DecodeShape {
  static constexpr bool kWide = E::kBytes == 4 && D == 128;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kMinBlocks = (NW == 4 && !kWide) ? 2 : 1;
};

template <typename E, int D, int KIND, int NW>
__global__ __launch_bounds__((DecodeShape<E, D, NW>::kThreads), (DecodeShape<E, D, NW>::kMinBlocks))
void k_decode(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int flag;
  __shared__ int s_sel[64];
  __shared__ int n_sel;
  const int i = blockIdx.x;
  if (i < p.sel_wgs) {
    if (!select_role<E, D, KIND, NW>(p, i / p.splits, i % p.splits, smem, s_sel, &n_sel)) return;
    if constexpr (KIND != 2) {
      if (p.has_lead) lead_attention<E, D, NW>(p, i / p.splits, s_sel, n_sel, smem, &flag);
    }
    return;
  }
  if constexpr (KIND != 2) {
    const int j = i - p.sel_wgs;
    if (j < p.wc_wgs) {
      wc_attention<E, D, NW>(p, j % p.units, j / p.units, smem, &flag);
    } else {
      const int k = j - p.wc_wgs;
      slc_attention<E, D, NW>(p, k % p.units, k / p.units, smem, &flag);
    }
  }
}

template <typename E, int D, int NW>
static size_t attn_role_lds_bytes(int P) {
  const size_t merge = (size_t)NW * 16 * (D + 4 + 2) * sizeof(float) + NW * sizeof(int);
  const size_t spare = NW == 8 ? ((size_t)16 * D + 32) * sizeof(float) : 0;   // a parked window partial
  return std::max(std::max(attn_stage_bytes<E, D, NW>(), merge), (size_t)P * 48 * sizeof(float)) + spare;
}

template <typename E, int D, int KIND, int NW>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodeParams& dp) {
  const int total = dp.sel_wgs + dp.wc_wgs + dp.slc_wgs;
  size_t lds = 0;
  if (dp.sel_wgs) lds = std::max(lds, select_lds_bytes<NW>(dp.nb_pad, dp.splits == 1));
  if (dp.do_attn) lds = std::max(lds, attn_role_lds_bytes<E, D, NW>(dp.has_lead + dp.wg_slc + 2 * dp.wg_wc));
  hipLaunchKernelGGL((k_decode<E, D, KIND, NW>), dim3(total), dim3(64 * NW), lds, a.stream, dp);
  return hipGetLastError();
}

template <typename E, int D, int NW>
static hipError_t launch_decode_kind(const DecodeArgs& a, const DecodeParams& dp) {
  switch (a.so_kind) {
    case 0: return launch_decode_t<E, D, 0, NW>(a, dp);
    case 1: return launch_decode_t<E, D, 1, NW>(a, dp);
    case 2: return launch_decode_t<E, D, 2, NW>(a, dp);   // exact masses: scoring roles only
    case 3: return launch_decode_t<E, D, 3, NW>(a, dp);   // compressed storage
    case 4: return launch_decode_t<E, D, 4, NW>(a, dp);   // rank-r fp32 in a query subspace
    default: return launch_decode_t<E, D, 5, NW>(a, dp);  // compressed storage in a query subspace
  }
}

template <typename E, int D>
static hipError_t launch_decode_ed(const DecodeArgs& a, const DecodeParams& dp) {
  if constexpr (DecodeShape<E, D, 8>::kWide) return launch_decode_kind<E, D, 4>(a, dp);
  else return a.nw == 8 ? launch_decode_kind<E, D, 8>(a, dp) : launch_decode_kind<E, D, 4>(a, dp);
}

int decode_max_waves(bool bf16, int head_dim) { return (!bf16 && head_dim == 128) ? 4 : 8; }

size_t decode_select_lds_bytes(int nw, int nb_pad, bool raw_in_lds) {
  return nw == 8 ? select_lds_bytes<8>(nb_pad, raw_in_lds) : select_lds_bytes<4>(nb_pad, raw_in_lds);
}

hipError_t launch_decode(const DecodeArgs& a) {
  DecodeParams p;
  const int units = a.batch * a.hkv;
  p.units = units; p.hkv = a.hkv; p.group = a.group; p.max_len = a.max_len; p.nb_max = a.nb_max;
  p.nb_pad = (a.nb_max + 15) / 16 * 16; p.top_k = a.top_k; p.seq_lens = a.seq_lens; p.Q = a.Q;
  p.sel_wgs = a.do_select ? units * a.splits : 0;
  p.splits = a.splits; p.sel_tpw = a.sel_tpw; p.rank = a.rank; p.alpha = a.alpha; p.scale = a.scale;
  p.mu = a.mu; p.so = a.so; p.P = a.P; p.sub_s = a.sub_s; p.vlen = a.vlen; p.sel = a.sel; p.sel_score = a.sel_score;
  p.sel_counters = a.sel_counters; p.scores = a.scores; p.lse_part = a.lse_part;
  p.do_attn = a.do_attn ? 1 : 0;
  p.has_lead = (a.do_select && a.do_attn) ? 1 : 0;
  p.lead_tiles = p.has_lead ? a.lead_tiles : 0;
  p.wg_slc = a.do_attn ? a.wg_slc : 0;
  p.wg_wc = a.do_attn ? a.wg_wc : 0;
  p.pub = (p.has_lead && p.wg_slc > 0) ? a.ready : nullptr;
  p.wc_wgs = units * p.wg_wc;
  p.slc_wgs = units * p.wg_slc;
  p.nc_max = a.nc_max; p.window = a.window; p.cmp_on = a.cmp_on; p.tpw_slc = a.tpw_slc;
  p.scale_log2 = a.scale * kLog2e;
  p.K = a.K; p.V = a.V; p.kc = a.kc; p.vc = a.vc; p.gates = a.gates;
  p.sel_in = a.sel_in;
  p.out = a.out; p.attn_counters = a.attn_counters; p.part_ml = a.part_ml; p.part_o = a.part_o;
  p.status = a.status; p.poll_cap = a.poll_cap;
  if (a.bf16) return a.head_dim == 128 ? launch_decode_ed<EltBF16, 128>(a, p) : launch_decode_ed<EltBF16, 64>(a, p);
  return a.head_dim == 128 ? launch_decode_ed<EltF32, 128>(a, p) : launch_decode_ed<EltF32, 64>(a, p);
}

}  // namespace cobs
