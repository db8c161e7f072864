// Sparse decode attention over the three NSA branches with gated combine (gfx950).
//
// Branches (Janus issue #181 on NSA: compression, selection and sliding-window
// paths with gates; COBS explainer, Technisches Resuemee 2.3: only the selector
// changes): each branch is an exact softmax over its own key set,
//   SLC - the keys of the top-k selected 64-key blocks,
//   WIN - the last W positions,
//   CMP - the mean-pooled tokens (32 keys every 16 positions),
// and out = g_cmp o_cmp + g_slc o_slc + g_win o_win.
//
// Work is split into 64-key tiles.  One wavefront processes its tiles with an
// online softmax for the whole GQA group at once: S = K Q^T is a 64x16 tile
// computed with v_mfma_f32_16x16x32_bf16 (keys on the M side, the group's heads
// on the N side, head_dim as the contraction), so each lane owns one head and a
// fixed set of 16 keys; the probabilities it holds are exactly the B operand of
// O^T = V^T P^T, so P never leaves registers.  V is staged in LDS row-major and
// read as the transposed A operand.  K is loaded straight into the MFMA layout.
// Every tile is read once from HBM with 16-byte loads.
//
// The waves of a workgroup merge their (max, sum, O) in LDS into one partial per
// workgroup; the last workgroup of a (sequence, kv-head) (atomic counter) merges
// the partials of each branch by log-sum-exp rescaling and applies the gates.
#include "cobs_device.h"
#include "cobs_launch.h"
#include "attn_tile.h"

#include <algorithm>

namespace cobs {

struct AttnParams {
  int hkv, group, max_len, nc_max, top_k, window, cmp_on;
  int tiles_per_wave, wg_slc, wg_win, wg_cmp;
  float scale_log2;                 // scale * log2(e)
  const int32_t* seq_lens;
  const void *Q, *K, *V, *kc, *vc;
  const float* gates;
  const int32_t* sel;
  float* out;
  uint32_t* counters;
  float* part_ml;
  float* part_o;
};

template <typename E, int D>
__global__ __launch_bounds__(256) void k_attn_decode(AttnParams p) {
  using T = AttnTiling<E, D>;
  constexpr int NCH = T::kChunks, EPL = T::kEpl, NDT = T::kDt;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int last_flag;

  const int nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int head = blockIdx.y, seq = blockIdx.z;
  const int unit = seq * p.hkv + head;
  const int G = p.group;
  const int L = p.seq_lens[seq];
  const int P = p.wg_slc + p.wg_win + p.wg_cmp;

  int branch, local;                       // 0 = SLC, 1 = WIN, 2 = CMP
  if ((int)blockIdx.x < p.wg_slc) { branch = 0; local = blockIdx.x; }
  else if ((int)blockIdx.x < p.wg_slc + p.wg_win) { branch = 1; local = blockIdx.x - p.wg_slc; }
  else { branch = 2; local = blockIdx.x - p.wg_slc - p.wg_win; }

  // the group's queries as the B operand of S = K Q^T (heads >= G are zero)
  u32x4 qf[NCH];
  {
    const typename E::storage* Qh = reinterpret_cast<const typename E::storage*>(p.Q) +
                                    ((size_t)seq * p.hkv * G + (size_t)head * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qf[c] = ld16(Qh + (4 * c + g) * EPL);
      if (n >= G) qf[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  const typename E::storage* Ku = reinterpret_cast<const typename E::storage*>(p.K) + (size_t)unit * p.max_len * D;
  const typename E::storage* Vu = reinterpret_cast<const typename E::storage*>(p.V) + (size_t)unit * p.max_len * D;
  const typename E::storage* kcu = p.cmp_on ? reinterpret_cast<const typename E::storage*>(p.kc) + (size_t)unit * p.nc_max * D : nullptr;
  const typename E::storage* vcu = p.cmp_on ? reinterpret_cast<const typename E::storage*>(p.vc) + (size_t)unit * p.nc_max * D : nullptr;
  const int nc = (p.cmp_on && L >= 32) ? (L - 32) / 16 + 1 : 0;
  const int win_len = min(p.window, L);
  const int win_start = L - win_len;

  typename E::storage* lds = reinterpret_cast<typename E::storage*>(smem) + (size_t)wave * kBlock * T::kRowStride;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < p.tiles_per_wave; ++j) {
    const int tile = (local * nw + wave) * p.tiles_per_wave + j;
    const typename E::storage *Kt, *Vt;
    int nvalid = 0;
    if (branch == 0) {
      if (tile < p.top_k) {
        const int b = p.sel[(size_t)unit * p.top_k + tile];
        if (b >= 0) {
          nvalid = min(kBlock, L - b * kBlock);
          Kt = Ku + (size_t)b * kBlock * D;
          Vt = Vu + (size_t)b * kBlock * D;
        }
      }
    } else if (branch == 1) {
      const int start = win_start + tile * kBlock;
      if (start < L) {
        nvalid = min(kBlock, L - start);
        Kt = Ku + (size_t)start * D;
        Vt = Vu + (size_t)start * D;
      }
    } else {
      const int start = tile * kBlock;
      if (start < nc) {
        nvalid = min(kBlock, nc - start);
        Kt = kcu + (size_t)start * D;
        Vt = vcu + (size_t)start * D;
      }
    }
    if (nvalid <= 0) continue;
    attend_tile<E, D>(Kt, Vt, nvalid, qf, p.scale_log2, lds, m_run, l_run, acc_o);
  }
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);

  // ---- merge the waves of this workgroup in LDS ----------------------------
  __syncthreads();                                   // staging slices no longer needed
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
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += blockDim.x) {
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
    po.st4((uint32_t)((((int)blockIdx.x * G + h) * D + d4) * 4), o);
    if (d4 == 0) {
      pm.st1((uint32_t)(((blockIdx.x * 16 + h) * 2) * 4), M);
      pm.st1((uint32_t)(((blockIdx.x * 16 + h) * 2 + 1) * 4), Ls);
    }
  }

  // ---- the last workgroup of this (sequence, kv-head) combines ------------
  if (!arrive_last(p.counters + unit, (uint32_t)P, &last_flag)) return;

  // (max, sum) of every partial into LDS with one round of loads
  float* sm = reinterpret_cast<float*>(smem);          // [P][16][2]
  float* fac = sm + (size_t)P * 32;                    // [P][16]: gate / L_branch * 2^(m_q - M_branch)
  for (int i = threadIdx.x; i < P * G; i += blockDim.x) {
    const int q = i / G, h = i % G;
    sm[(q * 16 + h) * 2] = pm.ld1((uint32_t)(((q * 16 + h) * 2) * 4));
    sm[(q * 16 + h) * 2 + 1] = pm.ld1((uint32_t)(((q * 16 + h) * 2 + 1) * 4));
  }
  __syncthreads();
  const int pb[4] = {0, p.wg_slc, p.wg_slc + p.wg_win, P};   // SLC, WIN, CMP partial ranges
  // merge factor of partial q for head h: gate / L_branch * 2^(m_q - M_branch)
  for (int i = threadIdx.x; i < 3 * G; i += blockDim.x) {
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
  // out[h][d] = sum_q fac[q][h] O_q[h][d]; two output float4 per thread, partials in
  // chunks of 16 so that up to 32 coherent loads are in flight at once
  const int items = G * (D / 4);
  for (int i0 = threadIdx.x; i0 < items; i0 += 2 * blockDim.x) {
    const int i1 = i0 + blockDim.x;
    const bool has1 = i1 < items;
    const int h0 = i0 / (D / 4), d0 = (i0 % (D / 4)) * 4;
    const int h1 = has1 ? i1 / (D / 4) : h0, d1 = has1 ? (i1 % (D / 4)) * 4 : d0;
    f32x4 r0 = {0.f, 0.f, 0.f, 0.f}, r1 = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < P; c0 += 16) {
      f32x4 o0[16], o1[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int q = min(c0 + j, P - 1);
        o0[j] = po.ld4((uint32_t)(((q * G + h0) * D + d0) * 4));
        o1[j] = po.ld4((uint32_t)(((q * G + h1) * D + d1) * 4));
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + j < P) {
          r0 += fac[(c0 + j) * 16 + h0] * o0[j];
          r1 += fac[(c0 + j) * 16 + h1] * o1[j];
        }
      }
    }
    st_f32x4(p.out + ((size_t)seq * p.hkv * G + head * G + h0) * D + d0, r0);
    if (has1) st_f32x4(p.out + ((size_t)seq * p.hkv * G + head * G + h1) * D + d1, r1);
  }
  if (threadIdx.x == 0) reset_counter(p.counters + unit);
}

template <typename E, int D>
static hipError_t launch_attn_t(const AttnArgs& a, const AttnParams& ap) {
  const int P = a.wg_slc + a.wg_win + a.wg_cmp;
  dim3 grid(P, a.hkv, a.batch);
  const size_t lds = std::max(attn_lds_bytes<E, D>(a.waves_per_wg), (size_t)P * 48 * sizeof(float));
  hipLaunchKernelGGL((k_attn_decode<E, D>), grid, dim3(64 * a.waves_per_wg), lds, a.stream, ap);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnArgs& a) {
  AttnParams ap;
  ap.hkv = a.hkv; ap.group = a.group; ap.max_len = a.max_len; ap.nc_max = a.nc_max;
  ap.top_k = a.top_k; ap.window = a.window; ap.cmp_on = a.cmp_on;
  ap.tiles_per_wave = a.tiles_per_wave; ap.wg_slc = a.wg_slc; ap.wg_win = a.wg_win; ap.wg_cmp = a.wg_cmp;
  ap.scale_log2 = a.scale * kLog2e;
  ap.seq_lens = a.seq_lens; ap.Q = a.Q; ap.K = a.K; ap.V = a.V; ap.kc = a.kc; ap.vc = a.vc;
  ap.gates = a.gates; ap.sel = a.sel; ap.out = a.out; ap.counters = a.counters;
  ap.part_ml = a.part_ml; ap.part_o = a.part_o;
  if (a.bf16) return a.head_dim == 128 ? launch_attn_t<EltBF16, 128>(a, ap) : launch_attn_t<EltBF16, 64>(a, ap);
  return a.head_dim == 128 ? launch_attn_t<EltF32, 128>(a, ap) : launch_attn_t<EltF32, 64>(a, ap);
}

size_t attn_decode_lds_bytes(bool bf16, int head_dim, int waves) {
  if (bf16) return head_dim == 128 ? attn_lds_bytes<EltBF16, 128>(waves) : attn_lds_bytes<EltBF16, 64>(waves);
  return head_dim == 128 ? attn_lds_bytes<EltF32, 128>(waves) : attn_lds_bytes<EltF32, 64>(waves);
}

}  // namespace cobs
