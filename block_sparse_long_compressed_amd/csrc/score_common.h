// Block-score contraction shared by the decode and prefill selection kernels.
//
// COBS (gist.science explainer, Technisches Resuemee 2.2-2.3): the estimate of
// ln m_b is ln n_b + scale q.mu_b + alpha/2 scale^2 q^T Sigma_b q, with Sigma_b
// the diagonal variance or sum_i v_i v_i^T for the rank-r scaled eigenvectors.
// For a 16-block tile and the 16 heads of a GQA group this is an fp32 MFMA
// contraction (v_mfma_f32_16x16x4_f32): A = summary rows (blocks), B = query
// weights (heads).  Lane (n = l%16, g = l/16) supplies summary columns
// 16u + 4g + c of block n and the weights of head n for the same columns, and
// receives the scores of blocks 4g + i (i = 0..3) for head n.
#pragma once
#include "cobs_device.h"

namespace cobs {

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

// Weights of head n of the group whose first head's query starts at q_base:
// linear scale*q, quadratic alpha/2 scale^2 q^2 (diagonal form only).
template <typename E, int D, int KIND>
__device__ __forceinline__ void score_weights(const void* Q, size_t q_base, int n, int g, int G, float scale,
                                              float alpha, float (&wlin)[D / 16][4], float (&wquad)[D / 16][4]) {
  const bool hv = n < G;
  const size_t qoff = q_base + (size_t)(hv ? n : 0) * D;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    float q4[4];
    load_q4<E>(Q, qoff + 16 * u + 4 * g, q4);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float qv = hv ? q4[c] : 0.f;
      wlin[u][c] = scale * qv;
      wquad[u][c] = (KIND == 0) ? 0.5f * alpha * scale * scale * qv * qv : 0.f;
    }
  }
}

// Summary rows of one 16-block tile held in registers: this lane's mean columns
// and its second-order columns (the diagonal, or the first kRankGroup scaled
// eigenvectors; further groups are fetched while scoring).
constexpr int kRankGroup = 4;

template <int D, int KIND>
struct SumTile {
  f32x4 m4[D / 16];
  f32x4 v4[KIND == 0 ? 1 : kRankGroup][D / 16];
};

template <int D, int KIND>
__device__ __forceinline__ void sum_tile_load_group(const float* vrow, int r0, int rank, int g, SumTile<D, KIND>& t) {
#pragma unroll
  for (int rr = 0; rr < kRankGroup; ++rr) {
    if (r0 + rr < rank) {
#pragma unroll
      for (int u = 0; u < D / 16; ++u) t.v4[rr][u] = ld_f32x4(vrow + (r0 + rr) * D + 16 * u + 4 * g);
    }
  }
}

// Issue the loads of one tile (mrow / vrow: this lane's block row).
template <int D, int KIND>
__device__ __forceinline__ void sum_tile_load(const float* mrow, const float* vrow, int rank, int g, bool use_quad,
                                              SumTile<D, KIND>& t) {
#pragma unroll
  for (int u = 0; u < D / 16; ++u) t.m4[u] = ld_f32x4(mrow + 16 * u + 4 * g);
  if (use_quad) {
    if constexpr (KIND == 0) {
#pragma unroll
      for (int u = 0; u < D / 16; ++u) t.v4[0][u] = ld_f32x4(vrow + 16 * u + 4 * g);
    } else {
      sum_tile_load_group<D, KIND>(vrow, 0, rank, g, t);
    }
  }
}

// Scores (without ln n_b) of the tile's 16 blocks for the group's heads from the
// loaded rows.  Linear and quadratic terms are independent MFMA chains.
template <int D, int KIND>
__device__ __forceinline__ f32x4 sum_tile_score(SumTile<D, KIND>& t, const float* vrow, int rank, int g, bool use_quad,
                                                float alpha, const float (&wlin)[D / 16][4],
                                                const float (&wquad)[D / 16][4]) {
  constexpr int NU = D / 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NU; ++u) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mfma_f32_16x16x4(t.m4[u][c], wlin[u][c], acc);
  }
  if (!use_quad) return acc;
  if constexpr (KIND == 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc2 = mfma_f32_16x16x4(t.v4[0][u][c], wquad[u][c], acc2);
    }
  } else {
    // (v_i . q)^2 for each scaled eigenvector v_i: the projection is a linear MFMA
    // chain with the linear weights, squared on the VALU
#pragma unroll 1
    for (int r0 = 0; r0 < rank; r0 += kRankGroup) {
      if (r0 > 0) sum_tile_load_group<D, KIND>(vrow, r0, rank, g, t);
#pragma unroll
      for (int rr = 0; rr < kRankGroup; ++rr) {
        if (r0 + rr < rank) {
          f32x4 pr = {0.f, 0.f, 0.f, 0.f}, pr2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; u += 2) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              pr = mfma_f32_16x16x4(t.v4[rr][u][c], wlin[u][c], pr);
              pr2 = mfma_f32_16x16x4(t.v4[rr][u + 1][c], wlin[u + 1][c], pr2);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float dd = pr[i] + pr2[i];
            acc2[i] += 0.5f * alpha * dd * dd;
          }
        }
      }
    }
  }
  return acc + acc2;
}

// Load and score one tile in one step.
template <int D, int KIND>
__device__ __forceinline__ f32x4 score_tile(const float* mrow, const float* vrow, int rank, int g, bool use_quad,
                                            float alpha, const float (&wlin)[D / 16][4],
                                            const float (&wquad)[D / 16][4]) {
  SumTile<D, KIND> t;
  sum_tile_load<D, KIND>(mrow, vrow, rank, g, use_quad, t);
  return sum_tile_score<D, KIND>(t, vrow, rank, g, use_quad, alpha, wlin, wquad);
}

// Number of candidate blocks (a prefix [0, n)) for a query at position t of a
// sequence of length L: blocks whose keys all lie at positions <= t.
__device__ __forceinline__ int candidate_blocks(int L, int t) {
  return (t >= L - 1) ? (L + kBlock - 1) / kBlock : (t + 1) / kBlock;
}

// Adds 1 to hist[digit] for every active lane; lanes of the wave that share a
// digit are combined first (a few rounds), the rest use plain LDS atomics.
__device__ __forceinline__ void wave_histogram_add(uint32_t* hist, bool active, uint32_t digit) {
  uint64_t todo = __ballot(active);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    if (!todo) break;
    const int leader = __builtin_ctzll(todo);
    const uint32_t dl = __shfl(digit, leader, 64);
    const uint64_t same = __ballot(active && digit == dl) & todo;
    if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__builtin_popcountll(same));
    todo &= ~same;
  }
  if ((todo >> lane) & 1ull) atomicAdd(&hist[digit], 1u);
}

// Digit search of one radix pass: given the wave's four bins per lane (bins
// 4l..4l+3), find the bin holding the `need`-th largest key.  Returns the digit
// and updates need (rank within the bin) and eq_bin (the bin's size).
__device__ __forceinline__ uint32_t radix_digit(const u32x4& hb, int& need, int& eq_bin) {
  const int lane = threadIdx.x & 63;
  const int tot = (int)(hb[0] + hb[1] + hb[2] + hb[3]);
  const int incl = wave_inclusive_sum(tot);
  const int all = __builtin_amdgcn_readlane(incl, 63);
  int above = all - incl;                        // keys in bins above this lane's four
  int dig = 0, nn = 0, eb = 0;
  bool found = false;
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    const int h = (int)hb[j];
    if (!found && above < need && need <= above + h) { found = true; dig = 4 * lane + j; nn = need - above; eb = h; }
    above += h;
  }
  const int src = __builtin_ctzll(__ballot(found));
  need = __builtin_amdgcn_readlane(nn, src);
  eq_bin = __builtin_amdgcn_readlane(eb, src);
  return (uint32_t)__builtin_amdgcn_readlane(dig, src);
}

}  // namespace cobs
