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

// Linear weights scale*q of head n of the group whose first head's query starts
// at q_base (zero for columns n >= G).  The diagonal quadratic weight alpha/2
// scale^2 q^2 is formed from them inside the contraction, which keeps one set
// of weight registers.
template <typename E, int D, int KIND>
__device__ __forceinline__ void score_weights(const void* Q, size_t q_base, int n, int g, int G, float scale,
                                              float (&wlin)[D / 16][4]) {
  const bool hv = n < G;
  const size_t qoff = q_base + (size_t)(hv ? n : 0) * D;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    float q4[4];
    load_q4<E>(Q, qoff + 16 * u + 4 * g, q4);
#pragma unroll
    for (int c = 0; c < 4; ++c) wlin[u][c] = hv ? scale * q4[c] : 0.f;
  }
}

// Query weights of one wave, in B-operand layout.  lin: scale * q (fp32 MFMA);
// quad: scale * P q (subspace kinds).  For the compressed kinds with bf16 queries
// the contraction runs on v_mfma_f32_16x16x32_bf16 instead: lane (n, g)'s eight
// k-slots of chunk j are columns 16u + 4g + c for u = 2j, 2j+1 (the columns the
// compressed storage keeps together per lane), qb holds q in that order (bf16,
// exact), qh + ql the two-part bf16 split of scale * P q.  Members a kind does not
// use are never written and cost no registers.
template <int D>
struct ScoreW {
  float lin[D / 16][4];
  float quad[D / 16][4];
  u32x4 qb[D / 32];
  u32x4 qh[D / 32], ql[D / 32];
  u32x4 q2h[D / 32], q2l[D / 32];     // diagonal kind, bf16 queries: q^2 as exact hi + lo bf16 parts
};

template <int D>
__device__ __forceinline__ void score_weights_bf16(const void* Q, size_t q_base, int n, int g, int G,
                                                   u32x4 (&qb)[D / 32]) {
  const bool hv = n < G;
  const uint16_t* qh = static_cast<const uint16_t*>(Q) + q_base + (size_t)(hv ? n : 0) * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const uint2 a = *reinterpret_cast<const uint2*>(qh + 32 * j + 4 * g);
    const uint2 b = *reinterpret_cast<const uint2*>(qh + 32 * j + 16 + 4 * g);
    qb[j] = hv ? u32x4{a.x, a.y, b.x, b.y} : u32x4{0u, 0u, 0u, 0u};
  }
}

// scale * P q (fp32, [u][c] layout) as two bf16 parts in the chunk order above.
template <int D>
__device__ __forceinline__ void split_bf16(const float (&w)[D / 16][4], u32x4 (&hi)[D / 32], u32x4 (&lo)[D / 32]) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {           // slots 2h, 2h+1: u = 2j + h/2, c = 2(h%2), 2(h%2)+1
      const float a = w[2 * j + h / 2][2 * (h % 2)], b = w[2 * j + h / 2][2 * (h % 2) + 1];
      const uint32_t ah = f32_to_bf16_bits(a), bh = f32_to_bf16_bits(b);
      const uint32_t al = f32_to_bf16_bits(a - __uint_as_float(ah << 16));
      const uint32_t bl = f32_to_bf16_bits(b - __uint_as_float(bh << 16));
      hi[j][h] = ah | (bh << 16);
      lo[j][h] = al | (bl << 16);
    }
  }
}

// Score kinds: 0 diagonal, 1 rank-r fp32, 2 exact masses (no summaries), 3 rank-r
// in the compressed storage (bf16 mean; FP4 E2M1 vectors with one E8M0 exponent
// per 32 entries), 4 and 5 the rank-r kinds 1 and 3 with the vectors in a query
// subspace (length vlen = the subspace dimension rounded up to 32; the quadratic
// term contracts them with scale * P q instead of scale * q).  In the compressed
// storage a vector of length n has its entry 16u + 4g + c at nibble
// (g * n/16 + u) * 4 + c, so each lane's codes are contiguous.
template <int KIND>
struct Kind {
  static constexpr bool kFp4 = KIND == 3 || KIND == 5;
  static constexpr bool kSub = KIND == 4 || KIND == 5;
  static constexpr bool kRank = KIND == 1 || KIND >= 3;
  static constexpr bool kRankF32 = KIND == 1 || KIND == 4;
  // fp32 rank-r vectors held per scoring round: a group of four takes 128 registers;
  // the subspace kind, which also holds the projected weights, takes two
  static constexpr int kGroupF32 = KIND == 4 ? 2 : 4;
};

// Bytes of one block's compressed record: codes, exponents, padding to 16.
__host__ __device__ constexpr size_t fp4_record_bytes_dev(int rank, int n) {
  return ((size_t)rank * (n / 2 + n / 32) + 15) / 16 * 16;
}

// Summary rows of block row `row` (mean, second-order) for a score kind; vlen is
// the length of a rank-r vector (D without a subspace).
template <int D, int KIND>
__device__ __forceinline__ void summary_rows(const void* mu, const void* so, size_t row, int rank, int vlen,
                                             const void*& mr, const void*& vr) {
  if constexpr (Kind<KIND>::kFp4) {
    mr = static_cast<const uint16_t*>(mu) + row * D;
    vr = static_cast<const uint8_t*>(so) + row * fp4_record_bytes_dev(rank, vlen);
  } else {
    mr = static_cast<const float*>(mu) + row * D;
    vr = static_cast<const float*>(so) + row * (KIND == 0 ? (size_t)D : (size_t)rank * vlen);
  }
}

// Summary rows of one 16-block tile held in registers: this lane's mean columns
// and its second-order columns (the diagonal, or the first kRankGroup scaled
// eigenvectors, further groups fetched while scoring; for the compressed storage
// the bf16 mean and the first kRankGroup vectors' FP4 codes and exponents).
constexpr int kRankGroup = 4;

template <int D, int KIND>
struct SumTile {
  static constexpr bool kF = Kind<KIND>::kFp4;
  f32x4 m4[kF ? 1 : D / 16];
  f32x4 v4[Kind<KIND>::kRankF32 ? Kind<KIND>::kGroupF32 : 1][kF ? 1 : D / 16];
  uint2 mb[kF ? D / 16 : 1];           // bf16 mean columns 16u + 4g .. +3
  u32x4 code[kF ? kRankGroup : 1];     // this lane's vlen/4 codes of each vector of the group
  uint32_t ex[kF ? kRankGroup : 1];    // the vector's vlen/32 exponent bytes
  // subspace kinds: the record's exponent block (a 32-byte window) as loaded; each
  // vector's bytes are cut from it when the tile is scored (sub_tile_exponents)
  u32x4 exw[kF && Kind<KIND>::kSub ? 2 : 1];
};

// 16 bytes from a 4-byte aligned address (one dwordx4 load).
__device__ __forceinline__ u32x4 ld16_a4(const void* p) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

template <int D, int KIND>
__device__ __forceinline__ void sum_tile_load_group(const void* vrow, int r0, int rank, int vlen, int g,
                                                    SumTile<D, KIND>& t) {
  if constexpr (Kind<KIND>::kFp4) {
    const uint8_t* rec = static_cast<const uint8_t*>(vrow);
    // subspace kinds: the exponent block starts 16-aligned at rank * vlen/2 and the
    // record extends at least 16 bytes past it (32 when it holds more than 16 bytes).
    // Every load here is unconditional in its width and address (no branch on the
    // runtime vlen), so no value is moved or cut before it has arrived and the tile's
    // loads stay in flight while the wave scores other tiles.
    if constexpr (Kind<KIND>::kSub) {
      const uint8_t* ep = rec + rank * (vlen / 2);
      t.exw[0] = *reinterpret_cast<const u32x4*>(ep);
      t.exw[1] = *reinterpret_cast<const u32x4*>(ep + (rank * (vlen / 32) > 16 ? 16 : 0));
    }
    // vectors past the rank repeat the last one (loaded, never scored), so a tile
    // always has the same loads in flight
#pragma unroll
    for (int rr = 0; rr < kRankGroup; ++rr) {
      const int r = min(r0 + rr, rank - 1);
      {
        if constexpr (!Kind<KIND>::kSub) {
          const uint8_t* cp = rec + r * (D / 2) + g * (D / 8);
          if constexpr (D == 128) {
            t.code[rr] = *reinterpret_cast<const u32x4*>(cp);
            t.ex[rr] = *reinterpret_cast<const uint32_t*>(rec + rank * (D / 2) + r * (D / 32));
          } else {
            const uint2 c2 = *reinterpret_cast<const uint2*>(cp);
            t.code[rr] = u32x4{c2.x, c2.y, 0u, 0u};
            t.ex[rr] = *reinterpret_cast<const uint16_t*>(rec + rank * (D / 2) + r * (D / 32));
          }
        } else {
          // the lane's vlen/32 code words: one 16-byte load at 4-byte alignment.  Below
          // vlen = 128 it also reads up to 12 bytes that follow the run (the next lane's
          // codes or the exponent block), inside the record for every rank 1-8 and
          // vlen 32, 64, 96; words j >= vlen/32 are never decoded
          t.code[rr] = ld16_a4(rec + r * (vlen / 2) + g * (vlen / 8));
        }
      }
    }
  } else {
    // vectors past the rank and columns past vlen repeat the last ones (loaded, never
    // scored), so a tile always has the same loads in flight
    const float* vr = static_cast<const float*>(vrow);
#pragma unroll
    for (int rr = 0; rr < Kind<KIND>::kGroupF32; ++rr) {
      const int r = min(r0 + rr, rank - 1);
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const int ul = Kind<KIND>::kSub ? min(u, vlen / 16 - 1) : u;
        t.v4[rr][u] = ld_f32x4(vr + r * vlen + 16 * ul + 4 * g);
      }
    }
  }
}

// Issue the loads of one tile (mrow / vrow: this lane's block row).
template <int D, int KIND>
__device__ __forceinline__ void sum_tile_load(const void* mrow, const void* vrow, int rank, int vlen, int g,
                                              bool use_quad, SumTile<D, KIND>& t) {
  if constexpr (Kind<KIND>::kFp4) {
    const uint16_t* mr = static_cast<const uint16_t*>(mrow);
#pragma unroll
    for (int u = 0; u < D / 16; ++u) t.mb[u] = *reinterpret_cast<const uint2*>(mr + 16 * u + 4 * g);
    if (use_quad) sum_tile_load_group<D, KIND>(vrow, 0, rank, vlen, g, t);
  } else {
    const float* mr = static_cast<const float*>(mrow);
#pragma unroll
    for (int u = 0; u < D / 16; ++u) t.m4[u] = ld_f32x4(mr + 16 * u + 4 * g);
    if (use_quad) {
      if constexpr (KIND == 0) {
        const float* vr = static_cast<const float*>(vrow);
#pragma unroll
        for (int u = 0; u < D / 16; ++u) t.v4[0][u] = ld_f32x4(vr + 16 * u + 4 * g);
      } else {
        sum_tile_load_group<D, KIND>(vrow, 0, rank, vlen, g, t);
      }
    }
  }
}

// Subspace kinds: the vlen/32 exponent bytes of vectors r0 .. r0+3 from the loaded
// exponent window (called when the tile is scored, its loads complete).
template <int D, int KIND>
__device__ __forceinline__ void sub_tile_exponents(SumTile<D, KIND>& t, int r0, int vlen) {
  if constexpr (Kind<KIND>::kFp4 && Kind<KIND>::kSub) {
    const int nw = vlen / 32;
    const u32x4 a = t.exw[0], b = t.exw[1];
    auto ew = [&](int i) -> uint32_t {                // word i (0-7) of the 32-byte exponent window
      const u32x4 v = (i & 4) ? b : a;                // selects of values, no indexed memory
      const uint32_t lo = (i & 1) ? v[1] : v[0], hi = (i & 1) ? v[3] : v[2];
      return (i & 2) ? hi : lo;
    };
#pragma unroll
    for (int rr = 0; rr < kRankGroup; ++rr) {
      const int o = (r0 + rr) * nw, wi = o >> 2, sh = 8 * (o & 3);
      const uint32_t lo = ew(wi), hi = ew(wi + 1);
      const uint32_t ex = sh ? (lo >> sh) | (hi << (32 - sh)) : lo;
      t.ex[rr] = nw == 4 ? ex : ex & ((1u << (8 * nw)) - 1u);
    }
  }
}

// 2^(byte - 127) of an E8M0 exponent byte, as the fp32 scale operand of the gfx950
// scaled FP4 conversion (which multiplies by 2 to the scale's biased exponent - 127).
__device__ __forceinline__ float e8m0_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The compressed kinds with bf16 queries on the bf16 MFMA: the bf16 mean and the
// decoded FP4 entries (E2M1 times a power of two, exact in bf16) against q in bf16,
// products exact and accumulated in fp32; scale is applied to the sums.
template <int D, int KIND>
__device__ __forceinline__ f32x4 sum_tile_score_bf16(SumTile<D, KIND>& t, const void* vrow, int rank, int vlen, int g,
                                                     bool use_quad, float alpha, float scale, const ScoreW<D>& W) {
  constexpr int NJ = D / 32;
  constexpr bool kSub = Kind<KIND>::kSub;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    acc = mfma_bf16_16x16x32(u32x4{t.mb[2 * j].x, t.mb[2 * j].y, t.mb[2 * j + 1].x, t.mb[2 * j + 1].y}, W.qb[j],
                             acc);
  acc *= scale;
  if (!use_quad) return acc;
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int r0 = 0; r0 < rank; r0 += kRankGroup) {
    if (r0 > 0) sum_tile_load_group<D, KIND>(vrow, r0, rank, vlen, g, t);
    sub_tile_exponents<D, KIND>(t, r0, vlen);
#pragma unroll
    for (int rr = 0; rr < kRankGroup; ++rr) {
      if (r0 + rr < rank) {
        f32x4 pr = {0.f, 0.f, 0.f, 0.f}, pr2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (kSub && 32 * j >= vlen) break;
          // chunk j: the eight codes of word j, all in exponent group j
          const uint32_t w = t.code[rr][j];
          const float sc = e8m0_scale((t.ex[rr] >> (8 * j)) & 0xFFu);
          const u32x4 a = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3))};
          if constexpr (kSub) {
            pr = mfma_bf16_16x16x32(a, W.qh[j], pr);
            pr2 = mfma_bf16_16x16x32(a, W.ql[j], pr2);
          } else {
            pr = mfma_bf16_16x16x32(a, W.qb[j], pr);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dd = kSub ? pr[i] + pr2[i] : scale * pr[i];
          acc2[i] += 0.5f * alpha * dd * dd;
        }
      }
    }
  }
  return acc + acc2;
}

// Scores (without ln n_b) of the tile's 16 blocks for the group's heads from the
// loaded rows.  Linear and quadratic terms are independent MFMA chains.  wlin are
// the linear weights scale * q; wq the weights the rank-r vectors are contracted
// with (wlin, or scale * P q for the subspace kinds).
template <int D, int KIND>
__device__ __forceinline__ f32x4 sum_tile_score(SumTile<D, KIND>& t, const void* vrow, int rank, int vlen, int g,
                                                bool use_quad, float alpha, const float (&wlin)[D / 16][4],
                                                const float (&wq)[D / 16][4]) {
  constexpr int NU = D / 16;
  constexpr bool kSub = Kind<KIND>::kSub;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NU; ++u) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float m;
      if constexpr (Kind<KIND>::kFp4) {
        const uint32_t w = (c < 2) ? t.mb[u].x : t.mb[u].y;
        m = (c & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
      } else {
        m = t.m4[u][c];
      }
      acc = mfma_f32_16x16x4(m, wlin[u][c], acc);
    }
  }
  if (!use_quad) return acc;
  if constexpr (KIND == 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float w = wlin[u][c];
        acc2 = mfma_f32_16x16x4(t.v4[0][u][c], 0.5f * alpha * w * w, acc2);   // alpha/2 scale^2 q^2
      }
    }
  } else if constexpr (Kind<KIND>::kFp4) {
    // (v_i . q)^2 with v_i decoded on the fly by the hardware FP4 conversion: entry
    // 16u + 4g + c is nibble u*4 + c of this lane's codes, scaled by the exponent of
    // group u/2 of this lane's block (the scale must be applied on the A side: an
    // output row belongs to another lane's block)
#pragma unroll 1
    for (int r0 = 0; r0 < rank; r0 += kRankGroup) {
      if (r0 > 0) sum_tile_load_group<D, KIND>(vrow, r0, rank, vlen, g, t);
      sub_tile_exponents<D, KIND>(t, r0, vlen);
#pragma unroll
      for (int rr = 0; rr < kRankGroup; ++rr) {
        if (r0 + rr < rank) {
          f32x4 pr = {0.f, 0.f, 0.f, 0.f}, pr2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            if (kSub && 16 * u >= vlen) break;
            // codes of columns 16u + 4g + {0,1} and {2,3}: bytes 2(u&1) and 2(u&1)+1 of word u/2;
            // group u/2's exponent (columns 16u + 4g + c share group u/2)
            const uint32_t w = t.code[rr][u >> 1];
            const float sc = e8m0_scale((t.ex[rr] >> (8 * (u >> 1))) & 0xFFu);
            f32x2 lo, hi;
            if (u & 1) {
              lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
              hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
            } else {
              lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
              hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
            }
            const float v[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if (u & 1) pr2 = mfma_f32_16x16x4(v[c], wq[u][c], pr2);
              else pr = mfma_f32_16x16x4(v[c], wq[u][c], pr);
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
  } else {
    // (v_i . q)^2 for each scaled eigenvector v_i: the projection is a linear MFMA
    // chain with the weights, squared on the VALU
#pragma unroll 1
    for (int r0 = 0; r0 < rank; r0 += Kind<KIND>::kGroupF32) {
      if (r0 > 0) sum_tile_load_group<D, KIND>(vrow, r0, rank, vlen, g, t);
#pragma unroll
      for (int rr = 0; rr < Kind<KIND>::kGroupF32; ++rr) {
        if (r0 + rr < rank) {
          f32x4 pr = {0.f, 0.f, 0.f, 0.f}, pr2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; u += 2) {
            if (kSub && 16 * u >= vlen) break;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              pr = mfma_f32_16x16x4(t.v4[rr][u][c], wq[u][c], pr);
              pr2 = mfma_f32_16x16x4(t.v4[rr][u + 1][c], wq[u + 1][c], pr2);
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

// Whether a kind runs its contraction on the bf16 MFMA: the compressed kinds and the
// diagonal kind, with bf16 queries.
template <typename E, int KIND>
constexpr bool kBf16Path = E::kBytes == 2 && (Kind<KIND>::kFp4 || KIND == 0);

// x (eight fp32 values, two f32x4) as hi + lo bf16 parts: hi the nearest bf16 of x, lo
// the nearest bf16 of x - hi, so hi + lo keeps 16 of x's 24 significand bits (the
// dropped part is below 2^-16 of |x|).
__device__ __forceinline__ void split_bf16x8(const f32x4& x, const f32x4& y, u32x4& h, u32x4& l) {
  h = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  const float xs[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    l[e] = pack_bf16x2(xs[2 * e] - __uint_as_float(h[e] << 16), xs[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u));
}

// Diagonal kind with bf16 queries on v_mfma_f32_16x16x32_bf16: the tile's fp32 means
// and variances split into hi + lo bf16 parts, q (bf16, exact) and q^2 (exact in fp32,
// 16 significand bits, as an exact hi + lo pair) in the same chunk order (lane (n, g)'s
// eight k-slots of chunk j are columns 16u + 4g + c for u = 2j, 2j+1, the columns its
// fp32 summary loads hold).  Products are exact; sums accumulate in fp32.
template <int D, int KIND>
__device__ __forceinline__ f32x4 sum_tile_score_diag_split(const SumTile<D, KIND>& t, bool use_quad, float alpha,
                                                           float scale, const ScoreW<D>& W) {
  constexpr int NJ = D / 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u32x4 mh, ml;
    split_bf16x8(t.m4[2 * j], t.m4[2 * j + 1], mh, ml);
    acc = mfma_bf16_16x16x32(mh, W.qb[j], acc);
    acc = mfma_bf16_16x16x32(ml, W.qb[j], acc);
  }
  if (use_quad) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 vh, vl;
      split_bf16x8(t.v4[0][2 * j], t.v4[0][2 * j + 1], vh, vl);
      acc2 = mfma_bf16_16x16x32(vh, W.q2h[j], acc2);
      acc2 = mfma_bf16_16x16x32(vh, W.q2l[j], acc2);
      acc2 = mfma_bf16_16x16x32(vl, W.q2h[j], acc2);
      acc2 = mfma_bf16_16x16x32(vl, W.q2l[j], acc2);
    }
  }
  return scale * acc + (0.5f * alpha * scale * scale) * acc2;
}

// The wave's query weights other than the subspace ones (which need the workgroup).
template <typename E, int D, int KIND>
__device__ __forceinline__ void prepare_weights(const void* Q, size_t q_base, int n, int g, int G, float scale,
                                                ScoreW<D>& W) {
  if constexpr (!(kBf16Path<E, KIND> && KIND == 0)) score_weights<E, D, KIND>(Q, q_base, n, g, G, scale, W.lin);
  if constexpr (kBf16Path<E, KIND>) score_weights_bf16<D>(Q, q_base, n, g, G, W.qb);
  if constexpr (kBf16Path<E, KIND> && KIND == 0) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __uint_as_float(W.qb[j][e] << 16), b = __uint_as_float(W.qb[j][e] & 0xFFFF0000u);
        const float a2 = a * a, b2 = b * b;
        W.q2h[j][e] = pack_bf16x2(a2, b2);
        W.q2l[j][e] = pack_bf16x2(a2 - __uint_as_float(W.q2h[j][e] << 16), b2 - __uint_as_float(W.q2h[j][e] & 0xFFFF0000u));
      }
    }
  }
}

// After W.quad holds scale * P q: its bf16 split for the bf16 path.
template <typename E, int D, int KIND>
__device__ __forceinline__ void finish_subspace_weights(ScoreW<D>& W) {
  if constexpr (kBf16Path<E, KIND> && Kind<KIND>::kSub) split_bf16<D>(W.quad, W.qh, W.ql);
}

// Score a loaded tile on the kind's path.
template <typename E, int D, int KIND>
__device__ __forceinline__ f32x4 tile_score(SumTile<D, KIND>& t, const void* vrow, int rank, int vlen, int g,
                                            bool use_quad, float alpha, float scale, const ScoreW<D>& W) {
  if constexpr (kBf16Path<E, KIND> && KIND == 0)
    return sum_tile_score_diag_split<D, KIND>(t, use_quad, alpha, scale, W);
  else if constexpr (kBf16Path<E, KIND>)
    return sum_tile_score_bf16<D, KIND>(t, vrow, rank, vlen, g, use_quad, alpha, scale, W);
  else
    return sum_tile_score<D, KIND>(t, vrow, rank, vlen, g, use_quad, alpha, W.lin,
                                   Kind<KIND>::kSub ? W.quad : W.lin);
}

// Load and score one tile in one step.
template <typename E, int D, int KIND>
__device__ __forceinline__ f32x4 score_tile(const void* mrow, const void* vrow, int rank, int vlen, int g,
                                            bool use_quad, float alpha, float scale, const ScoreW<D>& W) {
  SumTile<D, KIND> t;
  sum_tile_load<D, KIND>(mrow, vrow, rank, vlen, g, use_quad, t);
  return tile_score<E, D, KIND>(t, vrow, rank, vlen, g, use_quad, alpha, scale, W);
}

// Quadratic weights of the subspace kinds, scale * P q, in the B-operand layout:
// wq[u][c] of lane (n, g) = scale * (P q_n)[16u + 4g + c] for column tiles u < vlen/16
// (rows of P at or beyond s are zero).  The contraction over d is an MFMA chain whose
// A operand is P's row 16u + n and whose B operand is the linear weights, so the
// output (rows 16u + 4g + i, column n) lands in exactly this layout.  Column tiles
// are split over `nparts` waves (this one computes u = part, part + nparts, ...) and
// exchanged through `xch` ([D/16][64] f32x4 in LDS) when nparts > 1; the caller
// synchronises the waves between the two halves.
template <int D>
__device__ __forceinline__ void subspace_weights_part(const float* P, int s, int vlen, int part, int nparts, int n,
                                                      int g, const float (&wlin)[D / 16][4], f32x4* xch,
                                                      float (&wq)[D / 16][4]) {
  constexpr int NU = D / 16;
  const int lane = 16 * g + n;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (16 * u >= vlen || u % nparts != part) continue;
    const int row = 16 * u + n;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const f32x4 p4 = row < s ? ld_f32x4(P + (size_t)row * D + 16 * j + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_f32_16x16x4(p4[c], wlin[j][c], acc);
    }
    if (nparts > 1) xch[u * 64 + lane] = acc;
#pragma unroll
    for (int c = 0; c < 4; ++c) wq[u][c] = acc[c];
  }
}

// The same split into a load step and a contraction step, so that a caller can put
// other loads between them: P's rows of the column tiles u = part and part + nparts
// (those below vlen), then scale * P q for them into `xch`; after a barrier every
// wave takes all column tiles with subspace_weights_gather (part = -1).
template <int D>
struct SubspaceRows {
  f32x4 r[2][D / 16];
};

template <int D>
__device__ __forceinline__ void subspace_rows_load(const float* P, int s, int vlen, int part, int nparts, int n,
                                                   int g, SubspaceRows<D>& pr) {
  constexpr int NU = D / 16;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = part + k * nparts, row = 16 * u + n;
    const bool ok = u < NU && 16 * u < vlen && row < s;
#pragma unroll
    for (int j = 0; j < NU; ++j)
      pr.r[k][j] = ok ? ld_f32x4(P + (size_t)row * D + 16 * j + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int D>
__device__ __forceinline__ void subspace_rows_project(const SubspaceRows<D>& pr, int vlen, int part, int nparts,
                                                      int n, int g, const float (&wlin)[D / 16][4], f32x4* xch) {
  constexpr int NU = D / 16;
  const int lane = 16 * g + n;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = part + k * nparts;
    if (u >= NU || 16 * u >= vlen) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NU; ++j) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_f32_16x16x4(pr.r[k][j][c], wlin[j][c], acc);
    }
    xch[u * 64 + lane] = acc;
  }
}

template <int D>
__device__ __forceinline__ void subspace_weights_gather(int vlen, int part, int nparts, int n, int g,
                                                        const f32x4* xch, float (&wq)[D / 16][4]) {
  constexpr int NU = D / 16;
  const int lane = 16 * g + n;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (16 * u >= vlen || u % nparts == part) continue;
    const f32x4 v = xch[u * 64 + lane];
#pragma unroll
    for (int c = 0; c < 4; ++c) wq[u][c] = v[c];
  }
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

// Exclusive prefix sum over the NW waves of a workgroup, in thread order.
template <int NW = 4>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_inclusive_sum(v);
  if (lane == 63) lds_w[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = lds_w[i];
    base += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Top-k of the orderable keys[0, ncand) by a workgroup of NW waves, ties to the
// lower block index (MSB-first 8-bit radix select).  Thread tid owns blocks
// [tid * per, tid * per + per).  Each wave fills a private 256-bin histogram
// (double-buffered across passes, `hist` is [2][NW][256]); after one barrier every
// wave sums the NW histograms and finds the digit itself; the passes stop as soon as the
// bin holding the k-th key is taken whole.  Calls emit(pos, b) for every selected
// block b with its position in ascending block order and returns how many were
// selected (min(top_k, ncand)).
template <int NW = 4, typename Emit>
__device__ __forceinline__ int wg_select_topk(const uint32_t* keys, int ncand, int per, int top_k,
                                              uint32_t* hist, int* scan_w, Emit&& emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b0 = threadIdx.x * per;
  const int e_end = max(0, min(per, ncand - b0));
  const int kk = min(top_k, ncand);
  uint32_t prefix = 0u, hi_mask = 0u;
  int need = kk, eq_bin = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4 && kk > 0; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* hp = hist + (pass & 1) * (NW * 256);
    uint32_t* mine = hp + wave * 256;
    *reinterpret_cast<u32x4*>(&mine[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int e = 0; e < per; ++e) {               // uniform trip count: wave-wide ballots inside
      const uint32_t key = (e < e_end) ? keys[b0 + e] : 0u;
      wave_histogram_add(mine, e < e_end && (key & hi_mask) == prefix, (key >> shift) & 255u);
    }
    __syncthreads();
    u32x4 hb = *reinterpret_cast<const u32x4*>(&hp[4 * lane]);
#pragma unroll
    for (int w = 1; w < NW; ++w) hb += *reinterpret_cast<const u32x4*>(&hp[w * 256 + 4 * lane]);
    prefix |= radix_digit(hb, need, eq_bin) << shift;
    hi_mask |= 255u << shift;
    if (need == eq_bin) break;                    // every key with this prefix is taken
  }
  // taken: (key & hi_mask) > prefix, or == prefix among the first `need` by block index
  int eq_rank = 0;
  if (kk > 0 && need < eq_bin) {                  // a tie straddles the cut: rank the equal keys
    int eq_count = 0;
#pragma unroll 1
    for (int e = 0; e < e_end; ++e) eq_count += ((keys[b0 + e] & hi_mask) == prefix) ? 1 : 0;
    int eq_total;
    eq_rank = block_exclusive_scan<NW>(eq_count, scan_w, &eq_total);
  }
  int take_count = 0;
  if (kk > 0) {
    int r = eq_rank;
#pragma unroll 1
    for (int e = 0; e < e_end; ++e) {
      const uint32_t km = keys[b0 + e] & hi_mask;
      if (km > prefix) ++take_count;
      else if (km == prefix) { take_count += (r < need) ? 1 : 0; ++r; }
    }
  }
  int sel_total;
  const int pos0 = block_exclusive_scan<NW>(take_count, scan_w, &sel_total);
  if (kk > 0) {
    int r = eq_rank, pos = pos0;
#pragma unroll 1
    for (int e = 0; e < e_end; ++e) {
      const uint32_t km = keys[b0 + e] & hi_mask;
      bool tk = km > prefix;
      if (km == prefix) { tk = r < need; ++r; }
      if (tk) emit(pos++, b0 + e);
    }
  }
  return sel_total;
}

}  // namespace cobs
