// One 64-key tile of exact softmax attention for a whole GQA group (gfx950),
// shared by the decode and prefill attention kernels.
//
// S = K Q^T is a 64x16 tile computed with v_mfma_f32_16x16x32_bf16 (keys on the
// M side, the group's heads on the N side, head_dim as the contraction), so each
// lane owns one head and a fixed set of 16 keys; the probabilities it holds are
// exactly the B operand of O^T = V^T P^T, so P never leaves registers.  V is
// staged in LDS row-major (padded so the transposed reads are conflict-free) and
// read as the A operand (bf16: with gfx950's transposing LDS read).  K is loaded straight into the MFMA layout.  fp32
// inputs use v_mfma_f32_16x16x4_f32 with the same lane layout.  The softmax is
// online, in the log2 domain.  The steps are separate so that a caller walking
// several tiles can issue the next tile's K loads once the scores are formed and
// its V loads once V is staged, overlapping memory with the softmax and P V.
#pragma once
#include "cobs_device.h"

namespace cobs {

template <typename E, int D>
struct AttnTiling {
  static constexpr int kEpl = E::kPer16;                  // elements per 16-byte chunk
  static constexpr int kChunks = D * E::kBytes / 64;      // 16-byte chunks per lane per key row
  static constexpr int kLanesPerRow = D * E::kBytes / 16;
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  static constexpr int kLoads = kBlock / kRowsPerLoad;    // V staging loads per lane
  // LDS row stride (elements): bf16 rows 8 banks apart for the transposing reads,
  // fp32 rows one bank apart for the column reads
  static constexpr int kRowStride = E::kBytes == 2 ? D + 16 : D + 4;
  static constexpr int kDt = D / 16;                      // 16-wide output column tiles
};

template <typename E, int D>
constexpr size_t attn_lds_bytes(int waves) {
  using T = AttnTiling<E, D>;
  const size_t stage = (size_t)waves * kBlock * T::kRowStride * E::kBytes;
  const size_t merge = (size_t)waves * 16 * (D + 2) * sizeof(float);
  return stage > merge ? stage : merge;
}

// Registers of one 64-key tile in flight: K in the MFMA A layout, V rows as
// loaded (for LDS staging).
template <typename E, int D>
struct TileRegs {
  u32x4 kf[4][AttnTiling<E, D>::kChunks];
  u32x4 vf[AttnTiling<E, D>::kLoads];
};

// Issue the K loads of rows [0, nvalid) of Kt (row stride D elements; rows past
// nvalid repeat the last valid row and are masked in the softmax).
template <typename E, int D>
__device__ __forceinline__ void tile_load_k(const typename E::storage* __restrict__ Kt, int nvalid,
                                            TileRegs<E, D>& r) {
  using T = AttnTiling<E, D>;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = min(16 * t + n, nvalid - 1);
#pragma unroll
    for (int c = 0; c < T::kChunks; ++c) r.kf[t][c] = ld16(Kt + (size_t)row * D + (4 * c + g) * T::kEpl);
  }
}

template <typename E, int D>
__device__ __forceinline__ void tile_load_v(const typename E::storage* __restrict__ Vt, int nvalid,
                                            TileRegs<E, D>& r) {
  using T = AttnTiling<E, D>;
  const int lane = threadIdx.x & 63;
  const int col = (lane % T::kLanesPerRow) * T::kEpl, r0 = lane / T::kLanesPerRow;
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    const int row = min(T::kRowsPerLoad * i + r0, nvalid - 1);
    r.vf[i] = ld16(Vt + (size_t)row * D + col);
  }
}

// S = K Q^T : s[t][i] = q_n . k_{16t + 4g + i}
template <typename E, int D>
__device__ __forceinline__ void tile_scores(const TileRegs<E, D>& r, const u32x4 (&qf)[AttnTiling<E, D>::kChunks],
                                            f32x4 (&s)[4]) {
  constexpr int NCH = AttnTiling<E, D>::kChunks;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (E::kBytes == 2) {
        a = mfma_bf16_16x16x32(r.kf[t][c], qf[c], a);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) a = mfma_f32_16x16x4(__uint_as_float(r.kf[t][c][e]), __uint_as_float(qf[c][e]), a);
      }
    }
    s[t] = a;
  }
}

// V rows into this wave's LDS slice (row-major, padded).
template <typename E, int D>
__device__ __forceinline__ void tile_stage_v(const TileRegs<E, D>& r, typename E::storage* lds) {
  using T = AttnTiling<E, D>;
  const int lane = threadIdx.x & 63;
  const int col = (lane % T::kLanesPerRow) * T::kEpl, r0 = lane / T::kLanesPerRow;
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    st16(lds + (T::kRowsPerLoad * i + r0) * T::kRowStride + col, r.vf[i]);    // 16-byte aligned rows
  }
}

// Online softmax of the tile's scores (log2 domain; lane owns head n) and
// O^T += V^T P^T from the staged V.  l_run is the head's whole running sum in
// every lane of its column (bf16: from the same rounded P as the numerator, as one
// more MFMA output tile with an all-ones A operand).
template <typename E, int D>
__device__ __forceinline__ void tile_softmax_pv(f32x4 (&acc_s)[4], int nvalid, float scale_log2,
                                                const typename E::storage* lds, float& m_run, float& l_run,
                                                f32x4 (&acc_o)[AttnTiling<E, D>::kDt]) {
  using T = AttnTiling<E, D>;
  constexpr int SV = T::kRowStride;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  // max of the raw scores over the tile's valid keys (no mask on a full tile); the
  // softmax runs in log2 units, x = s * scale_log2
  float mt = -INFINITY;
  if (nvalid == kBlock) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, acc_s[t][i]);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * t + 4 * g + i;
        const float x = (key < nvalid) ? acc_s[t][i] : -INFINITY;
        acc_s[t][i] = x;
        mt = fmaxf(mt, x);
      }
    }
  }
  mt = fmaxf(mt, shfl_xor_f(mt, 16));
  mt = fmaxf(mt, shfl_xor_f(mt, 32));
  const float m_new = fmaxf(m_run, mt * scale_log2);
  const float corr = fast_exp2(m_run - m_new);     // 0 when m_run = -inf
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_s[t][i] = fast_exp2(fmaf(acc_s[t][i], scale_log2, -m_new));
  }
  l_run *= corr;
  m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < T::kDt; ++dt) acc_o[dt] *= corr;

  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): V stores visible to this wave
  __builtin_amdgcn_wave_barrier();

  if constexpr (E::kBytes == 2) {
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    f32x4 lt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 pb;
      pb[0] = pack_bf16x2(acc_s[2 * s][0], acc_s[2 * s][1]);
      pb[1] = pack_bf16x2(acc_s[2 * s][2], acc_s[2 * s][3]);
      pb[2] = pack_bf16x2(acc_s[2 * s + 1][0], acc_s[2 * s + 1][1]);
      pb[3] = pack_bf16x2(acc_s[2 * s + 1][2], acc_s[2 * s + 1][3]);
      // A operand of lane (n, g): V[kb + j][16 dt + n], kb = 32s + 16h + 4g, j = 0..3.
      // ds_read_b64_tr_b16 over 16 lanes returns to lane 4a + b the b-th 16-bit
      // element of the rows read by lanes a, a + 4, a + 8, a + 12, so lane (n, g)
      // reads row kb + n/4, columns 16 dt + 4(n%4) .. +3.
      const uint16_t* vl = reinterpret_cast<const uint16_t*>(lds);
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
      for (int dt = 0; dt < T::kDt; ++dt) {
        u32x4 va;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint16_t* src = vl + (32 * s + 16 * h + 4 * g + (n >> 2)) * SV + 16 * dt + 4 * (n & 3);
          const uint2 w = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
          va[2 * h] = w.x;
          va[2 * h + 1] = w.y;
        }
        acc_o[dt] = mfma_bf16_16x16x32(va, pb, acc_o[dt]);
      }
      lt = mfma_bf16_16x16x32(ones, pb, lt);
    }
    l_run += lt[0];
  } else {
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) psum += acc_s[t][i];
    psum += shfl_xor_f(psum, 16);
    psum += shfl_xor_f(psum, 32);
    l_run += psum;
    const float* vl = reinterpret_cast<const float*>(lds);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * t + 4 * g + i;
#pragma unroll
        for (int dt = 0; dt < T::kDt; ++dt)
          acc_o[dt] = mfma_f32_16x16x4(vl[key * SV + 16 * dt + n], acc_s[t][i], acc_o[dt]);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();      // LDS slice reused by the next tile
}

// One whole 64-key tile: rows [0, nvalid) of Kt / Vt (row stride D elements).
template <typename E, int D>
__device__ __forceinline__ void attend_tile(const typename E::storage* __restrict__ Kt,
                                            const typename E::storage* __restrict__ Vt, int nvalid,
                                            const u32x4 (&qf)[AttnTiling<E, D>::kChunks],
                                            float scale_log2, typename E::storage* lds,
                                            float& m_run, float& l_run,
                                            f32x4 (&acc_o)[AttnTiling<E, D>::kDt]) {
  TileRegs<E, D> r;
  tile_load_k<E, D>(Kt, nvalid, r);
  tile_load_v<E, D>(Vt, nvalid, r);
  f32x4 s[4];
  tile_scores<E, D>(r, qf, s);
  tile_stage_v<E, D>(r, lds);
  tile_softmax_pv<E, D>(s, nvalid, scale_log2, lds, m_run, l_run, acc_o);
}

}  // namespace cobs
