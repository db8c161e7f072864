// Per-block key summaries and pooled tokens (gfx950).
//
// COBS (gist.science explainer, Technisches Resuemee 2.2-2.3): each block of 64
// keys is summarised, independently of any query, by its mean key (kappa_1) and a
// compressed form of its key covariance (kappa_2).  The diagonal form stores the
// per-coordinate variance (1/n_b normalisation).  The compressed branch of NSA
// (Janus issue #181, compression path) attends over mean-pooled tokens: the mean
// of 32 consecutive keys (values) every 16 positions.
//
// One wavefront reduces one block of one (sequence, kv-head) and one tensor (keys:
// mean, variance, pooled keys; values: pooled values), so a block's rows take 64
// registers and three waves share a SIMD; a workgroup takes four consecutive
// blocks.  Every 16-byte load instruction reads 1 KiB of contiguous rows, the
// block stays in registers for the two-pass variance, and row sums are reduced
// with lane shuffles.  Pooled token j = (chunk_j + chunk_{j+1}) / 32 where chunk_c
// is the sum of rows [16c, 16c+16): a token across two blocks of the workgroup
// takes the first block's last chunk from LDS; the one after the workgroup's last
// block reads that block's first chunk again (the halo, 1/16 of the rows).
#include "cobs_device.h"
#include "cobs_launch.h"

namespace cobs {

template <typename E, int D>
struct RowTiling {
  static constexpr int kLanesPerRow = D * E::kBytes / 16;     // lanes covering one row
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;   // rows per load instruction
  static constexpr int kLoads = kBlock / kRowsPerLoad;        // load instructions per block
  static constexpr int kEpl = E::kPer16;                      // elements per lane per load
  static_assert(kLanesPerRow >= 8 && kLanesPerRow <= 32, "unsupported row width");
  static_assert(16 % kRowsPerLoad == 0, "a 16-row chunk must be whole loads");
};

// Sum over the lanes that share a column chunk (xor over the row-group bits).
template <int kLanesPerRow>
__device__ __forceinline__ float reduce_rows(float v) {
#pragma unroll
  for (int m = kLanesPerRow; m < kWave; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}

template <typename E, int D>
__device__ __forceinline__ void store_pooled(typename E::storage* dst, const float* v) {
  constexpr int kEpl = E::kPer16;
  if constexpr (E::kBytes == 2) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = f32_to_bf16_bits(v[2 * e]) | (f32_to_bf16_bits(v[2 * e + 1]) << 16);
    st16(dst, w);
  } else {
    f32x4 w;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) w[e] = v[e];
    st_f32x4(reinterpret_cast<float*>(dst), w);
  }
}

// Store this lane's EPL mean columns: fp32, or rounded to bf16 (nearest, ties to
// even) for the compressed storage.
template <int EPL>
__device__ __forceinline__ void store_mean(void* mu_u, bool mu_bf16, int b, int D, int col, const float* mean) {
  if (mu_bf16) {
    uint16_t* dst = static_cast<uint16_t*>(mu_u) + (size_t)b * D + col;
    uint32_t w[EPL / 2];
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e) w[e] = f32_to_bf16_bits(mean[2 * e]) | (f32_to_bf16_bits(mean[2 * e + 1]) << 16);
    if constexpr (EPL == 8) st16(dst, u32x4{w[0], w[1], w[2], w[3]});
    else *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
  } else {
    float* dst = static_cast<float*>(mu_u) + (size_t)b * D + col;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) st_f32x4(dst + e, f32x4{mean[e], mean[e + 1], mean[e + 2], mean[e + 3]});
  }
}

// Lane partial sums of chunk q = rows [16q, 16q+16) of a block held as loaded.
template <typename E, int D>
__device__ __forceinline__ void chunk_partials(const u32x4 (&x)[RowTiling<E, D>::kLoads], float (&part)[4][E::kPer16]) {
  using T = RowTiling<E, D>;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int e = 0; e < T::kEpl; ++e) {
      float a = 0.f;
#pragma unroll
      for (int i = q * 16 / T::kRowsPerLoad; i < (q + 1) * 16 / T::kRowsPerLoad; ++i) a += E::get(x[i], e);
      part[q][e] = a;
    }
  }
}

constexpr int kDiagWaves = 4;        // consecutive blocks per build workgroup, one per wave

template <typename E, int D>
__global__ __launch_bounds__(64 * kDiagWaves, 2) void k_build_diag(
    const int32_t* __restrict__ seq_lens, int max_len, int nb_max, int nc_max,
    const typename E::storage* __restrict__ K, const typename E::storage* __restrict__ V,
    void* __restrict__ mu, float* __restrict__ var,
    typename E::storage* __restrict__ kc, typename E::storage* __restrict__ vc,
    int want_var, int want_pool, int mu_bf16) {
  using T = RowTiling<E, D>;
  constexpr int LPR = T::kLanesPerRow, RPL = T::kRowsPerLoad, NL = T::kLoads, EPL = T::kEpl;
  __shared__ float last_chunk[kDiagWaves][D];   // each wave's rows [48, 64) summed, for its neighbour
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cc = lane % LPR;          // column chunk: columns [cc*EPL, cc*EPL+EPL)
  const int rg = lane / LPR;          // row group: rows rg, rg+RPL, ...
  const int hkv = gridDim.y;
  const int head = blockIdx.y, seq = blockIdx.z;
  // With pooled tokens, even workgroups take the keys (mean, variance, pooled keys)
  // and odd ones the values (pooled values) of the same run of blocks.
  const bool is_v = want_pool && (blockIdx.x & 1);
  const int run = want_pool ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;
  const int L = seq_lens[seq];
  const int nb = (L + kBlock - 1) / kBlock;
  if (run * kDiagWaves >= nb) return;           // the whole workgroup
  const int b = run * kDiagWaves + wave;
  const bool active = b < nb;
  const int nc = (want_pool && L >= 32) ? (L - 32) / 16 + 1 : 0;

  const size_t unit = (size_t)seq * hkv + head;
  const typename E::storage* X = (is_v ? V : K) + unit * (size_t)max_len * D;
  void* mu_u = mu_bf16 ? (void*)(static_cast<uint16_t*>(mu) + unit * (size_t)nb_max * D)
                       : (void*)(static_cast<float*>(mu) + unit * (size_t)nb_max * D);
  float* var_u = var ? var + unit * (size_t)nb_max * D : nullptr;
  typename E::storage* xc_u = want_pool ? (is_v ? vc : kc) + unit * (size_t)nc_max * D : nullptr;

  float ch[4][EPL];                   // sums of the block's four 16-row chunks
  if (active) {
    u32x4 x[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int r = min(b * kBlock + i * RPL + rg, L - 1);
      x[i] = ld16(X + (size_t)r * D + cc * EPL);
    }
    const int nrows = min(kBlock, L - b * kBlock);
    if (nrows < kBlock) {             // the last block of a sequence: rows past its end count as zero
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (i * RPL + rg >= nrows) x[i] = u32x4{0u, 0u, 0u, 0u};
    }
    float part[4][EPL];
    chunk_partials<E, D>(x, part);
    if (!is_v) {
      float mean[EPL];
      const float inv_n = 1.0f / (float)nrows;
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        mean[e] = reduce_rows<LPR>((part[0][e] + part[1][e]) + (part[2][e] + part[3][e])) * inv_n;
      if (rg == 0) store_mean<EPL>(mu_u, mu_bf16 != 0, b, D, cc * EPL, mean);
      if (want_var) {
        // unpack the raw rows again (keeping all 64 rows unpacked since the sums
        // would double the registers this wave holds)
#pragma unroll
        for (int i = 0; i < NL; ++i) asm volatile("" : "+v"(x[i]));
        float sq[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) sq[e] = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float ok = (i * RPL + rg < nrows) ? 1.f : 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float dlt = (E::get(x[i], e) - mean[e]) * ok;
            sq[e] = fmaf(dlt, dlt, sq[e]);
          }
        }
        float v[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = reduce_rows<LPR>(sq[e]) * inv_n;
        if (rg == 1 % RPL) {
          float* dst = var_u + (size_t)b * D + cc * EPL;
#pragma unroll
          for (int e = 0; e < EPL; e += 4) st_f32x4(dst + e, f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]});
        }
      }
    }
    if (want_pool) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) ch[q][e] = reduce_rows<LPR>(part[q][e]);
      }
      // pooled token c = 4b + q - 1 spans chunk q - 1 and chunk q of this block (q = 1..3)
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const int c = 4 * b + q - 1;
        if (c < nc) {
          float t[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) t[e] = (ch[q - 1][e] + ch[q][e]) * (1.0f / 32.0f);
          if (rg == q % RPL) store_pooled<E, D>(xc_u + (size_t)c * D + cc * EPL, t);
        }
      }
      if (rg == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) last_chunk[wave][cc * EPL + e] = ch[3][e];
      }
    }
  }
  if (!want_pool) return;
  __syncthreads();
  if (!active) return;
  // token 4b - 1 spans the previous block's last chunk and this block's first: the
  // previous wave's sums from LDS; the first wave's is emitted by the workgroup
  // before, whose last wave reads this block's first 16 rows once more (the halo)
  if (wave > 0) {
    const int c = 4 * b - 1;
    if (c < nc) {
      float t[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) t[e] = (last_chunk[wave - 1][cc * EPL + e] + ch[0][e]) * (1.0f / 32.0f);
      if (rg == 0) store_pooled<E, D>(xc_u + (size_t)c * D + cc * EPL, t);
    }
  }
  if (wave == kDiagWaves - 1) {
    const int c = 4 * b + 3;
    if (c < nc) {   // then rows [64(b+1), 64(b+1) + 16) are all < L
      const int row0 = (b + 1) * kBlock;
      float a[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a[e] = 0.f;
#pragma unroll
      for (int i = 0; i < 16 / RPL; ++i) {
        const u32x4 xh = ld16(X + (size_t)(row0 + i * RPL + rg) * D + cc * EPL);
#pragma unroll
        for (int e = 0; e < EPL; ++e) a[e] += E::get(xh, e);
      }
      float t[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) t[e] = (ch[3][e] + reduce_rows<LPR>(a[e])) * (1.0f / 32.0f);
      if (rg == 0) store_pooled<E, D>(xc_u + (size_t)c * D + cc * EPL, t);
    }
  }
}

// Incremental update after tokens are appended (positions [L_old, L_new) of each
// sequence are new): every block holding a new position gets its mean and
// diagonal variance recomputed from its keys, and every pooled token whose 32
// rows become complete is emitted; nothing else is written.  One wave walks the
// touched blocks b = L_old/64 + blockIdx.x, + gridDim.x, ...; pooled token c is
// emitted by the wave of the block holding its last row 16c + 31.
template <typename E, int D>
__global__ __launch_bounds__(64) void k_append_diag(
    const int32_t* __restrict__ old_lens, const int32_t* __restrict__ new_lens, int max_len, int nb_max,
    int nc_max, const typename E::storage* __restrict__ K, const typename E::storage* __restrict__ V,
    void* __restrict__ mu, float* __restrict__ var, typename E::storage* __restrict__ kc,
    typename E::storage* __restrict__ vc, int want_pool, int mu_bf16) {
  using T = RowTiling<E, D>;
  constexpr int LPR = T::kLanesPerRow, RPL = T::kRowsPerLoad, NL = T::kLoads, EPL = T::kEpl;
  const int lane = threadIdx.x;
  const int cc = lane % LPR, rg = lane / LPR;
  const int hkv = gridDim.y;
  const int head = blockIdx.y, seq = blockIdx.z;
  const int L0 = old_lens[seq], L = new_lens[seq];
  const size_t unit = (size_t)seq * hkv + head;
  const typename E::storage* Ku = K + unit * (size_t)max_len * D;
  const typename E::storage* Vu = V + unit * (size_t)max_len * D;
  void* mu_u = mu_bf16 ? (void*)(static_cast<uint16_t*>(mu) + unit * (size_t)nb_max * D)
                       : (void*)(static_cast<float*>(mu) + unit * (size_t)nb_max * D);
  float* var_u = var ? var + unit * (size_t)nb_max * D : nullptr;
#pragma unroll 1
  for (int b = L0 / kBlock + blockIdx.x; b * kBlock < L; b += gridDim.x) {
    const int row0 = b * kBlock;
    const int nrows = min(kBlock, L - row0);
    u32x4 xk[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) xk[i] = ld16(Ku + (size_t)min(row0 + i * RPL + rg, L - 1) * D + cc * EPL);
    float sum[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float ok = (i * RPL + rg < nrows) ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sum[e] += ok * E::get(xk[i], e);
    }
    float mean[EPL];
    const float inv_n = 1.0f / (float)nrows;
#pragma unroll
    for (int e = 0; e < EPL; ++e) mean[e] = reduce_rows<LPR>(sum[e]) * inv_n;
    if (rg == 0) store_mean<EPL>(mu_u, mu_bf16 != 0, b, D, cc * EPL, mean);
    if (var_u) {
      float sq[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) sq[e] = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float ok = (i * RPL + rg < nrows) ? 1.f : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float dlt = E::get(xk[i], e) - mean[e];
          sq[e] += ok * dlt * dlt;
        }
      }
      float v[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = reduce_rows<LPR>(sq[e]) * inv_n;
      if (rg == 1 % RPL) {
        float* dst = var_u + (size_t)b * D + cc * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4) st_f32x4(dst + e, f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]});
      }
    }
    if (want_pool) {
      // pooled tokens c with last row 16c+31 in [max(row0, L0), min(row0+64, L)): newly complete here
      const int lo = max(row0, L0), hi = min(row0 + kBlock, L);
      const int c_lo = max(0, (lo - 31 + 15) / 16);
      const int c_hi = hi >= 32 ? (hi - 32) / 16 + 1 : 0;       // 16c + 31 <= hi - 1
      typename E::storage* kc_u = kc + unit * (size_t)nc_max * D;
      typename E::storage* vc_u = vc + unit * (size_t)nc_max * D;
#pragma unroll 1
      for (int c = c_lo; c < c_hi; ++c) {
        float a[EPL], w[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) a[e] = w[e] = 0.f;
#pragma unroll
        for (int i = 0; i < 32 / RPL; ++i) {
          const int r = 16 * c + i * RPL + rg;               // r <= 16c + 31 < L
          const u32x4 xa = ld16(Ku + (size_t)r * D + cc * EPL);
          const u32x4 xb = ld16(Vu + (size_t)r * D + cc * EPL);
#pragma unroll
          for (int e = 0; e < EPL; ++e) { a[e] += E::get(xa, e); w[e] += E::get(xb, e); }
        }
        float tk[EPL], tv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          tk[e] = reduce_rows<LPR>(a[e]) * (1.0f / 32.0f);
          tv[e] = reduce_rows<LPR>(w[e]) * (1.0f / 32.0f);
        }
        if (rg == 0) store_pooled<E, D>(kc_u + (size_t)c * D + cc * EPL, tk);
        if (rg == 1 % RPL) store_pooled<E, D>(vc_u + (size_t)c * D + cc * EPL, tv);
      }
    }
  }
}

template <typename E, int D>
static hipError_t launch_diag(const BuildArgs& a) {
  const int runs = (a.nb_max + kDiagWaves - 1) / kDiagWaves;
  dim3 grid(a.kc != nullptr ? 2 * runs : runs, a.hkv, a.batch);
  hipLaunchKernelGGL((k_build_diag<E, D>), grid, dim3(64 * kDiagWaves), 0, a.stream,
                     a.seq_lens, a.max_len, a.nb_max, a.nc_max,
                     (const typename E::storage*)a.K, (const typename E::storage*)a.V,
                     a.mu, a.var, (typename E::storage*)a.kc, (typename E::storage*)a.vc,
                     a.var != nullptr ? 1 : 0, a.kc != nullptr ? 1 : 0, a.fp4 ? 1 : 0);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_append(const BuildArgs& a) {
  dim3 grid(a.touch_blocks, a.hkv, a.batch);
  hipLaunchKernelGGL((k_append_diag<E, D>), grid, dim3(64), 0, a.stream, a.old_lens, a.seq_lens, a.max_len,
                     a.nb_max, a.nc_max, (const typename E::storage*)a.K, (const typename E::storage*)a.V,
                     a.mu, a.var, (typename E::storage*)a.kc, (typename E::storage*)a.vc, a.kc != nullptr ? 1 : 0,
                     a.fp4 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_append_diag(const BuildArgs& a) {
  if (a.bf16) return a.head_dim == 128 ? launch_append<EltBF16, 128>(a) : launch_append<EltBF16, 64>(a);
  return a.head_dim == 128 ? launch_append<EltF32, 128>(a) : launch_append<EltF32, 64>(a);
}

hipError_t launch_build_diag(const BuildArgs& a) {
  if (a.bf16) {
    if (a.head_dim == 128) return launch_diag<EltBF16, 128>(a);
    return launch_diag<EltBF16, 64>(a);
  }
  if (a.head_dim == 128) return launch_diag<EltF32, 128>(a);
  return launch_diag<EltF32, 64>(a);
}

}  // namespace cobs
