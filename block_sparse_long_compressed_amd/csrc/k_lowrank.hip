// Rank-r covariance summaries (gfx950).
//
// COBS (gist.science explainer, Technisches Resuemee 2.3, "Low-Rank-
// Faktorisierung"): the within-block key covariance C_b = (1/n) sum_r
// (k_r - mu)(k_r - mu)^T is stored as its top-r eigenvectors scaled by the
// square roots of their eigenvalues, v_i = sqrt(lambda_i) u_i, so that
// sum_i v_i v_i^T is the best rank-r approximation of C_b.
//
// A block holds n <= 64 keys of dimension d = 64 or 128 > n, so the work is
// done on the n x n Gram matrix G = X X^T / n of the centred keys X (same
// non-zero eigenvalues as C_b): if G w = lambda w with |w| = 1, then
// X^T w / sqrt(n) = sqrt(lambda) u.  G is diagonalised by a parallel cyclic
// Jacobi method in fp64 (32 disjoint rotations per round, round-robin pairing,
// rotations accumulated in V), which agrees with a reference fp64 symmetric
// eigensolver to rounding.  One 256-thread workgroup per block; G and V live in
// LDS (2 x 32 KiB).  Eigenvalues <= 0 give v = 0; each v is signed so that its
// largest-magnitude entry is positive.
//
// Query-subspace projection (Technisches Resuemee 2.3, "Subraum-Projektion"):
// with P [s][d] (orthonormal rows spanning the queries' dominant directions) the
// covariance is first projected, C' = P C P^T.  Its Gram matrix is that of the
// projected keys Y = X P^T (formed 16 columns at a time in fp64), and its scaled
// eigenvectors are Y^T w / sqrt(n) = P (X^T w / sqrt(n)), stored with length
// vlen = s rounded up to 32 (zeros beyond s).
#include "cobs_device.h"
#include "cobs_launch.h"
#include "score_common.h"

namespace cobs {

constexpr int kLrThreads = 256;
constexpr int kN = 64;              // Gram size (keys per block)
constexpr int kMaxSweeps = 16;

// Round-robin pairing: round r (0..62), pair k (0..31) -> (p, q), p != q; every
// unordered pair of 0..63 occurs exactly once in 63 rounds.
__device__ __forceinline__ int rr_index(int pos, int r) { return pos == 0 ? 0 : 1 + (pos - 1 + r) % (kN - 1); }

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  const double t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

// FP4 E2M1 code of y (a value already divided by its group scale): the nearest of
// 0, .5, 1, 1.5, 2, 3, 4, 6 (ties to the even code, saturating at 6), sign in bit 3
// (none for zero).  The code is the number of midpoints between neighbouring
// magnitudes that lie below |y|, moved up at an exact midpoint to an even code.
__device__ __forceinline__ uint32_t e2m1_code(double y) {
  const double a = fabs(y);
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  uint32_t c = 0;
  bool tie = false;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    c += (mid[i] < a) ? 1u : 0u;
    tie |= (mid[i] == a);
  }
  if (tie && (c & 1u)) ++c;
  return (c != 0u && y < 0.0) ? (c | 8u) : c;
}

// The compressed record of one block from its rank scaled eigenvectors (fp64, of
// length len, a multiple of 32): per vector len/2 bytes of codes, then per vector
// len/32 exponent bytes, then zero padding to 16 bytes.  Each group of 32 entries
// shares the exponent e = floor(log2 max|v|) - 2 (stored as e + 127, 0 for an
// all-zero group), and entry 16u + 4g + c sits at nibble (g * len/16 + u) * 4 + c
// of its vector, low nibble first, so that a scoring lane reads its columns as one
// contiguous run.
template <int D>
__device__ void quantize_record(const double (*vout)[D], int (*gexp)[D / 32], uint8_t* rec, int rank, int len,
                                int tid) {
  const int NG = len / 32;
  for (int idx = tid; idx < rank * NG; idx += kLrThreads) {
    const int i = idx / NG, q = idx % NG;
    double amax = 0.0;
    for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs(vout[i][32 * q + j]));
    int e = -127;
    if (amax > 0.0) {
      int ex;
      frexp(amax, &ex);                    // amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
      e = max(-127, min(127, ex - 3));
    }
    gexp[i][q] = e;
  }
  __syncthreads();
  const int code_bytes = rank * (len / 2);
  const int total = (int)fp4_record_bytes_dev(rank, len);
  for (int idx = tid; idx < total; idx += kLrThreads) {
    uint32_t byte = 0;
    if (idx < code_bytes) {
      const int i = idx / (len / 2), bb = idx % (len / 2);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int P = 2 * bb + h;                       // nibble position within the vector
        const int g = P / (len / 4), kk = P % (len / 4);
        const int entry = 16 * (kk / 4) + 4 * g + (kk % 4);
        const double y = ldexp(vout[i][entry], -gexp[i][entry / 32]);
        byte |= e2m1_code(y) << (4 * h);
      }
    } else if (idx < code_bytes + rank * NG) {
      const int k = idx - code_bytes;
      byte = (uint32_t)(gexp[k / NG][k % NG] + 127);
    }
    rec[idx] = (uint8_t)byte;
  }
  __syncthreads();
}

template <typename E, int D>
__global__ __launch_bounds__(kLrThreads) void k_build_lowrank(const int32_t* __restrict__ seq_lens,
                                                              const int32_t* __restrict__ old_lens, int max_len,
                                                              int nb_max, int rank,
                                                              const typename E::storage* __restrict__ K,
                                                              void* __restrict__ lowrank, int fp4,
                                                              const float* __restrict__ Psub, int sub_s,
                                                              int vlen) {
  __shared__ double A[kN][kN + 1];      // Gram matrix, diagonalised in place (+1: bank spread)
  // the block's keys (fp32, exact for bf16) until G is built, then the rotations
  __shared__ union { float k[kN][D + 1]; double v[kN][kN + 1]; } kv;
  __shared__ double mu[D];
  __shared__ double cs[kN / 2][2];
  __shared__ int pq[kN / 2][2];
  __shared__ double red[4];
  __shared__ int order[8];
  __shared__ double lam_sel[8];
  __shared__ double vout[8][D];
  __shared__ int gexp[8][D / 32];
  __shared__ __align__(16) uint8_t rec[8 * (D / 2 + D / 32) + 16];
  auto& Vm = kv.v;

  const int tid = threadIdx.x;
  const int hkv = gridDim.y;
  const int head = blockIdx.y, seq = blockIdx.z;
  const int L = seq_lens[seq];
  // full build: block blockIdx.x; incremental update: the blocks holding positions
  // >= old_lens[seq], walked with a stride of the grid width
  const int b_first = (old_lens ? old_lens[seq] / kBlock : 0) + blockIdx.x;
#pragma unroll 1
  for (int b = b_first; b * kBlock < L; b += gridDim.x) {
  const int row0 = b * kBlock;
  const int n = min(kBlock, L - row0);
  const size_t unit = (size_t)seq * hkv + head;
  const typename E::storage* Kb = K + (unit * (size_t)max_len + row0) * D;
  auto kval = [&](int r, int c) -> double {
    if constexpr (E::kBytes == 2) return (double)bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(Kb)[(size_t)r * D + c]);
    else return (double)reinterpret_cast<const float*>(Kb)[(size_t)r * D + c];
  };

  // stage the keys (rows >= n are zero) and the mean (fp64)
  for (int idx = tid; idx < kN * D; idx += kLrThreads) {
    const int r = idx / D, c = idx % D;
    kv.k[r][c] = (r < n) ? (float)kval(r, c) : 0.f;
  }
  __syncthreads();
  for (int c = tid; c < D; c += kLrThreads) {
    double s = 0.0;
    for (int r = 0; r < n; ++r) s += (double)kv.k[r][c];
    mu[c] = s / (double)n;
  }
  __syncthreads();
  // Gram matrix G = X X^T / n (or, with a query subspace P, G = Y Y^T / n for the
  // projected keys Y = X P^T, whose covariance is P C P^T): each thread a 4x4 tile,
  // zero outside the n x n corner
  {
    const int ta = tid / 16, tb = tid % 16;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    if (Psub) {
      // 16 columns of Y = X P^T at a time, staged in A's space (A is written after)
      double (*ych)[17] = reinterpret_cast<double (*)[17]>(&A[0][0]);
      const float* Pu = Psub + (size_t)head * sub_s * D;
      for (int j0 = 0; j0 < sub_s; j0 += 16) {
        for (int idx = tid; idx < kN * 16; idx += kLrThreads) {
          const int r = idx / 16, jj = idx % 16, j = j0 + jj;
          double y = 0.0;
          if (r < n && j < sub_s) {
            const float* pr = Pu + (size_t)j * D;
            for (int c = 0; c < D; ++c) y += ((double)kv.k[r][c] - mu[c]) * (double)pr[c];
          }
          ych[r][jj] = y;
        }
        __syncthreads();
        for (int jj = 0; jj < 16; ++jj) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += ych[4 * ta + i][jj] * ych[4 * tb + j][jj];
        }
        __syncthreads();
      }
    } else {
      for (int c = 0; c < D; ++c) {
        const double m = mu[c];
        double xi[4], xj[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          xi[k] = (4 * ta + k < n) ? (double)kv.k[4 * ta + k][c] - m : 0.0;
          xj[k] = (4 * tb + k < n) ? (double)kv.k[4 * tb + k][c] - m : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] += xi[i] * xj[j];
      }
    }
    const double inv_n = 1.0 / (double)n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) A[4 * ta + i][4 * tb + j] = acc[i][j] * inv_n;
  }
  __syncthreads();
  for (int idx = tid; idx < kN * kN; idx += kLrThreads) Vm[idx / kN][idx % kN] = (idx / kN == idx % kN) ? 1.0 : 0.0;
  __syncthreads();

  // cyclic Jacobi sweeps
  double fro2 = 0.0;
  for (int idx = tid; idx < kN * kN; idx += kLrThreads) fro2 += A[idx / kN][idx % kN] * A[idx / kN][idx % kN];
  fro2 = block_sum_f64(fro2, red);
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    double off2 = 0.0;
    for (int idx = tid; idx < kN * kN; idx += kLrThreads) {
      const int i = idx / kN, j = idx % kN;
      if (i != j) off2 += A[i][j] * A[i][j];
    }
    off2 = block_sum_f64(off2, red);
    if (!(off2 > 1e-30 * fro2)) break;            // converged (also stops on an all-zero block)
    for (int r = 0; r < kN - 1; ++r) {
      if (tid < kN / 2) {
        const int p = rr_index(tid, r), q = rr_index(kN - 1 - tid, r);
        const double app = A[p][p], aqq = A[q][q], apq = A[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0 && fabs(apq) > 1e-300) {
          const double theta = (aqq - app) / (2.0 * apq);
          double t;
          if (fabs(theta) > 1e150) t = 0.5 / theta;
          else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(t * t + 1.0);
          s = t * c;
        }
        cs[tid][0] = c; cs[tid][1] = s;
        pq[tid][0] = p; pq[tid][1] = q;
      }
      __syncthreads();
      // rows: A <- J^T A
      for (int idx = tid; idx < (kN / 2) * kN; idx += kLrThreads) {
        const int k = idx / kN, j = idx % kN;
        const int p = pq[k][0], q = pq[k][1];
        const double c = cs[k][0], s = cs[k][1];
        const double ap = A[p][j], aq = A[q][j];
        A[p][j] = c * ap - s * aq;
        A[q][j] = s * ap + c * aq;
      }
      __syncthreads();
      // columns: A <- A J, V <- V J
      for (int idx = tid; idx < (kN / 2) * kN; idx += kLrThreads) {
        const int k = idx / kN, i = idx % kN;
        const int p = pq[k][0], q = pq[k][1];
        const double c = cs[k][0], s = cs[k][1];
        const double ap = A[i][p], aq = A[i][q];
        A[i][p] = c * ap - s * aq;
        A[i][q] = s * ap + c * aq;
        const double vp = Vm[i][p], vq = Vm[i][q];
        Vm[i][p] = c * vp - s * vq;
        Vm[i][q] = s * vp + c * vq;
      }
      __syncthreads();
    }
  }

  // top-r eigenvalues (ties to the lower index), by one wave
  if (tid < 64) {
    double lam = A[tid][tid];
    bool taken = false;
    for (int i = 0; i < rank; ++i) {
      double best = taken ? -INFINITY : lam;
      int bi = tid;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ob = __shfl_xor(best, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (tid == bi) taken = true;
      if (tid == 0) { order[i] = bi; lam_sel[i] = best; }
    }
  }
  __syncthreads();
  // v_i = X^T w_i / sqrt(n)
  const double inv_sqrt_n = 1.0 / sqrt((double)n);
  for (int idx = tid; idx < rank * D; idx += kLrThreads) {
    const int i = idx / D, c = idx % D;
    const int j = order[i];
    double s = 0.0;
    if (lam_sel[i] > 0.0) {
      for (int r = 0; r < n; ++r) s += (kval(r, c) - mu[c]) * Vm[r][j];
      s *= inv_sqrt_n;
    }
    vout[i][c] = s;
  }
  __syncthreads();
  // subspace: the vectors of P C P^T are P X^T w / sqrt(n) = P v (entries >= sub_s are 0)
  const int vl = Psub ? vlen : D;
  if (Psub) {
    const float* Pu = Psub + (size_t)head * sub_s * D;
    double pv[8 * D / kLrThreads];
#pragma unroll
    for (int k = 0; k < 8 * D / kLrThreads; ++k) {
      const int idx = tid + k * kLrThreads, i = idx / vl, j = idx % vl;
      double s = 0.0;
      if (i < rank && j < sub_s)
        for (int c = 0; c < D; ++c) s += (double)Pu[(size_t)j * D + c] * vout[i][c];
      pv[k] = s;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8 * D / kLrThreads; ++k) {
      const int idx = tid + k * kLrThreads;
      if (idx < rank * vl) vout[idx / vl][idx % vl] = pv[k];
    }
    __syncthreads();
  }
  // sign: largest-magnitude entry positive (first such entry on ties)
  if (tid < 64) {
    for (int i = 0; i < rank; ++i) {
      double best = -1.0;
      int bi = D;
      for (int c = tid; c < vl; c += 64) {
        const double a = fabs(vout[i][c]);
        if (a > best) { best = a; bi = c; }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ob = __shfl_xor(best, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (tid == 0) red[0] = (bi < vl && vout[i][bi] < 0.0) ? -1.0 : 1.0;
      __builtin_amdgcn_wave_barrier();
      const double sg = red[0];
      for (int c = tid; c < vl; c += 64) vout[i][c] *= sg;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  if (fp4) {
    quantize_record<D>(vout, gexp, rec, rank, vl, tid);
    const int words = (int)(fp4_record_bytes_dev(rank, vl) / 4);
    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(lowrank) +
                                                (unit * (size_t)nb_max + b) * fp4_record_bytes_dev(rank, vl));
    for (int w = tid; w < words; w += kLrThreads) dst[w] = reinterpret_cast<const uint32_t*>(rec)[w];
  } else {
    float* dst = static_cast<float*>(lowrank) + ((unit * (size_t)nb_max + b) * rank) * vl;
    for (int idx = tid; idx < rank * vl; idx += kLrThreads) dst[idx] = (float)vout[idx / vl][idx % vl];
  }
  __syncthreads();                         // shared arrays are reused by the next block
  }
}

template <typename E, int D>
static hipError_t launch_lr(const BuildArgs& a) {
  dim3 grid(a.old_lens ? a.touch_blocks : a.nb_max, a.hkv, a.batch);
  hipLaunchKernelGGL((k_build_lowrank<E, D>), grid, dim3(kLrThreads), 0, a.stream, a.seq_lens, a.old_lens,
                     a.max_len, a.nb_max, a.rank, (const typename E::storage*)a.K, a.lowrank, a.fp4 ? 1 : 0,
                     a.P, a.sub_s, a.vlen);
  return hipGetLastError();
}

hipError_t launch_build_lowrank(const BuildArgs& a) {
  if (a.rank < 1 || a.rank > 8) return hipErrorInvalidValue;
  if (a.bf16) return a.head_dim == 128 ? launch_lr<EltBF16, 128>(a) : launch_lr<EltBF16, 64>(a);
  return a.head_dim == 128 ? launch_lr<EltF32, 128>(a) : launch_lr<EltF32, 64>(a);
}

}  // namespace cobs
