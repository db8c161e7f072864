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
// X^T w / sqrt(n) = sqrt(lambda) u.  One 256-thread workgroup per block, G in
// LDS, in fp64: G is reduced to a tridiagonal T = Q^T G Q by 62 Householder
// reflections; the r largest eigenvalues of T come from bisection on Sturm counts
// (one half-wave per eigenvalue, 32 shifts per step); each eigenvector of T from
// the twisted factorisation T - lambda I = L+ D+ L+^T = U- D- U-^T (one solve, no
// iteration), made orthogonal to the earlier ones (a repeated eigenvalue takes one
// inverse-iteration step for each further direction); then w = Q z.  This agrees
// with a reference fp64 symmetric eigensolver to rounding wherever the eigenvalue
// is not repeated.  Eigenvalues <= 0 give v = 0; each v is signed so that its
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
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kN = 64;              // Gram size (keys per block)
constexpr double kEps = 0x1p-52;          // fp64 unit roundoff (2^-53) times 2
constexpr double kSafeMin = 0x1p-1021;    // safe minimum (1 / it does not overflow)

// A double moved between lanes by a DPP pattern (two 32-bit moves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Reductions over the 16 lanes of a row with DPP: lane pairs i^1, i^2 within a
// quad, then the mirrored quads and half-rows, so every lane adds the same two
// partial results (a + b and b + a) and ends with the same bits.
template <typename Op>
__device__ __forceinline__ double row_reduce(double v, Op op) {
  v = op(v, dpp_f64<0xB1>(v));      // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_f64<0x4E>(v));      // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_f64<0x141>(v));     // row_half_mirror
  v = op(v, dpp_f64<0x140>(v));     // row_mirror
  return v;
}
struct AddOp { __device__ double operator()(double a, double b) const { return a + b; } };
struct MaxOp { __device__ double operator()(double a, double b) const { return fmax(a, b); } };
struct MinOp { __device__ double operator()(double a, double b) const { return fmin(a, b); } };

// Sum, maximum and minimum over the 32 lanes of a half-wave, and the sum over the wave.
__device__ __forceinline__ double half_sum(double v) {
  v = row_reduce(v, AddOp{});
  return v + __shfl_xor(v, 16, 64);
}
__device__ __forceinline__ double half_max(double v) {
  v = row_reduce(v, MaxOp{});
  return fmax(v, __shfl_xor(v, 16, 64));
}
__device__ __forceinline__ double half_min(double v) {
  v = row_reduce(v, MinOp{});
  return fmin(v, __shfl_xor(v, 16, 64));
}
// The value of lane i (i the same in every lane).
__device__ __forceinline__ double readlane_f64(double v, int i) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, i);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), i);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_max(double v) {
  v = half_max(v);
  return fmax(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ double wave_sum(double v) {
  v = half_sum(v);
  return v + __shfl_xor(v, 32, 64);
}

// Number of eigenvalues below sig of the symmetric tridiagonal matrix with
// diagonal d and squared off-diagonal e2 (Sturm sequence of the LDL^T pivots of
// T - sig I; a pivot smaller in magnitude than pivmin is replaced by -pivmin).
__device__ __forceinline__ int sturm_count(const double* d, const double* e2, double sig, double pivmin) {
  double q = d[0] - sig;
  if (fabs(q) < pivmin) q = -pivmin;
  int c = q < 0.0 ? 1 : 0;
  for (int i = 1; i < kN; ++i) {
    double r = __builtin_amdgcn_rcp(q);           // 1 / q: hardware estimate and one Newton step
    r = fma(r, fma(-q, r, 1.0), r);
    q = (d[i] - sig) - e2[i - 1] * r;
    if (fabs(q) < pivmin) q = -pivmin;
    c += q < 0.0 ? 1 : 0;
  }
  return c;
}

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

template <typename E, int D, bool SUB>
__global__ __launch_bounds__(kLrThreads) void k_build_lowrank(const int32_t* __restrict__ seq_lens,
                                                              const int32_t* __restrict__ old_lens, int max_len,
                                                              int nb_max, int rank,
                                                              const typename E::storage* __restrict__ K,
                                                              void* __restrict__ lowrank, int fp4,
                                                              const float* __restrict__ Psub, int sub_s,
                                                              int vlen) {
  __shared__ double A[kN][kN + 1];      // Gram matrix, reduced in place (+1: bank spread)
  // the block's keys (fp32, exact for bf16) until G is built, then the Householder vectors
  // (with a query subspace, the projected keys Y = X P^T replace the keys before G)
  __shared__ union {
    float k[kN][D + 1];
    double v[kN][kN + 1];
    double y[SUB ? kN : 1][SUB ? D + 1 : 1];
  } kv;
  __shared__ double mu[D];
  __shared__ double red[4];
  __shared__ double lam_sel[8];
  // the output vectors, and before them the eigensolver's scratch
  __shared__ union {
    double vout[8][D];
    struct { double part[4][kN], col[2][kN], d[kN], e[kN], e2[kN]; } ev;
  } ov;
  auto& vout = ov.vout;
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
  // projected keys Y = X P^T, whose covariance is P C P^T) on the fp64 MFMA
  // (v_mfma_f64_16x16x4_f64: lane (r, q) = (lane % 16, lane / 16) holds A[r][q] and
  // B[q][r] of a 16x16x4 step and rows q, q + 4, q + 8, q + 12 of column r of the
  // 16x16 result):
  // wave w forms rows 16w..16w+15, the four waves together the 64 x 64 corner
  // (zero outside n x n, as the centred rows >= n are zero)
  {
    const int lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const int ra = 16 * wv + r16;
    const double inv_n = 1.0 / (double)n;
    auto xc = [&](int r, int c) -> double { return (r < n) ? (double)kv.k[r][c] - mu[c] : 0.0; };
    f64x4 acc[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) acc[tj] = f64x4{0.0, 0.0, 0.0, 0.0};
    if constexpr (SUB) {
      // Y = X P^T, 16 columns per tile (columns >= sub_s are zero), into LDS over the keys
      const float* Pu = Psub + (size_t)head * sub_s * D;
      const int ntj = (sub_s + 15) / 16;
      f64x4 yacc[D / 16];
#pragma unroll
      for (int tj = 0; tj < D / 16; ++tj) yacc[tj] = f64x4{0.0, 0.0, 0.0, 0.0};
      // 32 columns of P per round: all their loads go out before the contraction
      for (int c1 = 0; c1 < D; c1 += 32) {
        float pb[8][D / 16];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
#pragma unroll
          for (int tj = 0; tj < D / 16; ++tj) {
            const int j = 16 * tj + r16;
            pb[s8][tj] = (tj < ntj && j < sub_s) ? Pu[(size_t)j * D + c1 + 4 * s8 + kq] : 0.f;
          }
        }
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const double a = xc(ra, c1 + 4 * s8 + kq);
#pragma unroll
          for (int tj = 0; tj < D / 16; ++tj)
            if (tj < ntj) yacc[tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)pb[s8][tj], yacc[tj], 0, 0, 0);
        }
      }
      __syncthreads();                             // every wave is done with the keys
#pragma unroll
      for (int tj = 0; tj < D / 16; ++tj) {
        if (tj < ntj) {
#pragma unroll
          for (int i = 0; i < 4; ++i) kv.y[16 * wv + kq + 4 * i][16 * tj + r16] = yacc[tj][i];
        }
      }
      __syncthreads();
      for (int j0 = 0; j0 < 16 * ntj; j0 += 4) {
        const int j = j0 + kq;
        const double a = kv.y[ra][j];
#pragma unroll
        for (int tj = 0; tj < 4; ++tj)
          acc[tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, kv.y[16 * tj + r16][j], acc[tj], 0, 0, 0);
      }
    } else {
      for (int c0 = 0; c0 < D; c0 += 4) {
        const int c = c0 + kq;
        const double a = xc(ra, c);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) acc[tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, xc(16 * tj + r16, c), acc[tj], 0, 0, 0);
      }
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
#pragma unroll
      for (int i = 0; i < 4; ++i) A[16 * wv + kq + 4 * i][16 * tj + r16] = acc[tj][i] * inv_n;
    }
  }
  __syncthreads();
  // ---- top-r eigenpairs of G ------------------------------------------------
  // (1) Householder tridiagonalisation G = Q T Q^T, Q = H_0 ... H_61, H_k = I - u_k u_k^T
  //     (|u_k|^2 = 2, zero in entries 0..k); u_k is kept in row k of Vm.
  double fro2 = 0.0;
  for (int idx = tid; idx < kN * kN; idx += kLrThreads) fro2 += A[idx / kN][idx % kN] * A[idx / kN][idx % kN];
  fro2 = block_sum_f64(fro2, red);
  const int lane = tid & 63, wv = tid >> 6;
  // wave w keeps rows 16w..16w+15 of G in registers (lane = column); the column a
  // step reduces is row k of the symmetric G, published through LDS by its wave
  const int grow0 = __builtin_amdgcn_readfirstlane(16 * wv);
  double arow[16];
#pragma unroll
  for (int ii = 0; ii < 16; ++ii) arow[ii] = A[grow0 + ii][lane];
  auto own_row = [&](int r) {                        // arow[r - grow0] (r in this wave's rows)
    double v = 0.0;
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) v = (grow0 + ii == r) ? arow[ii] : v;
    return v;
  };
  if (wv == 0) ov.ev.col[0][lane] = arow[0];
  __syncthreads();
  for (int k = 0; k < kN - 2; ++k) {
    const double* colk = ov.ev.col[k & 1];
    double* coln = ov.ev.col[(k + 1) & 1];
    const bool owner_next = wv == (k + 1) / 16;
    // the reflector of column k below the diagonal, formed by every wave from the
    // same LDS values with bit-identical reductions (so all take the same branch)
    const double xi = (lane > k) ? colk[lane] : 0.0;
    const double sigma = wave_sum(xi * xi);
    if (!(sigma > 1e-40 * fro2)) {                  // the column is negligible: H_k = I
      if (wv == 0) Vm[k][lane] = 0.0;
      if (owner_next) coln[lane] = own_row(k + 1);
      __syncthreads();
      continue;
    }
    const double x0 = colk[k + 1];
    const double alpha = -copysign(sqrt(sigma), x0);
    const double sc = sqrt(1.0 / (sigma - alpha * x0));
    const double uj = (lane > k) ? (xi - (lane == k + 1 ? alpha : 0.0)) * sc : 0.0;
    if (wv == 0) Vm[k][lane] = uj;
    // p = G u: wave w sums its rows (G is symmetric, so a row serves as a column)
    {
      double sp = 0.0;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) sp += arow[ii] * readlane_f64(uj, grow0 + ii);
      ov.ev.part[wv][lane] = sp;
    }
    __syncthreads();
    // w = p - (u^T p / 2) u;  G <- G - u w^T - w u^T on this wave's rows
    {
      const double pj = (ov.ev.part[0][lane] + ov.ev.part[1][lane]) + (ov.ev.part[2][lane] + ov.ev.part[3][lane]);
      const double K = 0.5 * wave_sum(uj * pj);
      const double wj = pj - K * uj;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const double ui = readlane_f64(uj, grow0 + ii), wi = readlane_f64(wj, grow0 + ii);
        arow[ii] -= ui * wj + wi * uj;
      }
    }
    if (owner_next) coln[lane] = own_row(k + 1);
    __syncthreads();
  }
  // T: the diagonal, and the subdiagonal e_i = G[i+1][i] (row i + 1, lane i)
#pragma unroll
  for (int ii = 0; ii < 16; ++ii) {
    const int r = grow0 + ii;
    if (lane == r) ov.ev.d[r] = arow[ii];
    if (r >= 1 && lane == r - 1) { ov.ev.e[r - 1] = arow[ii]; ov.ev.e2[r - 1] = arow[ii] * arow[ii]; }
  }
  if (tid == 0) { ov.ev.e[kN - 1] = 0.0; ov.ev.e2[kN - 1] = 0.0; }
  __syncthreads();
  // (2) the j-th largest eigenvalue of T by bisection, one half-wave per eigenvalue:
  //     32 Sturm counts per step narrow the bracket 33-fold
  double* const Af = &A[0][0];                      // G is no longer needed: scratch
  double* const Wv = Af + 24 * kN;                  // eigenvectors, [j][kN]
  const int jv = tid >> 5, g = tid & 31;
  if (jv < rank) {
    const double* d = ov.ev.d;
    const double* e = ov.ev.e;
    const double* e2 = ov.ev.e2;
    double lo = INFINITY, hi = -INFINITY, emax2 = 0.0;
    for (int i = 0; i < kN; ++i) {
      const double r = fabs(e[i]) + (i > 0 ? fabs(e[i - 1]) : 0.0);
      lo = fmin(lo, d[i] - r);
      hi = fmax(hi, d[i] + r);
      emax2 = fmax(emax2, e2[i]);
    }
    const double pivmin = kSafeMin * fmax(1.0, emax2);
    const double tnorm = fmax(fabs(lo), fabs(hi));
    lo -= 2.0 * kEps * tnorm + 2.0 * pivmin;
    hi += 2.0 * kEps * tnorm + 2.0 * pivmin;
    const int target = kN - 1 - jv;                 // its index in ascending order
    for (int it = 0; it < 64; ++it) {
      if (hi - lo <= 2.0 * kEps * fmax(fabs(lo), fabs(hi)) + kEps * tnorm + pivmin) break;
      const double sig = lo + (hi - lo) * ((double)(g + 1) / 33.0);
      const int c = sturm_count(d, e2, sig, pivmin);
      const double nlo = half_max(c <= target ? sig : -INFINITY);
      const double nhi = half_min(c > target ? sig : INFINITY);
      if (nlo > -INFINITY) lo = nlo;
      if (nhi < INFINITY) hi = nhi;
    }
    // (3) its eigenvector of T from the twisted factorisation of T - lam I:
    //     T - lam I = L+ D+ L+^T = U- D- U-^T; at the twist k where
    //     |gamma_k| = |D+_k + D-_k - (d_k - lam)| is smallest, z_k = 1 and
    //     z_i = -L+_i z_i+1 above, z_i+1 = -U-_i z_i below
    if (g == 0) {
      const double lam = 0.5 * (lo + hi);
      lam_sel[jv] = lam;
      const double tiny = kSafeMin * 0x1p14;
      double* Lp = Af + jv * 3 * kN;
      double* Um = Lp + kN;
      double* Dp = Um + kN;
      double dp = d[0] - lam;
      for (int i = 0; i < kN - 1; ++i) {
        if (fabs(dp) < tiny) dp = -tiny;
        Dp[i] = dp;
        Lp[i] = e[i] / dp;
        dp = (d[i + 1] - lam) - Lp[i] * e[i];
      }
      Dp[kN - 1] = dp;
      double dm = d[kN - 1] - lam;
      double best = fabs(Dp[kN - 1] + dm - (d[kN - 1] - lam));
      int kt = kN - 1;
      for (int i = kN - 2; i >= 0; --i) {
        if (fabs(dm) < tiny) dm = -tiny;
        Um[i] = e[i] / dm;
        dm = (d[i] - lam) - Um[i] * e[i];
        const double gam = fabs(Dp[i] + dm - (d[i] - lam));
        if (gam < best) { best = gam; kt = i; }
      }
      double* z = Wv + jv * kN;
      z[kt] = 1.0;
      double zc = 1.0;
      for (int i = kt - 1; i >= 0; --i) { zc = -Lp[i] * zc; z[i] = zc; }
      zc = 1.0;
      for (int i = kt; i < kN - 1; ++i) { zc = -Um[i] * zc; z[i + 1] = zc; }
    }
  }
  __syncthreads();
  // (4) normalise, orthogonal to the earlier vectors.  A repeated eigenvalue gives
  //     the same twisted vector again; then one inverse-iteration step from the
  //     first unit vector (made orthogonal to the earlier vectors) that leaves a
  //     new direction: (T - lam I) y = b solved with the forward factorisation,
  //     pivots held at least eps |T| away from zero.
  if (wv == 0) {
    const double tn = wave_max(fabs(ov.ev.d[lane])) + 2.0 * wave_max(fabs(ov.ev.e[lane]));
    const double pfloor = kEps * tn;
    for (int jj = 0; jj < rank; ++jj) {
      double z = Wv[jj * kN + lane];
      double nz = 0.0;
      for (int attempt = -1; attempt < kN; ++attempt) {
        if (attempt >= 0) {
          double bv = (lane == attempt) ? 1.0 : 0.0;
          for (int pv = 0; pv < jj; ++pv) {
            const double v = Wv[pv * kN + lane];
            bv -= wave_sum(v * bv) * v;
          }
          Wv[jj * kN + lane] = bv;
          __builtin_amdgcn_wave_barrier();
          if (lane == 0) {
            const double* Lp = Af + jj * 3 * kN;
            const double* Dp = Lp + 2 * kN;
            double* y = Wv + jj * kN;
            for (int t = 1; t < kN; ++t) y[t] -= Lp[t - 1] * y[t - 1];
            for (int t = 0; t < kN; ++t) {
              double dd = Dp[t];
              if (fabs(dd) < pfloor) dd = dd < 0.0 ? -pfloor : pfloor;
              y[t] /= dd;
            }
            for (int t = kN - 2; t >= 0; --t) y[t] -= Lp[t] * y[t + 1];
          }
          __builtin_amdgcn_wave_barrier();
          z = Wv[jj * kN + lane];
          const double zm = wave_max(fabs(z));
          if (!(zm > 0.0 && zm < INFINITY)) continue;
          z /= zm;
        }
        nz = sqrt(wave_sum(z * z));
        if (!(nz > 0.0 && nz < INFINITY)) continue;
        z /= nz;
        for (int pv = 0; pv < jj; ++pv) {
          const double v = Wv[pv * kN + lane];
          z -= wave_sum(v * z) * v;
        }
        nz = sqrt(wave_sum(z * z));
        if (nz > 0.5) break;
      }
      Wv[jj * kN + lane] = (nz > 0.5) ? z / nz : 0.0;
    }
  }
  __syncthreads();
  // (5) back to G's basis: w = H_0 ... H_61 z, one half-wave per vector
  if (jv < rank) {
    double z0 = Wv[jv * kN + g], z1 = Wv[jv * kN + g + 32];
    for (int k = kN - 3; k >= 0; --k) {
      const double u0 = Vm[k][g], u1 = Vm[k][g + 32];
      const double dot = half_sum(u0 * z0 + u1 * z1);
      z0 -= dot * u0;
      z1 -= dot * u1;
    }
    Wv[jv * kN + g] = z0;
    Wv[jv * kN + g + 32] = z1;
  }
  __syncthreads();
  // the keys again (the Householder vectors took their space)
  for (int idx = tid; idx < kN * D; idx += kLrThreads) {
    const int r = idx / D, c = idx % D;
    kv.k[r][c] = (r < n) ? (float)kval(r, c) : 0.f;
  }
  __syncthreads();
  // v_i = X^T w_i / sqrt(n)
  const double inv_sqrt_n = 1.0 / sqrt((double)n);
  for (int idx = tid; idx < rank * D; idx += kLrThreads) {
    const int i = idx / D, c = idx % D;
    double s = 0.0;
    if (lam_sel[i] > 0.0) {
      for (int r = 0; r < n; ++r) s += ((double)kv.k[r][c] - mu[c]) * Wv[i * kN + r];
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
  // the query-subspace build keeps the projected keys in LDS (its own instantiation,
  // so the plain build keeps the smaller LDS footprint)
  if (a.P)
    hipLaunchKernelGGL((k_build_lowrank<E, D, true>), grid, dim3(kLrThreads), 0, a.stream, a.seq_lens, a.old_lens,
                       a.max_len, a.nb_max, a.rank, (const typename E::storage*)a.K, a.lowrank, a.fp4 ? 1 : 0,
                       a.P, a.sub_s, a.vlen);
  else
    hipLaunchKernelGGL((k_build_lowrank<E, D, false>), grid, dim3(kLrThreads), 0, a.stream, a.seq_lens, a.old_lens,
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
