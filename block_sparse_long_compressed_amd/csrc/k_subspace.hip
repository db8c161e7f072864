// Query subspace for the covariance projection (gfx950).
//
// COBS (gist.science explainer, Technisches Resuemee 2.3, "Subraum-Projektion"):
// block covariances are projected into the low-dimensional subspace spanned by
// the top eigenvectors of the queries' second moment.  From calibration queries
// of each GQA group this computes M = (1/N) sum q q^T (uncentred, fp64) and its
// top-s eigenvectors, returned as the rows of P [s][d] (fp32), each signed so its
// largest-magnitude entry is positive.
//
// Two launches per call:
//   k_second_moment  one workgroup per (kv-head, 16-row band of M): the group's
//                    queries stream through LDS in chunks, each thread keeps its
//                    entries of M in fp64 registers.
//   k_top_eigvecs    one workgroup per kv-head: a parallel cyclic Jacobi sweep in
//                    fp64 (d/2 disjoint rotations per round, round-robin pairing),
//                    with M in LDS and the accumulated rotations in the workspace
//                    (stored by column, so a rotation's reads are contiguous);
//                    then the eigenvalues are ranked (ties to the lower index) and
//                    the top s columns written out.
#include "cobs_device.h"
#include "cobs_launch.h"

namespace cobs {

constexpr int kSmThreads = 256;
constexpr int kSmChunk = 32;          // queries staged per LDS round
constexpr int kEgThreads = 512;
constexpr int kEgMaxSweeps = 30;

template <typename E, int D>
__global__ __launch_bounds__(kSmThreads) void k_second_moment(const typename E::storage* __restrict__ Q, int n,
                                                              int hq, int group, double* __restrict__ M) {
  __shared__ float qs[kSmChunk][D + 1];
  const int head = blockIdx.y, band = blockIdx.x;       // rows [16 band, 16 band + 16) of M
  const int tid = threadIdx.x;
  constexpr int PER = 16 * D / kSmThreads;              // entries of M per thread (8 or 4)
  double acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0;
  const int total = n * group;                          // queries of this group
  for (int q0 = 0; q0 < total; q0 += kSmChunk) {
    for (int idx = tid; idx < kSmChunk * D; idx += kSmThreads) {
      const int r = idx / D, c = idx % D, qi = q0 + r;
      float v = 0.f;
      if (qi < total) {
        const int t = qi / group, h = head * group + qi % group;
        const size_t off = ((size_t)t * hq + h) * D + c;
        if constexpr (E::kBytes == 2) v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(Q)[off]);
        else v = reinterpret_cast<const float*>(Q)[off];
      }
      qs[r][c] = v;
    }
    __syncthreads();
    const int rows = min(kSmChunk, total - q0);
    for (int r = 0; r < rows; ++r) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + k * kSmThreads, i = 16 * band + e / D, j = e % D;
        acc[k] += (double)qs[r][i] * (double)qs[r][j];
      }
    }
    __syncthreads();
  }
  const double inv = 1.0 / (double)total;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + k * kSmThreads, i = 16 * band + e / D, j = e % D;
    M[((size_t)head * D + i) * D + j] = acc[k] * inv;
  }
}

// Round-robin pairing over d indices: round r, slot k -> (p, q); every unordered
// pair occurs exactly once in d-1 rounds.
template <int D>
__device__ __forceinline__ int eg_index(int pos, int r) { return pos == 0 ? 0 : 1 + (pos - 1 + r) % (D - 1); }

template <int D>
__device__ __forceinline__ double eg_block_sum(double v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kEgThreads / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}

template <int D>
__global__ __launch_bounds__(kEgThreads) void k_top_eigvecs(const double* __restrict__ Mall, double* __restrict__ Vall,
                                                            int s, float* __restrict__ P) {
  extern __shared__ __align__(16) unsigned char smem[];
  double (*A)[D + 1] = reinterpret_cast<double (*)[D + 1]>(smem);
  double* cs = reinterpret_cast<double*>(smem + sizeof(double) * D * (D + 1));   // [D/2][2]
  int* pq = reinterpret_cast<int*>(cs + D);                                       // [D/2][2]
  double* red = reinterpret_cast<double*>(pq + D);                                // [kEgThreads/64]
  int* order = reinterpret_cast<int*>(red + kEgThreads / 64);                     // [D]
  const int head = blockIdx.x, tid = threadIdx.x;
  const double* M = Mall + (size_t)head * D * D;
  double* V = Vall + (size_t)head * D * D;
  for (int idx = tid; idx < D * D; idx += kEgThreads) {
    const int i = idx / D, j = idx % D;
    A[i][j] = M[idx];
    V[idx] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  double fro2 = 0.0;
  for (int idx = tid; idx < D * D; idx += kEgThreads) fro2 += A[idx / D][idx % D] * A[idx / D][idx % D];
  fro2 = eg_block_sum<D>(fro2, red);
  for (int sweep = 0; sweep < kEgMaxSweeps; ++sweep) {
    double off2 = 0.0;
    for (int idx = tid; idx < D * D; idx += kEgThreads) {
      const int i = idx / D, j = idx % D;
      if (i != j) off2 += A[i][j] * A[i][j];
    }
    off2 = eg_block_sum<D>(off2, red);
    if (!(off2 > 1e-30 * fro2)) break;                  // converged (also stops on an all-zero M)
    for (int r = 0; r < D - 1; ++r) {
      if (tid < D / 2) {
        const int p = eg_index<D>(tid, r), q = eg_index<D>(D - 1 - tid, r);
        const double app = A[p][p], aqq = A[q][q], apq = A[p][q];
        double c = 1.0, sn = 0.0;
        if (apq != 0.0 && fabs(apq) > 1e-300) {
          const double theta = (aqq - app) / (2.0 * apq);
          double t;
          if (fabs(theta) > 1e150) t = 0.5 / theta;
          else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(t * t + 1.0);
          sn = t * c;
        }
        cs[2 * tid] = c; cs[2 * tid + 1] = sn;
        pq[2 * tid] = p; pq[2 * tid + 1] = q;
      }
      __syncthreads();
      // rows: A <- J^T A
      for (int idx = tid; idx < (D / 2) * D; idx += kEgThreads) {
        const int k = idx / D, j = idx % D;
        const int p = pq[2 * k], q = pq[2 * k + 1];
        const double c = cs[2 * k], sn = cs[2 * k + 1];
        const double ap = A[p][j], aq = A[q][j];
        A[p][j] = c * ap - sn * aq;
        A[q][j] = sn * ap + c * aq;
      }
      __syncthreads();
      // columns: A <- A J, V <- V J
      for (int idx = tid; idx < (D / 2) * D; idx += kEgThreads) {
        const int k = idx / D, i = idx % D;
        const int p = pq[2 * k], q = pq[2 * k + 1];
        const double c = cs[2 * k], sn = cs[2 * k + 1];
        const double ap = A[i][p], aq = A[i][q];
        A[i][p] = c * ap - sn * aq;
        A[i][q] = sn * ap + c * aq;
        const double vp = V[(size_t)p * D + i], vq = V[(size_t)q * D + i];      // V stored by column
        V[(size_t)p * D + i] = c * vp - sn * vq;
        V[(size_t)q * D + i] = sn * vp + c * vq;
      }
      __syncthreads();
    }
  }
  // rank the eigenvalues (descending, ties to the lower index): position of each
  if (tid < D) {
    const double lam = A[tid][tid];
    int pos = 0;
    for (int j = 0; j < D; ++j) {
      const double o = A[j][j];
      pos += (o > lam || (o == lam && j < tid)) ? 1 : 0;
    }
    order[pos] = tid;
  }
  __syncthreads();
  // row i of P = column order[i] of V, signed by its largest-magnitude entry (first on ties)
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = wave; i < s; i += kEgThreads / 64) {
    const int j = order[i];
    double best = -1.0;
    int bi = D;
    for (int c = lane; c < D; c += 64) {
      const double a = fabs(V[(size_t)j * D + c]);
      if (a > best) { best = a; bi = c; }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const double ob = __shfl_xor(best, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    const double sg = V[(size_t)j * D + bi] < 0.0 ? -1.0 : 1.0;
    for (int c = lane; c < D; c += 64) P[((size_t)head * s + i) * D + c] = (float)(sg * V[(size_t)j * D + c]);
  }
}

size_t subspace_ws_bytes(int hkv, int d) { return (size_t)hkv * d * d * sizeof(double) * 2; }

template <typename E, int D>
static hipError_t launch_sub(const SubspaceArgs& a) {
  double* M = static_cast<double*>(a.ws);
  double* V = M + (size_t)a.hkv * D * D;
  hipLaunchKernelGGL((k_second_moment<E, D>), dim3(D / 16, a.hkv), dim3(kSmThreads), 0, a.stream,
                     (const typename E::storage*)a.Q, a.n, a.hq, a.group, M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(double) * D * (D + 1) + sizeof(double) * D + sizeof(int) * D +
                     sizeof(double) * (kEgThreads / 64) + sizeof(int) * D;
  hipLaunchKernelGGL((k_top_eigvecs<D>), dim3(a.hkv), dim3(kEgThreads), lds, a.stream, M, V, a.s, a.P);
  return hipGetLastError();
}

hipError_t launch_query_subspace(const SubspaceArgs& a) {
  if (a.bf16) return a.head_dim == 128 ? launch_sub<EltBF16, 128>(a) : launch_sub<EltBF16, 64>(a);
  return a.head_dim == 128 ? launch_sub<EltF32, 128>(a) : launch_sub<EltF32, 64>(a);
}

}  // namespace cobs
