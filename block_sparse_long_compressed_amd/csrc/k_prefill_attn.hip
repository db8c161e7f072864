// Token-blocked chunked-prefill attention (gfx950, bf16 K/V).
//
// NSA branches (Janus issue #181) for each query token t of a chunk, with the
// readings of the decode path: selected blocks (the token's own top-k), the
// window [t-W+1, t] and the pooled tokens j with 16j + 31 <= t, each an exact
// softmax, combined as g_cmp o_cmp + g_slc o_slc + g_win o_win.
//
// A workgroup of 8 waves owns 16 consecutive tokens of one kv-head group (two per
// wave, so a wave's B operand covers 2 x 16 query heads) and runs the three
// branches one after the other over 64-key tiles staged once in LDS for all 16
// tokens, two tiles per barrier (two LDS buffer pairs; the global loads of the
// next two tiles are in flight in registers while the current pair is consumed);
// every token masks its own keys:
//   window and pooled tokens: consecutive tokens' key ranges nearly coincide, so
//   each tile of the union range is staged once and a token masks positions
//   outside its range;
//   selected blocks: the workgroup stages the union of its tokens' selections
//   (consecutive tokens pick largely the same blocks: about 22 distinct blocks for
//   16 x 16 picks on the 32k workload) and a token keeps a tile only if the block is
//   one of its own; a wave whose two tokens both skip a tile does no arithmetic.
// Staged tiles:
//   K rows padded to d+8 elements, read as the A operand of S = K Q^T with
//   16-byte reads;
//   V rows padded to d+16 elements, its transpose (the A operand of O^T = V^T P^T)
//   read with gfx950's transposing LDS read (ds_read_b64_tr_b16: four lanes' 4 x
//   16-bit rows come back as columns), shared by both tokens of a wave.
#include "attn_tile.h"
#include "cobs_device.h"
#include "cobs_launch.h"
#include "score_common.h"

#include <algorithm>

namespace cobs {

constexpr int kPfThreads = 512;       // 8 waves
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kPfTokens = 2 * kPfWaves;   // query tokens per workgroup (two per wave)
constexpr int kPfMaxBlocks = 4096;    // longest prefix (blocks) the selected-block union supports
constexpr int kPfMaskWords = kPfMaxBlocks / 32;

// Selected-block bookkeeping of a workgroup (LDS, after the staging buffers): one
// bitmap per token over the prefix's blocks, their union as an ascending list.
struct PfSel {
  uint32_t mask[kPfTokens][kPfMaskWords];
  int32_t list[kPfTokens * 64];
  int scan_w[kPfWaves];
  int count;
};

// Exclusive prefix sum over the workgroup's threads, in thread order.
__device__ __forceinline__ int pf_block_scan(int v, int* lds_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_inclusive_sum(v);
  if (lane == 63) lds_w[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPfWaves; ++i) {
    const int c = lds_w[i];
    base += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

template <int D>
struct PfShape {
  static constexpr int kNch = D / 32;                    // 32-wide contraction slices of head_dim
  static constexpr int kDt = D / 16;                     // 16-row output tiles of O^T
  static constexpr int kKs = D + 8;                      // LDS row stride of staged K (elements)
  static constexpr int kRowChunks = D / 8;               // 16-byte chunks per K/V row
  static constexpr int kLoads = kBlock * kRowChunks / kPfThreads;   // 16-byte loads per thread per tile (K or V)
  static constexpr int kVs = D + 16;                     // LDS row stride of staged V (elements): 8 banks apart
  static constexpr int kKElems = kBlock * kKs;
  static constexpr int kBufElems = kKElems + kBlock * kVs;   // one staged tile: K then V
};

struct PaParams {
  int tokens, hkv, group, seq_len, nc_max, top_k, window, cmp_on, q_pos0;
  float scale_log2;
  const uint16_t *Q, *K, *V, *kc, *vc;
  const float* gates;
  const int32_t* sel;
  float* out;
};

template <int D>
struct StageRegs {
  u32x4 k[PfShape<D>::kLoads], v[PfShape<D>::kLoads];
};

// Global loads of one 64-row K/V tile (rows past nvalid repeat the last valid row).
template <int D>
__device__ __forceinline__ void stage_load(const uint16_t* __restrict__ Ks, const uint16_t* __restrict__ Vs,
                                           int nvalid, StageRegs<D>& r) {
  using S = PfShape<D>;
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int id = threadIdx.x + kPfThreads * i;
    const int row = min(id / S::kRowChunks, nvalid - 1), cc = id % S::kRowChunks;
    r.k[i] = ld16(Ks + (size_t)row * D + cc * 8);
    r.v[i] = ld16(Vs + (size_t)row * D + cc * 8);
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const StageRegs<D>& r, uint16_t* buf) {
  using S = PfShape<D>;
  uint16_t* vs = buf + S::kKElems;
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int id = threadIdx.x + kPfThreads * i;
    const int row = id / S::kRowChunks, cc = id % S::kRowChunks;
    st16(buf + row * S::kKs + cc * 8, r.k[i]);
    st16(vs + row * S::kVs + cc * 8, r.v[i]);
  }
}

// One staged tile for the wave's two tokens: keys at positions tile_start + 0..63,
// token u sees positions [lo[u], hi[u]].
template <int D>
__device__ __forceinline__ void shared_tile(const uint16_t* buf, int tile_start, const int (&lo)[2], const int (&hi)[2],
                                            const u32x4 (&qf)[2][PfShape<D>::kNch], float scale_log2,
                                            float (&m)[2], f32x4 (&lsum)[2], f32x4 (&acc)[2][PfShape<D>::kDt]) {
  using S = PfShape<D>;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  f32x4 s[2][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S::kNch; ++c) {
      const u32x4 kop = *reinterpret_cast<const u32x4*>(buf + (16 * t + n) * S::kKs + (4 * c + g) * 8);
      a0 = mfma_bf16_16x16x32(kop, qf[0][c], a0);
      a1 = mfma_bf16_16x16x32(kop, qf[1][c], a1);
    }
    s[0][t] = a0;
    s[1][t] = a1;
  }
  u32x4 pb[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // max of the raw scores over the token's visible keys (the mask is skipped for a
    // tile the token sees whole); the softmax runs in log2 units, x = s * scale_log2
    float mt = -INFINITY;
    if (tile_start >= lo[u] && tile_start + kBlock - 1 <= hi[u]) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[u][t][i]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = tile_start + 16 * t + 4 * g + i;
          const float x = (pos >= lo[u] && pos <= hi[u]) ? s[u][t][i] : -INFINITY;
          s[u][t][i] = x;
          mt = fmaxf(mt, x);
        }
      }
    }
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    // Rescale l and the output only when some lane's running max (log2 units) moved:
    // the factor is exactly 1 otherwise.  (Letting the max lag behind, so that P may
    // exceed 1, skips more rescales but loses the exact P = 1 at the maximum and
    // measured 3x the output error.)  A token with no visible key yet keeps
    // (m, l, acc) = (-inf, 0, 0); its P is all zero.
    const float m_cand = fmaxf(m[u], mt * scale_log2);
    if (__builtin_amdgcn_ballot_w64(m_cand > m[u])) {
      const float corr = (m_cand == -INFINITY) ? 1.f : fast_exp2(m[u] - m_cand);
      lsum[u] *= corr;
#pragma unroll
      for (int dt = 0; dt < S::kDt; ++dt) acc[u][dt] *= corr;
      m[u] = m_cand;
    }
    const float mref = (m[u] == -INFINITY) ? 0.f : m[u];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(fmaf(s[u][t][i], scale_log2, -mref));
        s[u][t][i] = pv;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pb[u][h][0] = pack_bf16x2(s[u][2 * h][0], s[u][2 * h][1]);
      pb[u][h][1] = pack_bf16x2(s[u][2 * h][2], s[u][2 * h][3]);
      pb[u][h][2] = pack_bf16x2(s[u][2 * h + 1][0], s[u][2 * h + 1][1]);
      pb[u][h][3] = pack_bf16x2(s[u][2 * h + 1][2], s[u][2 * h + 1][3]);
    }
  }
  // O^T += V^T P^T.  The A operand of lane (n, g) is V[kb + j][16 dt + n] for the
  // key runs kb = 32h + 4g and 32h + 16 + 4g, j = 0..3.  ds_read_b64_tr_b16 over a
  // group of 16 lanes returns to lane 4a + b the b-th 16-bit element of the rows
  // read by lanes a, a + 4, a + 8, a + 12; so lane (n, g) points at row kb + n/4,
  // columns 16 dt + 4(n%4) .. +3.
  const uint16_t* vs = buf + S::kKElems;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int dt = 0; dt < S::kDt; ++dt) {
      u32x4 vop;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint16_t* src = vs + (32 * h + 16 * e + 4 * g + (n >> 2)) * S::kVs + 16 * dt + 4 * (n & 3);
        const uint2 w = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
        vop[2 * e] = w.x;
        vop[2 * e + 1] = w.y;
      }
      acc[0][dt] = mfma_bf16_16x16x32(vop, pb[0][h], acc[0][dt]);
      acc[1][dt] = mfma_bf16_16x16x32(vop, pb[1][h], acc[1][dt]);
    }
    // the softmax denominator as one more output tile with an all-ones A operand:
    // every row is sum_k P[k][n] over the tile's keys, from the same bf16 P as the
    // numerator
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    lsum[0] = mfma_bf16_16x16x32(ones, pb[0][h], lsum[0]);
    lsum[1] = mfma_bf16_16x16x32(ones, pb[1][h], lsum[1]);
  }
}

// The three branches for the workgroup's 16 tokens; writes
// out = g_win o_win + g_cmp o_cmp + g_slc o_slc (a branch with no keys adds 0).
template <int D>
__global__ __launch_bounds__(kPfThreads, 1) void k_prefill_shared(PaParams p) {
  using S = PfShape<D>;
  constexpr int NCH = S::kNch, NDT = S::kDt;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* bufs = reinterpret_cast<uint16_t*>(smem);
  PfSel& ps = *reinterpret_cast<PfSel*>(smem + (size_t)4 * S::kBufElems * sizeof(uint16_t));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int head = blockIdx.y, G = p.group, L = p.seq_len;
  const int tok0 = blockIdx.x * kPfTokens;
  const int last_tok = min(tok0 + kPfTokens, p.tokens) - 1;
  const int hcol = min(n, G - 1);           // columns n >= G repeat head G-1 and are never written
  const int nb = (L + kBlock - 1) / kBlock;

  // this wave's two tokens (a token past the chunk sees nothing and writes nothing)
  int tok[2], t[2];
  bool live[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = tok0 + 2 * wave + u;
    live[u] = k < p.tokens;
    tok[u] = live[u] ? k : last_tok;
    t[u] = p.q_pos0 + tok[u];
  }
  u32x4 qf[2][NCH];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint16_t* Qh = p.Q + ((size_t)tok[u] * p.hkv * G + (size_t)head * G + hcol) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[u][c] = ld16(Qh + (4 * c + g) * 8);
  }

  // the tokens' selections as bitmaps (bounds-checked block indices) and their
  // union as an ascending list
  for (int i = threadIdx.x; i < kPfTokens * kPfMaskWords; i += kPfThreads) (&ps.mask[0][0])[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < kPfTokens * p.top_k; i += kPfThreads) {
    const int u = i / p.top_k, k = tok0 + u;
    if (k < p.tokens) {
      const int b = p.sel[((size_t)k * p.hkv + head) * p.top_k + i % p.top_k];
      if (b >= 0 && b < nb) atomicOr(&ps.mask[u][b >> 5], 1u << (b & 31));
    }
  }
  __syncthreads();
  {
    const int nwords = (nb + 31) / 32;
    int cnt = 0;                               // thread i owns word i (at most 4096 blocks: 128 words)
    for (int w = threadIdx.x; w < nwords; w += kPfThreads) {
      uint32_t x = 0u;
#pragma unroll
      for (int u = 0; u < kPfTokens; ++u) x |= ps.mask[u][w];
      cnt += __builtin_popcount(x);
    }
    int total;
    int pos = pf_block_scan(cnt, ps.scan_w, &total);
    for (int w = threadIdx.x; w < nwords; w += kPfThreads) {
      uint32_t x = 0u;
#pragma unroll
      for (int u = 0; u < kPfTokens; ++u) x |= ps.mask[u][w];
      while (x) {
        const int bit = __builtin_ctz(x);
        ps.list[pos++] = 32 * w + bit;
        x &= x - 1u;
      }
    }
    if (threadIdx.x == 0) ps.count = total;
    __syncthreads();
  }

  const int t_first = p.q_pos0 + tok0, t_last = p.q_pos0 + last_tok;
  bool have_out = false;                     // uniform: an earlier branch already wrote the outputs
#pragma unroll 1
  for (int br = 0; br < 3; ++br) {             // 0 = window, 1 = pooled tokens, 2 = selected blocks
    int lo[2], hi[2], base = 0, count = 0;
    const uint16_t *Ksrc, *Vsrc;
    if (br == 0) {
      if (p.window > 0) {
        base = max(0, t_first - p.window + 1);
        count = t_last + 1 - base;
      }
      Ksrc = p.K + (size_t)head * L * D;
      Vsrc = p.V + (size_t)head * L * D;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        lo[u] = max(0, t[u] - p.window + 1);
        hi[u] = live[u] ? t[u] : -1;
      }
    } else if (br == 1) {
      if (p.cmp_on) count = t_last >= 31 ? (t_last - 31) / 16 + 1 : 0;
      Ksrc = p.kc + (size_t)head * p.nc_max * D;
      Vsrc = p.vc + (size_t)head * p.nc_max * D;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        lo[u] = 0;
        hi[u] = (live[u] && t[u] >= 31) ? (t[u] - 31) / 16 : -1;
      }
    } else {
      count = ps.count * kBlock;               // tiles = the union's blocks
      Ksrc = p.K + (size_t)head * L * D;
      Vsrc = p.V + (size_t)head * L * D;
    }
    // tile j's first position (the union's j-th block for the selected branch, else
    // the j-th 64 positions from base); its valid rows are min(64, lim - start)
    const int lim = (br == 2) ? L : base + count;
    auto tile_start = [&](int j) -> int { return (br == 2) ? ps.list[j] * kBlock : base + j * kBlock; };
    const int ntiles = (count + kBlock - 1) / kBlock;
    float m[2] = {-INFINITY, -INFINITY};
    f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 acc[2][NDT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (ntiles > 0) {
      // Tiles go in pairs (stages): stage s, tiles 2s and 2s+1, is computed from LDS
      // buffer pair s&1 after one barrier, while the global loads of the next stage
      // are in flight in the two register sets; after the compute those are stored
      // to the other buffer pair and the sets load the stage after.
      StageRegs<D> sr0, sr1;
      auto load_tile = [&](int j, StageRegs<D>& r) {
        const int st = tile_start(j);
        stage_load<D>(Ksrc + (size_t)st * D, Vsrc + (size_t)st * D, min(kBlock, lim - st), r);
      };
      auto tile_buf = [&](int j) { return bufs + ((j >> 1) & 1) * 2 * S::kBufElems + (j & 1) * S::kBufElems; };
      auto compute_tile = [&](int j) {
        const int tstart = tile_start(j);
        const int nvj = min(kBlock, lim - tstart);
        bool any = true;
        if (br == 2) {                         // a token keeps the block only if it selected it
          const int b = tstart / kBlock;
          any = false;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bool mine = live[u] && ((ps.mask[2 * wave + u][b >> 5] >> (b & 31)) & 1u);
            lo[u] = mine ? tstart : 1;
            hi[u] = mine ? tstart + nvj - 1 : 0;
            any |= mine;
          }
        }
        if (any) shared_tile<D>(tile_buf(j), tstart, lo, hi, qf, p.scale_log2, m, lsum, acc);
      };
      load_tile(0, sr0);
      if (ntiles > 1) load_tile(1, sr1);
      __syncthreads();                         // the previous branch is done with the buffers
      stage_store<D>(sr0, tile_buf(0));
      if (ntiles > 1) stage_store<D>(sr1, tile_buf(1));
      if (ntiles > 2) load_tile(2, sr0);
      if (ntiles > 3) load_tile(3, sr1);
#pragma unroll 1
      for (int j = 0; j < ntiles; j += 2) {
        __syncthreads();                       // stage j/2 staged by every thread
        compute_tile(j);
        if (j + 1 < ntiles) compute_tile(j + 1);
        if (j + 2 < ntiles) stage_store<D>(sr0, tile_buf(j + 2));
        if (j + 3 < ntiles) stage_store<D>(sr1, tile_buf(j + 3));
        if (j + 4 < ntiles) load_tile(j + 4, sr0);
        if (j + 5 < ntiles) load_tile(j + 5, sr1);
      }
    }
    // this branch's gated, normalised output goes straight to (or onto) the outputs
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float lt = lsum[u][0];                 // every row of the ones tile holds the sum
      if (live[u] && n < G) {
        const size_t row = (size_t)tok[u] * p.hkv * G + (size_t)head * G + n;
        // (cmp, slc, win); without gates the selected branch alone, weight 1
        const float gate = p.gates ? p.gates[row * 3 + (br == 0 ? 2 : br == 1 ? 0 : 1)] : (br == 2 ? 1.f : 0.f);
        const float f = lt > 0.f ? gate / lt : 0.f;
        float* op = p.out + row * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 prev = have_out ? ld_f32x4(op + 16 * dt) : f32x4{0.f, 0.f, 0.f, 0.f};
          st_f32x4(op + 16 * dt, prev + f * acc[u][dt]);   // loads see this lane's own stores
        }
      }
    }
    have_out = true;
  }
}

template <int D>
static hipError_t launch_pa(const PrefillArgs& a) {
  PaParams p;
  p.tokens = a.tokens; p.hkv = a.hkv; p.group = a.group; p.seq_len = a.max_len; p.nc_max = a.nc_max;
  p.top_k = a.top_k; p.window = a.window; p.cmp_on = a.cmp_on; p.q_pos0 = a.q_pos0;
  p.scale_log2 = a.scale * kLog2e;
  p.Q = static_cast<const uint16_t*>(a.Q); p.K = static_cast<const uint16_t*>(a.K);
  p.V = static_cast<const uint16_t*>(a.V); p.kc = static_cast<const uint16_t*>(a.kc);
  p.vc = static_cast<const uint16_t*>(a.vc); p.gates = a.gates; p.sel = a.sel; p.out = a.out;
  if ((a.max_len + kBlock - 1) / kBlock > kPfMaxBlocks || a.top_k > 64) return hipErrorInvalidValue;
  dim3 g1((a.tokens + kPfTokens - 1) / kPfTokens, a.hkv, 1);
  const size_t lds = (size_t)4 * PfShape<D>::kBufElems * sizeof(uint16_t) + sizeof(PfSel);
  hipLaunchKernelGGL((k_prefill_shared<D>), g1, dim3(kPfThreads), lds, a.stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_attn_bf16(const PrefillArgs& a) {
  return a.head_dim == 128 ? launch_pa<128>(a) : launch_pa<64>(a);
}

}  // namespace cobs
