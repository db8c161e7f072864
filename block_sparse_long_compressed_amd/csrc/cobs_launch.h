// Host-side launch descriptors between the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cobs {

struct BuildArgs {
  int batch, hkv, max_len, nb_max, nc_max, head_dim, rank;
  bool bf16;
  int blocks_per_wave;
  const int32_t* seq_lens;
  const void *K, *V;
  float *mu, *var, *lowrank;   // var: diag channel or null; lowrank: [..][NB][rank][d] or null
  void *kc, *vc;               // null when the compressed branch is off
  hipStream_t stream;
};

// Workspace carve-up shared by selection and attention (decode: tokens = 1).
struct SelectArgs {
  int batch, tokens, hkv, group, head_dim, max_len, nb_max, top_k, rank, so_kind;
  int q_pos0;                  // < 0: decode at t = L-1
  bool bf16;
  float alpha, scale;
  int splits;                  // workgroups per (seq, token, kv-head) in the scoring phase
  int tiles_per_wave;          // 16-block tiles per wave
  const int32_t* seq_lens;
  const void* Q;
  const float *mu, *so;
  int32_t* sel;
  float* sel_score;
  // workspace
  uint32_t* counters;          // [batch*tokens*hkv]
  float* scores;               // [batch*tokens*hkv][16][nb_max]
  float* lse_part;             // [batch*tokens*hkv][splits][16][2]
  hipStream_t stream;
};

struct AttnArgs {
  int batch, hkv, group, head_dim, max_len, nb_max, nc_max, top_k, window, cmp_on;
  bool bf16;
  float scale;
  int waves_per_wg;            // 1, 2 or 4
  int tiles_per_wave;
  int wg_slc, wg_win, wg_cmp;  // workgroups per (seq, kv-head) for each branch
  const int32_t* seq_lens;
  const void *Q, *K, *V, *kc, *vc;
  const float* gates;
  const int32_t* sel;          // [batch][hkv][top_k]
  float* out;
  // workspace
  uint32_t* counters;          // [batch*hkv]
  float* part_ml;              // [batch*hkv][P][16][2]
  float* part_o;               // [batch*hkv][P][group][d]
  hipStream_t stream;
};

// Chunked prefill (and selection for queries at explicit positions).
struct PrefillArgs {
  int batch, tokens, hkv, group, head_dim, max_len, nb_max, nc_max, top_k, window, cmp_on, rank, so_kind;
  int q_pos0;                  // query i at t = q_pos0 + i
  bool bf16;
  float alpha, scale;
  const int32_t* seq_lens;     // device [batch] or null (then every length is max_len)
  const void *Q, *K, *V, *kc, *vc;
  const float *mu, *so, *gates;
  int32_t* sel;
  float* sel_score;
  float* out;
  hipStream_t stream;
};

hipError_t launch_build_diag(const BuildArgs& a);
hipError_t launch_build_lowrank(const BuildArgs& a);
hipError_t launch_select(const SelectArgs& a);
hipError_t launch_attn_decode(const AttnArgs& a);
size_t attn_decode_lds_bytes(bool bf16, int head_dim, int waves);
hipError_t launch_prefill_select(const PrefillArgs& a);
hipError_t launch_prefill_attn(const PrefillArgs& a);

}  // namespace cobs
