// Host-side launch descriptors between the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cobs {

struct BuildArgs {
  int batch, hkv, max_len, nb_max, nc_max, head_dim, rank;
  bool bf16;
  const int32_t* seq_lens;     // lengths the summaries are built for
  const int32_t* old_lens;     // incremental update: lengths they were valid for (else null)
  int touch_blocks;            // incremental update: workgroups per (sequence, kv-head)
  const void *K, *V;
  void* mu;                    // fp32 [..][NB][d], or bf16 when fp4 is set
  float* var;                  // diagonal channel, or null
  void* lowrank;               // fp32 [..][NB][rank][d], or FP4 records when fp4 is set; or null
  bool fp4;                    // compressed storage: bf16 mean, MX FP4 vectors
  const float* P;              // query subspaces [hkv][sub_s][d], or null
  int sub_s, vlen;             // subspace dimension (0: none); length of a rank-r vector
  void *kc, *vc;               // null when the compressed branch is off
  hipStream_t stream;
};

// One decode launch: scoring/selection and/or attention (see k_decode.hip).
struct DecodeArgs {
  int batch, hkv, group, head_dim, max_len, nb_max, nc_max, top_k, window, cmp_on, rank, so_kind;
  bool bf16;
  float alpha, scale;
  bool do_select, do_attn;
  int splits, sel_tpw;         // scoring workgroups per (sequence, kv-head), 16-block tiles per wave
  int lead_tiles;              // selected tiles the selecting workgroup attends to itself
  int wg_slc, tpw_slc;         // further selected-branch workgroups per unit, tiles per wave
  int wg_wc;                   // window/pooled workgroups per unit
  int nw;                      // waves per workgroup (4 or 8)
  const int32_t* seq_lens;
  const void *Q, *K, *V, *kc, *vc;
  const void *mu, *so;         // summaries in the layout of so_kind (3, 5: compressed storage)
  const float* P;              // query subspaces [hkv][sub_s][d] (so_kind 4, 5), else null
  int sub_s, vlen;             // subspace dimension; length of a rank-r vector
  const float* gates;
  int32_t* sel;                // written by the selection role
  const int32_t* sel_in;       // caller's selection (attention only)
  float* sel_score;
  float* out;
  // workspace
  uint32_t *sel_counters, *attn_counters, *ready, *status;
  float *scores, *lse_part, *part_ml, *part_o;
  uint32_t poll_cap;           // polls of one selection code before a wave gives up
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
  const void *mu, *so;
  const float* P;
  int sub_s, vlen;
  const float* gates;
  int32_t* sel;
  float* sel_score;
  float* out;
  hipStream_t stream;
};

// Query-subspace calibration (see k_subspace.hip).
struct SubspaceArgs {
  int hkv, hq, group, head_dim, n, s;
  bool bf16;
  const void* Q;               // [n][hq][d] calibration queries
  float* P;                    // [hkv][s][d] out
  void* ws;                    // subspace_ws_bytes(hkv, d)
  hipStream_t stream;
};

hipError_t launch_build_diag(const BuildArgs& a);
hipError_t launch_build_lowrank(const BuildArgs& a);
hipError_t launch_append_diag(const BuildArgs& a);     // mean, diagonal, pooled tokens of touched blocks
hipError_t launch_decode(const DecodeArgs& a);
int decode_max_waves(bool bf16, int head_dim);  // most waves a decode workgroup can have
size_t decode_select_lds_bytes(int nw, int nb_pad, bool raw_in_lds);
hipError_t launch_prefill_select(const PrefillArgs& a);
hipError_t launch_prefill_attn(const PrefillArgs& a);
hipError_t launch_prefill_attn_bf16(const PrefillArgs& a);   // token-blocked, bf16 K/V
hipError_t launch_query_subspace(const SubspaceArgs& a);
size_t subspace_ws_bytes(int hkv, int d);
void* static_scratch_of_current_device();       // cobs_sparse_attn_decode_static's array, or null

}  // namespace cobs
