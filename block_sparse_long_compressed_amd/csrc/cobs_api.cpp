// C ABI of the library: argument validation, workspace planning and launches.
// Every check happens on the host before the first HIP call, so an invalid call
// enqueues nothing (see include/cobs.h for the contract).
#include "cobs.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "cobs_launch.h"

namespace {

using namespace cobs;

constexpr size_t kAlign = 256;
constexpr int kMaxBlocks = 4096;        // per sequence (selection keeps <= 16 keys per thread)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

int64_t nb_of(int max_len) { return (max_len + 63) / 64; }
int64_t nc_of(const cobs_params* p, int max_len) {
  return (p->cmp_len > 0 && max_len >= 32) ? (max_len - 32) / 16 + 1 : 0;
}
// bytes of one block's compressed low-rank record: codes, exponents, padding to 16
size_t fp4_record_bytes(int rank, int d) { return ((size_t)rank * (d / 2 + d / 32) + 15) / 16 * 16; }
// kernel-side score kinds: 0 diag, 1 low-rank fp32, 2 exact masses, 3 low-rank fp4,
// 4 and 5 the low-rank kinds in a query subspace
int kernel_kind(const cobs_params* p) {
  const int k = p->so_kind == COBS_SO_LOWRANK_FP4 ? 3 : p->so_kind;
  return p->subspace_dim > 0 ? (k == 1 ? 4 : 5) : k;
}
// length of a stored rank-r vector: the subspace dimension rounded up to 32, else d
int vec_len(const cobs_params* p) { return p->subspace_dim > 0 ? (p->subspace_dim + 31) / 32 * 32 : p->head_dim; }
float scale_of(const cobs_params* p) { return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim); }
int group_of(const cobs_params* p) { return p->n_q_heads / p->n_kv_heads; }

cobs_status check_params(const cobs_params* p) {
  if (!p) return COBS_ERR_INVALID_ARG;
  if (p->n_q_heads < 1 || p->n_kv_heads < 1 || p->n_q_heads % p->n_kv_heads) return COBS_ERR_INVALID_ARG;
  if (p->top_k < 1 || p->top_k > 64) return COBS_ERR_INVALID_ARG;
  if (p->window < 0) return COBS_ERR_INVALID_ARG;
  if (p->cmp_len < 0 || p->cmp_stride < 0) return COBS_ERR_INVALID_ARG;
  if (p->so_kind != COBS_SO_DIAG && p->so_kind != COBS_SO_LOWRANK && p->so_kind != COBS_SO_LOWRANK_FP4)
    return COBS_ERR_INVALID_ARG;
  if (p->so_kind != COBS_SO_DIAG && (p->rank < 1 || p->rank > 8)) return COBS_ERR_INVALID_ARG;
  if (p->subspace_dim < 0) return COBS_ERR_INVALID_ARG;
  if (p->subspace_dim > 0) {
    if (p->so_kind == COBS_SO_DIAG || !p->subspace || p->subspace_dim > p->head_dim) return COBS_ERR_INVALID_ARG;
  }
  if (!(p->alpha >= 0.f) || !isfinite(p->alpha)) return COBS_ERR_INVALID_ARG;
  if (!(p->scale >= 0.f) || !isfinite(p->scale)) return COBS_ERR_INVALID_ARG;
  if (p->kv_dtype != COBS_BF16 && p->kv_dtype != COBS_F32) return COBS_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return COBS_ERR_UNSUPPORTED;
  if (p->block_size != 64) return COBS_ERR_UNSUPPORTED;
  const int G = group_of(p);
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return COBS_ERR_UNSUPPORTED;
  if (p->cmp_len != 0 && !(p->cmp_len == 32 && p->cmp_stride == 16)) return COBS_ERR_UNSUPPORTED;
  return COBS_OK;
}

cobs_status check_sizes(int batch, int max_len, int tokens) {
  if (batch < 1 || max_len < 1 || tokens < 1) return COBS_ERR_INVALID_ARG;
  if (nb_of(max_len) > kMaxBlocks) return COBS_ERR_UNSUPPORTED;
  return COBS_OK;
}

// Launch shapes and the workspace carve-up; a pure function of the sizes so that
// cobs_workspace_bytes and every call agree.  Decode workgroups have NW waves (8, or 4
// for fp32 keys at d = 128, whose attention tile needs a SIMD's whole register file).
constexpr int kWideUnits = 64;          // units from which eight-wave workgroups pay off
constexpr int kLeadTilesPerWave = 2;    // selected tiles each wave of the selecting workgroup runs
constexpr int kSlcTilesPerWave = 2;     // selected tiles per wave of the other selected-branch workgroups
constexpr int kLeadTilesPerWaveNarrow = 1;   // the same with four-wave workgroups
constexpr int kSlcTilesPerWaveNarrow = 1;
constexpr int kScoreTilesPerWave = 4;   // 16-block summary tiles per wave of a whole-unit scoring workgroup
constexpr int kScoreWaves = 2048;       // scoring waves of a launch with split scoring
constexpr int kWcTilesPerWave = 5;      // target window/pooled tiles per wave (eight-wave workgroups)
constexpr int kWcTilesPerWaveNarrow = 4;   // the same with four-wave workgroups
constexpr int kFillWorkgroups = 256;    // workgroups that fill the chip once (one per CU)
constexpr size_t kDecodeLdsBudget = 150 * 1024;

struct Plan {
  int nw, splits, sel_tpw, tpw_slc;
  int lead_tiles, wg_slc, wg_wc;         // with a selecting workgroup (the fused step)
  int wg_slc_in;                         // with the caller's selection (attention only)
  size_t off_cnt_sel, off_cnt_attn, off_ready, off_status, off_scores, off_lse, off_sel, off_ml, off_o, total;
};

Plan make_plan(const cobs_params* p, int batch, int max_len, int tokens) {
  Plan pl;
  const int hkv = p->n_kv_heads, G = group_of(p), d = p->head_dim;
  const bool bf16 = p->kv_dtype == COBS_BF16;
  const int nb = (int)nb_of(max_len);
  const int nb_pad = (nb + 15) / 16 * 16;
  const int units_sel = batch * tokens * hkv;
  const int units = batch * hkv;
  const int tiles = cdiv(nb, 16);
  // Eight-wave workgroups when there are units enough to fill the chip and one
  // workgroup can score a whole unit (its scores then stay in LDS); otherwise four
  // (two per CU), with the scoring spread over many waves and handed off.
  const bool wide = decode_max_waves(bf16, d) == 8 && units >= kWideUnits &&
                    tiles <= 8 * kScoreTilesPerWave && decode_select_lds_bytes(8, nb_pad, true) <= kDecodeLdsBudget;
  pl.nw = wide ? 8 : 4;
  if (wide) {
    pl.splits = 1;
    pl.sel_tpw = cdiv(tiles, pl.nw);
  } else {
    pl.sel_tpw = std::min(8, std::max(1, cdiv(units_sel * tiles, kScoreWaves)));
    pl.splits = cdiv(tiles, pl.nw * pl.sel_tpw);
  }
  // selected branch: the lead's share, then workgroups that wait for the rest
  pl.lead_tiles = std::min(p->top_k, pl.nw * (wide ? kLeadTilesPerWave : kLeadTilesPerWaveNarrow));
  const int tpw_slc = wide ? kSlcTilesPerWave : kSlcTilesPerWaveNarrow;
  pl.tpw_slc = tpw_slc;
  pl.wg_slc = cdiv(p->top_k - pl.lead_tiles, pl.nw * tpw_slc);
  pl.wg_slc_in = cdiv(p->top_k, pl.nw * tpw_slc);
  // window and pooled tiles: about kWcTilesPerWave per wave, spread wider when the
  // units are too few to fill the chip
  const int t_win = p->window > 0 ? cdiv(std::min(p->window, max_len), 64) : 0;
  const int t_cmp = cdiv((int)nc_of(p, max_len), 64);
  const int t_wc = t_win + t_cmp;
  const int wc_tpw = wide ? kWcTilesPerWave : kWcTilesPerWaveNarrow;
  pl.wg_wc = t_wc == 0 ? 0 : std::max(cdiv(t_wc, pl.nw * wc_tpw),
                                      std::min(cdiv(t_wc, pl.nw), cdiv(kFillWorkgroups, std::max(units, 1)) - 1));
  if (t_wc > 0) pl.wg_wc = std::max(pl.wg_wc, 1);
  const int P = std::max(1 + pl.wg_slc, pl.wg_slc_in) + 2 * pl.wg_wc;   // partial slots, either mode

  // with several query tokens only the selection buffer is used (prefill path)
  const bool decode = tokens == 1;
  size_t off = 0;
  pl.off_cnt_sel = off;  off = align_up(off + sizeof(uint32_t) * units_sel);
  pl.off_cnt_attn = off; off = align_up(off + sizeof(uint32_t) * units);
  pl.off_ready = off;    off = align_up(off + sizeof(uint32_t) * (size_t)units * p->top_k);
  pl.off_status = off;   off = align_up(off + sizeof(uint32_t));
  pl.off_scores = off;   off = align_up(off + (decode && pl.splits > 1 ? sizeof(float) * (size_t)units_sel * 16 * nb_pad : 0));
  pl.off_lse = off;      off = align_up(off + (decode && pl.splits > 1 ? sizeof(float) * (size_t)units_sel * pl.splits * 32 : 0));
  pl.off_sel = off;      off = align_up(off + sizeof(int32_t) * (size_t)units_sel * p->top_k);
  pl.off_ml = off;       off = align_up(off + (decode ? sizeof(float) * (size_t)units * P * 32 : 0));
  pl.off_o = off;        off = align_up(off + (decode ? sizeof(float) * (size_t)units * P * G * d : 0));
  pl.total = off;
  return pl;
}

// Polls of one published selection code before a selected-branch wave gives up
// (about 0.1 s); lowered only by tests, through cobs_set_poll_limit.
constexpr uint32_t kDefaultPollCap = 1u << 21;
std::atomic<uint32_t> g_poll_cap{kDefaultPollCap};

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

cobs_status hip_status(hipError_t e) { return e == hipSuccess ? COBS_OK : COBS_ERR_HIP; }

}  // namespace

extern "C" {

const char* cobs_status_string(int32_t status) {
  switch (status) {
    case COBS_OK: return "ok";
    case COBS_ERR_INVALID_ARG: return "invalid argument";
    case COBS_ERR_UNSUPPORTED: return "unsupported configuration";
    case COBS_ERR_WORKSPACE: return "workspace too small";
    case COBS_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

cobs_status cobs_validate_params(const cobs_params* p) { return check_params(p); }

cobs_status cobs_summary_shapes(const cobs_params* p, int32_t batch, int32_t max_len, int64_t* nb_max,
                                int64_t* nc_max, size_t* mu_bytes, size_t* so_bytes, size_t* pooled_bytes) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, 1)) != COBS_OK) return st;
  const int64_t nb = nb_of(max_len), nc = nc_of(p, max_len);
  const size_t rows = (size_t)batch * p->n_kv_heads;
  const size_t esz = p->kv_dtype == COBS_BF16 ? 2 : 4;
  if (nb_max) *nb_max = nb;
  if (nc_max) *nc_max = nc;
  const bool fp4 = p->so_kind == COBS_SO_LOWRANK_FP4;
  if (mu_bytes) *mu_bytes = rows * nb * p->head_dim * (fp4 ? 2 : sizeof(float));
  if (so_bytes) {
    if (fp4) *so_bytes = rows * nb * fp4_record_bytes(p->rank, vec_len(p));
    else if (p->so_kind == COBS_SO_LOWRANK) *so_bytes = rows * nb * vec_len(p) * sizeof(float) * p->rank;
    else *so_bytes = rows * nb * p->head_dim * sizeof(float);
  }
  if (pooled_bytes) *pooled_bytes = rows * nc * p->head_dim * esz;
  return COBS_OK;
}

size_t cobs_workspace_bytes(const cobs_params* p, int32_t batch, int32_t max_len, int32_t n_q_tokens) {
  if (check_params(p) != COBS_OK || check_sizes(batch, max_len, n_q_tokens) != COBS_OK) return 0;
  return make_plan(p, batch, max_len, n_q_tokens).total;
}

cobs_status cobs_build_summaries(const cobs_params* p, int32_t batch, int32_t max_len, const int32_t* seq_lens,
                                 const void* K, const void* V, void* mu, void* so, void* kc, void* vc,
                                 void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, 1)) != COBS_OK) return st;
  const bool pool = p->cmp_len > 0 && nc_of(p, max_len) > 0;
  if (!seq_lens || !K || !mu || !so) return COBS_ERR_INVALID_ARG;
  if (pool && (!V || !kc || !vc)) return COBS_ERR_INVALID_ARG;
  BuildArgs a;
  a.batch = batch; a.hkv = p->n_kv_heads; a.max_len = max_len;
  a.nb_max = (int)nb_of(max_len); a.nc_max = (int)nc_of(p, max_len);
  a.head_dim = p->head_dim; a.rank = p->rank; a.bf16 = p->kv_dtype == COBS_BF16;
  a.seq_lens = seq_lens; a.K = K; a.V = pool ? V : K;
  a.mu = mu;
  a.var = p->so_kind == COBS_SO_DIAG ? static_cast<float*>(so) : nullptr;
  a.lowrank = p->so_kind == COBS_SO_DIAG ? nullptr : so;
  a.fp4 = p->so_kind == COBS_SO_LOWRANK_FP4;
  a.P = p->subspace_dim > 0 ? p->subspace : nullptr; a.sub_s = p->subspace_dim; a.vlen = vec_len(p);
  a.kc = pool ? kc : nullptr; a.vc = pool ? vc : nullptr;
  a.old_lens = nullptr; a.touch_blocks = 0;
  a.stream = (hipStream_t)stream;
  if ((st = hip_status(launch_build_diag(a))) != COBS_OK) return st;
  if (a.lowrank) st = hip_status(launch_build_lowrank(a));
  return st;
}

cobs_status cobs_update_summaries(const cobs_params* p, int32_t batch, int32_t max_len, const int32_t* old_lens,
                                  const int32_t* new_lens, int32_t max_append, const void* K, const void* V,
                                  void* mu, void* so, void* kc, void* vc, void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, 1)) != COBS_OK) return st;
  if (max_append < 1 || max_append > max_len) return COBS_ERR_INVALID_ARG;
  const bool pool = p->cmp_len > 0 && nc_of(p, max_len) > 0;
  if (!old_lens || !new_lens || !K || !mu || !so) return COBS_ERR_INVALID_ARG;
  if (pool && (!V || !kc || !vc)) return COBS_ERR_INVALID_ARG;
  BuildArgs a;
  a.batch = batch; a.hkv = p->n_kv_heads; a.max_len = max_len;
  a.nb_max = (int)nb_of(max_len); a.nc_max = (int)nc_of(p, max_len);
  a.head_dim = p->head_dim; a.rank = p->rank; a.bf16 = p->kv_dtype == COBS_BF16;
  a.seq_lens = new_lens; a.old_lens = old_lens;
  a.touch_blocks = std::min((int)a.nb_max, cdiv(max_append - 1, 64) + 2);   // blocks a run of new positions can touch
  a.K = K; a.V = pool ? V : K;
  a.mu = mu;
  a.var = p->so_kind == COBS_SO_DIAG ? static_cast<float*>(so) : nullptr;
  a.lowrank = p->so_kind == COBS_SO_DIAG ? nullptr : so;
  a.fp4 = p->so_kind == COBS_SO_LOWRANK_FP4;
  a.P = p->subspace_dim > 0 ? p->subspace : nullptr; a.sub_s = p->subspace_dim; a.vlen = vec_len(p);
  a.kc = pool ? kc : nullptr; a.vc = pool ? vc : nullptr;
  a.stream = (hipStream_t)stream;
  if ((st = hip_status(launch_append_diag(a))) != COBS_OK) return st;
  if (a.lowrank) st = hip_status(launch_build_lowrank(a));
  return st;
}

static PrefillArgs prefill_args(const cobs_params* p, int32_t batch, int32_t max_len, const int32_t* seq_lens,
                                int32_t tokens, int32_t q_pos0, hipStream_t stream) {
  PrefillArgs a;
  a.batch = batch; a.tokens = tokens; a.hkv = p->n_kv_heads; a.group = group_of(p); a.head_dim = p->head_dim;
  a.max_len = max_len; a.nb_max = (int)nb_of(max_len); a.nc_max = (int)nc_of(p, max_len); a.top_k = p->top_k;
  a.window = p->window; a.cmp_on = (p->cmp_len > 0 && nc_of(p, max_len) > 0) ? 1 : 0; a.rank = p->rank;
  a.so_kind = kernel_kind(p); a.q_pos0 = q_pos0; a.bf16 = p->kv_dtype == COBS_BF16; a.alpha = p->alpha;
  a.scale = scale_of(p); a.seq_lens = seq_lens; a.Q = a.K = a.V = a.kc = a.vc = nullptr;
  a.mu = a.so = a.gates = nullptr; a.sel = nullptr; a.sel_score = nullptr; a.out = nullptr; a.stream = stream;
  a.P = p->subspace_dim > 0 ? p->subspace : nullptr; a.sub_s = p->subspace_dim; a.vlen = vec_len(p);
  return a;
}

static DecodeArgs decode_args(const cobs_params* p, const Plan& pl, int32_t batch, int32_t max_len,
                              const int32_t* seq_lens, void* ws, hipStream_t stream) {
  DecodeArgs a;
  a.batch = batch; a.hkv = p->n_kv_heads; a.group = group_of(p); a.head_dim = p->head_dim;
  a.max_len = max_len; a.nb_max = (int)nb_of(max_len); a.nc_max = (int)nc_of(p, max_len); a.top_k = p->top_k;
  a.window = p->window; a.cmp_on = (p->cmp_len > 0 && nc_of(p, max_len) > 0) ? 1 : 0; a.rank = p->rank;
  a.so_kind = kernel_kind(p); a.bf16 = p->kv_dtype == COBS_BF16; a.alpha = p->alpha; a.scale = scale_of(p);
  a.do_select = a.do_attn = false;
  a.splits = pl.splits; a.sel_tpw = pl.sel_tpw;
  a.lead_tiles = pl.lead_tiles; a.wg_slc = pl.wg_slc; a.tpw_slc = pl.tpw_slc; a.wg_wc = pl.wg_wc; a.nw = pl.nw;
  a.seq_lens = seq_lens; a.Q = a.K = a.V = a.kc = a.vc = nullptr; a.mu = a.so = a.gates = nullptr;
  a.sel = nullptr; a.sel_in = nullptr; a.sel_score = nullptr; a.out = nullptr;
  a.P = p->subspace_dim > 0 ? p->subspace : nullptr; a.sub_s = p->subspace_dim; a.vlen = vec_len(p);
  a.sel_counters = at<uint32_t>(ws, pl.off_cnt_sel);
  a.attn_counters = at<uint32_t>(ws, pl.off_cnt_attn);
  a.ready = at<uint32_t>(ws, pl.off_ready);
  a.status = at<uint32_t>(ws, pl.off_status);
  a.scores = at<float>(ws, pl.off_scores);
  a.lse_part = at<float>(ws, pl.off_lse);
  a.part_ml = at<float>(ws, pl.off_ml);
  a.part_o = at<float>(ws, pl.off_o);
  a.poll_cap = g_poll_cap.load(std::memory_order_relaxed);
  a.stream = stream;
  return a;
}

cobs_status cobs_select_topk(const cobs_params* p, int32_t batch, int32_t max_len, const int32_t* seq_lens,
                             int32_t n_q_tokens, int32_t q_pos0, const void* Q, const void* mu, const void* so,
                             int32_t* sel, float* sel_score, void* ws, size_t ws_bytes, void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, n_q_tokens)) != COBS_OK) return st;
  if (q_pos0 < 0 && n_q_tokens != 1) return COBS_ERR_INVALID_ARG;
  if (q_pos0 >= 0 && (int64_t)q_pos0 + n_q_tokens > max_len) return COBS_ERR_INVALID_ARG;
  if (!seq_lens || !Q || !mu || !so || !sel || !ws) return COBS_ERR_INVALID_ARG;
  const Plan pl = make_plan(p, batch, max_len, n_q_tokens);
  if (ws_bytes < pl.total) return COBS_ERR_WORKSPACE;
  if (q_pos0 >= 0) {           // queries at explicit positions: one wave per (token, group)
    PrefillArgs a = prefill_args(p, batch, max_len, seq_lens, n_q_tokens, q_pos0, (hipStream_t)stream);
    a.Q = Q; a.mu = mu; a.so = so; a.sel = sel; a.sel_score = sel_score;
    return hip_status(launch_prefill_select(a));
  }
  DecodeArgs a = decode_args(p, pl, batch, max_len, seq_lens, ws, (hipStream_t)stream);
  a.do_select = true;
  a.Q = Q; a.mu = mu; a.so = so; a.sel = sel; a.sel_score = sel_score;
  return hip_status(launch_decode(a));
}

cobs_status cobs_select_topk_exact(const cobs_params* p, int32_t batch, int32_t max_len, const int32_t* seq_lens,
                                   const void* Q, const void* K, int32_t* sel, float* sel_score, void* ws,
                                   size_t ws_bytes, void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, 1)) != COBS_OK) return st;
  if (!seq_lens || !Q || !K || !sel || !ws) return COBS_ERR_INVALID_ARG;
  const Plan pl = make_plan(p, batch, max_len, 1);
  if (ws_bytes < pl.total) return COBS_ERR_WORKSPACE;
  DecodeArgs a = decode_args(p, pl, batch, max_len, seq_lens, ws, (hipStream_t)stream);
  a.do_select = true;
  a.so_kind = 2;                               // exact masses from K
  a.Q = Q; a.K = K; a.sel = sel; a.sel_score = sel_score;
  return hip_status(launch_decode(a));
}

cobs_status cobs_sparse_attn_decode(const cobs_params* p, int32_t batch, int32_t max_len, const int32_t* seq_lens,
                                    const void* Q, const void* K, const void* V, const void* mu, const void* so,
                                    const void* kc, const void* vc, const float* gates, const int32_t* sel_in,
                                    int32_t* sel_out, float* out, void* ws, size_t ws_bytes, void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, 1)) != COBS_OK) return st;
  const bool cmp_on = p->cmp_len > 0 && nc_of(p, max_len) > 0;
  if (!seq_lens || !Q || !K || !V || !out || !ws) return COBS_ERR_INVALID_ARG;
  if (!sel_in && (!mu || !so)) return COBS_ERR_INVALID_ARG;
  if (cmp_on && (!kc || !vc)) return COBS_ERR_INVALID_ARG;
  const Plan pl = make_plan(p, batch, max_len, 1);
  if (ws_bytes < pl.total) return COBS_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (sel_in && sel_out && sel_out != sel_in) {
    if (hipMemcpyAsync(sel_out, sel_in, sizeof(int32_t) * (size_t)batch * p->n_kv_heads * p->top_k,
                       hipMemcpyDeviceToDevice, s) != hipSuccess)
      return COBS_ERR_HIP;
  }
  DecodeArgs a = decode_args(p, pl, batch, max_len, seq_lens, ws, s);
  a.do_select = sel_in == nullptr;
  a.do_attn = true;
  if (sel_in) { a.lead_tiles = 0; a.wg_slc = pl.wg_slc_in; }
  a.Q = Q; a.K = K; a.V = V; a.kc = kc; a.vc = vc; a.mu = mu; a.so = so; a.gates = gates; a.out = out;
  a.sel = sel_out ? sel_out : at<int32_t>(ws, pl.off_sel);
  a.sel_in = sel_in;
  return hip_status(launch_decode(a));
}

cobs_status cobs_sparse_attn_prefill(const cobs_params* p, int32_t seq_len, int32_t n_q_tokens, int32_t q_pos0,
                                     const void* Q, const void* K, const void* V, const void* mu, const void* so,
                                     const void* kc, const void* vc, const float* gates, int32_t* sel_out,
                                     float* out, void* ws, size_t ws_bytes, void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(1, seq_len, n_q_tokens)) != COBS_OK) return st;
  if (q_pos0 < 0 || (int64_t)q_pos0 + n_q_tokens > seq_len) return COBS_ERR_INVALID_ARG;
  if (!Q || !K || !V || !mu || !so || !out || !ws) return COBS_ERR_INVALID_ARG;
  const bool cmp_on = p->cmp_len > 0 && nc_of(p, seq_len) > 0;
  if (cmp_on && (!kc || !vc)) return COBS_ERR_INVALID_ARG;
  const Plan pl = make_plan(p, 1, seq_len, n_q_tokens);
  if (ws_bytes < pl.total) return COBS_ERR_WORKSPACE;
  PrefillArgs a = prefill_args(p, 1, seq_len, nullptr, n_q_tokens, q_pos0, (hipStream_t)stream);
  a.Q = Q; a.K = K; a.V = V; a.kc = kc; a.vc = vc; a.mu = mu; a.so = so; a.gates = gates; a.out = out;
  a.sel = sel_out ? sel_out : at<int32_t>(ws, pl.off_sel);
  cobs_status st2 = hip_status(launch_prefill_select(a));
  if (st2 != COBS_OK) return st2;
  return hip_status(launch_prefill_attn(a));
}

cobs_status cobs_decode_status(const cobs_params* p, int32_t batch, int32_t max_len, void* ws, size_t ws_bytes,
                               uint32_t* flags, void* stream) {
  cobs_status st = check_params(p);
  if (st != COBS_OK) return st;
  if ((st = check_sizes(batch, max_len, 1)) != COBS_OK) return st;
  if (!flags) return COBS_ERR_INVALID_ARG;
  const Plan pl = make_plan(p, batch, max_len, 1);
  if (!ws && ws_bytes == 0) {                   // the array of cobs_sparse_attn_decode_static
    ws = static_scratch_of_current_device();
    ws_bytes = COBS_STATIC_SCRATCH_BYTES;
    if (!ws) { *flags = 0u; return COBS_OK; }   // no call on this device yet
  }
  if (!ws) return COBS_ERR_INVALID_ARG;
  if (ws_bytes < pl.total) return COBS_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* dev = at<uint32_t>(ws, pl.off_status);
  if (hipMemcpyAsync(flags, dev, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return COBS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return COBS_ERR_HIP;
  if (*flags != 0u) {
    if (hipMemsetAsync(dev, 0, sizeof(uint32_t), s) != hipSuccess) return COBS_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return COBS_ERR_HIP;
  }
  return COBS_OK;
}

void cobs_set_poll_limit(uint32_t polls) { g_poll_cap.store(polls == 0xFFFFFFFFu ? kDefaultPollCap : polls); }

size_t cobs_query_subspace_workspace_bytes(const cobs_params* p) {
  if (!p || p->n_kv_heads < 1 || (p->head_dim != 64 && p->head_dim != 128)) return 0;
  return align_up(subspace_ws_bytes(p->n_kv_heads, p->head_dim));
}

cobs_status cobs_query_subspace(const cobs_params* p, int32_t n_tokens, const void* Q, float* P_out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!p || !P_out || !Q || !ws || n_tokens < 1) return COBS_ERR_INVALID_ARG;
  cobs_params q = *p;
  q.subspace = P_out;                          // validated as the subspace it will become
  cobs_status st = check_params(&q);
  if (st != COBS_OK) return st;
  if (q.subspace_dim < 1) return COBS_ERR_INVALID_ARG;
  if (ws_bytes < cobs_query_subspace_workspace_bytes(p)) return COBS_ERR_WORKSPACE;
  SubspaceArgs a;
  a.hkv = p->n_kv_heads; a.hq = p->n_q_heads; a.group = group_of(p); a.head_dim = p->head_dim;
  a.n = n_tokens; a.s = p->subspace_dim; a.bf16 = p->kv_dtype == COBS_BF16;
  a.Q = Q; a.P = P_out; a.ws = ws; a.stream = (hipStream_t)stream;
  return hip_status(launch_query_subspace(a));
}

}  // extern "C"
