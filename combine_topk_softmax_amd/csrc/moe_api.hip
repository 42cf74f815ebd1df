// C ABI of the fused MoE layer: host-side validation, workspace planning and
// launch sequencing on the caller's streams.  No allocation, no host
// synchronisation, no device reads: everything is stream-ordered and can be
// captured into a hipGraph.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe_device.h"

using namespace moe;

// Library-held workspace of moe_forward_noalloc, used instead of a caller
// buffer.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` is only a host-side stand-in for the symbol:
// its device address on the current GPU comes from hipGetSymbolAddress (once
// per device, static_scratch below) and only that address is handed to
// kernels.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxExperts = 1024;
constexpr int64_t kInt32Max = 2147483647;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int64_t act_elem_bytes(int32_t dt) { return dt == MOE_DTYPE_F32 ? 4 : 2; }

int64_t w_elem_bytes(int32_t dt) { return dt == MOE_DTYPE_F32 ? 4 : dt == MOE_DTYPE_BF16 ? 2 : 1; }

bool fp8_path(const moe_problem &p) { return p.w_dtype == MOE_DTYPE_FP8_E4M3; }

// Checks of _moe_problem_size, the activation's 2:1 width rule,
// the format agreement of FusedMoEModularKernel.__init__ and the
// unsupported-activation error (all on the modular_kernel.py page), plus
// this library's tile and index limits.
moe_status validate(const moe_problem *pp) {
  if (!pp) return MOE_ERR_INVALID_ARG;
  const moe_problem &p = *pp;
  if (p.E < 1 || p.M < 0 || p.N < 2 || p.K < 1 || p.topk < 1) return MOE_ERR_INVALID_ARG;
  if (p.global_E < 0 || p.chunk_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (p.chunk_tokens > 0 && p.format != MOE_FORMAT_STANDARD) return MOE_ERR_UNSUPPORTED;
  const int64_t Eg = router_width(p);
  if (p.N % 2 != 0 || p.topk > Eg || p.E > Eg) return MOE_ERR_INVALID_ARG;
  if (!p.expert_map && Eg != p.E) return MOE_ERR_INVALID_ARG;   // no map: global == local
  if (p.format != MOE_FORMAT_STANDARD && p.format != MOE_FORMAT_BATCHED_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (p.scoring != MOE_SCORING_SOFTMAX && p.scoring != MOE_SCORING_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (p.align < 0 || p.shared_N < 0) return MOE_ERR_INVALID_ARG;
  if (p.format == MOE_FORMAT_BATCHED_EXPERTS && p.max_tokens_per_expert < 1) return MOE_ERR_INVALID_ARG;
  if (p.act_dtype != MOE_DTYPE_F32 && p.act_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (p.w_dtype != MOE_DTYPE_F32 && p.w_dtype != MOE_DTYPE_BF16 && p.w_dtype != MOE_DTYPE_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  if (p.act_quant != MOE_QUANT_NONE && p.act_quant != MOE_QUANT_FP8_TOKEN_GROUP_128) return MOE_ERR_INVALID_ARG;
  if (p.activation != MOE_ACTIVATION_SILU && p.activation != MOE_ACTIVATION_GELU) return MOE_ERR_UNSUPPORTED;
  if (p.apply_router_weight_on_input != 0 && p.apply_router_weight_on_input != 1) return MOE_ERR_INVALID_ARG;
  if (p.apply_router_weight_on_input && p.topk != 1) return MOE_ERR_INVALID_ARG;   // topk == 1 only
  if (p.reserved != 0) return MOE_ERR_INVALID_ARG;
  if (p.weight_layout != MOE_WEIGHTS_ROW_MAJOR && p.weight_layout != MOE_WEIGHTS_PACKED) return MOE_ERR_INVALID_ARG;
  if (Eg > kMaxExperts || p.topk > 64) return MOE_ERR_UNSUPPORTED;
  const int64_t I = p.N / 2;
  if (p.K % 128 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // dtype combinations: fp32 x fp32, bf16 x bf16, fp8-quantised x fp8
  if (fp8_path(p)) {
    if (p.act_quant != MOE_QUANT_FP8_TOKEN_GROUP_128 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  } else {
    if (p.act_quant != MOE_QUANT_NONE || p.w_dtype != p.act_dtype) return MOE_ERR_UNSUPPORTED;
  }
  if (p.shared_N > 0 && (p.shared_N % 128 != 0 || fp8_path(p))) return MOE_ERR_UNSUPPORTED;
  if (p.weight_layout == MOE_WEIGHTS_PACKED && I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t align = p.align > 0 ? p.align : 1;
  if (align > 4096) return MOE_ERR_UNSUPPORTED;
  const int64_t pairs = p.M * p.topk;
  if (pairs + p.E * (align - 1) > kInt32Max / 2) return MOE_ERR_UNSUPPORTED;
  if (p.format == MOE_FORMAT_BATCHED_EXPERTS && p.E * p.max_tokens_per_expert > kInt32Max / 2)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Tokens whose intermediates the workspace holds at once: one chunk when the
// experts step is chunked, else the whole batch.
int64_t chunk_of(const moe_problem &p) { return p.chunk_tokens > 0 ? std::min(p.M, p.chunk_tokens) : p.M; }
bool chunked(const moe_problem &p) { return p.chunk_tokens > 0 && p.chunk_tokens < p.M; }

// Picks an expert-parallel shard expects of `pairs`: its share E / global_E.
int64_t local_pairs_of(const moe_problem &p, int64_t pairs) {
  return p.global_E > p.E ? pairs * p.E / p.global_E : pairs;
}

// Weight streaming while the average expert holds no more rows than one
// streaming tile (weights then dominate the bytes); MFMA tiles otherwise.
bool streaming_of(const moe_problem &p, int64_t local_pairs) {
  const int64_t I = p.N / 2;
  return p.w_dtype != MOE_DTYPE_F32 && stream_gemm_fits(p.w_dtype, p.K, I) &&
         local_pairs <= p.E * (int64_t)stream_gemm_tile_rows(p.w_dtype);
}

// K splits of the down GEMM for an experts call over `pairs` (Standard format).
int64_t down_split_of(const moe_problem &p, int64_t pairs) {
  const int64_t lp = local_pairs_of(p, pairs);
  if (p.format != MOE_FORMAT_STANDARD || !streaming_of(p, lp)) return 1;
  return stream_gemm_down_split(p.w_dtype, p.E, lp, p.K, p.N / 2);
}

void layout(const moe_problem &p, moe_ws_layout &L) {
  memset(&L, 0, sizeof(L));
  const int64_t n = p.M * p.topk;        // pairs of the batch
  const int64_t nc = chunk_of(p) * p.topk;   // pairs of one chunk
  const int64_t E = p.E, I = p.N / 2;
  const bool standard = p.format == MOE_FORMAT_STANDARD;
  const int64_t align = p.align > 0 ? p.align : 1;
  const int64_t cap = standard ? 0 : p.max_tokens_per_expert;
  const int64_t eb = act_elem_bytes(p.act_dtype);
  const bool fp8 = fp8_path(p);

  L.perm_len = standard ? nc + E * (align - 1) : 0;
  // pairs per counting chunk, each one wavefront of the rank kernel, which
  // steps through its chunk 64 pairs at a time: 64 chunks of up to 512 pairs,
  // then up to 256 chunks (the scan walks each expert's column of chunk
  // counts, so more chunks pay only where the ranking is long)
  L.chunk = std::max<int64_t>(64, round_up((nc + 63) / 64, 64));
  if (L.chunk > 512) L.chunk = std::max<int64_t>(512, round_up((nc + 255) / 256, 64));
  L.n_chunks = std::max<int64_t>(1, (nc + L.chunk - 1) / L.chunk);
  L.tile_rows = kTileRows;
  const int64_t tiled_rows = standard ? nc : std::min(n, E * cap);
  L.max_tiles = std::max<int64_t>(1, (tiled_rows + E * (kMinPlanTileRows - 1)) / kMinPlanTileRows);
  L.act_rows = standard ? L.perm_len : E * cap;

  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    size_t at = (size_t)off;
    off = round_up(off + std::max<int64_t>(bytes, 0), kAlign);
    return at;
  };
  L.status = take(4);
  L.counts = take(4 * E);
  L.offsets = take(4 * (E + 1));
  L.chunk_hist = take(4 * L.n_chunks * E);
  L.tiles = take(4 * (L.max_tiles * 4 + 1));
  L.perm = take(4 * L.perm_len);
  L.inv = take(4 * n);
  L.act = take(L.act_rows * I * (fp8 ? 4 : eb));
  L.act_q = take(fp8 ? L.act_rows * I : 0);
  L.act_scale = take(fp8 ? L.act_rows * (I / 128) * 4 : 0);
  L.topk_weights = take(4 * n);
  L.topk_ids = take(4 * n);
  const int64_t a_rows = standard ? p.M : E * cap;
  const bool need_a = !standard || fp8 || p.apply_router_weight_on_input;
  L.a_q = take(need_a ? a_rows * p.K * (fp8 ? 1 : eb) : 0);
  L.a_scale = take(need_a && fp8 ? a_rows * (p.K / 128) * 4 : 0);
  L.fused_out = take((standard ? n : E * cap) * p.K * eb);
  L.shared_act = take(p.shared_N > 0 ? p.M * (p.shared_N / 2) * eb : 0);
  L.down_split = down_split_of(p, nc);
  L.down_partial = take(L.down_split > 1 ? L.down_split * L.perm_len * p.K * 4 : 0);
  L.total_bytes = (size_t)off;
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<uint8_t *>(ws) + off);
}

#define MOE_HIP(call)                      \
  do {                                     \
    if ((call) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

moe_status check_ws(const moe_problem &p, void *ws, size_t ws_bytes, moe_ws_layout &L) {
  layout(p, L);
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total_bytes) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

void record(const moe_stage_events *ev, int i, hipStream_t s) {
  if (ev && ev->ev[i]) (void)hipEventRecord(ev->ev[i], s);
}

// Whether prepare writes the activations the experts read (a_out), rather
// than the experts reading x directly.
bool prepared_rows(const moe_problem &p) {
  return p.format == MOE_FORMAT_BATCHED_EXPERTS || p.act_quant == MOE_QUANT_FP8_TOKEN_GROUP_128 ||
         p.apply_router_weight_on_input;
}

// Rows per tile of the grouped GEMMs' plan: the streaming kernels' (wide
// fp8 panels take shorter tiles), the 256-row MFMA tiles, or the general
// kernel's.
int gemm_tile_rows(const moe_problem &p, const moe_ws_layout &L) {
  const int64_t I = p.N / 2;
  const int64_t local_pairs = local_pairs_of(p, p.M * p.topk);
  const bool streaming = streaming_of(p, local_pairs);
  const bool big = !streaming && mfma_gemm_fits(p.w_dtype, p.act_dtype, p.K, I, p.M);
  const bool wide = streaming && stream_gemm_gated_wide(p.w_dtype, p.E, local_pairs, p.K, I);
  return wide ? stream_gemm_wide_tile_rows() : streaming ? stream_gemm_tile_rows(p.w_dtype)
                                             : big       ? mfma_gemm_tile_rows()
                                                         : (int)L.tile_rows;
}

// Counts and permutation of p.M tokens' pairs (ids), their pair -> slot map
// written from inv_pair0 on (a chunk's pairs within the batch's map).  With
// plan set, small batches also get the GEMMs' tile plan from the same
// kernel; returns through *planned whether they did.
moe_status do_count(const moe_problem &p, const int32_t *ids, int32_t *expert_num_tokens, void *ws,
                    const moe_ws_layout &L, int64_t inv_pair0, hipStream_t s, bool plan = false,
                    bool *planned = nullptr) {
  DispatchBufs b;
  b.status = at<int32_t>(ws, L.status);
  b.counts = at<int32_t>(ws, L.counts);
  b.offsets = at<int32_t>(ws, L.offsets);
  b.chunk_hist = at<int32_t>(ws, L.chunk_hist);
  b.perm = at<int32_t>(ws, L.perm);
  b.inv = at<int32_t>(ws, L.inv) + inv_pair0;
  b.perm_len = L.perm_len;
  b.n_chunks = L.n_chunks;
  b.chunk = L.chunk;
  b.clear_status = inv_pair0 == 0;
  b.tiles = at<int32_t>(ws, L.tiles);
  b.max_tiles = (int)L.max_tiles;
  b.plan_rows = plan && count_fused(p) ? gemm_tile_rows(p, L) : 0;
  MOE_HIP(launch_count_and_permute(p, ids, expert_num_tokens, b, s));
  if (planned) *planned = b.plan_rows > 0;
  return MOE_OK;
}

// The rows the experts read, when prepare writes them (quantised, batched or
// router-weighted); the batched scatter reads the pair -> row map.
moe_status do_rows(const moe_problem &p, const void *x, const float *topk_w, void *a_out, float *a_scale_out,
                   void *ws, const moe_ws_layout &L, hipStream_t s) {
  if (!prepared_rows(p)) return MOE_OK;
  const bool batched = p.format == MOE_FORMAT_BATCHED_EXPERTS;
  MOE_HIP(launch_dispatch_rows(p, x, at<int32_t>(ws, L.inv), p.apply_router_weight_on_input ? topk_w : nullptr,
                               a_out, a_scale_out, batched, s));
  return MOE_OK;
}

moe_status do_prepare(const moe_problem &p, const void *x, const int32_t *ids, const float *topk_w,
                      void *a_out, float *a_scale_out, int32_t *expert_num_tokens, void *ws,
                      const moe_ws_layout &L, hipStream_t s, bool plan = false, bool *planned = nullptr) {
  moe_status st = do_count(p, ids, expert_num_tokens, ws, L, 0, s, plan, planned);
  if (st != MOE_OK) return st;
  return do_rows(p, x, topk_w, a_out, a_scale_out, ws, L, s);
}

// The shared expert's launch on its aux stream, started from the main stream's
// position at the time of the call.
struct SharedStart {
  const moe_problem *p;
  const void *x;
  const moe_shared *shared;
  void *ws;
  const moe_ws_layout *L;
};

moe_status do_shared(const moe_problem &p, const void *x, const void *w1, const void *w2, void *out,
                     void *ws, const moe_ws_layout &L, hipStream_t s);

moe_status start_shared(const SharedStart &sh, hipStream_t main) {
  MOE_HIP(hipEventRecord(sh.shared->input_ready, main));
  MOE_HIP(hipStreamWaitEvent(sh.shared->aux_stream, sh.shared->input_ready, 0));
  const moe_status st = do_shared(*sh.p, sh.x, sh.shared->w1, sh.shared->w2, sh.shared->out, sh.ws, *sh.L,
                                  sh.shared->aux_stream);
  if (st != MOE_OK) return st;
  MOE_HIP(hipEventRecord(sh.shared->output_ready, sh.shared->aux_stream));
  return MOE_OK;
}

// The down GEMM's K-split partial sums, when the caller combines them itself.
struct SplitPartials {
  const float *part = nullptr;   // null: the rows were reduced into fused_out
  int S = 0;
  int64_t stride = 0;
};

// sh: start the shared expert once the gated grouped GEMM is queued.  Its
// GEMMs fill every compute unit: started with the layer, they held the units
// the short counting and planning kernels waited for (DeepSeek-V3 shape:
// 0.33 ms instead of 0.04); overlapping the gated GEMM, they slowed it by
// 0.35 ms; overlapping the down GEMM costs about 0.3 ms and measured best.
moe_status do_experts(const moe_problem &p, const void *a, const float *a_scale, const moe_weights &w,
                      const int32_t *counts, void *fused_out, void *ws, const moe_ws_layout &L,
                      hipStream_t s, const moe_stage_events *ev, const SharedStart *sh = nullptr,
                      SplitPartials *sp = nullptr, bool planned = false) {
  const bool standard = p.format == MOE_FORMAT_STANDARD;
  const bool fp8 = fp8_path(p);
  const int64_t I = p.N / 2;
  int32_t *tiles = at<int32_t>(ws, L.tiles);
  int32_t *status = at<int32_t>(ws, L.status);
  int32_t *perm = standard ? at<int32_t>(ws, L.perm) : nullptr;
  const int64_t local_pairs = local_pairs_of(p, p.M * p.topk);
  const bool streaming = streaming_of(p, local_pairs);
  // Past that point the GEMMs are bound by the matrix cores: 128 x 256 tiles
  // where the shapes allow, the general 128 x 128 kernel otherwise.
  const bool big = !streaming && mfma_gemm_fits(p.w_dtype, p.act_dtype, p.K, I, p.M);
  const bool wide = streaming && stream_gemm_gated_wide(p.w_dtype, p.E, local_pairs, p.K, I);
  // (a small batch's counting kernel already wrote the plan)
  if (!planned)
    MOE_HIP(launch_plan_tiles(p, counts, at<int32_t>(ws, L.offsets), L.perm_len, gemm_tile_rows(p, L),
                              (int)L.max_tiles, tiles, status, s));
  record(ev, 2, s);
  GemmTiles gt;
  gt.tiles = tiles;
  gt.tile_count = tiles + L.max_tiles * 4;
  gt.max_tiles = (int)L.max_tiles;
  gt.dense_rows = 0;

  GemmParams g1;
  memset(&g1, 0, sizeof(g1));
  g1.a = a;
  g1.a_scale = a_scale;
  g1.perm = perm;
  g1.topk = (int)p.topk;
  g1.n_pairs = (int)(p.M * p.topk);
  g1.w = w.w1;
  g1.w_scale = w.w1_scale;
  g1.Nw = p.N;
  g1.Kred = p.K;
  g1.out = at<void>(ws, L.act);
  g1.ldo = I;
  g1.half_n = I;
  g1.act = p.activation;
  g1.w_packed = p.weight_layout == MOE_WEIGHTS_PACKED;
  g1.t = gt;
  if (streaming && fp8) {
    // the gated GEMM quantises act itself (one 128-column group per tile)
    g1.out = at<void>(ws, L.act_q);
    g1.out_scale = at<float>(ws, L.act_scale);
  }
  if (streaming) {
    MOE_HIP(launch_stream_gemm(p.w_dtype, fp8 ? MOE_DTYPE_F32 : p.act_dtype, kGemmGatedAct, g1, (int)(I / 128),
                               wide ? 4 : 2, s));
  }
  else if (big)
    MOE_HIP(launch_mfma_gemm(kGemmGatedAct, g1, mfma_gemm_n_tiles(kGemmGatedAct, g1.Nw), s));
  else
    MOE_HIP(launch_grouped_gemm(p.w_dtype, fp8 ? MOE_DTYPE_F32 : p.act_dtype, kGemmGatedAct, g1,
                                (int)(I / 64), s));
  record(ev, 3, s);
  if (sh) {
    const moe_status st = start_shared(*sh, s);
    if (st != MOE_OK) return st;
  }
  if (fp8 && !streaming)
    MOE_HIP(launch_quant_rows(at<float>(ws, L.act), tiles, (int)L.max_tiles, I, at<uint8_t>(ws, L.act_q),
                              at<float>(ws, L.act_scale), s));

  GemmParams g2;
  memset(&g2, 0, sizeof(g2));
  g2.a = fp8 ? at<void>(ws, L.act_q) : at<void>(ws, L.act);
  g2.a_scale = fp8 ? at<float>(ws, L.act_scale) : nullptr;
  g2.perm = nullptr;
  g2.topk = (int)p.topk;
  g2.n_pairs = (int)(p.M * p.topk);
  g2.w = w.w2;
  g2.w_scale = w.w2_scale;
  g2.Nw = p.K;
  g2.Kred = I;
  g2.out = fused_out;
  g2.ldo = p.K;
  g2.out_perm = perm;
  g2.half_n = 0;
  g2.w_packed = p.weight_layout == MOE_WEIGHTS_PACKED;
  g2.t = gt;
  // a split needs the partial-sum buffer the layout reserved for it (a
  // shorter last chunk may pick a split its layout did not)
  const int64_t split = down_split_of(p, p.M * p.topk);
  if (streaming && split > 1 && split == L.down_split) {
    g2.out = at<void>(ws, L.down_partial);
    g2.out_perm = nullptr;
    g2.k_split = (int)split;
    g2.split_stride = L.perm_len * p.K;
    MOE_HIP(launch_stream_gemm(p.w_dtype, MOE_DTYPE_F32, kGemmDown, g2, (int)(p.K / 128), 2, s));
    if (sp) {
      // sp: the caller's combine reads the partial sums (fused_out stays unwritten)
      sp->part = at<float>(ws, L.down_partial);
      sp->S = (int)split;
      sp->stride = g2.split_stride;
    } else {
      MOE_HIP(launch_split_reduce(at<float>(ws, L.down_partial), (int)split, g2.split_stride, perm, L.perm_len,
                                  g2.n_pairs, (int)p.K, p.act_dtype, fused_out, s));
    }
  } else if (streaming) {
    const int nbw = stream_gemm_down_plan(p.w_dtype, p.E, local_pairs, p.K, I, &g2.bal_p, &g2.bal_h);
    MOE_HIP(launch_stream_gemm(p.w_dtype, p.act_dtype, kGemmDown, g2, (int)(p.K / 128), nbw, s));
  }
  else if (big)
    MOE_HIP(launch_mfma_gemm(kGemmDown, g2, mfma_gemm_n_tiles(kGemmDown, g2.Nw), s));
  else
    MOE_HIP(launch_grouped_gemm(p.w_dtype, p.act_dtype, kGemmDown, g2, (int)(p.K / 128), s));
  record(ev, 4, s);
  return MOE_OK;
}

moe_status do_shared(const moe_problem &p, const void *x, const void *w1, const void *w2, void *out,
                     void *ws, const moe_ws_layout &L, hipStream_t s) {
  const int64_t Is = p.shared_N / 2;
  GemmTiles gt;
  gt.tiles = nullptr;
  gt.tile_count = nullptr;
  gt.max_tiles = 0;
  gt.dense_rows = (int)p.M;
  GemmParams g1;
  memset(&g1, 0, sizeof(g1));
  g1.a = x;
  g1.topk = 1;
  g1.n_pairs = (int)p.M;
  g1.w = w1;
  g1.Nw = p.shared_N;
  g1.Kred = p.K;
  g1.out = at<void>(ws, L.shared_act);
  g1.ldo = Is;
  g1.half_n = Is;
  g1.act = p.activation;
  g1.t = gt;
  const bool big = mfma_gemm_fits(p.act_dtype, p.act_dtype, p.K, Is, p.M);
  if (big)
    MOE_HIP(launch_mfma_gemm(kGemmGatedAct, g1, mfma_gemm_n_tiles(kGemmGatedAct, g1.Nw), s));
  else
    MOE_HIP(launch_grouped_gemm(p.act_dtype, p.act_dtype, kGemmGatedAct, g1, (int)(Is / 64), s));
  GemmParams g2;
  memset(&g2, 0, sizeof(g2));
  g2.a = at<void>(ws, L.shared_act);
  g2.topk = 1;
  g2.n_pairs = (int)p.M;
  g2.w = w2;
  g2.Nw = p.K;
  g2.Kred = Is;
  g2.out = out;
  g2.ldo = p.K;
  g2.t = gt;
  if (big)
    MOE_HIP(launch_mfma_gemm(kGemmDown, g2, mfma_gemm_n_tiles(kGemmDown, g2.Nw), s));
  else
    MOE_HIP(launch_grouped_gemm(p.act_dtype, p.act_dtype, kGemmDown, g2, (int)(p.K / 128), s));
  return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream`, which must be
// the current device (the lookup is made with that device current).
moe_status static_scratch(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_HIP;
    if (sdev != dev) return MOE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The argument checks of moe_forward (M > 0).
moe_status forward_args(const moe_problem &p, const float *logits, const void *x, const moe_weights *w,
                        const void *out, const moe_shared *shared) {
  if (!logits || !x || !w || !w->w1 || !w->w2 || !out) return MOE_ERR_INVALID_ARG;
  if (fp8_path(p) && (!w->w1_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
  if (shared) {
    if (!shared->w1 || !shared->w2 || !shared->out || !shared->aux_stream || !shared->input_ready ||
        !shared->output_ready)
      return MOE_ERR_INVALID_ARG;
    if (out == x || shared->out == x) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

// ------------------------------------------- two-microbatch (DBO) schedule
// The routed layer of one microbatch, in the three parts the two-microbatch
// schedule puts on different streams: route + prepare (dispatch), the
// experts, and finalize (combine).
struct FwdBatch {
  moe_problem p;              // M = this microbatch's tokens
  const float *logits;
  const void *x;
  void *out;
  const moe_shared *shared;   // this microbatch's shared-expert streams and events, or null
  void *ws;
  moe_ws_layout L;
  SplitPartials sp;
  bool planned = false;       // the counting kernel wrote the tile plan
};

moe_status fwd_route_prepare(FwdBatch &b, hipStream_t s) {
  const moe_problem &p = b.p;
  float *tw = at<float>(b.ws, b.L.topk_weights);
  int32_t *ti = at<int32_t>(b.ws, b.L.topk_ids);
  MOE_HIP(launch_route(p, b.logits, tw, ti, s));
  void *a_q = prepared_rows(p) ? at<void>(b.ws, b.L.a_q) : nullptr;
  float *a_s = p.act_quant == MOE_QUANT_FP8_TOKEN_GROUP_128 ? at<float>(b.ws, b.L.a_scale) : nullptr;
  return do_prepare(p, b.x, ti, tw, a_q, a_s, at<int32_t>(b.ws, b.L.counts), b.ws, b.L, s, true, &b.planned);
}

moe_status fwd_experts(FwdBatch &b, const moe_weights &w, hipStream_t s) {
  const moe_problem &p = b.p;
  void *a_q = prepared_rows(p) ? at<void>(b.ws, b.L.a_q) : nullptr;
  float *a_s = p.act_quant == MOE_QUANT_FP8_TOKEN_GROUP_128 ? at<float>(b.ws, b.L.a_scale) : nullptr;
  const SharedStart sh{&b.p, b.x, b.shared, b.ws, &b.L};
  return do_experts(p, a_q ? a_q : b.x, a_s, w, at<int32_t>(b.ws, b.L.counts), at<void>(b.ws, b.L.fused_out), b.ws,
                    b.L, s, nullptr, b.shared ? &sh : nullptr, &b.sp, b.planned);
}

moe_status fwd_finalize(FwdBatch &b, hipStream_t s) {
  const moe_problem &p = b.p;
  const float *cw = p.apply_router_weight_on_input ? nullptr : at<float>(b.ws, b.L.topk_weights);
  const int32_t *inv = at<int32_t>(b.ws, b.L.inv);
  if (b.sp.part)
    MOE_HIP(launch_combine_split(p, b.sp.part, b.sp.S, b.sp.stride, cw, inv, b.out, s));
  else
    MOE_HIP(launch_combine(p, at<void>(b.ws, b.L.fused_out), cw, inv, p.format != MOE_FORMAT_STANDARD, b.out, s));
  return MOE_OK;
}

__global__ void copy_status_kernel(const int32_t *__restrict__ from, int32_t *__restrict__ to) { *to = *from; }

}  // namespace

extern "C" {

const char *moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int moe_version(void) { return 5; }

moe_status moe_validate(const moe_problem *p) { return validate(p); }

moe_status moe_workspace_layout(const moe_problem *p, moe_ws_layout *out) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_INVALID_ARG;
  layout(*p, *out);
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_problem *p, size_t *bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_ws_layout L;
  moe_status st = moe_workspace_layout(p, &L);
  if (st == MOE_OK) *bytes = L.total_bytes;
  return st;
}

moe_status moe_pack_weights(const moe_problem *p, const moe_weights *src, void *w1_packed,
                            void *w2_packed, hipStream_t stream) {
  if (!p) return MOE_ERR_INVALID_ARG;
  moe_problem q = *p;
  q.weight_layout = MOE_WEIGHTS_PACKED;   // the target layout's constraints apply
  moe_status st = validate(&q);
  if (st != MOE_OK) return st;
  if (!src || !src->w1 || !src->w2 || !w1_packed || !w2_packed) return MOE_ERR_INVALID_ARG;
  if (w1_packed == src->w1 || w2_packed == src->w2) return MOE_ERR_INVALID_ARG;
  const int64_t eb = w_elem_bytes(p->w_dtype), I = p->N / 2;
  MOE_HIP(launch_pack_weights(src->w1, w1_packed, p->E, p->N, p->K * eb, true, stream));
  MOE_HIP(launch_pack_weights(src->w2, w2_packed, p->E, p->K, I * eb, false, stream));
  return MOE_OK;
}

moe_status moe_route(const moe_problem *p, const float *logits, float *topk_weights,
                     int32_t *topk_ids, hipStream_t stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->M == 0) return MOE_OK;
  if (!logits || !topk_weights || !topk_ids) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_route(*p, logits, topk_weights, topk_ids, stream));
  return MOE_OK;
}

moe_status moe_prepare(const moe_problem *p, const void *x, const int32_t *topk_ids,
                       const float *topk_weights, void *a_out, float *a_scale_out,
                       int32_t *expert_num_tokens, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->M == 0) return MOE_OK;
  if (chunked(*p)) return MOE_ERR_UNSUPPORTED;   // chunking is moe_forward's
  moe_ws_layout L;
  if ((st = check_ws(*p, workspace, workspace_bytes, L)) != MOE_OK) return st;
  if (!x || !topk_ids || !expert_num_tokens) return MOE_ERR_INVALID_ARG;
  const bool quant = p->act_quant == MOE_QUANT_FP8_TOKEN_GROUP_128;
  const bool rows = prepared_rows(*p);
  if (rows && !a_out) return MOE_ERR_INVALID_ARG;
  if (quant && !a_scale_out) return MOE_ERR_INVALID_ARG;
  if (!rows && (a_out || a_scale_out)) return MOE_ERR_INVALID_ARG;
  if (p->apply_router_weight_on_input && !topk_weights) return MOE_ERR_INVALID_ARG;
  return do_prepare(*p, x, topk_ids, topk_weights, a_out, a_scale_out, expert_num_tokens, workspace, L,
                    stream);
}

moe_status moe_experts(const moe_problem *p, const void *a, const float *a_scale,
                       const moe_weights *w, const int32_t *expert_num_tokens, void *fused_out,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->M == 0) return MOE_OK;
  if (chunked(*p)) return MOE_ERR_UNSUPPORTED;
  moe_ws_layout L;
  if ((st = check_ws(*p, workspace, workspace_bytes, L)) != MOE_OK) return st;
  if (!a || !w || !w->w1 || !w->w2 || !expert_num_tokens || !fused_out) return MOE_ERR_INVALID_ARG;
  if (fp8_path(*p) && (!a_scale || !w->w1_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
  return do_experts(*p, a, a_scale, *w, expert_num_tokens, fused_out, workspace, L, stream, nullptr);
}

moe_status moe_finalize(const moe_problem *p, const void *fused_out, const float *topk_weights,
                        void *out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->M == 0) return MOE_OK;
  moe_ws_layout L;
  if ((st = check_ws(*p, workspace, workspace_bytes, L)) != MOE_OK) return st;
  if (!fused_out || !out || (!topk_weights && !p->apply_router_weight_on_input)) return MOE_ERR_INVALID_ARG;
  const bool batched = p->format == MOE_FORMAT_BATCHED_EXPERTS;
  // the pair -> slot map moe_prepare wrote masks every pair it did not place
  // (bad ids, other shards' picks, dropped batched picks), whose rows of
  // fused_out the experts step never wrote
  MOE_HIP(launch_combine(*p, fused_out, p->apply_router_weight_on_input ? nullptr : topk_weights,
                         at<int32_t>(workspace, L.inv), batched, out, stream));
  return MOE_OK;
}

moe_status moe_shared_expert(const moe_problem *p, const void *x, const void *w1, const void *w2,
                             void *out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->shared_N <= 0) return MOE_ERR_INVALID_ARG;
  if (p->M == 0) return MOE_OK;
  moe_ws_layout L;
  if ((st = check_ws(*p, workspace, workspace_bytes, L)) != MOE_OK) return st;
  if (!x || !w1 || !w2 || !out) return MOE_ERR_INVALID_ARG;
  return do_shared(*p, x, w1, w2, out, workspace, L, stream);
}

moe_status moe_forward(const moe_problem *p, const float *logits, const void *x,
                       const moe_weights *w, void *out, const moe_shared *shared,
                       void *workspace, size_t workspace_bytes, hipStream_t stream,
                       const moe_stage_events *events) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if ((shared != nullptr) != (p->shared_N > 0)) return MOE_ERR_INVALID_ARG;
  if (p->M == 0) return MOE_OK;
  moe_ws_layout L;
  if ((st = check_ws(*p, workspace, workspace_bytes, L)) != MOE_OK) return st;
  if ((st = forward_args(*p, logits, x, w, out, shared)) != MOE_OK) return st;
  record(events, 0, stream);
  // Shared expert on the aux stream, overlapping the routed path: from the
  // down GEMM on, or from the start when the experts step is chunked.
  const SharedStart sh{p, x, shared, workspace, &L};
  if (shared && chunked(*p) && (st = start_shared(sh, stream)) != MOE_OK) return st;
  float *tw = at<float>(workspace, L.topk_weights);
  int32_t *ti = at<int32_t>(workspace, L.topk_ids);
  MOE_HIP(launch_route(*p, logits, tw, ti, stream));
  record(events, 1, stream);

  const bool standard = p->format == MOE_FORMAT_STANDARD;
  const bool quant = p->act_quant == MOE_QUANT_FP8_TOKEN_GROUP_128;
  void *a_q = prepared_rows(*p) ? at<void>(workspace, L.a_q) : nullptr;
  float *a_s = quant ? at<float>(workspace, L.a_scale) : nullptr;
  int32_t *counts = at<int32_t>(workspace, L.counts);
  void *fused = at<void>(workspace, L.fused_out);
  SplitPartials sp;   // set when the down GEMM split K: the combine reads its partial sums
  if (!chunked(*p)) {
    bool planned = false;
    if ((st = do_prepare(*p, x, ti, tw, a_q, a_s, counts, workspace, L, stream, true, &planned)) != MOE_OK)
      return st;
    if ((st = do_experts(*p, a_q ? a_q : x, a_s, *w, counts, fused, workspace, L, stream, events,
                         shared ? &sh : nullptr, &sp, planned)) != MOE_OK)
      return st;
  } else {
    // Prepare the whole batch's rows, then count, permute and run the experts
    // chunk by chunk (stage events then mark the last chunk's boundaries).
    if ((st = do_rows(*p, x, tw, a_q, a_s, workspace, L, stream)) != MOE_OK) return st;
    const int64_t a_row_bytes = a_q ? (quant ? p->K : p->K * act_elem_bytes(p->act_dtype))
                                    : p->K * act_elem_bytes(p->act_dtype);
    const int64_t out_row_bytes = p->K * act_elem_bytes(p->act_dtype);
    for (int64_t m0 = 0; m0 < p->M; m0 += p->chunk_tokens) {
      moe_problem pc = *p;
      pc.M = std::min(p->chunk_tokens, p->M - m0);
      const int64_t pair0 = m0 * p->topk;
      bool planned = false;
      if ((st = do_count(pc, ti + pair0, counts, workspace, L, pair0, stream, true, &planned)) != MOE_OK) return st;
      const uint8_t *a = reinterpret_cast<const uint8_t *>(a_q ? a_q : x) + m0 * a_row_bytes;
      const float *as = a_s ? a_s + m0 * (p->K / 128) : nullptr;
      void *fo = reinterpret_cast<uint8_t *>(fused) + pair0 * out_row_bytes;
      if ((st = do_experts(pc, a, as, *w, counts, fo, workspace, L, stream, events, nullptr, nullptr, planned)) !=
          MOE_OK)
        return st;
    }
  }
  // the permutation prepare just wrote masks dropped / other shards' pairs
  const float *cw = p->apply_router_weight_on_input ? nullptr : tw;
  if (sp.part)
    MOE_HIP(launch_combine_split(*p, sp.part, sp.S, sp.stride, cw, at<int32_t>(workspace, L.inv), out, stream));
  else
    MOE_HIP(launch_combine(*p, fused, cw, at<int32_t>(workspace, L.inv), !standard, out, stream));
  record(events, 5, stream);
  if (shared) MOE_HIP(hipStreamWaitEvent(stream, shared->output_ready, 0));
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_problem *p, const float *logits, const void *x,
                               const moe_weights *w, void *out, const moe_shared *shared,
                               hipStream_t stream, const moe_stage_events *events, int32_t *status_out) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if ((shared != nullptr) != (p->shared_N > 0)) return MOE_ERR_INVALID_ARG;
  if (p->M == 0) return MOE_OK;
  moe_ws_layout L;
  layout(*p, L);
  if (L.total_bytes > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if ((st = forward_args(*p, logits, x, w, out, shared)) != MOE_OK) return st;
  void *ws = nullptr;
  if ((st = static_scratch(stream, &ws)) != MOE_OK) return st;
  if ((st = moe_forward(p, logits, x, w, out, shared, ws, MOE_STATIC_SCRATCH_BYTES, stream, events)) != MOE_OK)
    return st;
  if (status_out) {
    copy_status_kernel<<<1, 1, 0, stream>>>(at<int32_t>(ws, L.status), status_out);
    MOE_HIP(hipGetLastError());
  }
  return MOE_OK;
}

moe_status moe_prepare_async(const moe_problem *p, const void *x, const int32_t *topk_ids,
                             const float *topk_weights, void *a_out, float *a_scale_out,
                             int32_t *expert_num_tokens, void *workspace, size_t workspace_bytes,
                             hipStream_t stream, hipEvent_t done) {
  if (!done) return MOE_ERR_INVALID_ARG;
  const moe_status st = moe_prepare(p, x, topk_ids, topk_weights, a_out, a_scale_out, expert_num_tokens, workspace,
                                    workspace_bytes, stream);
  if (st != MOE_OK) return st;
  MOE_HIP(hipEventRecord(done, stream));
  return MOE_OK;
}

moe_status moe_finalize_async(const moe_problem *p, const void *fused_out, const float *topk_weights,
                              void *out, void *workspace, size_t workspace_bytes, hipStream_t stream,
                              hipEvent_t done) {
  if (!done) return MOE_ERR_INVALID_ARG;
  const moe_status st = moe_finalize(p, fused_out, topk_weights, out, workspace, workspace_bytes, stream);
  if (st != MOE_OK) return st;
  MOE_HIP(hipEventRecord(done, stream));
  return MOE_OK;
}

moe_status moe_receive(hipStream_t stream, hipEvent_t done) {
  if (!done) return MOE_ERR_INVALID_ARG;
  MOE_HIP(hipStreamWaitEvent(stream, done, 0));
  return MOE_OK;
}

moe_status moe_forward_dbo(const moe_problem *p, const float *logits, const void *x, const moe_weights *w,
                           void *out, const moe_shared *shared, void *workspace0, void *workspace1,
                           size_t workspace_bytes, hipStream_t compute_stream, hipStream_t comm_stream,
                           const moe_dbo_events *ev) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if ((shared != nullptr) != (p->shared_N > 0)) return MOE_ERR_INVALID_ARG;
  if (chunked(*p)) return MOE_ERR_UNSUPPORTED;
  if (p->M == 0) return MOE_OK;
  if (!ev) return MOE_ERR_INVALID_ARG;
  for (int u = 0; u < 2; ++u)
    if (!ev->prepared[u] || !ev->computed[u] || !ev->finalized[u]) return MOE_ERR_INVALID_ARG;
  if (!logits || !x || !out) return MOE_ERR_INVALID_ARG;
  // microbatch 0: the first (M + 1) / 2 tokens, microbatch 1: the rest
  const int64_t Mu[2] = {(p->M + 1) / 2, p->M / 2};
  const int64_t row_bytes = p->K * act_elem_bytes(p->act_dtype);
  void *ws[2] = {workspace0, workspace1};
  FwdBatch b[2];
  const int nb = Mu[1] > 0 ? 2 : 1;
  for (int u = 0; u < nb; ++u) {
    const int64_t m0 = u == 0 ? 0 : Mu[0];
    b[u].p = *p;
    b[u].p.M = Mu[u];
    b[u].logits = logits + m0 * router_width(*p);
    b[u].x = reinterpret_cast<const uint8_t *>(x) + m0 * row_bytes;
    b[u].out = reinterpret_cast<uint8_t *>(out) + m0 * row_bytes;
    b[u].shared = shared ? &shared[u] : nullptr;
    b[u].ws = ws[u];
    if ((st = check_ws(b[u].p, ws[u], workspace_bytes, b[u].L)) != MOE_OK) return st;
    if ((st = forward_args(b[u].p, b[u].logits, b[u].x, w, b[u].out, b[u].shared)) != MOE_OK) return st;
  }
  if (nb == 2 && workspace0 == workspace1) return MOE_ERR_INVALID_ARG;
  // The comm stream starts from the compute stream's position.
  MOE_HIP(hipEventRecord(ev->finalized[1], compute_stream));
  MOE_HIP(hipStreamWaitEvent(comm_stream, ev->finalized[1], 0));
  // Dispatch side: both microbatches' route + prepare, back to back; the
  // second overlaps the first one's expert GEMMs.
  for (int u = 0; u < nb; ++u) {
    if ((st = fwd_route_prepare(b[u], comm_stream)) != MOE_OK) return st;
    MOE_HIP(hipEventRecord(ev->prepared[u], comm_stream));
  }
  // Compute side: each microbatch's experts once its dispatch is in; the
  // combine of microbatch 0 runs on the comm stream beside microbatch 1's
  // experts.
  for (int u = 0; u < nb; ++u) {
    MOE_HIP(hipStreamWaitEvent(compute_stream, ev->prepared[u], 0));
    if ((st = fwd_experts(b[u], *w, compute_stream)) != MOE_OK) return st;
    MOE_HIP(hipEventRecord(ev->computed[u], compute_stream));
    MOE_HIP(hipStreamWaitEvent(comm_stream, ev->computed[u], 0));
    if ((st = fwd_finalize(b[u], comm_stream)) != MOE_OK) return st;
    MOE_HIP(hipEventRecord(ev->finalized[u], comm_stream));
  }
  // Join: the compute stream passes the end once every combine (and shared
  // expert) is done.
  MOE_HIP(hipStreamWaitEvent(compute_stream, ev->finalized[nb - 1], 0));
  for (int u = 0; u < nb; ++u)
    if (b[u].shared) MOE_HIP(hipStreamWaitEvent(compute_stream, b[u].shared->output_ready, 0));
  return MOE_OK;
}

}  // extern "C"
