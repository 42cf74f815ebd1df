// Device helpers and internal launch interfaces of the gfx950 fused-MoE
// library.  Everything here is CDNA4-specific: 64-lane wavefronts, MFMA
// builtins, LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, which on every non-NaN input gives the bit-level rule
// (add 0x7fff plus the kept LSB to the fp32 pattern, keep the top 16 bits).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 bits (lo in bits 0-15), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// float in [-448, 448] -> OCP e4m3fn code, round to nearest even (the callers
// clamp; NaN is clamped to -448 by fminf/fmaxf).  gfx950's v_cvt_pk_fp8_f32
// converts to the OCP format on this chip; on that range it gives the
// bit-level rule: subnormal codes (|v| < 2^-6) are the nearest multiple of
// 2^-9, ties to even; normal codes keep 3 mantissa bits, the 20 dropped bits
// rounded to nearest even with a carry moving into the exponent.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
}

// One token-group-128 quantisation step: scale from the group's |max|, codes
// of clamp(x / scale).  Both divisions are IEEE fp32 (hipcc's default).
__device__ __forceinline__ float group_scale(float amax) { return fmaxf(amax, 1e-10f) / 448.0f; }

__device__ __forceinline__ uint32_t quant_e4m3(float x, float scale) {
  float t = x / scale;
  t = fminf(fmaxf(t, -448.0f), 448.0f);
  return f32_to_e4m3(t);
}

// The same with the reciprocal of the scale (the second-stage quantisation
// of act in GEMM epilogues): x * inv is within 2 ulp of x / scale, which can
// move a code only for values that close to an e4m3 rounding boundary.
__device__ __forceinline__ uint32_t quant_e4m3_inv(float x, float inv) {
  float t = x * inv;
  t = fminf(fmaxf(t, -448.0f), 448.0f);
  return f32_to_e4m3(t);
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15), returned in
// every lane: rotations by 8, 4, 2 and 1 within the row, each combined with
// fmaxf, with no LDS traffic.
__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x128, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x124, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x122, 0xf, 0xf, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x121, 0xf, 0xf, false)));
  return m;
}

// ------------------------------------------------------------ activation

// act(gate) * up of the gated GEMM epilogues: silu_and_mul, or gelu_and_mul
// with the exact GELU g * Phi(g) = 0.5 g (1 + erf(g / sqrt 2)).  silu is
// g / (1 + 2^(-g log2 e)) with the hardware 2^x and reciprocal (about 1 ulp
// each, the exponent argument rounded once): a few fp32 ulps from the exact
// value, in about a tenth of the instructions of expf and an IEEE division.
template <int ACT>
__device__ __forceinline__ float gated_act(float g, float u) {
  if constexpr (ACT == MOE_ACTIVATION_GELU)
    return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f)) * u;
  else
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}

__device__ __forceinline__ float gated_act(float g, float u, int act) {
  return act == MOE_ACTIVATION_GELU ? gated_act<MOE_ACTIVATION_GELU>(g, u) : gated_act<MOE_ACTIVATION_SILU>(g, u);
}

// ------------------------------------------------------- expert-parallel shard

// Router width: the global experts of an expert-parallel shard, else E.
inline int64_t router_width(const moe_problem &p) { return p.global_E > 0 ? p.global_E : p.E; }

// Local expert of a routed (global) id: >= 0 local, -1 held by another shard,
// -2 invalid (id outside [0, Eg) or a map entry outside [-1, E)).
__device__ __forceinline__ int local_expert(int id, int Eg, const int32_t *map, int E) {
  if (id < 0 || id >= Eg) return -2;
  const int l = map ? map[id] : id;
  return l == -1 ? -1 : (l >= 0 && l < E ? l : -2);
}

// ------------------------------------------------------------- wave utils

__device__ __forceinline__ uint64_t lanemask_lt() {
  uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Wavefront reductions: the four 16-lane DPP rows reduce by row rotations
// (no LDS traffic), then lanes 0, 16, 32 and 48 are read into scalar
// registers and combined there, so every lane gets the same value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ float row_lane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x122>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x121>(__float_as_uint(v)));
  return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0x128>(v));
  v = max_u64(v, dpp_u64<0x124>(v));
  v = max_u64(v, dpp_u64<0x122>(v));
  v = max_u64(v, dpp_u64<0x121>(v));
  auto lane_u64 = [&](int l) -> uint64_t {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  };
  return max_u64(max_u64(lane_u64(0), lane_u64(16)), max_u64(lane_u64(32), lane_u64(48)));
}

// ------------------------------------------------------- packed weights
// MOE_WEIGHTS_PACKED: weight rows are grouped in panels of 128 rows ("gated"
// w1: gate rows [128 P, 128 P + 128) together with the matching up rows;
// "down" w2: rows [128 P, 128 P + 128)).  For each (expert, panel, K-step of
// 128 bytes, wavefront w of 8, block b of nbw, piece p of 2, lane l of 64) one
// 16-byte piece holds bytes [32 (l / 16) + 16 p, +16) of the K-step of panel
// row 16 w + l % 16 of block b.  So a wavefront's K-step (nbw x 2 KB) is
// contiguous and every 1 KB of it is exactly one 64-lane 16-byte load in MFMA
// fragment order.  Sizes are those of the row-major tensors.
struct PackedGeom {
  int64_t half;      // rows per block kind: I (gated) or Nw (down)
  int64_t n_panels;  // half / 128
  int64_t nk;        // K-steps per row: row_bytes / 128
  int nbw;           // 2 (gated: gate + up) or 1 (down)
};

__host__ __device__ inline PackedGeom packed_geom(int64_t Nw, int64_t row_bytes, bool gated) {
  PackedGeom g;
  g.half = gated ? Nw / 2 : Nw;
  g.n_panels = g.half / 128;
  g.nk = row_bytes / 128;
  g.nbw = gated ? 2 : 1;
  return g;
}

// Byte offset of the 16-byte piece holding bytes [16 c, 16 c + 16) of K-step
// ks of row `row` of expert e.
__host__ __device__ inline int64_t packed_piece(const PackedGeom &g, int64_t e, int64_t row, int64_t ks, int c) {
  int b = 0;
  int64_t rr = row;
  if (g.nbw == 2 && row >= g.half) {
    b = 1;
    rr = row - g.half;
  }
  const int64_t panel = rr / 128;
  const int w = (int)((rr % 128) / 16), r16 = (int)(rr % 16);
  const int lane = (c >> 1) * 16 + r16, p = c & 1;
  return ((((((e * g.n_panels + panel) * g.nk + ks) * 8 + w) * g.nbw + b) * 2 + p) * 64 + lane) * 16;
}

// Bytes between consecutive K-steps of one row in the packed layout.
__host__ __device__ inline int64_t packed_kstep_stride(const PackedGeom &g) { return (int64_t)g.nbw * 16384; }

// ------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; shapes are validated by the
// C ABI before these are called.

struct GemmTiles {
  const int32_t *tiles;       // [max_tiles][4] = {expert, seg_base, row0, nrows}
  const int32_t *tile_count;  // device count of valid tiles
  int max_tiles;
  int dense_rows;             // > 0: dense (one expert, rows 0..dense_rows)
};

enum GemmKind { kGemmGatedAct = 0, kGemmDown = 1 };

struct GemmParams {
  // A operand: activation rows
  const void *a;
  const float *a_scale;       // fp8: [rows, Kred/128]
  const int32_t *perm;        // slot -> pair (gather by perm[slot] / topk); NULL: row = slot
  int topk;
  int n_pairs;                // bound of perm values (M*topk)
  // B operand: weights [E, Nw, Kred]
  const void *w;
  const float *w_scale;       // fp8: [E, Nw/128, Kred/128]
  int64_t Nw;
  int64_t Kred;
  // output
  void *out;
  int64_t ldo;
  const int32_t *out_perm;    // down GEMM: slot -> output row; NULL: row = slot
  float *out_scale;           // gated fp8 streaming GEMM: if set, act is written as e4m3 codes
                              // (out, ldo bytes per row) with one scale per row and 128 columns
  int64_t half_n;             // gated: I (up rows start here)
  int act;                    // gated: MOE_ACTIVATION_*
  int w_packed;               // weights in MOE_WEIGHTS_PACKED order
  // streaming down GEMM split over K: work item s of a panel reduces K-steps
  // [s, s + 1) * nk / k_split and writes fp32 partial sums by slot to
  // out + s * split_stride (out_perm unused); 0 or 1: no split
  int k_split;
  int64_t split_stride;
  // streaming fp8 down GEMM, balanced plan (stream_gemm_down_plan): each row
  // tile's columns form bal_h items of the wide width, then bal_p - bal_h of
  // one block fewer per wavefront; 0: one width
  int bal_p, bal_h;
  GemmTiles t;
};

hipError_t launch_route(const moe_problem &p, const float *logits, float *w, int32_t *ids,
                        hipStream_t s);

struct DispatchBufs {
  int32_t *status, *counts, *offsets, *chunk_hist, *perm, *inv;
  int64_t perm_len, n_chunks, chunk;
  int clear_status;   // reset the status word first (not for the later chunks of one batch)
  // the grouped GEMMs' tile plan, written by the counting kernel itself when
  // count_fused() holds and plan_rows > 0 (rows per tile)
  int32_t *tiles;
  int max_tiles;
  int plan_rows;
};

// Whether a batch is counted, ranked (and planned) by one single-block kernel.
bool count_fused(const moe_problem &p);
hipError_t launch_count_and_permute(const moe_problem &p, const int32_t *ids, int32_t *expert_num_tokens,
                                    const DispatchBufs &b, hipStream_t s);
// Row quantise / scatter; topk_w non-NULL applies each token's (single)
// router weight to its input row first (apply_router_weight_on_input).
hipError_t launch_dispatch_rows(const moe_problem &p, const void *x, const int32_t *inv, const float *topk_w,
                                void *a_out, float *a_scale_out, bool batched, hipStream_t s);
hipError_t launch_plan_tiles(const moe_problem &p, const int32_t *counts, const int32_t *offsets,
                             int64_t perm_len, int tile_rows, int max_tiles, int32_t *tiles,
                             int32_t *status, hipStream_t s);
hipError_t launch_quant_rows(const float *in, const int32_t *tiles, int max_tiles, int64_t cols,
                             uint8_t *q, float *scale, hipStream_t s);
hipError_t launch_grouped_gemm(int w_dtype, int out_dtype, GemmKind kind, const GemmParams &g,
                               int n_tiles, hipStream_t s);
// Weight-streaming variant (HBM-bound regime): gated tiles cover 128 gate
// columns, down tiles 128 output columns; rows per tile below.
int stream_gemm_tile_rows(int w_dtype);
bool stream_gemm_fits(int w_dtype, int64_t K, int64_t I);
// 16-row weight blocks per wavefront for the down GEMM (1, 2 or, fp8 with
// wide gated panels, 4), from the problem's shape: two when that still leaves
// enough work items.
int stream_gemm_down_blocks(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I);
// blocks per wavefront of the down GEMM's (wide) items, and the balanced plan
// if one is taken (bal_p = 0 otherwise)
int stream_gemm_down_plan(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I, int *bal_p, int *bal_h);
// K splits of the streaming down GEMM (1: none): bf16 shapes whose panels of
// two weight blocks leave too few work items to fill the chip (few experts,
// wide K) take two blocks per wavefront and split the reduction instead; the
// partial sums then go through launch_split_reduce.
int stream_gemm_down_split(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I);
// out[perm[slot]] = sum over s of part[s * stride + slot * K] (rows of K
// values) for the slots whose perm entry is a pair below n_pairs.
hipError_t launch_split_reduce(const float *part, int S, int64_t stride, const int32_t *perm, int64_t n_slots,
                               int n_pairs, int K, int out_dtype, void *out, hipStream_t s);
// Whether the gated GEMM takes wide panels (fp8: 256 act columns per work
// item, 2 gate + 2 up weight blocks per wavefront); launched with blocks = 4.
bool stream_gemm_gated_wide(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I);
int stream_gemm_wide_tile_rows();   // row tiles of the plan when the gated GEMM is wide
// blocks: gated GEMM 2, or 4 for wide panels; down GEMM weight blocks per
// wavefront (1 or 2).
hipError_t launch_stream_gemm(int w_dtype, int out_dtype, GemmKind kind, const GemmParams &g, int n_tiles,
                              int blocks, hipStream_t s);
// Compute-bound variant (bf16, many rows per expert): 256-row tiles; gated
// tiles cover 128 act columns, down tiles 256 output columns.
int mfma_gemm_tile_rows();
bool mfma_gemm_fits(int w_dtype, int act_dtype, int64_t K, int64_t I, int64_t M);
int mfma_gemm_n_tiles(GemmKind kind, int64_t Nw);
hipError_t launch_mfma_gemm(GemmKind kind, const GemmParams &g, int n_tiles, hipStream_t s);
hipError_t launch_pack_weights(const void *src, void *dst, int64_t E, int64_t Nw, int64_t row_bytes, bool gated,
                               hipStream_t s);
// Combine.  Rows: inv[pair] with rows_from_inv (batched), else pair; with
// inv non-NULL a pair whose inv is negative adds nothing.  topk_w NULL: the
// outputs are added unweighted (router weight applied on the input).
hipError_t launch_combine(const moe_problem &p, const void *fused_out, const float *topk_w,
                          const int32_t *inv, bool rows_from_inv, void *out, hipStream_t s);
// The combine of moe_forward when the down GEMM split K (bf16, Standard): the
// pair rows come from the split's fp32 partial slices by slot (inv[pair]).
hipError_t launch_combine_split(const moe_problem &p, const float *part, int S, int64_t stride,
                                const float *topk_w, const int32_t *inv, void *out, hipStream_t s);

constexpr int kTileRows = 128;   // grouped-GEMM rows per tile (BM)
constexpr int kMinPlanTileRows = 96;   // the smallest row tile any GEMM's plan uses (wide fp8 panels)
constexpr int kTileCols = 128;   // grouped-GEMM weight rows per tile (BN)

}  // namespace moe
