// Weight-streaming grouped GEMM for the HBM-bound regime (a few hundred rows
// per expert at most): decode-sized batches and prefill whose per-expert row
// count is below the MFMA/HBM ridge.  Same computation as grouped_gemm.hip --
// the gated GEMM act = silu(A w1_gate) * (A w1_up) or the down GEMM
// out = act w2^T with the unpermute in its epilogue (modular_kernel.py page,
// FusedMoEPermuteExpertsUnpermute: GEMM, gated activation, optional
// quantisation, GEMM; the worst-tokens page: the grouped GEMM is masked by
// per-expert counts read on the device) -- organised around reading every
// weight byte exactly once:
//
//  * one workgroup = one expert's rows (up to TMAX, masked by the device
//    count in 16-row MFMA blocks) x a panel of weight rows, so an expert's
//    weights are streamed once whatever its row count;
//  * each of the 8 wavefronts owns its own 16-row weight blocks, which no
//    other wavefront needs: they go straight from HBM into MFMA B fragments in
//    registers, prefetched D K-steps ahead (no LDS round trip);
//  * the activation rows, shared by all wavefronts, are staged through a
//    double-buffered LDS tile (XOR-swizzled 16-byte chunks) two K-steps ahead;
//  * the number of 16-row blocks is rounded up (1, 2, 4, 6, ...) and each
//    value gets its own fully unrolled main loop, so no load, LDS access or
//    MFMA sits behind a branch (branches around memory operations make the
//    compiler wait for every outstanding load);
//  * work items are dealt out XCD by XCD: consecutive items of one expert land
//    on the same XCD, so its activation rows stay in that XCD's L2;
//  * the fp8 down GEMM can deal each row tile's output columns out as items of
//    two widths (NBW and NBW - 1 blocks per wavefront), the wide ones first,
//    so that every compute unit streams the same number of weight bytes where
//    one width would leave the last round of items part-empty.  A column's
//    arithmetic does not depend on the item that holds it, so the outputs are
//    the same bits either way.
//
// MFMA: v_mfma_f32_16x16x32_bf16, or for fp8 v_mfma_scale_f32_16x16x128_f8f6f4
// with unit block scales (OCP e4m3; the layer's fp32 block scales applied per
// 128-wide K block).  Inside each 128-byte K-step a lane of group q = lane/16
// holds 32 contiguous bytes; MFMA step t takes bytes [t*F, t*F + F) of them
// (F = 16 for bf16: two steps; F = 32 for fp8: one step).  A and B use the
// same mapping, so the k permutation this implies cancels in the dot product.
#include <algorithm>
#include <utility>

#include "moe_device.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int EB>
struct Mfma16;

template <>
struct Mfma16<2> {
  static constexpr int kSteps = 2;  // 16x16x32 steps per 128-byte K-step
  typedef bf16x8 frag;
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// fp8: gfx950's 16x16x128 MFMA takes a whole 128-byte K-step per instruction
// (a lane's 32 bytes of its row), four times the K of the 16x16x32 form.  It
// exists only with per-32-element E8M0 block scales; 127 encodes 2^0, so the
// product is the plain e4m3 one (format 0 = OCP e4m3 for both operands) and
// the layer's fp32 scales are applied per 128-wide K block as before.
template <>
struct Mfma16<1> {
  static constexpr int kSteps = 1;
  typedef i32x8 frag;
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// Swizzled LDS address of byte b of a 128-byte tile row: the 16-byte chunk
// index is XORed with (row / 2) % 8 so that 16 consecutive rows (one 128-bit
// access pass over gfx950's 64 banks) hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int b) {
  return row * 128 + ((((b >> 4) ^ ((row >> 1) & 7)) << 4) | (b & 15));
}

// Staging registers are native vectors: HIP's uint4 is a struct whose copies
// become memcpy, which can keep a staging array in memory.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <typename F>
__device__ __forceinline__ F frag_at(const u32x4 (&v)[2], int t) {
  if constexpr (sizeof(F) == 32) {
    return __builtin_bit_cast(F, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
  } else if constexpr (sizeof(F) == 16) {
    return __builtin_bit_cast(F, v[t]);
  } else {
    const u32x4 q = v[t >> 1];
    const u32x2 h = (t & 1) ? q.zw : q.xy;
    return __builtin_bit_cast(F, h);
  }
}

// A fragment from the swizzled LDS tile: bytes [off, off + sizeof(F)) of a row;
// a 32-byte fragment spans two 16-byte chunks, which the swizzle places apart.
template <typename F>
__device__ __forceinline__ F lds_frag(const uint8_t *A, int row, int off) {
  if constexpr (sizeof(F) == 32) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(A + swz(row, off));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(A + swz(row, off + 16));
    return __builtin_bit_cast(F, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    return *reinterpret_cast<const F *>(A + swz(row, off));
  }
}

constexpr int kThreads = 512;
constexpr int kXcdUnits = 32;   // compute units per XCD (256 in 8 XCDs)
#ifndef MOE_STREAM_SPLIT_TAIL
#define MOE_STREAM_SPLIT_TAIL 1
#endif
#ifndef MOE_STREAM_FRAG_AHEAD
#define MOE_STREAM_FRAG_AHEAD 2
#endif

// 16-byte weight load; packed weights stream once in whole cache lines, so
// they are read non-temporally (the row-major pattern touches half lines per
// instruction and is faster through the cache).
template <bool NT>
__device__ __forceinline__ u32x4 load_w16(const uint8_t *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  else
    return *reinterpret_cast<const u32x4 *>(p);
}

template <int EB, bool GATED, bool OUT_BF16, int NBW, int D, int TMAX, bool PACKED>
__global__ __launch_bounds__(kThreads) void stream_gemm_kernel(const GemmParams g, int n_tiles) {
  using MM = Mfma16<EB>;
  using frag = typename MM::frag;
  constexpr bool kScaled = EB == 1;
  constexpr int kFrag = 32 / MM::kSteps;    // bytes per lane per MFMA step
  constexpr int U = D % 2 == 0 ? D : 2 * D; // unroll = lcm(2, D); the host checks nk % U == 0
  // gated: a wavefront holds GB gate blocks and the GB matching up blocks
  static_assert(!GATED || NBW == 2 || NBW == 4, "gated: 1 or 2 gate blocks per wavefront");
  constexpr int GB = GATED ? NBW / 2 : 1;
  static_assert(TMAX % 64 == 0 && TMAX <= 256, "row tile");
  // the balanced down plan (fp8, 3 or 4 blocks per wavefront): items of NBW
  // and NBW - 1 blocks
  constexpr bool kBal = !GATED && kScaled && NBW >= 3;

  __shared__ __attribute__((aligned(16))) uint8_t As[2][TMAX * 128];
  __shared__ __attribute__((aligned(16))) float Sa[2][TMAX];
  __shared__ int32_t Orow[GATED ? 1 : TMAX];   // down: output row of each tile row

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tiles_n = *g.t.tile_count;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int S = GATED || g.k_split <= 1 ? 1 : g.k_split;
  int c, sk = 0, nt = 0, half = -1;
  int64_t col0 = 0;   // down: the item's first output column (weight row)
  bool narrow = false;   // balanced down plan: the item holds NBW - 1 blocks per wavefront
  if (kBal && g.bal_p > 0) {
    // Balanced down plan: a row tile's K / 128 column units form bal_h items
    // of NBW blocks per wavefront, then bal_p - bal_h items of NBW - 1; the
    // wide items of all tiles come first, each group dealt out XCD by XCD.
    const int n_wide = tiles_n * g.bal_h, n_narrow = tiles_n * (g.bal_p - g.bal_h);
    const int per_wide = (n_wide + 7) >> 3;
    if (local < per_wide) {
      const int item = xcd * per_wide + local;
      if (item >= n_wide) return;
      c = item / g.bal_h;
      col0 = (int64_t)(item - c * g.bal_h) * (128 * NBW);
    } else {
      const int per_narrow = (n_narrow + 7) >> 3, li = local - per_wide;
      if (li >= per_narrow) return;
      const int item = xcd * per_narrow + li, np = g.bal_p - g.bal_h;
      if (item >= n_narrow) return;
      c = item / np;
      col0 = (int64_t)g.bal_h * (128 * NBW) + (int64_t)(item - c * np) * (128 * (NBW - 1));
      narrow = true;
    }
  } else {
    const int total = tiles_n * n_tiles;
    const int per = (total + 7) >> 3;
    // An XCD's items past its last whole round (32 compute units), or all of
    // them when there are fewer than a round, leave units idle; when they fill
    // at most half a round, each of them becomes two work items over the two
    // halves of its rows, adjacent so that the pair shares its weight panel
    // through L2.  The outputs are the same: every row is computed as in the
    // whole item (the fp8 epilogue's quantisation groups are per row).
    const int whole = per & ~(kXcdUnits - 1), rem = per - whole;
    const bool split_tail = MOE_STREAM_SPLIT_TAIL && GATED && rem <= kXcdUnits / 2;
    int li = local;
    if (split_tail && local >= whole) {
      li = whole + ((local - whole) >> 1);
      half = (local - whole) & 1;
    }
    if (li >= per) return;
    const int item = xcd * per + li;
    if (item >= total) return;
    // item -> (row tile c, K split sk, panel nt): the panels of one split are
    // adjacent, so concurrent items share the split's activation K range
    c = item / n_tiles;
    const int n_panels = n_tiles / S;
    sk = S > 1 ? (item - c * n_tiles) / n_panels : 0;
    nt = item - c * n_tiles - sk * n_panels;
    col0 = (int64_t)nt * (128 * NBW);
  }
  const int32_t *tile = g.t.tiles + (int64_t)c * 4;
  const int e = tile[0];
  int64_t row0 = (int64_t)tile[1] + tile[2];
  int T = tile[3];
  if (half >= 0) {
    const int first = ((T + 1) / 2 + 15) & ~15;   // rows of the first half, whole blocks of 16
    if (half == 0) {
      T = min(T, first);
    } else {
      row0 += first;
      T -= first;
      if (T <= 0) return;
    }
  }
  const int64_t row_bytes = g.Kred * EB;
  const int nk = (int)(row_bytes / 128) / S;   // K-steps of this item, from k0
  const int k0 = sk * nk;
  // partial sums of a K split: fp32 rows by slot, one slice per split
  void *const out = S > 1 ? static_cast<void *>(reinterpret_cast<float *>(g.out) + sk * g.split_stride) : g.out;
  const int32_t *const out_perm = S > 1 ? nullptr : g.out_perm;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t kblocks = g.Kred / 128;

  const PackedGeom pg = packed_geom(g.Nw, row_bytes, GATED);
  const int64_t kstride = PACKED ? packed_kstep_stride(pg) : 128;   // bytes between K-steps
  constexpr int64_t pstride = PACKED ? 1024 : 16;                    // bytes between the two pieces
  // A row (in the activation tensor) of tile row r.  Rows past the count map
  // to the last real row (so their loads share its cache lines) and padding
  // slots to row 0: an A row only feeds its own output row, which the
  // epilogue does not store for those rows, so no mask is needed.
  auto a_row_of = [&](int r) -> int64_t {
    const int64_t s = row0 + min(r, T - 1);
    if (!g.perm) return s;
    const int f = g.perm[s];
    return (f < 0 || f >= g.n_pairs) ? 0 : f / g.topk;
  };
  const int ach = tid & 7;
  const uint8_t *abase = reinterpret_cast<const uint8_t *>(g.a) + ach * 16 + (int64_t)k0 * 128;

  // Gated fp8: the item's act columns are whole quantisation groups of 128
  // (one, or two with wide panels), so the epilogue quantises them directly
  // (the per-token-group e4m3 scheme that the layer applies to its input,
  // applied again to act before the down GEMM): row maxima are reduced across
  // the 16 lanes holding a row's columns in a wavefront, then across the
  // wavefronts of the group through LDS; the codes are staged in LDS and
  // written as whole rows.
  auto quant_epilogue = [&]<int NMB, int ACT>(f32x4 (&acc)[NMB][NBW]) {
    constexpr int kGroupWaves = 8 / GB;   // wavefronts whose columns form one group
    constexpr int kRowCodes = 128 * GB;   // code bytes per row of the item
    static_assert(NMB * 16 * kRowCodes <= 2 * TMAX * 128, "the codes fit the A buffers");
    __syncthreads();   // every wavefront is done reading the A tiles
    float *rmax = reinterpret_cast<float *>(&As[0][0]);   // [TMAX][8]
    uint8_t *codes = &As[0][0];                           // [TMAX][kRowCodes], once rmax is read
    const int grp = wv / kGroupWaves;
    float v[NMB][GB][4];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) {
          v[mb][gb][i] = gated_act<ACT>(acc[mb][gb][i], acc[mb][gb + GB][i]);
          m = fmaxf(m, fabsf(v[mb][gb][i]));
        }
        m = row16_max(m);
        if (r16 == 0) rmax[(mb * 16 + q * 4 + i) * 8 + wv] = m;
      }
    }
    __syncthreads();
    // The 16 lanes of a row group (same q) hold the same 4 * NMB rows: each
    // lane works out the scale of one or two of them (two IEEE divisions per
    // row, done once instead of in every lane), then every lane fetches the
    // reciprocals of its rows from the lanes that computed them.
    constexpr int kRowsQ = NMB * 4, kPer = (kRowsQ + 15) / 16;
    float my_inv[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int idx = t * 16 + r16, idc = min(idx, kRowsQ - 1);   // (mb, i) = (idc / 4, idc % 4)
      const int r = (idc >> 2) * 16 + q * 4 + (idc & 3);
      // the group's per-wavefront maxima are contiguous: 16-byte reads
      float amax = 0.0f;
#pragma unroll
      for (int w = 0; w < kGroupWaves; w += 4) {
        const float4 m4 = *reinterpret_cast<const float4 *>(&rmax[r * 8 + grp * kGroupWaves + w]);
        amax = fmaxf(amax, fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w)));
      }
      const float sc = group_scale(amax);
      my_inv[t] = 1.0f / sc;
      if (wv % kGroupWaves == 0 && idx < kRowsQ && r < T)
        g.out_scale[(row0 + r) * (g.ldo / 128) + (int64_t)nt * GB + grp] = sc;
    }
    float inv[NMB][4];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = mb * 4 + i;
        inv[mb][i] = __shfl(my_inv[idx >> 4], q * 16 + (idx & 15), 64);
      }
    __syncthreads();   // the row maxima are read: their space takes the codes
    // A row's consecutive codes sit in consecutive lanes: the first lane of
    // each quad gathers its quad's four bytes (DPP quad permutes) and writes
    // them as one 32-bit word, instead of four single-byte LDS writes.
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) {
          const int b = (int)quant_e4m3_inv(v[mb][gb][i], inv[mb][i]);
          const int b1 = __builtin_amdgcn_update_dpp(0, b, 0x55, 0xF, 0xF, false);   // quad lane 1
          const int b2 = __builtin_amdgcn_update_dpp(0, b, 0xAA, 0xF, 0xF, false);   // quad lane 2
          const int b3 = __builtin_amdgcn_update_dpp(0, b, 0xFF, 0xF, 0xF, false);   // quad lane 3
          if ((r16 & 3) == 0)
            *reinterpret_cast<uint32_t *>(&codes[(mb * 16 + q * 4 + i) * kRowCodes + wv * 16 * GB + gb * 16 + r16]) =
                (uint32_t)(b & 0xff) | ((uint32_t)(b1 & 0xff) << 8) | ((uint32_t)(b2 & 0xff) << 16) |
                ((uint32_t)(b3 & 0xff) << 24);
        }
    __syncthreads();
    // kRowCodes / 16 threads per row, 16 bytes each
    constexpr int kChunksRow = kRowCodes / 16;
    for (int c = tid; c < NMB * 16 * kChunksRow; c += kThreads) {
      const int r = c / kChunksRow, b = (c % kChunksRow) * 16;
      if (r < T)
        *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(g.out) + (row0 + r) * g.ldo + (int64_t)nt * kRowCodes +
                                   b) = *reinterpret_cast<const u32x4 *>(&codes[r * kRowCodes + b]);
    }
  };

  // The main loop for NMB blocks of 16 rows (NMB * 16 >= T) and NB weight
  // blocks per wavefront: every load, LDS access and MFMA is unconditional.
  auto body = [&]<int NMB, int NB>() {
    // Weight rows of this wavefront: NB blocks of 16 rows.  A lane reads two
    // 16-byte pieces per block and K-step: bytes [32 q, 32 q + 32) of its row.
    const uint8_t *wsrc[NB];
    const float *wscale[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      int64_t wrow0;
      if (GATED)
        wrow0 = (b >= GB ? g.half_n : 0) + (int64_t)nt * 128 * GB + wv * 16 * GB + (b % GB) * 16;
      else
        wrow0 = col0 + wv * (16 * NB) + b * 16;
      if (PACKED)
        wsrc[b] = reinterpret_cast<const uint8_t *>(g.w) + packed_piece(pg, e, wrow0 + r16, 0, 2 * q) +
                  (int64_t)k0 * kstride;
      else
        wsrc[b] = reinterpret_cast<const uint8_t *>(g.w) + ((int64_t)e * g.Nw + wrow0 + r16) * row_bytes +
                  q * 32 + (int64_t)k0 * 128;
      wscale[b] = kScaled ? g.w_scale + ((int64_t)e * (g.Nw / 128) + wrow0 / 128) * kblocks + k0 : nullptr;
    }
    constexpr int kPasses = (NMB * 16 + 63) / 64;   // A rows per thread per K-step
    int64_t arow[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) arow[i] = a_row_of((tid >> 3) + 64 * i);
    const int64_t srow = kScaled ? a_row_of(tid) : 0;

    u32x4 ra[2][kPasses];
    float rsa[2] = {0.0f, 0.0f};
    auto loadA = [&](int j, int ks) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i)
        ra[j][i] = *reinterpret_cast<const u32x4 *>(abase + arow[i] * row_bytes + (int64_t)ks * 128);
      if constexpr (kScaled) rsa[j] = g.a_scale[srow * kblocks + k0 + ks];
    };
    auto storeA = [&](int j, int st) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i) {
        const int r = (tid >> 3) + 64 * i;
        *reinterpret_cast<u32x4 *>(&As[st][swz(r, ach * 16)]) = ra[j][i];
      }
      if constexpr (kScaled)
        if (tid < TMAX) Sa[st][tid] = rsa[j];
    };

    u32x4 wb[D][NB][2];
    float wsv[D][NB];
    auto loadW = [&](int j, int ks) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint8_t *p = wsrc[b] + (int64_t)ks * kstride;
        wb[j][b][0] = load_w16<PACKED>(p);
        wb[j][b][1] = load_w16<PACKED>(p + pstride);
        if constexpr (kScaled) wsv[j][b] = wscale[b][ks];
      }
    };

    f32x4 acc[NMB][NB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[mb][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // One K-step of MFMAs from LDS stage st and weight registers j.
    auto compute = [&](int st, int j) {
      const uint8_t *A = As[st];
      if constexpr (!kScaled && MM::kSteps > 1) {
        // Sub-step outermost, so the MFMAs into one accumulator are NMB * NBW
        // instructions apart; A fragments are read kAhead (sub-step, block)
        // positions ahead of their MFMAs to cover LDS latency (the fully
        // unrolled ring keeps kAhead + 1 fragments live).
        constexpr int S = MM::kSteps * NMB;
        constexpr int kAhead = MOE_STREAM_FRAG_AHEAD < S ? MOE_STREAM_FRAG_AHEAD : S;
        frag f[S];
#pragma unroll
        for (int x = 0; x < kAhead; ++x) f[x] = lds_frag<frag>(A, (x % NMB) * 16 + r16, q * 32 + (x / NMB) * kFrag);
#pragma unroll
        for (int x = 0; x < S; ++x) {
          if (x + kAhead < S) {
            const int y = x + kAhead;
            f[y] = lds_frag<frag>(A, (y % NMB) * 16 + r16, q * 32 + (y / NMB) * kFrag);
          }
          const int mb = x % NMB, t = x / NMB;
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[mb][b] = MM::mma(f[x], frag_at<frag>(wb[j][b], t), acc[mb][b]);
          // keep the read-ahead in place (the scheduler would otherwise move
          // each read next to its MFMAs and wait for it there)
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // fp8: one MFMA step per K-step and block.  Blocks in order, A fragments
        // read kAhead blocks ahead (pinned like the bf16 ring); a block's
        // partial sums are scaled by its row and weight-block scales and folded
        // after the next block's MFMAs are issued, so the FMAs never wait on
        // the MFMA that produced them.
        static_assert(MM::kSteps == 1, "scaled path: one MFMA step per K-step");
        constexpr int kAhead = MOE_STREAM_FRAG_AHEAD < NMB ? MOE_STREAM_FRAG_AHEAD : NMB;
        frag f[NMB];
        f32x4 part[2][NB];
#pragma unroll
        for (int x = 0; x < kAhead; ++x) f[x] = lds_frag<frag>(A, x * 16 + r16, q * 32);
        auto issue = [&](int mb) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            part[mb & 1][b] = MM::mma(f[mb], frag_at<frag>(wb[j][b], 0), f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        };
        auto fold = [&](int mb) {
          const float4 sa4 = *reinterpret_cast<const float4 *>(&Sa[st][mb * 16 + q * 4]);
          const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[mb][b][i] += part[mb & 1][b][i] * (sa[i] * wsv[j][b]);
          // Fold each block here: without this the compiler sinks all blocks'
          // scale FMAs to the end of the K-step and keeps every block's partial
          // sums live at once.
#pragma unroll
          for (int b = 0; b < NB; ++b) asm volatile("" : "+v"(acc[mb][b]));
        };
        issue(0);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          if (mb + kAhead < NMB) f[mb + kAhead] = lds_frag<frag>(A, (mb + kAhead) * 16 + r16, q * 32);
          if (mb + 1 < NMB) issue(mb + 1);
          fold(mb);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // Down: the output row of tile row tid (slot order, or through out_perm;
    // padding slots and rows past the count give -1), loaded first so that no
    // later wait stops on it.
    int orow_t = -1;
    if constexpr (!GATED) {
      if (tid < T) {
        orow_t = (int)(row0 + tid);   // slots are int32 in the tile plan
        if (out_perm) {
          orow_t = out_perm[orow_t];
          if (orow_t >= g.n_pairs) orow_t = -1;
        }
      }
    }

    // Pipeline: A two K-steps ahead (registers -> LDS), weights D ahead.
    loadA(0, 0);
    loadA(1, min(1, nk - 1));
#pragma unroll
    for (int j = 0; j < D; ++j) loadW(j, min(j, nk - 1));
    storeA(0, 0);
    if constexpr (!GATED) {
      // the first barrier publishes the output rows read before the loads
      if (tid < NMB * 16) Orow[tid] = orow_t;
    }
    __syncthreads();
    // (the fp8 gated kernel with two blocks per wavefront keeps the plain
    // loop for 6 and 8 row blocks, where the peeled steps spill registers)
    constexpr bool kPeel = !(GATED && kScaled && NBW == 2 && NMB > 4);
    int kb = 0;
    for (; kb < (kPeel ? nk - U : nk); kb += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kb + u;
        loadA(u & 1, min(k + 2, nk - 1));
        compute(u & 1, u % D);
        loadW(u % D, min(k + D, nk - 1));
        storeA((u + 1) & 1, (u + 1) & 1);
        __syncthreads();
      }
    }
    // The last U K-steps issue no loads for steps past the end: loads still
    // in flight when the loop ends would hold the epilogue at its first use of
    // their registers until they land (about 2 us per item, measured).
    auto last_step = [&]<int u>() {
      if constexpr (u + 2 < U) loadA(u & 1, kb + u + 2);
      compute(u & 1, u % D);
      if constexpr (u + D < U) loadW(u % D, kb + u + D);
      if constexpr (u + 1 < U) storeA((u + 1) & 1, (u + 1) & 1);
      __syncthreads();
    };
    if constexpr (kPeel) {
      [&]<int... us>(std::integer_sequence<int, us...>) {
        (last_step.template operator()<us>(), ...);
      }(std::make_integer_sequence<int, U>{});
    }

    // Epilogue: in a 16x16 block, lane holds column r16 of rows 4*q + i.  The
    // activation is resolved once per item, outside the per-element code.
    auto epilogue = [&]<int ACT>() {
      if constexpr (GATED && kScaled) {
        if (g.out_scale) {
          quant_epilogue.template operator()<NMB, ACT>(acc);
          return;
        }
      }
      if constexpr (OUT_BF16) {
        // bf16 tiles go through LDS and leave as whole rows of 16-byte stores
        // (one 2-byte store per element cost a fifth of the down GEMM on the
        // DeepSeek shapes).  Rows are staged in passes that fit the A buffers;
        // the 16-byte row padding spreads the 4 rows a store instruction
        // touches over different banks.
        constexpr int kCols = GATED ? 128 * GB : 128 * NB;
        constexpr int kRowBytes = kCols * 2;
        constexpr int kPitch = kRowBytes + 16;
        constexpr int kFit = (2 * TMAX * 128 / kPitch) / 16 * 16;
        constexpr int RP = kFit < NMB * 16 ? kFit : NMB * 16;
        constexpr int kChunks = kRowBytes / 16;
        static_assert(RP >= 16, "staging buffer holds at least one row block");
        uint8_t *stage = &As[0][0];
        const int64_t ocol0 = GATED ? (int64_t)nt * kCols : col0;
        __syncthreads();   // every wavefront is done reading the A tiles
#pragma unroll
        for (int p0 = 0; p0 < NMB * 16; p0 += RP) {
#pragma unroll
          for (int mb = p0 / 16; mb < (p0 + RP) / 16 && mb < NMB; ++mb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint8_t *row = stage + (mb * 16 + q * 4 + i - p0) * kPitch;
              // a row's consecutive columns sit in consecutive lanes: the
              // first lane of each quad gathers the quad's four bf16 values
              // (DPP quad permutes) and writes them as one 8-byte word
              auto put4 = [&](int col, uint32_t h) {
                const uint32_t h1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x55, 0xF, 0xF, false);
                const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0xAA, 0xF, 0xF, false);
                const uint32_t h3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0xFF, 0xF, 0xF, false);
                if ((r16 & 3) == 0)
                  *reinterpret_cast<u32x2 *>(row + col * 2) = u32x2{(h & 0xffffu) | (h1 << 16), (h2 & 0xffffu) | (h3 << 16)};
              };
              if constexpr (GATED) {
#pragma unroll
                for (int gb = 0; gb < GB; ++gb) {
                  const float v = gated_act<ACT>(acc[mb][gb][i], acc[mb][gb + GB][i]);
                  put4(wv * 16 * GB + gb * 16 + r16, f32_to_bf16_bits(v));
                }
              } else {
                // (down: single 2-byte writes, measured 3% faster than the
                // gathered words on the DeepSeek-V3 shapes)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                  *reinterpret_cast<uint16_t *>(row + (wv * 16 * NB + b * 16 + r16) * 2) =
                      f32_to_bf16_bits(acc[mb][b][i]);
              }
            }
          }
          __syncthreads();
          const int nrows = min(RP, T - p0);
          for (int c = tid; c < nrows * kChunks; c += kThreads) {
            const int rl = c / kChunks, off = (c - rl * kChunks) * 16;
            int64_t orow = row0 + p0 + rl;
            if constexpr (!GATED) {
              orow = Orow[p0 + rl];
              if (orow < 0) continue;
            }
            *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(out) + (orow * g.ldo + ocol0) * 2 + off) =
                *reinterpret_cast<const u32x4 *>(stage + rl * kPitch + off);
          }
          __syncthreads();
        }
        return;
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mb * 16 + q * 4 + i;
          if (r >= T) continue;
          const int64_t slot = row0 + r;
          if constexpr (GATED) {
#pragma unroll
            for (int gb = 0; gb < GB; ++gb) {
              const float v = gated_act<ACT>(acc[mb][gb][i], acc[mb][gb + GB][i]);
              const int64_t col = (int64_t)nt * 128 * GB + wv * 16 * GB + gb * 16 + r16;
              if constexpr (OUT_BF16)
                reinterpret_cast<uint16_t *>(out)[slot * g.ldo + col] = f32_to_bf16_bits(v);
              else
                reinterpret_cast<float *>(out)[slot * g.ldo + col] = v;
            }
          } else {
            const int64_t orow = Orow[r];
            if (orow < 0) continue;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const int64_t col = col0 + wv * (16 * NB) + b * 16 + r16;
              if constexpr (OUT_BF16)
                reinterpret_cast<uint16_t *>(out)[orow * g.ldo + col] = f32_to_bf16_bits(acc[mb][b][i]);
              else
                reinterpret_cast<float *>(out)[orow * g.ldo + col] = acc[mb][b][i];
            }
          }
        }
      }
    };
    if constexpr (GATED) {
      if (g.act == MOE_ACTIVATION_GELU)
        epilogue.template operator()<MOE_ACTIVATION_GELU>();
      else
        epilogue.template operator()<MOE_ACTIVATION_SILU>();
    } else {
      epilogue.template operator()<MOE_ACTIVATION_SILU>();
    }
  };

  // Row blocks rounded up to 1, 2, 4, 6, ... (one specialised loop each); fp8
  // also has a loop for 5, the count of decode M=256's experts of 65-80 rows
  // (1-1.5% faster gated and down GEMMs than rounding them to 6).  Loops for
  // 3 and 7 as well put 608 bytes per lane of the gated kernels' arrays in
  // scratch memory.
  const int nmb = (T + 15) >> 4;
  const int nq = (EB == 1 && nmb == 5) ? 5 : nmb <= 1 ? 1 : (nmb + 1) & ~1;
  auto run = [&]<int NB>() {
    switch (nq) {
      case 1: body.template operator()<1, NB>(); break;
      case 2: body.template operator()<2, NB>(); break;
      case 4: body.template operator()<4, NB>(); break;
      case 5: if constexpr (EB == 1) body.template operator()<5, NB>(); break;
      case 6: body.template operator()<6, NB>(); break;
      case 8:
        // four weight blocks per wavefront (wide fp8 panels) take tiles of at
        // most 96 rows
        if constexpr (NBW != 4) body.template operator()<8, NB>();
        break;
      default:
        if constexpr (TMAX >= 256) {
          switch (nq) {
            case 10: body.template operator()<10, NB>(); break;
            case 12: body.template operator()<12, NB>(); break;
            case 14: body.template operator()<14, NB>(); break;
            default: body.template operator()<16, NB>(); break;
          }
        }
        break;
    }
  };
  if constexpr (kBal) {
    if (narrow)
      run.template operator()<NBW - 1>();
    else
      run.template operator()<NBW>();
  } else {
    run.template operator()<NBW>();
  }
}

template <int EB, bool GATED, int NBW, int D, int TMAX>
hipError_t launch_cfg(int out_dtype, const GemmParams &g, int n_tiles, hipStream_t s) {
  const int64_t items = (int64_t)g.t.max_tiles * n_tiles;
  // gated: room for a split tail (at most half a round more per XCD)
  const int64_t extra = MOE_STREAM_SPLIT_TAIL && GATED ? 8 * (kXcdUnits / 2) : 0;
  int64_t blocks = ((items + 7) / 8) * 8 + extra;
  if (!GATED && g.bal_p > 0) {
    // balanced down plan: the wide items of every tile, then the narrow ones
    const int64_t mt = g.t.max_tiles;
    blocks = 8 * ((mt * g.bal_h + 7) / 8 + (mt * (g.bal_p - g.bal_h) + 7) / 8);
  }
  dim3 grid((unsigned)blocks), block(kThreads);
  const bool bf = out_dtype == MOE_DTYPE_BF16;
  if constexpr (EB == 1 && GATED) {
    // the fp8 gated GEMM writes fp32 or re-quantised act, never bf16
    if (bf) return hipErrorInvalidValue;
    if (g.w_packed)
      stream_gemm_kernel<EB, GATED, false, NBW, D, TMAX, true><<<grid, block, 0, s>>>(g, n_tiles);
    else
      stream_gemm_kernel<EB, GATED, false, NBW, D, TMAX, false><<<grid, block, 0, s>>>(g, n_tiles);
  } else if (g.w_packed) {
    if (bf)
      stream_gemm_kernel<EB, GATED, true, NBW, D, TMAX, true><<<grid, block, 0, s>>>(g, n_tiles);
    else
      stream_gemm_kernel<EB, GATED, false, NBW, D, TMAX, true><<<grid, block, 0, s>>>(g, n_tiles);
  } else {
    if (bf)
      stream_gemm_kernel<EB, GATED, true, NBW, D, TMAX, false><<<grid, block, 0, s>>>(g, n_tiles);
    else
      stream_gemm_kernel<EB, GATED, false, NBW, D, TMAX, false><<<grid, block, 0, s>>>(g, n_tiles);
  }
  return hipGetLastError();
}

// Sum of the K splits of the down GEMM: one block per slot, 8 columns per
// thread and pass (two 16-byte loads per split), fp32 in split order.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ part, int S, int64_t stride,
                                                           const int32_t *__restrict__ perm, int n_pairs, int K,
                                                           void *__restrict__ out) {
  const int64_t slot = blockIdx.x;
  const int pair = perm[slot];
  if (pair < 0 || pair >= n_pairs) return;   // alignment padding
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sk = 0; sk < S; ++sk) {
      const float4 *src = reinterpret_cast<const float4 *>(part + sk * stride + slot * K + c);
      const float4 a = src[0], b = src[1];
      acc[0] += a.x, acc[1] += a.y, acc[2] += a.z, acc[3] += a.w;
      acc[4] += b.x, acc[5] += b.y, acc[6] += b.z, acc[7] += b.w;
    }
    if constexpr (OUT_BF16) {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + (int64_t)pair * K + c) =
          make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (int64_t)pair * K + c);
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

int stream_gemm_tile_rows(int w_dtype) { return w_dtype == MOE_DTYPE_FP8_E4M3 ? 128 : 256; }

// Prefetch depths (K-steps of weights in flight per wavefront), per dtype so
// that accumulators, staging and prefetch fit 256 registers.
#ifndef MOE_STREAM_GATED_D_BF16
#define MOE_STREAM_GATED_D_BF16 2
#endif
#ifndef MOE_STREAM_DOWN_D_BF16
#define MOE_STREAM_DOWN_D_BF16 4
#endif
#ifndef MOE_STREAM_GATED_D_FP8
#define MOE_STREAM_GATED_D_FP8 2
#endif
#ifndef MOE_STREAM_DOWN_D_FP8
#define MOE_STREAM_DOWN_D_FP8 4
#endif

// Down GEMM: 16-row weight blocks per wavefront.  Each wavefront reads the
// whole activation tile from LDS once per K-step, so two blocks halve the LDS
// bytes read per weight byte -- but also halve the number of work items, so
// the host keeps one block when two would leave CUs idle.
#ifndef MOE_STREAM_DOWN2_D_BF16
#define MOE_STREAM_DOWN2_D_BF16 2
#endif
#ifndef MOE_STREAM_DOWN4_FP8
#define MOE_STREAM_DOWN4_FP8 1
#endif
#ifndef MOE_STREAM_DOWN4_D_FP8
#define MOE_STREAM_DOWN4_D_FP8 1
#endif
#ifndef MOE_STREAM_DOWN2_D_FP8
#define MOE_STREAM_DOWN2_D_FP8 2
#endif

constexpr int unroll_of(int d) { return d % 2 == 0 ? d : 2 * d; }

bool stream_gemm_fits(int w_dtype, int64_t K, int64_t I) {
  const bool fp8 = w_dtype == MOE_DTYPE_FP8_E4M3;
  const int eb = fp8 ? 1 : 2;
  const int ug = unroll_of(fp8 ? MOE_STREAM_GATED_D_FP8 : MOE_STREAM_GATED_D_BF16);
  const int ud = unroll_of(fp8 ? MOE_STREAM_DOWN_D_FP8 : MOE_STREAM_DOWN_D_BF16);
  return I % 128 == 0 && (K * eb / 128) % ug == 0 && (I * eb / 128) % ud == 0;
}

// Wide gated panels for fp8: each wavefront holds 2 gate + 2 up blocks, so a
// work item covers 256 act columns (two quantisation groups) and re-reads the
// expert's activation rows half as often per weight byte; worth it once
// experts average 32 to 80 rows, and while the halved item count still gives
// every compute unit one (an expert-parallel shard of a few experts keeps
// the narrow panels).  Weights are prefetched one K-step ahead to leave
// registers for the doubled accumulators.
#ifndef MOE_STREAM_WIDE_FP8
#define MOE_STREAM_WIDE_FP8 1
#endif
#ifndef MOE_STREAM_WIDE_D_FP8
#define MOE_STREAM_WIDE_D_FP8 1
#endif
bool stream_gemm_gated_wide(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I) {
  return MOE_STREAM_WIDE_FP8 && w_dtype == MOE_DTYPE_FP8_E4M3 && I % 256 == 0 &&
         (K / 128) % unroll_of(MOE_STREAM_WIDE_D_FP8) == 0 && pairs >= 32 * E && pairs <= 80 * E &&
         E * (I / 256) >= 256;
}

// Their accumulators fit up to 6 blocks of 16 rows: the tile plan caps tiles
// at 96 rows (an expert above that takes two tiles).
int stream_gemm_wide_tile_rows() { return kMinPlanTileRows; }

int stream_gemm_down_blocks(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I) {
  const bool fp8 = w_dtype == MOE_DTYPE_FP8_E4M3;
  const int eb = fp8 ? 1 : 2;
  // fp8 with the wide gated panels' row tiles (experts of 32-80 rows): four
  // blocks, 512 output columns per item, half the activation re-reads
  if (MOE_STREAM_DOWN4_FP8 && fp8 && K % 512 == 0 && (I / 128) % unroll_of(MOE_STREAM_DOWN4_D_FP8) == 0 &&
      stream_gemm_gated_wide(w_dtype, E, pairs, K, I))
    return 4;
  const int u2 = unroll_of(fp8 ? MOE_STREAM_DOWN2_D_FP8 : MOE_STREAM_DOWN2_D_BF16);
  const int64_t items = std::min(E, pairs) * (K / 256);   // at most one row tile per expert
  return K % 256 == 0 && (I * eb / 128) % u2 == 0 && items >= 512 ? 2 : 1;
}

// Balanced fp8 down plan.  With one item width, the last round of items can
// leave compute units idle (decode M=256: 448 items of 512 columns on 256
// units, the second round three quarters full); these kernels stream at a
// rate per unit, not per chip, so a part-empty round costs a whole one.  Each
// row tile's K / 128 column units are then dealt out as bal_h items of w
// blocks per wavefront and bal_p - bal_h items of w - 1 (w = 4 where the
// uniform plan has 4, else 3), chosen so that the wide items fill whole rounds;
// the plan is kept only where a model of the rounds (time per item: its
// blocks plus a fixed quarter block for its prologue and epilogue) prefers it.
// The expected tile count is one per expert with tokens; a different count on
// the device changes the balance, not the result.
#ifndef MOE_STREAM_DOWN_BALANCE
#define MOE_STREAM_DOWN_BALANCE 1
#endif
#ifndef MOE_STREAM_DOWN3_D_FP8
#define MOE_STREAM_DOWN3_D_FP8 2
#endif
int stream_gemm_down_plan(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I, int *bal_p, int *bal_h) {
  *bal_p = *bal_h = 0;
  const int nb0 = stream_gemm_down_blocks(w_dtype, E, pairs, K, I);
  if (!MOE_STREAM_DOWN_BALANCE || w_dtype != MOE_DTYPE_FP8_E4M3 || nb0 < 2 || K % 128 != 0) return nb0;
  const int w = nb0 == 4 ? 4 : 3;
  if (w == 3 && (I / 128) % unroll_of(MOE_STREAM_DOWN3_D_FP8) != 0) return nb0;
  const int64_t tiles = std::min(E, pairs), units = K / 128, cus = 8 * kXcdUnits;
  if (tiles <= 0 || units % nb0 != 0) return nb0;
  const double o = 0.25;
  auto rounds = [&](int64_t n) { return (double)((n + cus - 1) / cus); };
  double best = rounds(tiles * (units / nb0)) * (nb0 + o);
  for (int64_t p = (units + w - 1) / w; p * (w - 1) <= units; ++p) {
    const int64_t h = units - p * (w - 1);   // items of w blocks; p - h of w - 1
    if (h <= 0 || h >= p || (tiles * h) % cus != 0) continue;
    const double cost = rounds(tiles * h) * (w + o) + rounds(tiles * (p - h)) * (w - 1 + o);
    if (cost < best - 1e-9) {
      best = cost;
      *bal_p = (int)p;
      *bal_h = (int)h;
    }
  }
  return *bal_p ? w : nb0;
}

#ifndef MOE_STREAM_DOWN_SPLIT
#define MOE_STREAM_DOWN_SPLIT 2
#endif
int stream_gemm_down_split(int w_dtype, int64_t E, int64_t pairs, int64_t K, int64_t I) {
  if (MOE_STREAM_DOWN_SPLIT <= 1 || w_dtype != MOE_DTYPE_BF16 || K % 256 != 0) return 1;
  if (stream_gemm_down_blocks(w_dtype, E, pairs, K, I) != 1) return 1;
  const int S = MOE_STREAM_DOWN_SPLIT;
  const int u2 = unroll_of(MOE_STREAM_DOWN2_D_BF16);
  // two-block panels of every split: at least one item per compute unit
  const int64_t items = std::min(E, pairs) * (K / 256) * S;
  return (I * 2 / 128) % ((int64_t)S * u2) == 0 && items >= 256 ? S : 1;
}

hipError_t launch_split_reduce(const float *part, int S, int64_t stride, const int32_t *perm, int64_t n_slots,
                               int n_pairs, int K, int out_dtype, void *out, hipStream_t s) {
  if (n_slots <= 0) return hipSuccess;
  dim3 grid((unsigned)n_slots), block(256);
  if (out_dtype == MOE_DTYPE_BF16)
    split_reduce_kernel<true><<<grid, block, 0, s>>>(part, S, stride, perm, n_pairs, K, out);
  else
    split_reduce_kernel<false><<<grid, block, 0, s>>>(part, S, stride, perm, n_pairs, K, out);
  return hipGetLastError();
}

hipError_t launch_stream_gemm(int w_dtype, int out_dtype, GemmKind kind, const GemmParams &g, int n_tiles,
                              int blocks, hipStream_t s) {
  const bool fp8 = w_dtype == MOE_DTYPE_FP8_E4M3;
  if (kind == kGemmGatedAct) {
    // n_tiles = I / 128 from the caller; wide panels (blocks == 4) cover 256 act columns
    if (fp8)
      return blocks == 4 ? launch_cfg<1, true, 4, MOE_STREAM_WIDE_D_FP8, 128>(out_dtype, g, n_tiles / 2, s)
                         : launch_cfg<1, true, 2, MOE_STREAM_GATED_D_FP8, 128>(out_dtype, g, n_tiles, s);
    return launch_cfg<2, true, 2, MOE_STREAM_GATED_D_BF16, 256>(out_dtype, g, n_tiles, s);
  }
  const int down_blocks = blocks;
  if (g.k_split > 1) {
    // K split (bf16): two blocks per wavefront, fp32 partial sums by slot
    if (fp8 || down_blocks != 2) return hipErrorInvalidValue;
    return launch_cfg<2, false, 2, MOE_STREAM_DOWN2_D_BF16, 256>(MOE_DTYPE_F32, g, n_tiles / 2 * g.k_split, s);
  }
  // down: n_tiles = K / 128 from the caller, K / 256 with two blocks per
  // wavefront, K / 512 with four (fp8); the balanced plan sizes its own grid
  if (g.bal_p > 0) {
    if (!fp8 || g.bal_h <= 0 || g.bal_h >= g.bal_p) return hipErrorInvalidValue;
    if (down_blocks == 4) return launch_cfg<1, false, 4, MOE_STREAM_DOWN4_D_FP8, 128>(out_dtype, g, 0, s);
    if (down_blocks == 3) return launch_cfg<1, false, 3, MOE_STREAM_DOWN3_D_FP8, 128>(out_dtype, g, 0, s);
    return hipErrorInvalidValue;
  }
  if (down_blocks == 4 && fp8)
    return launch_cfg<1, false, 4, MOE_STREAM_DOWN4_D_FP8, 128>(out_dtype, g, n_tiles / 4, s);
  if (down_blocks == 2)
    return fp8 ? launch_cfg<1, false, 2, MOE_STREAM_DOWN2_D_FP8, 128>(out_dtype, g, n_tiles / 2, s)
               : launch_cfg<2, false, 2, MOE_STREAM_DOWN2_D_BF16, 256>(out_dtype, g, n_tiles / 2, s);
  return fp8 ? launch_cfg<1, false, 1, MOE_STREAM_DOWN_D_FP8, 128>(out_dtype, g, n_tiles, s)
             : launch_cfg<2, false, 1, MOE_STREAM_DOWN_D_BF16, 256>(out_dtype, g, n_tiles, s);
}

}  // namespace moe
