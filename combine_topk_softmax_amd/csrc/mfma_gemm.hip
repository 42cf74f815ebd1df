// Compute-bound grouped expert GEMMs (bf16) for prefill batches whose experts
// hold many rows: the same two products as grouped_gemm.hip (modular_kernel.py
// page, header comment and FusedMoEPermuteExpertsUnpermute: a first GEMM, the
// gated activation, optional quantisation, a second GEMM; per-expert row
// counts read on the device, as on the worst-tokens page),
//
//   gated GEMM   act[slot, j] = silu(A w1[e, j]) * (A w1[e, I + j])
//   down GEMM    out[row(slot), :] = act[slot, :] w2[e]^T
//
// laid out for gfx950's matrix cores when flops, not weight bytes, set the
// time:
//
//  * a workgroup computes a 256-row x 256-column tile (rows: one expert's
//    slots from the device tile plan; columns: 128 gate + the matching 128 up
//    weight rows, or 256 output columns), so every operand byte staged in LDS
//    feeds 256 MFMA columns or rows;
//  * 8 wavefronts in a 2 x 4 grid, each owning 128 x 64 as 4 x 2 blocks of
//    v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane, two
//    wavefronts per SIMD);
//  * K advances 64 elements per step; both operands go global -> registers ->
//    a double-buffered, padded LDS tile (72 KB per stage), the next
//    step's global loads being in flight during the current step's 32 MFMAs
//    per wavefront; one barrier per step;
//  * all loads are unconditional (rows past the count read a valid row whose
//    products are never stored), so the compiler never waits for every
//    outstanding load in front of the MFMAs; the MFMAs of a wavefront's
//    32-row blocks past the count are skipped (the main loop is instantiated
//    per count of live blocks), which on the skewed prefill's 567 row tiles
//    (10.7% of their rows padding) took the gated GEMM from 3.83 to 3.62 ms
//    and the down GEMM from 2.21 to 1.96 ms;
//  * work items are dealt out XCD by XCD and, inside an XCD's range, grouped
//    eight row tiles at a time per column tile, so the workgroups resident on
//    one XCD share both activation rows and weight panels through its L2.
#include "moe_device.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Staging registers are native vectors: HIP's uint4 is a struct whose copies
// become memcpy, which keeps a staging array in memory (LDS or scratch).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kRows = 256;            // tile rows (slots)
constexpr int kCols = 256;            // tile columns (weight rows)
constexpr int kStep = 128;            // bytes of K per step (64 bf16)
#ifndef MOE_MFMA_GROUP_M
#define MOE_MFMA_GROUP_M 8
#endif
constexpr int kGroupM = MOE_MFMA_GROUP_M;   // row tiles per L2 group

// LDS tiles are [rows][144 B]: 128 bytes of K plus 16 bytes of padding.  A
// fragment read is one 16-byte chunk of 16 consecutive rows per 128-bit access
// pass; with a 144-byte pitch those rows start 36 banks apart, which covers
// gfx950's 64 banks exactly once.  Unlike an XOR swizzle, the padding keeps
// every K sub-step at a constant offset from the row's address, so a fragment
// needs one address register per row block instead of one per sub-step.
constexpr int kPitch = kStep + 16;
__device__ __forceinline__ int lds_at(int row, int b) { return row * kPitch + b; }

template <bool GATED, bool PACKED>
__global__ __launch_bounds__(kThreads) void mfma_gemm_kernel(const GemmParams g, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kRows * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kCols * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;
  const bool dense = g.t.dense_rows > 0;
  const int m_tiles = dense ? (g.t.dense_rows + kRows - 1) / kRows : *g.t.tile_count;
  const int total = m_tiles * n_tiles;

  // XCD-contiguous item ranges, then row-tile groups inside each range.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  const int item = xcd * per + local;
  if (local >= per || item >= total) return;
  const int grp = item / (kGroupM * n_tiles);
  const int gm = min(kGroupM, m_tiles - grp * kGroupM);
  const int within = item - grp * kGroupM * n_tiles;
  const int mt = grp * kGroupM + within % gm;
  const int nt = within / gm;

  int e, T;
  int64_t row0;
  if (dense) {
    e = 0;
    row0 = (int64_t)mt * kRows;
    T = min(kRows, g.t.dense_rows - mt * kRows);
  } else {
    const int32_t *d = g.t.tiles + (int64_t)mt * 4;
    e = d[0];
    row0 = (int64_t)d[1] + d[2];
    T = d[3];
  }

  const int64_t row_bytes = g.Kred * 2;
  const int nk = (int)(row_bytes / kStep);
  const int chunk = tid & 7;
  const PackedGeom pg = packed_geom(g.Nw, row_bytes, GATED);
  const int64_t kstride = PACKED ? packed_kstep_stride(pg) : kStep;

  // This thread stages chunk `chunk` of rows (tid / 8) + 64 i, i < 4, of both
  // operand tiles.  Rows past the tile's count and padding slots read row 0
  // instead: an A row only feeds its own output row, and the epilogue writes
  // nothing for those rows, so their contents never matter (and no select on
  // loaded data forces an early wait for the loads).
  const uint8_t *a_src[4];
  // Weight rows: base_i + (tid / 8) with base_i a multiple of 64, so in both
  // layouts the address splits into a per-lane part (row within the 64-row
  // group, chunk) shared by all four rows and a wavefront-uniform part per row
  // group, which stays in scalar registers.
  int64_t b_uni[4];
  auto wbase = [&](int i) -> int64_t {
    if (GATED) return i < 2 ? (int64_t)nt * 128 + 64 * i : g.half_n + (int64_t)nt * 128 + 64 * (i - 2);
    return (int64_t)nt * kCols + 64 * i;
  };
  const int r0 = tid >> 3;
  int64_t b_lane;
  if (PACKED)
    b_lane = packed_piece(pg, e, wbase(0) + r0, 0, chunk) - packed_piece(pg, e, wbase(0), 0, 0);
  else
    b_lane = (int64_t)r0 * row_bytes + chunk * 16;
  const uint8_t *b_src = reinterpret_cast<const uint8_t *>(g.w) + b_lane;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    b_uni[i] = PACKED ? packed_piece(pg, e, wbase(i), 0, 0) : ((int64_t)e * g.Nw + wbase(i)) * row_bytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 64 * i;
    a_src[i] = reinterpret_cast<const uint8_t *>(g.a) + chunk * 16;
    if (r < T) {
      const int64_t s = row0 + r;
      int64_t arow = s;
      if (g.perm) {
        const int f = g.perm[s];
        arow = (f >= 0 && f < g.n_pairs) ? f / g.topk : -1;
      }
      if (arow >= 0) a_src[i] = reinterpret_cast<const uint8_t *>(g.a) + arow * row_bytes + chunk * 16;
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

  // Two register sets of staged operands: step j's loads land in set j % 2,
  // issued two steps before they are stored to LDS.
  u32x4 ra[2][4], rb[2][4];
  auto gload = [&](int set, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[set][i] = *reinterpret_cast<const u32x4 *>(a_src[i] + (int64_t)ks * kStep);
      rb[set][i] = *reinterpret_cast<const u32x4 *>(b_src + b_uni[i] + (int64_t)ks * kstride);
    }
  };
  auto lstore = [&](int st, int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 64 * i;
      *reinterpret_cast<u32x4 *>(&As[st][lds_at(r, chunk * 16)]) = ra[set][i];
      *reinterpret_cast<u32x4 *>(&Bs[st][lds_at(r, chunk * 16)]) = rb[set][i];
    }
  };
  // B rows of this wavefront's two column blocks: gate and up (gated), or two
  // adjacent 32-column blocks (down).
  const int brow0 = GATED ? wn * 32 : wn * 64;
  const int brow1 = GATED ? 128 + wn * 32 : wn * 64 + 32;
  // One K-step of MFMAs from LDS stage st over this wavefront's first NMB
  // 32-row blocks (the blocks past the tile's row count are skipped: their
  // rows are never stored).  The step's global loads for K-step ks go out
  // spread over the MFMAs, two per 16-element sub-step, into register set
  // `set`: issued back to back, a workgroup's loads fill the texture address
  // queue and every wavefront stalls at issue until it drains, with its MFMAs
  // queued behind the loads.
  auto compute = [&](auto NMB_, int st, int set, int ks) {
    constexpr int NMB = decltype(NMB_)::value;
    const uint8_t *A = As[st];
    const uint8_t *B = Bs[st];
#pragma unroll
    for (int kk = 0; kk < kStep / 32; ++kk) {
      const int boff = kk * 32 + (lane >> 5) * 16;
      bf16x8 b0, b1;
      if (NMB > 0) {
        b0 = *reinterpret_cast<const bf16x8 *>(B + lds_at(brow0 + (lane & 31), boff));
        b1 = *reinterpret_cast<const bf16x8 *>(B + lds_at(brow1 + (lane & 31), boff));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < NMB) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(A + lds_at(wm * 128 + mb * 32 + (lane & 31), boff));
          acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[mb][1], 0, 0, 0);
        }
        if (mb == 1) {
          ra[set][kk] = *reinterpret_cast<const u32x4 *>(a_src[kk] + (int64_t)ks * kStep);
          rb[set][kk] = *reinterpret_cast<const u32x4 *>(b_src + b_uni[kk] + (int64_t)ks * kstride);
        }
      }
      // keep each sub-step's two loads with its MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline: LDS stage s % 2 holds K-step s while it is multiplied; register
  // set s % 2 receives step s + 2 during that multiply (its step s was stored
  // to LDS before the barrier that opened it), and step s + 1, loaded during
  // the previous multiply, is stored to the other stage after it.  Every load
  // thus has about two steps of matrix work to arrive in, and steps past the
  // last reload the last one instead of branching around the loads.  nk is
  // even (the host requires K and I to be multiples of 128 elements), so the
  // loop runs in pairs and every register-set index is a constant.  The loop
  // is instantiated per count of this wavefront's 32-row blocks that hold
  // real rows (a tile's last rows of an expert are often fewer than 256).
  auto main_loop = [&](auto NMB) {
    gload(0, 0);
    lstore(0, 0);
    gload(1, min(1, nk - 1));
    __syncthreads();
    for (int ks = 0; ks < nk; ks += 2) {
      compute(NMB, 0, 0, min(ks + 2, nk - 1));
      lstore(1, 1);
      __syncthreads();
      compute(NMB, 1, 1, min(ks + 3, nk - 1));
      lstore(0, 0);
      __syncthreads();
    }
  };
  const int nmb = min(4, max(0, (T - wm * 128 + 31) / 32));
  switch (nmb) {
    case 4: main_loop(std::integral_constant<int, 4>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }

  // Epilogue.  Accumulator element i of a 32x32 block sits at column
  // (lane % 32) and row 8 (i / 4) + 4 (lane / 32) + i % 4.  The bf16 tile is
  // staged in LDS (rows 0-127 in the A buffers, 128-255 in the B buffers) and
  // leaves as whole rows of 16-byte stores; the 16-byte row padding puts the
  // two rows of each 2-byte store instruction on different banks.
  constexpr int kOutCols = GATED ? 128 : kCols;
  constexpr int kRowB = kOutCols * 2, kSP = kRowB + 16, kChunk = kRowB / 16;
  static_assert(128 * kSP <= 2 * kRows * kPitch, "half a tile fits each operand's LDS buffers");
  __syncthreads();   // every wavefront is done reading the operand tiles
  uint8_t *half = wm == 0 ? &As[0][0] : &Bs[0][0];   // rows wm*128 .. +128
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint8_t *row = half + (mb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3)) * kSP;
      if constexpr (GATED) {
        const float v = gated_act(acc[mb][0][i], acc[mb][1][i], g.act);
        *reinterpret_cast<uint16_t *>(row + (wn * 32 + (lane & 31)) * 2) = f32_to_bf16_bits(v);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          *reinterpret_cast<uint16_t *>(row + (wn * 64 + nb * 32 + (lane & 31)) * 2) = f32_to_bf16_bits(acc[mb][nb][i]);
      }
    }
  }
  __syncthreads();
  const int64_t col0 = (int64_t)nt * kOutCols;
  for (int c = tid; c < T * kChunk; c += kThreads) {
    const int r = c / kChunk, off = (c - r * kChunk) * 16;
    const int64_t slot = row0 + r;
    int64_t orow = slot;
    if constexpr (!GATED) {
      if (g.out_perm) {
        orow = g.out_perm[slot];
        if (orow < 0 || orow >= g.n_pairs) continue;
      }
    }
    const uint8_t *src = (r < 128 ? &As[0][0] : &Bs[0][0]) + (r & 127) * kSP + off;
    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(g.out) + (orow * g.ldo + col0) * 2 + off) =
        *reinterpret_cast<const u32x4 *>(src);
  }
}

}  // namespace

int mfma_gemm_tile_rows() { return kRows; }

bool mfma_gemm_fits(int w_dtype, int act_dtype, int64_t K, int64_t I) {
  // bf16 in and out; gated column tiles of 128 act columns, down column tiles
  // of 256 outputs, K-steps of 64 elements on both reductions.
  return w_dtype == MOE_DTYPE_BF16 && act_dtype == MOE_DTYPE_BF16 && I % 128 == 0 && K % 256 == 0 &&
         I % 64 == 0;
}

int mfma_gemm_n_tiles(GemmKind kind, int64_t Nw) { return (int)(kind == kGemmGatedAct ? Nw / 256 : Nw / kCols); }

hipError_t launch_mfma_gemm(GemmKind kind, const GemmParams &g, int n_tiles, hipStream_t s) {
  const int m_tiles = g.t.dense_rows > 0 ? (g.t.dense_rows + kRows - 1) / kRows : g.t.max_tiles;
  // whole rounds of 8 blocks: every XCD needs as many blocks as the longest
  // XCD range of items
  const dim3 grid((unsigned)(((m_tiles * n_tiles + 7) / 8) * 8)), block(kThreads);
  const bool gated = kind == kGemmGatedAct;
  if (gated)
    g.w_packed ? mfma_gemm_kernel<true, true><<<grid, block, 0, s>>>(g, n_tiles)
               : mfma_gemm_kernel<true, false><<<grid, block, 0, s>>>(g, n_tiles);
  else
    g.w_packed ? mfma_gemm_kernel<false, true><<<grid, block, 0, s>>>(g, n_tiles)
               : mfma_gemm_kernel<false, false><<<grid, block, 0, s>>>(g, n_tiles);
  return hipGetLastError();
}

}  // namespace moe
