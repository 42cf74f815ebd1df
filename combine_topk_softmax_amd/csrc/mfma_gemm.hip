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
//  * a workgroup computes a 128-row x 256-column tile (rows: one expert's
//    slots from the device tile plan; columns: 128 gate + the matching 128 up
//    weight rows, or 256 output columns) with 4 wavefronts side by side, each
//    owning 128 x 64 as 8 x 4 blocks of v_mfma_f32_16x16x32_bf16 (128 fp32
//    accumulators per lane).  Two workgroups share a CU, one wavefront of
//    each per SIMD: while one waits at its K-step barrier, the other's MFMAs
//    keep the SIMD busy (with one 8-wavefront workgroup per CU every SIMD
//    idled at each barrier, about a fifth of the K-step);
//  * the activation rows (A) are copied global -> LDS by the LDS DMA
//    (global_load_lds_dwordx4: no staging registers, no LDS store
//    instructions) into 4 stages of 128 rows x 128 bytes (64 elements of K),
//    the 16-byte chunks of a row XOR-swizzled by the row's low bits so that
//    the fragment reads of 8 consecutive rows hit distinct banks.  The copy
//    of K-step s + 3 is issued at the end of step s, into the stage the
//    step's barrier released, so it has more than two K-steps to land;
//  * the weights (B) never touch LDS: each wavefront loads its own 16-row
//    fragments (each loaded once per workgroup) straight from global memory
//    into registers, 1.5 K-steps ahead
//    through a ring of four sub-step slots.  With the packed weight layout a
//    wavefront's fragment of one 32-element sub-step is one contiguous 1 KB
//    (the layout stores exactly this lane order: lane l holds row l % 16, K
//    elements 16 (l / 16) + 8 p of each 64-element step, p the sub-step), so
//    every B load is fully coalesced; A fragments are read from LDS in the
//    same K order.  Against staging both operands through LDS this moves 37%
//    fewer LDS bytes per flop, and it spreads the global loads over all the
//    wavefronts of a CU (one wavefront's vector-memory throughput is limited: a probe
//    of plain 16-byte loads from L2 gave 32 GB/s per CU with 4 wavefronts per
//    CU, 76 GB/s with 8);
//  * one barrier per K-step, after an explicit `s_waitcnt vmcnt(16)` (all but
//    the loads of the last step and a half have landed).  The LDS copies are
//    issued in inline asm: the compiler cannot tell the four stages apart and
//    would otherwise wait for every copy in flight before each fragment read,
//    and a workgroup fence would do the same, so the barrier is a bare one;
//  * addressing stays out of the vector registers: the weights are read
//    through a buffer resource on the expert's block (a per-lane 32-bit
//    offset plus scalar block and step offsets), the A copies take a scalar
//    base plus one 32-bit row offset per lane, and the wavefront index is
//    made uniform, which leaves room for a sub-step's eight A fragments to be
//    read together ahead of its MFMAs (plus two of the next sub-step's during
//    the last MFMAs) instead of two at a time just before their MFMAs;
//  * all loads are unconditional (rows past the count read a valid row whose
//    products are never stored);
//  * work items are dealt out XCD by XCD and, inside an XCD's range, grouped
//    16 (gated) or 6 (down) row tiles at a time per column tile, so the
//    workgroups resident on one XCD share both activation rows and weight
//    panels through its L2.
//
// Measured on one MI355X on the skewed prefill's expert shapes (packed
// weights), same box and run, against the previous kernel (one 256-row tile
// per CU, both operands staged global -> registers -> LDS, 32x32x16 MFMAs):
// gated GEMM 3.52-3.64 -> 3.06 ms, down GEMM 1.91-1.99 -> 1.72 ms; the scalar
// addressing and early fragment reads then took 2.99 -> 2.87 ms and 1.74 ->
// 1.70 ms, and two 128-row workgroups per CU in place of one 256-row
// workgroup of 8 wavefronts (2 x 4) 2.87 -> 2.75 ms and 1.69 -> 1.64 ms.
// With both operands made cache-resident (a timing copy of an earlier
// schedule) the loop ran no faster: the loads are hidden.  The MFMA pipes are
// busy 69% of the gated GEMM's cycles; the rest goes to the K-step barrier,
// the copy issue and the empty rows of each expert's last, partial tile.
#include "moe_device.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 128;              // tile rows (slots)
constexpr int kCols = 256;              // tile columns (weight rows)
constexpr int kStep = 128;              // bytes of K per step (64 bf16)
constexpr int kStages = 4;              // A stages in LDS
constexpr int kStage = kRows * kStep;   // 16 KB
// row tiles per L2 group, measured on the skewed prefill (A/B runs on one
// box): 16 for the gated GEMM (12 column tiles per expert there; 1% faster
// than 8, while 12 and 32 were slower), 6 for the down GEMM (16 column tiles;
// 1.6% faster than 8, 4 in between, 16 slower)
constexpr int kGroupGated = 16, kGroupDown = 6;
constexpr int kPrefetch = 2;            // fragments of the second sub-step read early

#define MOE_LP(p) ((__attribute__((address_space(3))) void *)(p))

template <bool GATED, bool PACKED>
__global__ __launch_bounds__(kThreads, 2) void mfma_gemm_kernel(const GemmParams g, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];
  __shared__ int32_t Orow[GATED ? 1 : kRows];   // down: output row of each tile row (-1: none)

  // the wavefront index is uniform: block and step offsets derived from it
  // stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wv;   // the wavefront's 64 columns of the tile
  const bool dense = g.t.dense_rows > 0;
  const int m_tiles = dense ? (g.t.dense_rows + kRows - 1) / kRows : *g.t.tile_count;
  const int total = m_tiles * n_tiles;

  // XCD-contiguous item ranges, then row-tile groups inside each range.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  const int item = xcd * per + local;
  if (local >= per || item >= total) return;
  constexpr int kGroupM = GATED ? kGroupGated : kGroupDown;
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
  const PackedGeom pg = packed_geom(g.Nw, row_bytes, GATED);
  const int64_t kstride = PACKED ? packed_kstep_stride(pg) : kStep;

  // A copies: wavefront wv fills rows wv*32 + 8j + lane/8 (j < 4) of each
  // stage; lane l writes slot l % 8 of its row, which holds global chunk
  // (l % 8) ^ (row & 7) = (l % 8) ^ (l / 8).  Rows past the tile's count and
  // padding slots read the base row instead: an A row only feeds its own
  // output row, and the epilogue writes nothing for those.  Row offsets are
  // 32-bit from a wavefront-uniform base: the tile's first slot row when A
  // is indexed by slot, the start of A when rows are gathered through perm.
  const int rr = lane >> 3, cg = (lane & 7) ^ rr;
  const uint8_t *a_base = reinterpret_cast<const uint8_t *>(g.a) + (g.perm ? 0 : row0 * row_bytes);
  uint32_t a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = wv * 32 + 8 * j + rr;
    a_off[j] = (uint32_t)(cg * 16);
    if (q < T) {
      int64_t arow = q;
      if (g.perm) {
        const int f = g.perm[row0 + q];
        arow = (f >= 0 && f < g.n_pairs) ? f / g.topk : -1;
      }
      if (arow >= 0) a_off[j] = (uint32_t)(arow * row_bytes) + (uint32_t)(cg * 16);
    }
  }
  // B: this wavefront's four 16-row blocks -- gated: gate, gate, up, up (act
  // columns wn*32 + 16 (nb % 2)); down: four adjacent blocks of outputs.
  // Loaded through a buffer resource on expert e's weights (32-bit offsets:
  // a per-lane one, and wavefront-uniform block and step offsets).
  auto brow = [&](int nb) -> int64_t {
    if (GATED) return (nb < 2 ? (int64_t)0 : g.half_n) + (int64_t)nt * 128 + wn * 32 + (nb & 1) * 16;
    return (int64_t)nt * kCols + wn * 64 + nb * 16;
  };
  const int bc = 2 * (lane >> 4);   // lane's first 16-byte chunk of a K-step
  const int64_t e_bytes = g.Nw * row_bytes;
  const uint32_t b_lane = PACKED ? (uint32_t)(packed_piece(pg, e, brow(0) + (lane & 15), 0, bc) -
                                              packed_piece(pg, e, brow(0), 0, 0))
                                 : (uint32_t)((lane & 15) * row_bytes + bc * 16);
  uint32_t b_off[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    b_off[nb] = (uint32_t)((PACKED ? packed_piece(pg, e, brow(nb), 0, 0) : ((int64_t)e * g.Nw + brow(nb)) * row_bytes) -
                           (int64_t)e * e_bytes);
  // raw buffer (stride 0) over the expert's e_bytes (< 2^31, checked on the
  // host); word 3 gives the 32-bit data format that raw loads require
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(reinterpret_cast<const uint8_t *>(g.w)) + (int64_t)e * e_bytes, (short)0,
      (int)e_bytes, 0x00020000);
  constexpr uint32_t kPstep = PACKED ? 1024 : 16;   // the second sub-step of a K-step

  f32x4 acc[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 bf[4][4];   // [slot][nb]: B of four consecutive 32-element sub-steps

  // LDS byte address of this wavefront's first copy row in stage 0
  const uint32_t lds0 = (uint32_t)(uintptr_t)MOE_LP(smem) + (uint32_t)(wv * 32) * kStep;
  // A of K-step ks into `stage` (scalar base + the 32-bit row offsets).
  // Issued in asm: the compiler's wait counting cannot tell the four stages
  // apart and would wait for every copy in flight before each fragment read;
  // the copies' own waits are the explicit vmcnt before each barrier.
  auto copy_a = [&](int stage, int ks) {
    const uint8_t *src = a_base + (int64_t)ks * kStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(stage * kStage + 8 * j * kStep));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_nop 0"
                   :: "s"(m0v), "v"(a_off[j]), "s"(src) : "memory", "m0");
    }
  };
  // B of sub-step t (K-step t / 2, sub-step t % 2) into `slot`
  auto load_b = [&](int slot, int t) {
    const int ks = min(t >> 1, nk - 1), p = t & 1;
    const uint32_t so = (uint32_t)ks * (uint32_t)kstride + (uint32_t)p * kPstep;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bf[slot][nb] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, b_lane, b_off[nb] + so, 0));
  };
  // A fragment of 16-row block mb, sub-step p: lane l reads row
  // 16 mb + l % 16 of the stage, 16-byte chunk bc + p swizzled by the
  // row's low bits (= l % 8); one base per sub-step, the rest immediate offsets
  uint32_t a_rd[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    a_rd[p] = (uint32_t)((lane & 15) * kStep + (((bc + p) ^ (lane & 7)) << 4));
  auto read_a = [&](int stage, int p, int mb) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(smem + stage * kStage + mb * 16 * kStep + a_rd[p]);
  };

  // Prologue: A steps 0-2 copying, B sub-steps 0-2.  The order matters:
  // vmcnt counts loads in issue order.
  copy_a(0, 0);
  copy_a(1, min(1, nk - 1));
  load_b(0, 0);
  load_b(1, 1);
  load_b(2, 2);
  copy_a(2, min(2, nk - 1));
  // K-step ks (A stage ks % 4, B slots 2ks % 4 and (2ks + 1) % 4, all
  // compile-time): each sub-step t first issues the B loads of sub-step t + 3
  // into the slot sub-step t - 1 freed; the A copy of ks + 3 goes out at the
  // end, into the stage the barrier released.  Steps past the last re-copy
  // and reload the last one instead of branching around the loads.  A
  // sub-step's eight fragment reads are issued together ahead of its MFMAs,
  // and the first kPrefetch of the second sub-step's go out during the
  // first sub-step's last MFMAs, so neither sub-step starts on a bare LDS
  // latency (the compiler would otherwise read each pair of fragments just
  // before its MFMAs).
  auto kstep = [&](auto ST_, int ks) {
    constexpr int ST = decltype(ST_)::value, S0 = (2 * ST) & 3, S1 = (2 * ST + 1) & 3;
    // vmcnt(16): all but the last 16 loads (the previous step's B loads and
    // A copy, and the A copy before them) have landed, among them the A copy
    // of ks and the B of this step's first sub-step; after the barrier
    // everyone's A of ks is in and the stage of ks - 1 is free.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_b((S0 + 3) & 3, 2 * ks + 3);
    bf16x8 af[8], pf[kPrefetch];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) af[mb] = read_a(ST, 0, mb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bf[S0][nb], acc[mb][nb], 0, 0, 0);
      if (mb == 5) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) pf[i] = read_a(ST, 1, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_b((S1 + 3) & 3, 2 * ks + 4);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) af[mb] = mb < kPrefetch ? pf[mb] : read_a(ST, 1, mb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bf[S1][nb], acc[mb][nb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    copy_a((ST + 3) & 3, min(ks + 3, nk - 1));
  };
  // nk is even (K and I are multiples of 128 elements): groups of four steps,
  // then a last pair when nk % 4 == 2
  int ks = 0;
  for (; ks + 4 <= nk; ks += 4) {
    kstep(std::integral_constant<int, 0>{}, ks);
    kstep(std::integral_constant<int, 1>{}, ks + 1);
    kstep(std::integral_constant<int, 2>{}, ks + 2);
    kstep(std::integral_constant<int, 3>{}, ks + 3);
  }
  if (ks < nk) {
    kstep(std::integral_constant<int, 0>{}, ks);
    kstep(std::integral_constant<int, 1>{}, ks + 1);
  }

  // Epilogue.  A 16x16 accumulator block holds column l % 16 and rows
  // 4 (l / 16) + i in lane l.  The bf16 tile is staged in the (now idle) A
  // stages, rows of kRowB bytes with their 16-byte chunks XOR-swizzled by row,
  // and leaves as whole rows of 16-byte stores.
  constexpr int kOutCols = GATED ? 128 : kCols;
  constexpr int kRowB = kOutCols * 2, kChunk = kRowB / 16;
  static_assert(kRows * kRowB <= kStages * kStage, "the output tile fits the A stages");
  auto osw = [&](int r, int byte) { return r * kRowB + ((((byte >> 4) ^ (r & 7)) << 4) | (byte & 15)); };
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): the last (unused) copies have landed
  __syncthreads();
  // down: every tile row's output row, loaded once here (its latency runs
  // under the staging below) instead of once per 16-byte store
  int orow_t = -1;
  if constexpr (!GATED) {
    if (tid < T) {
      const int64_t slot = row0 + tid;
      orow_t = (int)slot;   // slots are int32 in the tile plan
      if (g.out_perm) {
        orow_t = g.out_perm[slot];
        if (orow_t >= g.n_pairs) orow_t = -1;
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mb * 16 + (lane >> 4) * 4 + i;
      if constexpr (GATED) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float v = gated_act(acc[mb][nb][i], acc[mb][nb + 2][i], g.act);
          *reinterpret_cast<uint16_t *>(smem + osw(r, (wn * 32 + nb * 16 + (lane & 15)) * 2)) = f32_to_bf16_bits(v);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          *reinterpret_cast<uint16_t *>(smem + osw(r, (wn * 64 + nb * 16 + (lane & 15)) * 2)) =
              f32_to_bf16_bits(acc[mb][nb][i]);
      }
    }
  }
  if constexpr (!GATED) {
    if (tid < kRows) Orow[tid] = orow_t;
  }
  __syncthreads();
  const int64_t col0 = (int64_t)nt * kOutCols;
  for (int c = tid; c < T * kChunk; c += kThreads) {
    const int r = c / kChunk, off = (c - r * kChunk) * 16;
    int64_t orow = row0 + r;
    if constexpr (!GATED) {
      orow = Orow[r];
      if (orow < 0) continue;
    }
    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(g.out) + (orow * g.ldo + col0) * 2 + off) =
        *reinterpret_cast<const u32x4 *>(smem + osw(r, off));
  }
}

}  // namespace

int mfma_gemm_tile_rows() { return kRows; }

bool mfma_gemm_fits(int w_dtype, int act_dtype, int64_t K, int64_t I, int64_t M) {
  // bf16 in and out; gated column tiles of 128 act columns, down column tiles
  // of 256 outputs, an even number of 64-element K-steps on both reductions;
  // 32-bit offsets within one expert's weights (2I x K) and within the M
  // token rows that the gated GEMM gathers.
  const int64_t lim = (int64_t)1 << 31;
  return w_dtype == MOE_DTYPE_BF16 && act_dtype == MOE_DTYPE_BF16 && I % 128 == 0 && K % 256 == 0 &&
         2 * I * K * 2 < lim && M * K * 2 < lim;
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
