// [Permute-Experts-Unpermute]: the two grouped expert GEMMs on gfx950 MFMA.
//
// The modular_kernel.py page's header comment splits the experts step into a
// first GEMM, the gated activation (FusedMoEPermuteExpertsUnpermute
// .activation, silu_and_mul, whose output is half as wide as its input), an
// optional quantisation and a second GEMM; the worst-tokens page has the grouped
// GEMM read the per-expert counts from a device tensor.  Here:
//
//   gated GEMM   act[slot, j] = silu(A w1[e, j]) * (A w1[e, I + j])
//   down GEMM    out[row(slot), :] = act[slot, :] w2[e]^T
//
// where A is the slot's activation row: x[perm[slot] / topk] (Standard: the
// permutation is applied by gathering rows, never materialised), or row `slot`
// of the batched buffer.  The down GEMM's epilogue writes row perm[slot]
// (= m*topk + j) of the (M, topk, K) output -- the unpermute -- or the same
// batched row.
//
// Work unit: a 128-row tile of one expert's rows (from the device tile plan,
// so counts never reach the host) times 128 weight rows.  Both operands are
// K-contiguous, so tiles are staged global -> registers -> LDS in 16-byte
// chunks with an XOR swizzle of the chunk index (conflict-free both for the
// row-wise stores and for the MFMA fragment reads), double-buffered so that the
// next K-step's global loads are in flight while MFMAs consume the current one.
// Four wavefronts each own a 64x64 sub-tile as 2x2 blocks of
// v_mfma_f32_32x32x16_bf16 (bf16), v_mfma_f32_32x32x16_fp8_fp8 (OCP fp8, with
// the fp32 block scales applied once per 128-wide K block) or
// v_mfma_f32_32x32x2_f32 (fp32).  For the gated GEMM a wave's two 32-column
// blocks are gate column j and up column I + j, so SiLU-and-mul happens in
// registers.  32-row blocks past the tile's row count are skipped.
#include "moe_device.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Staging registers are native vectors: HIP's uint4 is a struct whose copies
// become memcpy, which keeps a staging array in memory (LDS or scratch).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One MFMA flavour per element size.  A step consumes kLaneBytes per lane of
// each operand: lane l holds row (l % 32), k-half (l / 32).
template <int EB>
struct Mfma;

template <>
struct Mfma<2> {  // bf16, 32x32x16
  static constexpr int kLaneBytes = 16;
  typedef bf16x8 frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<1> {  // OCP fp8 e4m3, 32x32x16
  static constexpr int kLaneBytes = 8;
  typedef long frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<4> {  // fp32, 32x32x2
  static constexpr int kLaneBytes = 4;
  typedef float frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

constexpr int kRowBytes = 128;             // one K-step: 128 bytes of every row
constexpr int kTileBytes = 128 * kRowBytes; // 128 rows

// Byte address of (row, byte b of the row's K-step) in a swizzled LDS tile.
// gfx950 serves a 128-bit LDS access 16 lanes at a time over 64 banks (256
// bytes): with 128-byte rows, rows r and r+1 share a bank row, so the 16-byte
// chunk index is XORed with (row / 2) % 8 to give 16 consecutive rows of one
// logical chunk 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int b) {
  return row * kRowBytes + ((((b >> 4) ^ ((row >> 1) & 7)) << 4) | (b & 15));
}

template <int EB, bool GATED, bool OUT_BF16, bool PACKED>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(const GemmParams g) {
  using MM = Mfma<EB>;
  using frag = typename MM::frag;
  constexpr bool kScaled = EB == 1;
  constexpr int kSteps = kRowBytes / (2 * MM::kLaneBytes);

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];
  __shared__ float lds_sa[2][128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m_tiles = g.t.dense_rows > 0 ? (g.t.dense_rows + 127) / 128 : g.t.max_tiles;
  const int t = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;

  int e, nrows;
  int64_t row0;  // first slot of this tile
  if (g.t.dense_rows > 0) {
    e = 0;
    row0 = (int64_t)t * 128;
    nrows = min(128, g.t.dense_rows - t * 128);
  } else {
    if (t >= *g.t.tile_count) return;  // uniform: the device plan has fewer tiles
    const int32_t *d = g.t.tiles + (int64_t)t * 4;
    e = d[0];
    row0 = (int64_t)d[1] + d[2];
    nrows = d[3];
  }

  const int64_t row_bytes = g.Kred * EB;
  const int nk = (int)(row_bytes / kRowBytes);
  const int chunk = tid & 7;
  const PackedGeom pg = packed_geom(g.Nw, row_bytes, GATED);
  const int64_t kstride = PACKED ? packed_kstep_stride(pg) : kRowBytes;   // weight bytes between K-steps

  // Source rows of this thread's 4 A chunks and 4 B chunks per K-step.
  const uint8_t *a_src[4];
  bool a_ok[4];
  const uint8_t *b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    // rows past the count read row 0 (no branch around the load) and are
    // zeroed on their way into LDS
    a_src[i] = reinterpret_cast<const uint8_t *>(g.a) + chunk * 16;
    a_ok[i] = false;
    if (r < nrows) {
      const int64_t s = row0 + r;
      int64_t arow = s;
      if (g.perm) {
        const int f = g.perm[s];
        arow = (f >= 0 && f < g.n_pairs) ? f / g.topk : -1;
      }
      if (arow >= 0) {
        a_src[i] = reinterpret_cast<const uint8_t *>(g.a) + arow * row_bytes + chunk * 16;
        a_ok[i] = true;
      }
    }
    int64_t wrow;
    if (GATED)
      wrow = r < 64 ? (int64_t)nt * 64 + r : g.half_n + (int64_t)nt * 64 + (r - 64);
    else
      wrow = (int64_t)nt * 128 + r;
    if (PACKED)
      b_src[i] = reinterpret_cast<const uint8_t *>(g.w) + packed_piece(pg, e, wrow, 0, chunk);
    else
      b_src[i] = reinterpret_cast<const uint8_t *>(g.w) + ((int64_t)e * g.Nw + wrow) * row_bytes + chunk * 16;
  }
  // fp8: per-row activation scale (thread tid < 128 owns row tid), per-block weight scales.
  const float *sa_src = g.a_scale;
  bool sa_ok = false;
  const float *sw_src[2] = {nullptr, nullptr};
  const int64_t kblocks = g.Kred / 128;
  if constexpr (kScaled) {
    if (tid < nrows) {
      const int64_t s = row0 + tid;
      int64_t arow = s;
      if (g.perm) {
        const int f = g.perm[s];
        arow = (f >= 0 && f < g.n_pairs) ? f / g.topk : -1;
      }
      if (arow >= 0) {
        sa_src = g.a_scale + arow * kblocks;
        sa_ok = true;
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      int64_t wrow0;
      if (GATED)
        wrow0 = (nb ? g.half_n : 0) + (int64_t)nt * 64 + wn * 32;
      else
        wrow0 = (int64_t)nt * 128 + wn * 64 + nb * 32;
      sw_src[nb] = g.w_scale + ((int64_t)e * (g.Nw / 128) + wrow0 / 128) * kblocks;
    }
  }

  bool active[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) active[mb] = wm * 64 + mb * 32 < nrows;

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

  u32x4 ra[4], rb[4];
  float sa_reg = 0.0f;
  auto gload = [&](int ks) {
    const int64_t off = (int64_t)ks * kRowBytes;   // activation bytes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + off);
      rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + (int64_t)ks * kstride);
    }
    if constexpr (kScaled) sa_reg = sa_src[ks];
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4 *>(&lds[st][0][swz(r, chunk * 16)]) = a_ok[i] ? ra[i] : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4 *>(&lds[st][1][swz(r, chunk * 16)]) = rb[i];
    }
    if constexpr (kScaled)
      if (tid < 128) lds_sa[st][tid] = sa_ok ? sa_reg : 0.0f;
  };
  auto compute = [&](int st, int ks) {
    const uint8_t *As = lds[st][0];
    const uint8_t *Bs = lds[st][1];
    f32x16 part[2][2];
    if constexpr (kScaled) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) part[mb][nb][i] = 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
      const int boff = kk * 2 * MM::kLaneBytes + (lane >> 5) * MM::kLaneBytes;
      frag bfr[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int brow = GATED ? nb * 64 + wn * 32 + (lane & 31) : wn * 64 + nb * 32 + (lane & 31);
        bfr[nb] = *reinterpret_cast<const frag *>(Bs + swz(brow, boff));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (!active[mb]) continue;
        const frag af = *reinterpret_cast<const frag *>(As + swz(wm * 64 + mb * 32 + (lane & 31), boff));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if constexpr (kScaled)
            part[mb][nb] = MM::mma(af, bfr[nb], part[mb][nb]);
          else
            acc[mb][nb] = MM::mma(af, bfr[nb], acc[mb][nb]);
        }
      }
    }
    if constexpr (kScaled) {
      const float sw0 = sw_src[0][ks], sw1 = sw_src[1][ks];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (!active[mb]) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * 64 + mb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          const float sa = lds_sa[st][r];
          acc[mb][0][i] += part[mb][0][i] * (sa * sw0);
          acc[mb][1][i] += part[mb][1][i] * (sa * sw1);
        }
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  // The last step reloads itself instead of branching around the loads.
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    gload(min(ks + 1, nk - 1));
    compute(st, ks);
    lstore(st ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element i of a 32x32 block sits at column (lane % 32)
  // and row 8*(i/4) + 4*(lane/32) + i%4.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (!active[mb]) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = wm * 64 + mb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      if (r >= nrows) continue;
      const int64_t slot = row0 + r;
      if constexpr (GATED) {
        const float gt = acc[mb][0][i], up = acc[mb][1][i];
        const float v = gated_act(gt, up, g.act);
        const int64_t col = (int64_t)nt * 64 + wn * 32 + (lane & 31);
        if constexpr (OUT_BF16)
          reinterpret_cast<uint16_t *>(g.out)[slot * g.ldo + col] = f32_to_bf16_bits(v);
        else
          reinterpret_cast<float *>(g.out)[slot * g.ldo + col] = v;
      } else {
        const int64_t orow = g.out_perm ? g.out_perm[slot] : slot;
        if (orow < 0 || (g.out_perm && orow >= g.n_pairs)) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int64_t col = (int64_t)nt * 128 + wn * 64 + nb * 32 + (lane & 31);
          if constexpr (OUT_BF16)
            reinterpret_cast<uint16_t *>(g.out)[orow * g.ldo + col] = f32_to_bf16_bits(acc[mb][nb][i]);
          else
            reinterpret_cast<float *>(g.out)[orow * g.ldo + col] = acc[mb][nb][i];
        }
      }
    }
  }
}

template <int EB, bool GATED>
hipError_t launch_typed(int out_dtype, const GemmParams &g, int n_tiles, hipStream_t s) {
  const int m_tiles = g.t.dense_rows > 0 ? (g.t.dense_rows + 127) / 128 : g.t.max_tiles;
  dim3 grid((unsigned)(m_tiles * n_tiles)), block(256);
  const bool bf = out_dtype == MOE_DTYPE_BF16;
  if (g.w_packed) {
    if (bf)
      grouped_gemm_kernel<EB, GATED, true, true><<<grid, block, 0, s>>>(g);
    else
      grouped_gemm_kernel<EB, GATED, false, true><<<grid, block, 0, s>>>(g);
  } else {
    if (bf)
      grouped_gemm_kernel<EB, GATED, true, false><<<grid, block, 0, s>>>(g);
    else
      grouped_gemm_kernel<EB, GATED, false, false><<<grid, block, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(int w_dtype, int out_dtype, GemmKind kind, const GemmParams &g,
                               int n_tiles, hipStream_t s) {
  const bool gated = kind == kGemmGatedAct;
  switch (w_dtype) {
    case MOE_DTYPE_BF16:
      return gated ? launch_typed<2, true>(out_dtype, g, n_tiles, s) : launch_typed<2, false>(out_dtype, g, n_tiles, s);
    case MOE_DTYPE_FP8_E4M3:
      return gated ? launch_typed<1, true>(out_dtype, g, n_tiles, s) : launch_typed<1, false>(out_dtype, g, n_tiles, s);
    default:
      return gated ? launch_typed<4, true>(out_dtype, g, n_tiles, s) : launch_typed<4, false>(out_dtype, g, n_tiles, s);
  }
}

}  // namespace moe
