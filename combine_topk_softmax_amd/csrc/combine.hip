// [Combine]: the top-k weighted reduce of the unweighted expert outputs.
//
// FusedMoEPrepareAndFinalize.finalize (modular_kernel.py page) applies
// topk_weights to the (M, topk, K) expert output and reduces over topk into
// the (M, K) output, which it overwrites; on one GPU there is no combine
// communication, only this gather-weight-reduce.  Rows come from
// fused_out[m*topk + j] (Standard) or from the batched row the dispatch placed
// pair (m, j) in (BatchedExperts); a dropped pair, or the pick of an expert
// another expert-parallel shard holds, adds nothing.  With the router weight
// applied on the input the outputs are added unweighted.
//
// HBM-bound: one block per token (and column range: a small batch spreads
// each token's columns over several blocks so that every CU has work), 8
// outputs per thread and pass.  The picks
// go in groups of up to 8: their slots and weights first, then every row's
// 16-byte loads at once (a dropped pick loads nothing), then the fp32 sums in
// j order, so a thread keeps up to 8 rows in flight instead of one.  Each
// expert-output row is read once, so bf16 rows are loaded non-temporally
// (skewed prefill combine 0.237 -> 0.203 ms, DeepSeek-V3 shape 0.109 -> 0.083).
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kGroup = 8;   // picks whose row loads are in flight together
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, int rows_from_inv,
                                                      int K, int k, T *__restrict__ out) {
  const int m = blockIdx.x;
  for (int c = (blockIdx.y * 256 + threadIdx.x) * 8; c < K; c += 256 * 8 * gridDim.y) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += kGroup) {
      int64_t row[kGroup];
      float wj[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        row[u] = -1;
        wj[u] = 0.0f;
        if (j0 + u < k) {
          const int64_t pair = (int64_t)m * k + j0 + u;
          const int64_t slot = inv ? (int64_t)inv[pair] : pair;
          if (slot >= 0) {                         // else dropped, or another shard's pick
            row[u] = rows_from_inv ? slot : pair;
            wj[u] = w ? w[pair] : 1.0f;
          }
        }
      }
      if constexpr (sizeof(T) == 2) {
        uint4 raw[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
          raw[u] = row[u] >= 0 ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                     reinterpret_cast<const u32x4 *>(y + row[u] * K + c)))
                               : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          if (row[u] < 0) continue;
          const uint32_t v[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wj[u] * bf16_bits_to_f32(v[i] & 0xffffu);
            acc[2 * i + 1] += wj[u] * bf16_bits_to_f32(v[i] >> 16);
          }
        }
      } else {
        float4 lo[kGroup], hi[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          if (row[u] >= 0) {
            const float4 *src = reinterpret_cast<const float4 *>(y + row[u] * K + c);
            lo[u] = src[0], hi[u] = src[1];
          } else {
            lo[u] = hi[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          }
        }
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          if (row[u] < 0) continue;
          const float a = wj[u];
          acc[0] += a * lo[u].x, acc[1] += a * lo[u].y, acc[2] += a * lo[u].z, acc[3] += a * lo[u].w;
          acc[4] += a * hi[u].x, acc[5] += a * hi[u].y, acc[6] += a * hi[u].z, acc[7] += a * hi[u].w;
        }
      }
    }
    if constexpr (sizeof(T) == 2) {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<uint4 *>(out + (int64_t)m * K + c) = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      float4 *dst = reinterpret_cast<float4 *>(out + (int64_t)m * K + c);
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// moe_forward with the down GEMM split over K (bf16): a pick's row is the sum
// of its slot's fp32 partial slices in split order, rounded to bf16, which is
// what the split's reduce would have stored; weighting and summing then go as
// in combine_kernel, so the output equals reduce-then-combine bit for bit
// without the reduce's launch and its bf16 round trip.  Groups of 4 picks keep
// 2 x S 16-byte loads per pick in flight; the partial rows are read once.
constexpr int kSplitGroup = 4;
typedef float f32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void combine_split_kernel(const float *__restrict__ part, int S, int64_t stride,
                                                            const float *__restrict__ w,
                                                            const int32_t *__restrict__ inv, int K, int k,
                                                            uint16_t *__restrict__ out) {
  const int m = blockIdx.x;
  for (int c = (blockIdx.y * 256 + threadIdx.x) * 8; c < K; c += 256 * 8 * gridDim.y) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += kSplitGroup) {
      int64_t slot[kSplitGroup];
      float wj[kSplitGroup];
#pragma unroll
      for (int u = 0; u < kSplitGroup; ++u) {
        slot[u] = -1;
        wj[u] = 0.0f;
        if (j0 + u < k) {
          const int64_t pair = (int64_t)m * k + j0 + u;
          const int64_t sl = inv[pair];
          if (sl >= 0) {                           // else dropped, or another shard's pick
            slot[u] = sl;
            wj[u] = w ? w[pair] : 1.0f;
          }
        }
      }
      float v[kSplitGroup][8];
#pragma unroll
      for (int u = 0; u < kSplitGroup; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
      for (int sk = 0; sk < S; ++sk) {
        f32x4v lo[kSplitGroup], hi[kSplitGroup];
#pragma unroll
        for (int u = 0; u < kSplitGroup; ++u) {
          if (slot[u] >= 0) {
            const f32x4v *src = reinterpret_cast<const f32x4v *>(part + sk * stride + slot[u] * K + c);
            lo[u] = __builtin_nontemporal_load(src);
            hi[u] = __builtin_nontemporal_load(src + 1);
          } else {
            lo[u] = hi[u] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
          }
        }
#pragma unroll
        for (int u = 0; u < kSplitGroup; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[u][i] += lo[u][i];
            v[u][4 + i] += hi[u][i];
          }
      }
#pragma unroll
      for (int u = 0; u < kSplitGroup; ++u) {
        if (slot[u] < 0) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wj[u] * bf16_bits_to_f32(f32_to_bf16_bits(v[u][i]));
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<uint4 *>(out + (int64_t)m * K + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

// Blocks per token: one for large batches, else one per 2048 columns.
static unsigned combine_col_blocks(const moe_problem &p) {
  return p.M >= 1024 ? 1u : (unsigned)((p.K + 2047) / 2048);
}

hipError_t launch_combine_split(const moe_problem &p, const float *part, int S, int64_t stride,
                                const float *topk_w, const int32_t *inv, void *out, hipStream_t s) {
  if (p.act_dtype != MOE_DTYPE_BF16 || !inv) return hipErrorInvalidValue;
  dim3 grid((unsigned)p.M, combine_col_blocks(p)), block(256);
  combine_split_kernel<<<grid, block, 0, s>>>(part, S, stride, topk_w, inv, (int)p.K, (int)p.topk,
                                              (uint16_t *)out);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_problem &p, const void *fused_out, const float *topk_w,
                          const int32_t *inv, bool rows_from_inv, void *out, hipStream_t s) {
  dim3 grid((unsigned)p.M, combine_col_blocks(p)), block(256);
  const int K = (int)p.K, k = (int)p.topk, r = rows_from_inv ? 1 : 0;
  if (p.act_dtype == MOE_DTYPE_BF16)
    combine_kernel<uint16_t><<<grid, block, 0, s>>>((const uint16_t *)fused_out, topk_w, inv, r, K, k,
                                                    (uint16_t *)out);
  else
    combine_kernel<float><<<grid, block, 0, s>>>((const float *)fused_out, topk_w, inv, r, K, k, (float *)out);
  return hipGetLastError();
}

}  // namespace moe
