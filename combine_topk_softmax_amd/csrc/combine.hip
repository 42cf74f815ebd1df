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
// HBM-bound: one block per token, 16-byte vector loads of each of the k rows,
// fp32 accumulation in j order, one 16-byte store per 8 outputs.
#include "moe_device.h"

namespace moe {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, int rows_from_inv,
                                                      int K, int k, T *__restrict__ out) {
  const int m = blockIdx.x;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const int64_t pair = (int64_t)m * k + j;
      const int64_t slot = inv ? (int64_t)inv[pair] : pair;
      if (slot < 0) continue;                      // dropped, or another shard's pick
      const int64_t row = rows_from_inv ? slot : pair;
      const float wj = w ? w[pair] : 1.0f;
      if constexpr (sizeof(T) == 2) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(y + row * K + c);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += wj * bf16_bits_to_f32(u[i] & 0xffffu);
          acc[2 * i + 1] += wj * bf16_bits_to_f32(u[i] >> 16);
        }
      } else {
        const float4 *src = reinterpret_cast<const float4 *>(y + row * K + c);
        const float4 a = src[0], b = src[1];
        acc[0] += wj * a.x, acc[1] += wj * a.y, acc[2] += wj * a.z, acc[3] += wj * a.w;
        acc[4] += wj * b.x, acc[5] += wj * b.y, acc[6] += wj * b.z, acc[7] += wj * b.w;
      }
    }
    if constexpr (sizeof(T) == 2) {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i]) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1]) << 16);
      *reinterpret_cast<uint4 *>(out + (int64_t)m * K + c) = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      float4 *dst = reinterpret_cast<float4 *>(out + (int64_t)m * K + c);
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_problem &p, const void *fused_out, const float *topk_w,
                          const int32_t *inv, bool rows_from_inv, void *out, hipStream_t s) {
  dim3 grid((unsigned)p.M), block(256);
  const int K = (int)p.K, k = (int)p.topk, r = rows_from_inv ? 1 : 0;
  if (p.act_dtype == MOE_DTYPE_BF16)
    combine_kernel<uint16_t><<<grid, block, 0, s>>>((const uint16_t *)fused_out, topk_w, inv, r, K, k,
                                                    (uint16_t *)out);
  else
    combine_kernel<float><<<grid, block, 0, s>>>((const float *)fused_out, topk_w, inv, r, K, k, (float *)out);
  return hipGetLastError();
}

}  // namespace moe
