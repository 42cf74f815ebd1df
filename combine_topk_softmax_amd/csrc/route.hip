// [Router]: top-k expert selection and routing weights, one wavefront per token.
//
// The modular_kernel.py page names the router as the first step of the fused
// MoE layer and FusedMoEModularKernel.forward consumes its outputs
// (topk_weights and topk_ids, one row of topk entries per token).  The
// selection compares fp32 logits, ties going to the lower expert index; the
// weights are the softmax over all E logits or the sigmoid of each logit,
// optionally renormalised over the k picks.
//
// gfx950 mapping: a token's E logits are spread over the 64 lanes of one
// wavefront (VPL per lane).  Each of the k rounds is one wave-wide max
// reduction of a 64-bit key (order-preserving logit bits, then the inverted
// expert index so that equal logits prefer the lower index).  The winner's
// lane retires its key; no LDS, no atomics, one pass over the logits.
#include "moe_device.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;                       // -0 ties with +0
  uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  uint32_t ord = (uint32_t)(key >> 32);
  uint32_t b = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(b);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int M, int E,
                                                    int k, int sigmoid, int renorm,
                                                    float *__restrict__ topk_w,
                                                    int32_t *__restrict__ topk_ids) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // wave-uniform
  const float *row = logits + (int64_t)m * E;

  float v[VPL];
  uint64_t key[VPL];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
      key[i] = route_key(v[i], e);
      mx = fmaxf(mx, v[i]);
    } else {
      v[i] = -INFINITY;
      key[i] = 0ull;
    }
  }
  float den = 0.0f;
  if (!sigmoid) {
    mx = wave_max(mx);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) den += expf(v[i] - mx);
    den = wave_sum(den);
  }

  float my_w = 0.0f, wsum = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (key[i] == best) key[i] = 0ull;
    const int e = (int)(~(uint32_t)best);
    const float l = key_logit(best);
    const float p = sigmoid ? 1.0f / (1.0f + expf(-l)) : expf(l - mx) / den;
    wsum += p;
    if (lane == j) {
      my_w = p;
      my_id = e;
    }
  }
  if (lane < k) {
    topk_w[(int64_t)m * k + lane] = renorm ? my_w / wsum : my_w;
    topk_ids[(int64_t)m * k + lane] = my_id;
  }
}

}  // namespace

hipError_t launch_route(const moe_problem &p, const float *logits, float *w, int32_t *ids,
                        hipStream_t s) {
  const int M = (int)p.M, E = (int)router_width(p), k = (int)p.topk;
  dim3 grid((M + 3) / 4), block(256);
  const int sig = p.scoring == MOE_SCORING_SIGMOID, ren = p.renormalize != 0;
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, M, E, k, sig, ren, w, ids);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, M, E, k, sig, ren, w, ids);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, M, E, k, sig, ren, w, ids);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, M, E, k, sig, ren, w, ids);
  return hipGetLastError();
}

}  // namespace moe
