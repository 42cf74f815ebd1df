// [Quantize-Dispatch] on one GPU: per-expert counting, the stable prefix-sum
// permutation of the (token, slot) pairs, the BatchedExperts row scatter and
// the token-group-128 fp8 quantiser, plus the tile plan the grouped GEMMs read.
//
// Sources: modular_kernel.py page -- FusedMoEPrepareAndFinalize.prepare
// (quantise and dispatch), ExpertTokensMetadata.expert_num_tokens (per-expert
// counts), FusedMoEActivationFormat (Standard vs BatchedExperts), and the
// worst-tokens page (counts kept in a device int32 tensor, read by a masked
// grouped GEMM with no host synchronisation).
//
// Determinism: a pair's slot is decided by counts and ranks only, never by the
// order in which atomics return.  The pairs are cut into chunks; chunk
// histograms (LDS atomics: only totals matter) are prefix-summed in a fixed
// order; then one wavefront per chunk walks its pairs 64 at a time and ranks
// each pair among the lanes holding the same expert with a ballot-based match
// (log2(E) ballots), so the order inside an expert segment is ascending pair
// index.
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxChunks = 256;   // counting chunks per batch (the workspace layout keeps to it)

// ----------------------------------------------------------- histogram

__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t *__restrict__ ids, int n,
                                                         int E, int Eg, const int32_t *__restrict__ map,
                                                         int chunk, int32_t *__restrict__ chunk_hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int f0 = c * chunk, f1 = min(n, f0 + chunk);
  for (int f = f0 + threadIdx.x; f < f1; f += blockDim.x) {
    const int e = local_expert(ids[f], Eg, map, E);
    if (e >= 0) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_hist[(int64_t)c * E + e] = h[e];
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 1024, 16
// waves): wave scans by shuffles, then wave 0 scans the 16 wave totals.
// *total (shared) receives the sum of all values.
__device__ int block_exclusive_scan(int v, int *total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int w = lane < 16 ? wsum[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int t = __shfl_up(wi, o, 64);
      if (lane >= o) wi += t;
    }
    if (lane < 16) wsum[lane] = wi - w;
    if (lane == 15) *total = wi;
  }
  __syncthreads();
  const int r = wsum[wid] + incl - v;
  __syncthreads();
  return r;
}

// One block of 1024 threads: chunk prefixes per expert, counts, padded
// segment offsets (STANDARD), pad slots of the permutation set to -1.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *__restrict__ chunk_hist, int n_chunks,
                                                    int E, int align, int standard,
                                                    int32_t *counts, int32_t *expert_num_tokens,
                                                    int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ perm, int64_t perm_len,
                                                    int32_t *__restrict__ status, int clear_status) {
  __shared__ int total_sh;
  const int e = threadIdx.x;
  if (e == 0 && clear_status) *status = 0;
  int run = 0;
  if (e < E) {
    // the expert's column of chunk counts, 64 at a time into registers, so
    // that the loads are in flight together rather than each behind the
    // last store
    for (int c0 = 0; c0 < n_chunks; c0 += 64) {
      int h[64];
#pragma unroll
      for (int c = 0; c < 64; ++c)
        if (c0 + c < n_chunks) h[c] = chunk_hist[(int64_t)(c0 + c) * E + e];
#pragma unroll
      for (int c = 0; c < 64; ++c)
        if (c0 + c < n_chunks) {
          chunk_hist[(int64_t)(c0 + c) * E + e] = run;
          run += h[c];
        }
    }
    counts[e] = run;
    expert_num_tokens[e] = run;
  }
  if (!standard) return;  // uniform
  int padded = e < E ? (run + align - 1) / align * align : 0;
  int start = block_exclusive_scan(padded, &total_sh);
  if (e < E) {
    offsets[e] = start;
    for (int s = start + run; s < start + padded; ++s) perm[s] = -1;
  }
  if (e == 0) offsets[E] = total_sh;
  for (int64_t s = total_sh + threadIdx.x; s < perm_len; s += blockDim.x) perm[s] = -1;
}

// One wavefront per chunk: stable rank of each pair inside its expert.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t *__restrict__ ids, int n, int E,
                                                  int Eg, const int32_t *__restrict__ map,
                                                  int nbits, int chunk, int standard, int64_t cap,
                                                  const int32_t *__restrict__ chunk_prefix,
                                                  const int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ perm,
                                                  int32_t *__restrict__ inv,
                                                  int32_t *__restrict__ status) {
  __shared__ int run[kMaxExperts];
  const int lane = threadIdx.x, c = blockIdx.x;
  for (int e = lane; e < E; e += 64)
    run[e] = chunk_prefix[(int64_t)c * E + e] + (standard ? offsets[e] : 0);
  __syncthreads();
  const int f0 = c * chunk, f1 = min(n, f0 + chunk);
  for (int base = f0; base < f1; base += 64) {
    const int f = base + lane;
    const bool valid = f < f1;
    const int e = valid ? local_expert(ids[f], Eg, map, E) : -1;
    const bool good = valid && e >= 0;
    if (valid && !good) {
      inv[f] = -1;                                   // another shard's pick, or invalid
      if (e == -2) atomicOr(status, MOE_DEVICE_BAD_EXPERT_ID);
    }
    uint64_t peers = __ballot(good);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = good && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    int pos = 0;
    if (good) {
      pos = run[e] + __popcll(peers & lanemask_lt());
      if (standard) {
        perm[pos] = f;
        inv[f] = pos;
      } else if (pos < cap) {
        inv[f] = (int32_t)(e * cap + pos);
      } else {
        inv[f] = -1;
        atomicOr(status, MOE_DEVICE_CAPACITY_OVERFLOW);
      }
    }
    __syncthreads();
    if (good && (peers & lanemask_lt()) == 0) run[e] += __popcll(peers);
    __syncthreads();
  }
}

// --------------------------------------------------- row quantise / scatter

// Blocks of 256 threads = 16 teams of 16 lanes; block (m, y) handles groups
// y * 16 + team (+ multiples of 16 * gridDim.y) of token row m.  A team
// handles one group of 128 channels, 8 per lane: |max| by shuffles inside the
// team, scale, codes.  Each row is read once and written to every destination
// row: the rows inv[] names for its topk pairs (batched), or row m (standard
// quantise).  Spreading a row's groups over blocks keeps the latency chain of
// a decode batch (few rows) short: one load-quantise-store round per block.
// With topk_w (router weight on the input, topk == 1) the row is first
// multiplied by the token's weight and rounded to the activation type.
template <typename TIn, bool QUANT>
__global__ __launch_bounds__(256) void dispatch_rows_kernel(const TIn *__restrict__ x, int K, int k,
                                                            const int32_t *__restrict__ inv,
                                                            const float *__restrict__ topk_w,
                                                            void *__restrict__ a_out,
                                                            float *__restrict__ a_scale) {
  const int m = blockIdx.x;
  const int team = threadIdx.x >> 4, tl = threadIdx.x & 15;
  const int G = K / 128;
  for (int g = blockIdx.y * 16 + team; g < G; g += 16 * gridDim.y) {
    const int c0 = g * 128 + tl * 8;
    float v[8];
    if constexpr (sizeof(TIn) == 2) {
      uint4 raw = *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + c0);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    } else {
      const float4 *src = reinterpret_cast<const float4 *>(x + (int64_t)m * K + c0);
      float4 a = src[0], b = src[1];
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
    if (topk_w) {
      const float wm = topk_w[m];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] *= wm;
        if constexpr (sizeof(TIn) == 2) v[i] = bf16_bits_to_f32(f32_to_bf16_bits(v[i]));
      }
    }
    if constexpr (QUANT) {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      amax = row16_max(amax);
      const float sc = group_scale(amax);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) lo |= quant_e4m3(v[i], sc) << (8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) hi |= quant_e4m3(v[4 + i], sc) << (8 * i);
      const uint2 q = make_uint2(lo, hi);
      for (int j = 0; j < (inv ? k : 1); ++j) {
        const int64_t d = inv ? inv[(int64_t)m * k + j] : m;
        if (d < 0) continue;
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(a_out) + d * K + c0) = q;
        if (tl == 0) a_scale[d * G + g] = sc;
      }
    } else {
      for (int j = 0; j < (inv ? k : 1); ++j) {
        const int64_t d = inv ? inv[(int64_t)m * k + j] : m;
        if (d < 0) continue;
        if constexpr (sizeof(TIn) == 2) {
          uint32_t u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
          *reinterpret_cast<uint4 *>(reinterpret_cast<TIn *>(a_out) + d * K + c0) = make_uint4(u[0], u[1], u[2], u[3]);
        } else {
          float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<TIn *>(a_out) + d * K + c0);
          dst[0] = make_float4(v[0], v[1], v[2], v[3]);
          dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
      }
    }
  }
}

// Re-quantise the first GEMM's fp32 output per token group of 128 (the
// modular_kernel.py page keeps a second activation scale so that the second
// GEMM's input is quantised the same way).  One block per tile of rows; only
// rows that hold real pairs are touched.  16 teams of 16 lanes, one
// (row, group) per team at a time, 8 values per lane.
__global__ __launch_bounds__(256) void quant_rows_kernel(const float *__restrict__ in,
                                                         const int32_t *__restrict__ tiles,
                                                         int max_tiles, int64_t cols,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ scale) {
  const int t = blockIdx.x;
  if (t >= tiles[(int64_t)max_tiles * 4]) return;
  const int32_t *d = tiles + (int64_t)t * 4;
  const int64_t row0 = (int64_t)d[1] + d[2];
  const int nrows = d[3];
  const int G = (int)(cols / 128);
  // gridDim.y blocks share a tile's (row, group) items, 16 teams each
  const int team = blockIdx.y * 16 + (threadIdx.x >> 4), tl = threadIdx.x & 15;
  const int teams = gridDim.y * 16;
  for (int pidx = team; pidx < nrows * G; pidx += teams) {
    const int64_t row = row0 + pidx / G;
    const int g = pidx % G;
    const float4 *src = reinterpret_cast<const float4 *>(in + row * cols + g * 128 + tl * 8);
    const float4 a = src[0], b = src[1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = row16_max(amax);
    const float sc = group_scale(amax);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= quant_e4m3(v[i], sc) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= quant_e4m3(v[4 + i], sc) << (8 * i);
    *reinterpret_cast<uint2 *>(q + row * cols + g * 128 + tl * 8) = make_uint2(lo, hi);
    if (tl == 0) scale[row * G + g] = sc;
  }
}

// Tile plan for the grouped GEMMs: expert e's rows [0, count_e) are cut into
// tiles of tile_rows; tiles[t] = {e, first row of e's segment, row0, nrows}.
// A count above the capacity (batched) or a plan that would overrun
// max_tiles is clamped, flagging the status word.
__global__ __launch_bounds__(1024) void plan_tiles_kernel(const int32_t *__restrict__ counts,
                                                          const int32_t *__restrict__ offsets,
                                                          int E, int standard, int64_t cap,
                                                          int64_t perm_len, int tile_rows,
                                                          int max_tiles, int32_t *__restrict__ tiles,
                                                          int32_t *__restrict__ status) {
  __shared__ int total_sh;
  const int e = threadIdx.x;
  int cnt = 0;
  int64_t seg = 0;
  if (e < E) {
    cnt = max(counts[e], 0);
    if (standard) {
      seg = offsets[e];
      int64_t room = perm_len - seg;
      if ((int64_t)cnt > room) cnt = (int)max<int64_t>(room, 0);
    } else {
      seg = (int64_t)e * cap;
      if ((int64_t)cnt > cap) {
        cnt = (int)cap;
        atomicOr(status, MOE_DEVICE_CAPACITY_OVERFLOW);
      }
    }
  }
  __shared__ int t0_sh[kMaxExperts], cnt_sh[kMaxExperts];
  __shared__ int64_t seg_sh[kMaxExperts];
  const int nt = (cnt + tile_rows - 1) / tile_rows;
  const int t0 = block_exclusive_scan(nt, &total_sh);
  if (e < E) {
    t0_sh[e] = t0;
    cnt_sh[e] = cnt;
    seg_sh[e] = seg;
  }
  __syncthreads();
  // every thread writes tiles (an expert of many rows has many): tile t
  // belongs to the last expert whose first tile is at or before t (experts
  // without tiles share their first index with the next one)
  const int total = total_sh;
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    if (t >= max_tiles) {
      atomicOr(status, MOE_DEVICE_CAPACITY_OVERFLOW);
      break;
    }
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (t0_sh[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int i = t - t0_sh[lo];
    int32_t *d = tiles + (int64_t)t * 4;
    d[0] = lo;
    d[1] = (int32_t)seg_sh[lo];
    d[2] = i * tile_rows;
    d[3] = min(tile_rows, cnt_sh[lo] - i * tile_rows);
  }
  if (e == 0) tiles[(int64_t)max_tiles * 4] = min(total, max_tiles);
}

// -------------------------------------------------- small batches, one block
// Counting, scan, stable ranking and (optionally) the tile plan of a batch of
// at most kSmallPairs pairs over at most kSmallExperts local experts in one
// workgroup of 1024 threads, instead of four launches (decode batches spend
// more time between those launches than in them).  Same outputs as
// chunk_hist + scan + rank + plan_tiles: each of the 16 wavefronts takes a
// contiguous run of pairs, the per-wavefront histograms are prefix-summed in
// wavefront order, and each wavefront ranks its run 64 pairs at a time with
// ballots, so every expert segment is in ascending pair order.
constexpr int kSmallPairs = 4096;
constexpr int kSmallExperts = 256;

__global__ __launch_bounds__(1024) void prepare_small_kernel(
    const int32_t *__restrict__ ids, int n, int E, int Eg, const int32_t *__restrict__ map, int nbits,
    int standard, int align, int64_t cap, int32_t *counts, int32_t *expert_num_tokens,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int64_t perm_len, int32_t *__restrict__ inv,
    int32_t *__restrict__ status, int clear_status, int tile_rows, int max_tiles, int32_t *__restrict__ tiles) {
  __shared__ int lid[kSmallPairs];
  __shared__ int whist[16][kSmallExperts];
  __shared__ int start_sh[kSmallExperts];
  __shared__ int total_sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0 && clear_status) *status = 0;
  for (int i = tid; i < 16 * kSmallExperts; i += 1024) (&whist[0][0])[i] = 0;
  __syncthreads();
  // pairs [w * run, (w + 1) * run) belong to wavefront w
  const int run = (n + 15) / 16;
  for (int f = tid; f < n; f += 1024) {
    const int e = local_expert(ids[f], Eg, map, E);
    lid[f] = e;
    if (e < 0) {
      inv[f] = -1;                                   // another shard's pick, or invalid
      if (e == -2) atomicOr(status, MOE_DEVICE_BAD_EXPERT_ID);
    } else {
      atomicAdd(&whist[f / run][e], 1);
    }
  }
  __syncthreads();
  // per expert: counts, the wavefronts' prefixes, padded segment offsets
  int cnt = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int h = whist[w][tid];
      whist[w][tid] = cnt;
      cnt += h;
    }
    counts[tid] = cnt;
    expert_num_tokens[tid] = cnt;
  }
  const int padded = tid < E ? (standard ? (cnt + align - 1) / align * align : 0) : 0;
  const int start = block_exclusive_scan(padded, &total_sh);
  if (tid < E) start_sh[tid] = standard ? start : 0;
  if (standard) {
    if (tid < E) {
      offsets[tid] = start;
      for (int sl = start + cnt; sl < start + padded; ++sl) perm[sl] = -1;
    }
    if (tid == 0) offsets[E] = total_sh;
    for (int64_t sl = total_sh + tid; sl < perm_len; sl += 1024) perm[sl] = -1;
  }
  __syncthreads();
  // stable ranks: wavefront wv walks its run of pairs 64 at a time
  for (int e = lane; e < E; e += 64) whist[wv][e] += start_sh[e];
  __syncthreads();
  const int f0 = wv * run, f1 = min(n, f0 + run);
  for (int base = f0; base < f1; base += 64) {
    const int f = base + lane;
    const int e = f < f1 ? lid[f] : -1;
    const bool good = e >= 0;
    uint64_t peers = __ballot(good);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = good && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    if (good) {
      const int pos = whist[wv][e] + __popcll(peers & lanemask_lt());
      if (standard) {
        perm[pos] = f;
        inv[f] = pos;
      } else if (pos < cap) {
        inv[f] = (int32_t)(e * cap + pos);
      } else {
        inv[f] = -1;
        atomicOr(status, MOE_DEVICE_CAPACITY_OVERFLOW);
      }
    }
    // every lane has read its run position before the leader of each expert
    // group moves it on (the wavefront executes in lockstep)
    __builtin_amdgcn_wave_barrier();
    if (good && (peers & lanemask_lt()) == 0) whist[wv][e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
  if (tile_rows <= 0) return;   // uniform
  // tile plan, as plan_tiles_kernel
  int c = cnt;
  int64_t seg = 0;
  if (tid < E) {
    if (standard) {
      seg = start;
      const int64_t room = perm_len - seg;
      if ((int64_t)c > room) c = (int)max<int64_t>(room, 0);
    } else {
      seg = (int64_t)tid * cap;
      if ((int64_t)c > cap) {
        c = (int)cap;
        atomicOr(status, MOE_DEVICE_CAPACITY_OVERFLOW);
      }
    }
  }
  const int nt = tid < E ? (c + tile_rows - 1) / tile_rows : 0;
  const int t0 = block_exclusive_scan(nt, &total_sh);
  if (tid < E) {
    for (int i = 0; i < nt; ++i) {
      const int t = t0 + i;
      if (t >= max_tiles) {
        atomicOr(status, MOE_DEVICE_CAPACITY_OVERFLOW);
        break;
      }
      int32_t *d = tiles + (int64_t)t * 4;
      d[0] = tid;
      d[1] = (int32_t)seg;
      d[2] = i * tile_rows;
      d[3] = min(tile_rows, c - i * tile_rows);
    }
  }
  if (tid == 0) tiles[(int64_t)max_tiles * 4] = min(total_sh, max_tiles);
}

int ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

}  // namespace

bool count_fused(const moe_problem &p) { return p.M * p.topk <= kSmallPairs && p.E <= kSmallExperts; }

hipError_t launch_count_and_permute(const moe_problem &p, const int32_t *ids,
                                    int32_t *expert_num_tokens, const DispatchBufs &b,
                                    hipStream_t s) {
  const int n = (int)(p.M * p.topk), E = (int)p.E, Eg = (int)router_width(p);
  const int standard = p.format == MOE_FORMAT_STANDARD;
  const int align = p.align > 0 ? (int)p.align : 1;
  if (count_fused(p)) {
    prepare_small_kernel<<<1, 1024, 0, s>>>(ids, n, E, Eg, p.expert_map, ceil_log2(E), standard, align,
                                            p.max_tokens_per_expert, b.counts, expert_num_tokens, b.offsets, b.perm,
                                            b.perm_len, b.inv, b.status, b.clear_status, b.plan_rows, b.max_tiles,
                                            b.tiles);
    return hipGetLastError();
  }
  chunk_hist_kernel<<<(unsigned)b.n_chunks, 256, 0, s>>>(ids, n, E, Eg, p.expert_map, (int)b.chunk,
                                                          b.chunk_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (b.n_chunks > kMaxChunks) return hipErrorInvalidValue;
  scan_kernel<<<1, 1024, 0, s>>>(b.chunk_hist, (int)b.n_chunks, E, align, standard, b.counts,
                                 expert_num_tokens, b.offsets, b.perm, b.perm_len, b.status, b.clear_status);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  rank_kernel<<<(unsigned)b.n_chunks, 64, 0, s>>>(ids, n, E, Eg, p.expert_map, ceil_log2(E), (int)b.chunk, standard,
                                                  p.max_tokens_per_expert, b.chunk_hist, b.offsets,
                                                  b.perm, b.inv, b.status);
  return hipGetLastError();
}

hipError_t launch_dispatch_rows(const moe_problem &p, const void *x, const int32_t *inv, const float *topk_w,
                                void *a_out, float *a_scale_out, bool batched, hipStream_t s) {
  const int K = (int)p.K, k = (int)p.topk;
  const bool quant = p.act_quant == MOE_QUANT_FP8_TOKEN_GROUP_128;
  const int32_t *d = batched ? inv : nullptr;
  // enough blocks for every group of a small batch to go at once
  const int G = K / 128;
  const int ny = p.M >= 1024 ? 1 : (G + 15) / 16;
  dim3 grid((unsigned)p.M, (unsigned)ny), block(256);
  if (p.act_dtype == MOE_DTYPE_BF16) {
    if (quant)
      dispatch_rows_kernel<uint16_t, true><<<grid, block, 0, s>>>((const uint16_t *)x, K, k, d, topk_w, a_out, a_scale_out);
    else
      dispatch_rows_kernel<uint16_t, false><<<grid, block, 0, s>>>((const uint16_t *)x, K, k, d, topk_w, a_out, a_scale_out);
  } else {
    if (quant)
      dispatch_rows_kernel<float, true><<<grid, block, 0, s>>>((const float *)x, K, k, d, topk_w, a_out, a_scale_out);
    else
      dispatch_rows_kernel<float, false><<<grid, block, 0, s>>>((const float *)x, K, k, d, topk_w, a_out, a_scale_out);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows(const float *in, const int32_t *tiles, int max_tiles, int64_t cols,
                             uint8_t *q, float *scale, hipStream_t s) {
  const dim3 grid((unsigned)max_tiles, 8);
  quant_rows_kernel<<<grid, 256, 0, s>>>(in, tiles, max_tiles, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_plan_tiles(const moe_problem &p, const int32_t *counts, const int32_t *offsets,
                             int64_t perm_len, int tile_rows, int max_tiles, int32_t *tiles,
                             int32_t *status, hipStream_t s) {
  const int standard = p.format == MOE_FORMAT_STANDARD;
  plan_tiles_kernel<<<1, 1024, 0, s>>>(counts, offsets, (int)p.E, standard, p.max_tokens_per_expert,
                                       perm_len, tile_rows, max_tiles, tiles, status);
  return hipGetLastError();
}

}  // namespace moe
