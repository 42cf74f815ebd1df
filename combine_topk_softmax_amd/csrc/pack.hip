// One-time reordering of row-major expert weights into the packed layout
// (see PackedGeom in moe_device.h): a gather copy in 16-byte pieces, writes
// contiguous.  Runs when weights are loaded, not on the per-step path.
#include "moe_device.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                   int64_t n_pieces, int64_t Nw, int64_t row_bytes, PackedGeom g) {
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n_pieces;
       o += (int64_t)gridDim.x * blockDim.x) {
    int64_t t = o;
    const int lane = (int)(t % 64);
    t /= 64;
    const int p = (int)(t % 2);
    t /= 2;
    const int b = (int)(t % g.nbw);
    t /= g.nbw;
    const int w = (int)(t % 8);
    t /= 8;
    const int64_t ks = t % g.nk;
    t /= g.nk;
    const int64_t panel = t % g.n_panels;
    const int64_t e = t / g.n_panels;
    const int64_t row = (int64_t)b * g.half + panel * 128 + w * 16 + (lane & 15);
    const int64_t kbyte = ks * 128 + (lane >> 4) * 32 + p * 16;
    *reinterpret_cast<uint4 *>(dst + o * 16) =
        *reinterpret_cast<const uint4 *>(src + (e * Nw + row) * row_bytes + kbyte);
  }
}

}  // namespace

hipError_t launch_pack_weights(const void *src, void *dst, int64_t E, int64_t Nw, int64_t row_bytes, bool gated,
                               hipStream_t s) {
  const PackedGeom g = packed_geom(Nw, row_bytes, gated);
  const int64_t n_pieces = E * Nw * row_bytes / 16;
  const int64_t blocks = std::min<int64_t>((n_pieces + 255) / 256, 65536);
  pack_kernel<<<(unsigned)blocks, 256, 0, s>>>(reinterpret_cast<const uint8_t *>(src),
                                                reinterpret_cast<uint8_t *>(dst), n_pieces, Nw, row_bytes, g);
  return hipGetLastError();
}

}  // namespace moe
