// Repack canonical NVFP4 codes/scales into the tile layout (and back).
// A pure byte permutation into the tile layout described in device_common.h,
// zero past the matrix edge.
#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

// A 16-byte slot of the packed buffer is either four 4-byte pieces of code
// rows (code region) or one 16-byte run of a scale row (scale region).
struct Piece {
  int64_t row;    // matrix row
  int64_t first;  // first canonical byte within the row
  int bytes;      // 4 (codes) or 16 (scales)
  bool is_scale;
};

__device__ __forceinline__ Piece slot_piece(int64_t slot, int64_t nkt, int d) {
  const int64_t tile = slot / (kTileBytes / 16);
  const int within = (int)(slot % (kTileBytes / 16));  // 0..575
  const int64_t rt = tile / nkt, kt = tile % nkt;
  Piece p;
  if (within < kTileCodeBytes / 16) {
    const int c = within / 64, l = within % 64, r = l & 31, h = l >> 5;
    p.row = rt * kTileRows + r + 32 * (d & 1);
    p.first = (kt * kTileK + c * kChunkK + 8 * h + 16 * (d >> 1)) / 2;
    p.bytes = 4;
    p.is_scale = false;
  } else {
    const int sl = within - kTileCodeBytes / 16;  // 0..63
    p.row = rt * kTileRows + (sl >> 1) + 32 * (sl & 1);
    p.first = kt * (kTileK / 16);
    p.bytes = 16;
    p.is_scale = true;
  }
  return p;
}

__global__ void pack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                            int64_t n, int64_t k, int64_t nkt, int64_t slots, uint8_t* __restrict__ packed) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= slots) return;
  uint8_t out[16];
  const Piece p0 = slot_piece(slot, nkt, 0);
  const int npieces = p0.is_scale ? 1 : 4;
  for (int d = 0; d < npieces; ++d) {
    const Piece p = d == 0 ? p0 : slot_piece(slot, nkt, d);
    const int64_t row_bytes = p.is_scale ? k / 16 : k / 2;
    const uint8_t* src = (p.is_scale ? scales : codes) + p.row * row_bytes;
    for (int i = 0; i < p.bytes; ++i) {
      const int64_t col = p.first + i;
      out[4 * d + i] = (p.row < n && col < row_bytes) ? src[col] : (uint8_t)0;
    }
  }
  uint4 v;
  v.x = out[0] | (out[1] << 8) | (out[2] << 16) | ((uint32_t)out[3] << 24);
  v.y = out[4] | (out[5] << 8) | (out[6] << 16) | ((uint32_t)out[7] << 24);
  v.z = out[8] | (out[9] << 8) | (out[10] << 16) | ((uint32_t)out[11] << 24);
  v.w = out[12] | (out[13] << 8) | (out[14] << 16) | ((uint32_t)out[15] << 24);
  *reinterpret_cast<uint4*>(packed + slot * 16) = v;
}

__global__ void unpack_kernel(const uint8_t* __restrict__ packed, int64_t n, int64_t k, int64_t nkt,
                              int64_t slots, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= slots) return;
  const uint4 v = *reinterpret_cast<const uint4*>(packed + slot * 16);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const Piece p0 = slot_piece(slot, nkt, 0);
  const int npieces = p0.is_scale ? 1 : 4;
  for (int d = 0; d < npieces; ++d) {
    const Piece p = d == 0 ? p0 : slot_piece(slot, nkt, d);
    if (p.row >= n) continue;
    const int64_t row_bytes = p.is_scale ? k / 16 : k / 2;
    uint8_t* dst = (p.is_scale ? scales : codes) + p.row * row_bytes;
    for (int i = 0; i < p.bytes; ++i) {
      const int64_t col = p.first + i;
      const int byte = 4 * d + i;
      if (col < row_bytes) dst[col] = (uint8_t)(w[byte / 4] >> (8 * (byte % 4)));
    }
  }
}

__global__ void fill_zero_kernel(uint4* __restrict__ p, size_t n16) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, const Geometry& g, void* packed,
                       hipStream_t s) {
  int64_t slots = (int64_t)(packed_bytes(g) / 16);
  if (slots == 0) return hipSuccess;
  unsigned blocks = (unsigned)((slots + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, codes, scales, g.n, g.k, g.nkt, slots,
                     static_cast<uint8_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, const Geometry& g, uint8_t* codes, uint8_t* scales,
                         hipStream_t s) {
  int64_t slots = (int64_t)(packed_bytes(g) / 16);
  if (slots == 0) return hipSuccess;
  unsigned blocks = (unsigned)((slots + 255) / 256);
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t*>(packed), g.n,
                     g.k, g.nkt, slots, codes, scales);
  return hipGetLastError();
}

// Zero-fill (16-byte aligned, size a multiple of 16) with a kernel rather than
// a memset node, so a caller may capture it in a graph.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace nvfp4
