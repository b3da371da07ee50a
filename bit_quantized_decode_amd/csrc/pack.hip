// a1: repack canonical NVFP4 codes/scales into the tile layout (and back).
// A pure byte permutation: every 16-byte lane slot of a tile is one 16-byte run
// of a canonical row (32 codes, or 16 scale bytes), zero past the matrix edge.
#include "device_common.h"
#include "launchers.h"

namespace nvfp4 {
namespace {

// Where tile slot `slot` (16 bytes) of the packed buffer comes from.
struct SlotSource {
  int64_t row;       // matrix row
  int64_t first;     // first canonical byte within the row (codes) or first block (scales)
  bool is_scale;
};

__device__ __forceinline__ SlotSource slot_source(int64_t slot, int64_t nkt) {
  int64_t tile = slot / (kTileBytes / 16);
  int within = (int)(slot % (kTileBytes / 16));  // 0..575
  int64_t rt = tile / nkt, kt = tile % nkt;
  SlotSource s;
  if (within < kTileCodeBytes / 16) {
    int c = within / 64, l = within % 64;
    s.row = rt * kTileRows + l;
    s.first = (kt * kTileK + c * kChunkK) / 2;
    s.is_scale = false;
  } else {
    int l = within - kTileCodeBytes / 16;
    s.row = rt * kTileRows + l;
    s.first = kt * (kTileK / 16);
    s.is_scale = true;
  }
  return s;
}

__global__ void pack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                            int64_t n, int64_t k, int64_t nkt, int64_t slots, uint8_t* __restrict__ packed) {
  int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= slots) return;
  SlotSource s = slot_source(slot, nkt);
  const int64_t row_bytes = s.is_scale ? k / 16 : k / 2;
  const uint8_t* src = (s.is_scale ? scales : codes) + s.row * row_bytes;
  uint8_t out[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int64_t col = s.first + i;
    out[i] = (s.row < n && col < row_bytes) ? src[col] : (uint8_t)0;
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
  int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= slots) return;
  SlotSource s = slot_source(slot, nkt);
  if (s.row >= n) return;
  const int64_t row_bytes = s.is_scale ? k / 16 : k / 2;
  uint8_t* dst = (s.is_scale ? scales : codes) + s.row * row_bytes;
  uint4 v = *reinterpret_cast<const uint4*>(packed + slot * 16);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int64_t col = s.first + i;
    if (col < row_bytes) dst[col] = (uint8_t)(w[i / 4] >> (8 * (i % 4)));
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
