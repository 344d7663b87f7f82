// tq_stream.hip -- tq_stream_read: the practical HBM read ceiling that the
// GEMV's weight stream is measured against.
//
// Page "the full arc: how the 1bit.systems ternary stack got from broken to
// 76.7 tok/s", TL;DR, and page "1bit.systems" project README, section
// "hardware": the GEMV is judged by the fraction of the memory bandwidth it
// reaches.  A published peak is not reachable by any kernel; this one reads
// a buffer with the GEMV's access (16-byte non-temporal loads, consecutive
// lanes on consecutive pieces, eight loads in flight per lane) and does
// nothing else, so its rate is the ceiling a streaming kernel can reach on
// the same buffers.  Each block XORs what it read into one 16-byte word of
// `sink`, which keeps every load live and gives an exact check.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;    // 16-byte loads in flight per lane
constexpr int kStreamPerCu = 8;     // resident blocks per CU

// Tiles of kStreamThreads * kStreamUnroll pieces, interleaved over the grid
// and read without predicates; the pieces past the last whole tile are read
// by the last block.  (Measured on MI355X over a 2 GiB buffer: 8 blocks per
// CU 7.02 TB/s, 4 blocks 6.98, 16 loads per lane 6.64, 1024-thread blocks
// 6.80, ordinary cached loads 6.27.)
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(
    const u32x4 *__restrict__ p, int64_t n16, u32x4 *__restrict__ sink) {
  __shared__ u32x4 wx[kStreamThreads / kWave];
  u32x4 x = {0u, 0u, 0u, 0u};
  constexpr int64_t kTile = (int64_t)kStreamThreads * kStreamUnroll;
  const int64_t tiles = n16 / kTile;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const u32x4 *q = p + t * kTile + threadIdx.x;
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      v[u] = __builtin_nontemporal_load(q + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= v[u];
  }
  if (blockIdx.x == gridDim.x - 1)
    for (int64_t i = tiles * kTile + threadIdx.x; i < n16; i += kStreamThreads)
      x ^= __builtin_nontemporal_load(p + i);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    x[c] = wave_allreduce(x[c], [](uint32_t a, uint32_t b) { return a ^ b; });
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) wx[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 t = wx[0];
#pragma unroll
    for (int w = 1; w < kStreamThreads / kWave; ++w) t ^= wx[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_stream_read(const void *buf, int64_t bytes, void *sink,
                                    int64_t sink_words, hipStream_t stream) {
  using namespace tq;
  if (bytes < 0 || bytes % 16 != 0 || sink_words < 1) return TQ_ERR_SHAPE;
  if (bytes == 0) return TQ_OK;
  if (!buf || !sink) return TQ_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 16)) return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t n16 = bytes / 16;
  const int64_t per_block = (int64_t)kStreamThreads * kStreamUnroll;
  int64_t blocks = n16 / per_block;  // whole tiles; the last block also reads the rest
  if (blocks < 1) blocks = 1;
  blocks = blocks < (int64_t)dev.num_cus * kStreamPerCu ? blocks : (int64_t)dev.num_cus * kStreamPerCu;
  blocks = blocks < sink_words ? blocks : sink_words;
  return launch(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0,
                stream, reinterpret_cast<const u32x4 *>(buf), n16,
                reinterpret_cast<u32x4 *>(sink));
}
