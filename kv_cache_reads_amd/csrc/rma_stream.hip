// Streaming-read ceiling for benchmarks (instrumentation, not a step of the
// method).  Each block reads one contiguous piece of a device range with the
// scan's load form (nontemporal 16-byte loads, 256 threads, two batches of
// eight loads per thread in flight) and nothing else, so its time is what the chip allows for
// reading those bytes with that grid.  Block b XOR-folds the 32-bit words of its
// piece into sink[b], which makes every byte count and lets a test check that
// the whole range was read exactly once.
#include "rma_device.hpp"
#include "rma_internal.hpp"

namespace rma {

constexpr int kStreamThreads = 256;
constexpr int kStreamBatch = 8;   // 16-byte loads per thread and batch: 32 KB per block, as a scan batch

__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const uint4* __restrict__ p, int64_t n16, int64_t per_block, uint32_t* __restrict__ sink) {
  const int64_t b0 = (int64_t)blockIdx.x * per_block;
  const int64_t b1 = min(n16, b0 + per_block);
  constexpr int64_t STEP = (int64_t)kStreamThreads * kStreamBatch;
  uint32_t acc = 0u;
  if (b0 < b1) {
    // two batches in flight, as in the scan: batch j + 2 is issued as soon as
    // batch j is folded.  Loads are unconditional (a piece past the end re-reads
    // the block's last one and is masked out).
    auto load = [&](uint4 (&v)[kStreamBatch], int64_t i) {
#pragma unroll
      for (int k = 0; k < kStreamBatch; ++k) v[k] = ld_stream16(p + min(i + k * kStreamThreads, b1 - 1));
    };
    auto fold = [&](const uint4 (&v)[kStreamBatch], int64_t i) {
#pragma unroll
      for (int k = 0; k < kStreamBatch; ++k)
        acc ^= (i + k * kStreamThreads < b1) ? (v[k].x ^ v[k].y ^ v[k].z ^ v[k].w) : 0u;
    };
    uint4 va[kStreamBatch], vb[kStreamBatch];
    const int64_t i0 = b0 + threadIdx.x;
    load(va, i0);
    if (i0 - threadIdx.x + STEP < b1) load(vb, i0 + STEP);
    for (int64_t i = i0; i - threadIdx.x < b1; i += 2 * STEP) {
      fold(va, i);
      if (i - threadIdx.x + 2 * STEP < b1) load(va, i + 2 * STEP);
      if (i - threadIdx.x + STEP >= b1) break;
      fold(vb, i + STEP);
      if (i - threadIdx.x + 3 * STEP < b1) load(vb, i + 3 * STEP);
    }
  }
  // the block's fold, one plain store per block (one word shared by all blocks
  // would serialise their atomics at the end of the launch)
  __shared__ uint32_t s_x[kStreamThreads / kWave];
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & (kWave - 1)) == 0) s_x[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0u;
#pragma unroll
    for (int w = 0; w < kStreamThreads / kWave; ++w) x ^= s_x[w];
    sink[blockIdx.x] = x;
  }
}

hipError_t launch_stream_read(const void* p, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = (n16 + blocks - 1) / blocks;
  return launch_kernel("stream_read_kernel", stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, st,
                       static_cast<const uint4*>(p), n16, per_block, sink);
}

}  // namespace rma
