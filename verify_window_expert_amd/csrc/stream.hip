// A plain streaming read of a device buffer: the bandwidth yardstick beside which the
// layer's kernels are measured (the spec's peak is not what a read of HBM reaches).
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kStreamThreads = 256, kStreamUnroll = 4;

// Every thread reads 16-byte words (non-temporal) at a grid stride, kStreamUnroll loads
// in flight, and folds them with xor; the fold is stored only if it equals a value the
// caller cannot arrange by accident, so the loads cannot be dropped and nearly nothing
// is written.
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(StreamArgs a) {
  const u32x4* src = (const u32x4*)a.src;
  const size_t n = a.words, stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kStreamUnroll - 1) * stride < n; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; u++) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == a.magic) a.sink[0] = f;
}

int launch_stream_read(const StreamArgs& a, hipStream_t s, const Prof* p) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  // 8 workgroups per compute unit, never more than there are words
  const size_t per = (size_t)kStreamThreads * kStreamUnroll;
  size_t grid = (size_t)cus * 8;
  if (grid * per > a.words) grid = (a.words + per - 1) / per;
  if (grid < 1) grid = 1;
  launch(k_stream_read, dim3((unsigned)grid), dim3(kStreamThreads), 0, s, p, a);
  return (int)hipGetLastError();
}

}  // namespace sw
