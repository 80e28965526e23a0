// A plain streaming read of a device buffer: the bandwidth yardstick beside which the
// layer's kernels are measured (the spec's peak is not what a read of HBM reaches).
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kStreamThreads = 512, kStreamDepth = 16;
constexpr int kStreamWaves = kStreamThreads / kWave;
constexpr size_t kStreamStep = (size_t)kWave * kStreamDepth * 16;   // bytes per wave per step

// Every wave reads one contiguous chunk, kStreamDepth 16-byte loads per lane in flight
// (non-temporal), through a buffer resource over its chunk: the hardware range check
// returns zeros past the end, so the last chunk needs no branch. The words are folded
// with xor and the fold is stored only if it equals a value the caller chooses, so the
// loads cannot be dropped and nearly nothing is written.
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(StreamArgs a) {
  const size_t bytes = a.words * 16;
  const size_t wv = (size_t)blockIdx.x * kStreamWaves + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const size_t per = a.chunk;                       // bytes per wave, a multiple of kStreamStep
  const size_t begin = wv * per;
  if (begin >= bytes) return;
  const size_t len = bytes - begin < per ? bytes - begin : per;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.src + begin), (short)0, (int)len, kRsrcWord3);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t off = 0; off < len; off += kStreamStep) {
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; d++)
      v[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, (int)(off + (size_t)d * kWave * 16), 2));
#pragma unroll
    for (int d = 0; d < kStreamDepth; d++) acc ^= v[d];
  }
  const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == a.magic) a.sink[0] = f;
}

int launch_stream_read(const StreamArgs& a0, hipStream_t s, const Prof* p) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  // 4 workgroups of 8 waves per compute unit, every wave one chunk (fewer when the
  // buffer is small: at least one step per wave)
  StreamArgs a = a0;
  const size_t bytes = a.words * 16;
  size_t waves = (size_t)cus * 4 * kStreamWaves;
  size_t per = (bytes + waves - 1) / waves;
  per = (per + kStreamStep - 1) / kStreamStep * kStreamStep;
  waves = (bytes + per - 1) / per;
  a.chunk = per;
  const size_t grid = (waves + kStreamWaves - 1) / kStreamWaves;
  launch(k_stream_read, dim3((unsigned)grid), dim3(kStreamThreads), 0, s, p, a);
  return (int)hipGetLastError();
}

}  // namespace sw
