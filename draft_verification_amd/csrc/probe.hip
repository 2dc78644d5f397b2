// libsdv_probe: the benchmark's measurement aid, built beside libsdv and not
// part of its interface.  A plain streaming read: 256-thread workgroups,
// each thread issuing 32 16-byte non-temporal loads together (128 KB per
// workgroup), folded to one word per workgroup.  Of the plain reads measured
// (32, 64 and 128 KB per workgroup, with and without a pause between two
// halves) this shape was the fastest, 7.0 against 6.7-6.8 TB/s over 1.79 GB;
// its duration over a buffer of the batch's size is the practical HBM read
// ceiling that the bandwidth pass is compared with.
//
//   long long probe_stream_read_sink_words(long long bytes)
//       uint32 words the sink needs for `bytes` (-1 for bytes < 0)
//   int probe_stream_read(hipStream_t s, const void* src, long long bytes, uint32_t* sink)
//       stream `bytes` (a multiple of 16) of 16-byte aligned device memory,
//       folding each workgroup's words into one sink word; SD_* return codes
//
// A second probe gives the ceiling of a mixed stream, for the drafting
// heads' bias kernel, which reads C_k and U_k and writes L_k (three bytes
// read per byte written for the Markov head, two for the RNN head):
//   int probe_stream_mix(hipStream_t s, const void* src, void* dst, long long wbytes, int ratio)
//       read ratio * wbytes of src (ratio in [1, 4]) and write wbytes of dst
//       (a multiple of 2048; both 16-byte aligned), non-temporal both ways:
//       each wave reads ratio * 2 KB and writes their XOR folded to 2 KB
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPer = 32;
constexpr long long kVecPerBlock = (long long)kThreads * kPer;

__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4* __restrict__ src, long long n,
                                                          uint32_t* sink) {
  const long long base = (long long)blockIdx.x * kVecPerBlock;
  uint4 v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const long long i = base + threadIdx.x + (long long)k * kThreads;
    v[k] = i < n ? sdv::ld_nt(src + i) : make_uint4(0, 0, 0, 0);
  }
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;  // one word per workgroup (wave 0's fold)
}

constexpr int kMixMaxRatio = 4;
constexpr long long kMixWaveBytes = 2048;  // written per wave: 128 vectors, two per lane

__global__ __launch_bounds__(kThreads) void k_stream_mix(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         long long chunks, int ratio) {
  const long long c = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (c >= chunks) return;
  const int lane = threadIdx.x & 63;
  const uint4* s = src + c * 128 * ratio;
  uint4 v[2 * kMixMaxRatio];
#pragma unroll
  for (int i = 0; i < 2 * kMixMaxRatio; ++i)
    v[i] = i < 2 * ratio ? sdv::ld_nt(s + i * 64 + lane) : make_uint4(0, 0, 0, 0);
  uint4 a = v[0], b = v[1];
#pragma unroll
  for (int i = 1; i < kMixMaxRatio; ++i) {
    a.x ^= v[2 * i].x; a.y ^= v[2 * i].y; a.z ^= v[2 * i].z; a.w ^= v[2 * i].w;
    b.x ^= v[2 * i + 1].x; b.y ^= v[2 * i + 1].y; b.z ^= v[2 * i + 1].z; b.w ^= v[2 * i + 1].w;
  }
  sdv::st_nt(dst + c * 128 + lane, a);
  sdv::st_nt(dst + c * 128 + 64 + lane, b);
}

}  // namespace

extern "C" int probe_stream_mix(hipStream_t stream, const void* src, void* dst, long long wbytes, int ratio) {
  if (wbytes < 0 || (wbytes % kMixWaveBytes) != 0 || ratio < 1 || ratio > kMixMaxRatio) return SD_EINVAL;
  if (wbytes == 0) return SD_OK;
  if (!src || !dst || ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) != 0) return SD_EINVAL;
  const long long chunks = wbytes / kMixWaveBytes;
  const long long blocks = (chunks + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0xFFFFFFFFLL / kThreads) return SD_EUNSUPPORTED;
  SDV_TRY_LAUNCH(sdv::launch(k_stream_mix, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                             (const uint4*)src, (uint4*)dst, chunks, ratio));
  return SD_OK;
}

extern "C" long long probe_stream_read_sink_words(long long bytes) {
  if (bytes < 0) return -1;
  return (bytes / 16 + kVecPerBlock - 1) / kVecPerBlock;
}

extern "C" int probe_stream_read(hipStream_t stream, const void* src, long long bytes, uint32_t* sink) {
  if (bytes < 0 || (bytes % 16) != 0) return SD_EINVAL;
  if (bytes == 0) return SD_OK;
  if (!src || !sink || (((uintptr_t)src) & 15) != 0) return SD_EINVAL;
  const long long n = bytes / 16;
  const long long blocks = (n + kVecPerBlock - 1) / kVecPerBlock;
  if (blocks > 0xFFFFFFFFLL / kThreads) return SD_EUNSUPPORTED;  // work-items of one launch
  SDV_TRY_LAUNCH(sdv::launch(k_stream_read, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                             (const uint4*)src, n, sink));
  return SD_OK;
}
