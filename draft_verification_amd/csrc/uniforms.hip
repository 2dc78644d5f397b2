// sd_uniforms: the uniforms behind the library's random decisions, for given
// (request, position, draw) counters.
//
// Every random decision of the method (the draft sample, the accept test and
// the correction sample; speculative-decoding history page, "1.1 mechanism",
// and DSpark summary, "innovation one") takes one uniform from the counter
// hash in sdv_common.h.  This entry point evaluates the same hash for a list
// of counters, so that a caller can replay or audit a step's decisions.
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_uniforms(uint64_t seed, long long n,
                                                       const int64_t* __restrict__ req,
                                                       const int64_t* __restrict__ pos,
                                                       uint64_t draw, float* __restrict__ out) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  // the 24-bit value is exact in fp32
  out[i] = (float)sdv::uniform24(seed, (uint64_t)req[i], (uint64_t)pos[i], draw);
}

}  // namespace

extern "C" int sd_uniforms(hipStream_t stream, uint64_t seed, long long n, const int64_t* req,
                           const int64_t* pos, int draw, float* out) {
  if (n < 0 || draw < 0) return SD_EINVAL;
  if (n == 0) return SD_OK;
  if (!req || !pos || !out) return SD_EINVAL;
  const long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFFLL) return SD_EUNSUPPORTED;
  SDV_TRY_LAUNCH(sdv::launch(k_uniforms, dim3((unsigned)blocks), dim3(kThreads), 0, stream, seed, n,
                             req, pos, (uint64_t)draw, out));
  return SD_OK;
}
