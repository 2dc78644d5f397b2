// sd_schedule: survival products, candidate sort and greedy Theta selection.
//
// DSpark summary, "2.2 hardware-aware prefix scheduler": maximise
// Theta = tau * SPS(B) with B = sum_r (1 + l_r) and tau = sum_r sum_{j<=l_r} a_{r,j},
// greedily over candidates sorted by survival, stopping once Theta falls;
// "challenge 2" adds the capped asynchronous variant.  Speculative-decoding
// history page, DSpark "move two": a_{r,j} is the product of the per-position
// confidences up to j.
//
// One workgroup of 1024 threads does everything in LDS (the problem is at most
// 16384 candidates, and latency-bound): keys are uint64 so that one ascending
// integer sort orders by survival descending, then request, then position.
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// key = (~bits(a)) << 32 | r << 8 | j.  a >= 0, so its bit pattern grows with
// a and the complement sorts larger survival first.
__device__ __forceinline__ uint64_t make_key(float a, int r, int j) {
  return ((uint64_t)(~__float_as_uint(a)) << 32) | ((uint64_t)(uint32_t)r << 8) | (uint32_t)j;
}
__device__ __forceinline__ float key_survival(uint64_t key) {
  return __uint_as_float(~(uint32_t)(key >> 32));
}
// q = rint(a * 2^32): exact in fp64 (a has 24 significant bits).
__device__ __forceinline__ uint64_t key_fixed_point(uint64_t key) {
  return (uint64_t)__builtin_rint((double)key_survival(key) * 4294967296.0);
}

__device__ __forceinline__ uint64_t wave_excl_scan_u64(uint64_t v, int lane) {
  uint64_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void k_schedule(
    int R, int gmax, const int32_t* __restrict__ gamma_r, const float* __restrict__ conf,
    const float* __restrict__ sps, int mode, const int32_t* __restrict__ cap_k,
    int32_t* __restrict__ ell, int32_t* __restrict__ batch_out, int32_t* __restrict__ n_sel_out,
    double* __restrict__ theta_out, float* __restrict__ surv, int npad) {
  __shared__ uint64_t keys[SD_MAX_SCHED_SLOTS];
  __shared__ uint64_t wave_tot[kWaves];
  __shared__ int s_count, s_fail, s_nstar;
  __shared__ double s_best_theta[kWaves];
  __shared__ int s_best_n[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { s_count = 0; s_fail = 0x7FFFFFFF; }
  __syncthreads();

  // 1. survival products, left to right in fp32, one thread per request.
  int my_count = 0;
  for (int r = tid; r < R; r += kThreads) {
    const int g = gamma_r ? sdv::clampi(gamma_r[r], 0, gmax) : gmax;
    float a = 1.0f;
    for (int j = 1; j <= gmax; ++j) {
      uint64_t key = ~0ull;
      float out = 0.0f;
      if (j <= g) {
        a = a * conf[(size_t)r * gmax + (j - 1)];
        key = make_key(a, r, j);
        out = a;
      }
      keys[r * gmax + (j - 1)] = key;
      if (surv) surv[(size_t)r * gmax + (j - 1)] = out;
    }
    my_count += g;
  }
  for (int i = R * gmax + tid; i < npad; i += kThreads) keys[i] = ~0ull;
  if (my_count) atomicAdd(&s_count, my_count);
  __syncthreads();
  const int N = s_count;

  // 2. bitonic sort of npad keys, ascending.
  for (int k = 2; k <= npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < (npad >> 1); t += kThreads) {
        const int i = 2 * t - (t & (j - 1));
        const int l = i + j;
        const uint64_t x = keys[i], y = keys[l];
        const bool asc = (i & k) == 0;
        if ((x > y) == asc) { keys[i] = y; keys[l] = x; }
      }
      __syncthreads();
    }
  }

  // 3. fixed-point tau scan over the sorted order: thread t owns the
  //    contiguous positions [t*seg, (t+1)*seg).
  const int seg = (npad + kThreads - 1) / kThreads;
  const int i0 = tid * seg;
  uint64_t my_sum = 0;
  for (int s = 0; s < seg; ++s) {
    const int i = i0 + s;
    if (i < N) my_sum += key_fixed_point(keys[i]);
  }
  uint64_t excl = wave_excl_scan_u64(my_sum, lane);
  if (lane == 63) wave_tot[wave] = excl + my_sum;
  __syncthreads();
  if (wave == 0) {
    uint64_t v = lane < kWaves ? wave_tot[lane] : 0;
    uint64_t e = wave_excl_scan_u64(v, lane);
    if (lane < kWaves) wave_tot[lane] = e;
  }
  __syncthreads();
  uint64_t T = excl + wave_tot[wave];

  // 4. Theta_n = (T_n * 2^-32) * SPS[R + n - 1]; first decline and argmax.
  double best = 0.0;   // Theta_0 = 0 at n = 0
  int best_n = 0;
  int fail = 0x7FFFFFFF;
  for (int s = 0; s < seg; ++s) {
    const int i = i0 + s;
    if (i >= N) break;
    const uint64_t q = key_fixed_point(keys[i]);
    const uint64_t Tprev = T;
    T += q;
    const int n = i + 1;
    const double th = (double)T * 0x1p-32 * (double)sps[R + n - 1];
    const double th_prev = (n == 1) ? 0.0 : (double)Tprev * 0x1p-32 * (double)sps[R + n - 2];
    if (th < th_prev && n < fail) fail = n;
    if (th > best) { best = th; best_n = n; }
  }
  fail = sdv::wave_min_i(fail);
  // argmax over the wave: larger Theta, then smaller n
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(best, o, 64);
    const int on = __shfl_xor(best_n, o, 64);
    if (ob > best || (ob == best && on < best_n)) { best = ob; best_n = on; }
  }
  if (lane == 0) {
    atomicMin(&s_fail, fail);
    s_best_theta[wave] = best;
    s_best_n[wave] = best_n;
  }
  __syncthreads();
  if (tid == 0) {
    double b = s_best_theta[0];
    int bn = s_best_n[0];
    for (int w = 1; w < kWaves; ++w)
      if (s_best_theta[w] > b || (s_best_theta[w] == b && s_best_n[w] < bn)) {
        b = s_best_theta[w];
        bn = s_best_n[w];
      }
    int nstar;
    if (mode == SD_SCHED_EARLY_STOP) nstar = (s_fail == 0x7FFFFFFF) ? N : s_fail - 1;
    else if (mode == SD_SCHED_GLOBAL_ARGMAX) nstar = bn;
    else nstar = sdv::clampi(*cap_k, 0, N);
    s_nstar = nstar;
  }
  __syncthreads();
  const int nstar = s_nstar;

  // 5. outputs.  Theta_{n*} is recomputed from the prefix sum by the owner.
  if (tid == 0) {
    if (batch_out) *batch_out = R + nstar;
    if (n_sel_out) *n_sel_out = nstar;
    if (theta_out && nstar == 0) *theta_out = 0.0;
  }
  if (theta_out && nstar > 0) {
    const int i = nstar - 1;
    if (i >= i0 && i < i0 + seg) {
      uint64_t Ti = excl + wave_tot[wave];
      for (int ii = i0; ii <= i; ++ii) Ti += key_fixed_point(keys[ii]);
      *theta_out = (double)Ti * 0x1p-32 * (double)sps[R + nstar - 1];
    }
  }
  // l_r = #{j : key(r, j) <= the n*-th smallest key}; the survival products
  // are recomputed with the same fp32 multiplies, so the keys are identical.
  const uint64_t kstar = nstar > 0 ? keys[nstar - 1] : 0;
  for (int r = tid; r < R; r += kThreads) {
    int cnt = 0;
    if (nstar > 0) {
      const int g = gamma_r ? sdv::clampi(gamma_r[r], 0, gmax) : gmax;
      float a = 1.0f;
      for (int j = 1; j <= g; ++j) {
        a = a * conf[(size_t)r * gmax + (j - 1)];
        if (make_key(a, r, j) <= kstar) cnt = j;
        else break;
      }
    }
    ell[r] = cnt;
  }
}

}  // namespace

extern "C" int sd_schedule(hipStream_t stream, int R, int gamma_max, const int32_t* gamma_r,
                           const float* conf, const float* sps, int sps_len, int mode,
                           const int32_t* cap_k, int32_t* ell, int32_t* batch, int32_t* n_sel,
                           double* theta, float* surv) {
  if (R < 0 || gamma_max < 0) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA) return SD_EUNSUPPORTED;
  if ((long long)R * gamma_max > SD_MAX_SCHED_SLOTS) return SD_EUNSUPPORTED;
  if (mode != SD_SCHED_EARLY_STOP && mode != SD_SCHED_GLOBAL_ARGMAX && mode != SD_SCHED_CAPPED_TOPK)
    return SD_EINVAL;
  if (mode == SD_SCHED_CAPPED_TOPK && !cap_k) return SD_EINVAL;
  if (R > 0 && (!ell || !sps || (gamma_max > 0 && !conf))) return SD_EINVAL;
  if ((long long)sps_len < (long long)R * (1 + gamma_max)) return SD_ERANGE;
  int npad = 1;
  while (npad < R * gamma_max) npad <<= 1;
  SDV_TRY_LAUNCH(sdv::launch(k_schedule, dim3(1), dim3(kThreads), 0, stream, R, gamma_max, gamma_r,
                             conf, sps, mode, cap_k, ell, batch, n_sel, theta, surv, npad));
  return SD_OK;
}
