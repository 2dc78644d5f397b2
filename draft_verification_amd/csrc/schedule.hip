// sd_schedule: survival products, candidate sort and greedy Theta selection.
//
// DSpark summary, "2.2 hardware-aware prefix scheduler": maximise
// Theta = tau * SPS(B) with B = sum_r (1 + l_r) and tau = sum_r sum_{j<=l_r} a_{r,j},
// greedily over candidates sorted by survival, stopping once Theta falls;
// "challenge 2" adds the capped asynchronous variant.  Speculative-decoding
// history page, DSpark "move two": a_{r,j} is the product of the per-position
// confidences up to j.
//
// Optional sequential temperature scaling (DSpark summary, "2.1 confidence
// head"): c' = sigmoid(logit(c) / T_j) per draft position j, in fp64 rounded
// to fp32, before the products.  Threshold mode (the confidence-threshold
// sweep of the same page) keeps every candidate whose survival is >= theta.
//
// Keys are uint64 so that one ascending integer order sorts by survival
// descending, then request, then position; they are unique.  Two kernels:
//   k_sched_rank    many workgroups: each rebuilds every key in LDS (one
//                   thread per request, fp32 products left to right, into a
//                   padded position-major table) and ranks 16 candidates by
//                   counting the smaller keys, 32 threads per candidate;
//                   writes sorted[rank] = key.  Sorting
//                   by counting is N^2 work, but spread over the whole chip it
//                   beats any single-CU network for these sizes (N <= 16384).
//   k_sched_select  one workgroup: the sorted keys in registers, the
//                   fixed-point tau scan, Theta, the mode's n*, and l_r.
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 1024;  // k_sched_select
constexpr int kWaves = kThreads / 64;
static_assert((kWaves & (kWaves - 1)) == 0 && kWaves <= 64, "wave results combine in one wave");
constexpr int kRankThreads = 512;  // measured: 256 threads 12.9, 512 11.9, 1024 12.3 us per headline schedule
constexpr int kRankCand = 16;   // candidates per ranking workgroup
constexpr int kRankSegs = kRankThreads / kRankCand;

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

// c' = 1 / (1 + ((1 - c) / c)^(1 / T)) = sigmoid(logit(c) / T); 0 and 1 are fixed.
__device__ __forceinline__ float sts_calibrate(float c, float T) {
  if (c != c) return c;  // NaN stays NaN
  if (!(c > 0.0f)) return 0.0f;
  if (c >= 1.0f) return 1.0f;
  const double odds = (1.0 - (double)c) / (double)c;
  return (float)(1.0 / (1.0 + pow(odds, 1.0 / (double)T)));
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint64_t wave_excl_scan_u64(uint64_t v, int lane) {
  uint64_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  return incl - v;
}


// Survival products of request r, fp32 left to right, straight from the
// confidences (recalibrated first when per-position temperatures are given):
// the key of position j goes to kT[(j-1) * ld + r] (position-major, ld =
// R + 1 so that neighbouring requests use neighbouring LDS words and the
// chain's accesses never share a bank); slots past gamma_r get the largest
// key.  The loads are independent of the chain and issue together; the
// products are sequential, as their definition is.
__device__ __forceinline__ void request_keys(int r, int gmax, int ld, const int32_t* gamma_r,
                                             const float* conf, const float* sts_temp,
                                             uint64_t* kT, float* surv) {
  const int g = gamma_r ? sdv::clampi(gamma_r[r], 0, gmax) : gmax;
  const float* cr = conf + (size_t)r * gmax;
  float a = 1.0f;
  constexpr int kU = 8;
  for (int j0 = 1; j0 <= gmax; j0 += kU) {
    float cv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) cv[u] = (j0 + u <= g) ? cr[j0 + u - 1] : 0.0f;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u;
      if (j > gmax) break;
      uint64_t key = ~0ull;
      float out = 0.0f;
      if (j <= g) {
        const float cj = sts_temp ? sts_calibrate(cv[u], sts_temp[j - 1]) : cv[u];
        a = a * cj;
        key = make_key(a, r, j);
        out = a;
      }
      kT[(j - 1) * ld + r] = key;
      if (surv) surv[(size_t)r * gmax + (j - 1)] = out;
    }
  }
}

// Candidates are the R * gmax slots in position-major order, kRankCand per
// workgroup (candidate c is slot (c / R) * ld + c % R of the table, so the
// padding adds no workgroup); kRankSegs segments of kRankCand threads count
// the smaller keys over the whole padded table, segment s reading keys s,
// s + kRankSegs, ... (the segments' concurrent reads are neighbouring words;
// a segment's threads read the same word).
__global__ __launch_bounds__(kRankThreads) void k_sched_rank(
    int R, int gmax, const int32_t* __restrict__ gamma_r, const float* __restrict__ conf,
    const float* __restrict__ sts_temp, float* __restrict__ surv, uint64_t* __restrict__ sorted) {
  extern __shared__ uint64_t kT[];
  __shared__ int part[kRankSegs][kRankCand];
  const int tid = threadIdx.x;
  const int ld = R + 1;
  const int nkeys = gmax * ld;  // padded table, the padding holds the largest key
  float* my_surv = blockIdx.x == 0 ? surv : nullptr;  // one workgroup writes it
  for (int i = tid; i < gmax; i += kRankThreads) kT[i * ld + R] = ~0ull;
  for (int r = tid; r < R; r += kRankThreads) request_keys(r, gmax, ld, gamma_r, conf, sts_temp, kT, my_surv);
  __syncthreads();
  const int cl = tid % kRankCand, seg = tid / kRankCand;
  const int cand = blockIdx.x * kRankCand + cl;
  const uint64_t mine = cand < R * gmax ? kT[(cand / R) * ld + cand % R] : ~0ull;
  int cnt = 0;
  int i = seg;
  for (; i + 7 * kRankSegs < nkeys; i += 8 * kRankSegs) {  // 8 independent LDS loads in flight
    uint64_t q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = kT[i + u * kRankSegs];
#pragma unroll
    for (int u = 0; u < 8; ++u) cnt += q[u] < mine ? 1 : 0;
  }
  for (; i < nkeys; i += kRankSegs) cnt += kT[i] < mine ? 1 : 0;
  part[seg][cl] = cnt;
  __syncthreads();
  if (tid < kRankCand && mine != ~0ull) {
    int rank = 0;
#pragma unroll
    for (int s2 = 0; s2 < kRankSegs; ++s2) rank += part[s2][tid];
    sorted[rank] = mine;
  }
}

template <int E>
__global__ __launch_bounds__(kThreads) void k_sched_select(
    int R, int gmax, const int32_t* __restrict__ gamma_r, const float* __restrict__ sps,
    int mode, const int32_t* __restrict__ cap_k, float threshold, const uint64_t* __restrict__ sorted,
    int32_t* __restrict__ ell, int32_t* __restrict__ batch_out, int32_t* __restrict__ n_sel_out,
    double* __restrict__ theta_out) {
  __shared__ int ell_lds[SD_MAX_SCHED_SLOTS];
  __shared__ uint64_t wave_tot[kWaves];
  __shared__ int s_count, s_fail, s_nstar, s_above;
  __shared__ double s_best_theta[kWaves];
  __shared__ int s_best_n[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nslots = R * gmax;
  const int i0 = tid * E;
  // issue the independent loads first: sorted keys (valid below N, known
  // after the count) and the throughput table entries this thread needs
  uint64_t key[E];
  float sps_n[E], sps_prev;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = i0 + e;
    key[e] = i < nslots ? sorted[i] : ~0ull;
    sps_n[e] = i < nslots ? sps[R + i] : 0.0f;
  }
  sps_prev = (i0 >= 1 && i0 - 1 < nslots) ? sps[R + i0 - 1] : 0.0f;
  if (tid == 0) { s_count = 0; s_fail = 0x7FFFFFFF; s_above = 0; }
  __syncthreads();
  // N = the number of candidates: R * gmax without per-request lengths
  int my_count = 0;
  for (int r = tid; r < R; r += kThreads) {
    if (gamma_r) my_count += sdv::clampi(gamma_r[r], 0, gmax);
    ell_lds[r] = 0;
  }
  if (gamma_r) {
    my_count = wave_sum_i(my_count);
    if (lane == 0 && my_count) atomicAdd(&s_count, my_count);
  }
  __syncthreads();
  const int N = gamma_r ? s_count : nslots;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (i0 + e >= N) key[e] = ~0ull;

  // 3. fixed-point tau scan over the sorted order.
  uint64_t my_sum = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (i0 + e < N) my_sum += key_fixed_point(key[e]);
  const uint64_t excl = wave_excl_scan_u64(my_sum, lane);
  if (lane == 63) wave_tot[wave] = excl + my_sum;
  __syncthreads();
  if (wave == 0) {
    const uint64_t v = lane < kWaves ? wave_tot[lane] : 0;
    const uint64_t e = wave_excl_scan_u64(v, lane);
    if (lane < kWaves) wave_tot[lane] = e;
  }
  __syncthreads();
  const uint64_t T0 = excl + wave_tot[wave];

  // 4. Theta_n = (T_n * 2^-32) * SPS[R + n - 1]; first decline and argmax.
  double best = 0.0;  // Theta_0 = 0 at n = 0
  int best_n = 0;
  int fail = 0x7FFFFFFF;
  uint64_t T = T0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = i0 + e;
    if (i < N) {
      const uint64_t Tprev = T;
      T += key_fixed_point(key[e]);
      const int n = i + 1;
      const double th = (double)T * 0x1p-32 * (double)sps_n[e];
      const double th_prev = (n == 1) ? 0.0 : (double)Tprev * 0x1p-32 * (double)(e == 0 ? sps_prev : sps_n[e - 1]);
      if (th < th_prev && n < fail) fail = n;
      if (th > best) { best = th; best_n = n; }
    }
  }
  if (mode == SD_SCHED_THRESHOLD) {  // candidates with survival >= theta (a prefix)
    int above = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (i0 + e < N && key_survival(key[e]) >= threshold) ++above;
    if (above) atomicAdd(&s_above, above);
  }
  fail = sdv::wave_min_i(fail);
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
  if (wave == 0) {
    // the waves' bests, combined in lanes 0..kWaves-1 by the same rule
    double b = lane < kWaves ? s_best_theta[lane] : 0.0;
    int bn = lane < kWaves ? s_best_n[lane] : 0x7FFFFFFF;
#pragma unroll
    for (int o = kWaves / 2; o > 0; o >>= 1) {
      const double ob = __shfl_xor(b, o, 64);
      const int on = __shfl_xor(bn, o, 64);
      if (ob > b || (ob == b && on < bn)) { b = ob; bn = on; }
    }
    if (lane == 0) {
      int nstar;
      if (mode == SD_SCHED_EARLY_STOP) nstar = (s_fail == 0x7FFFFFFF) ? N : s_fail - 1;
      else if (mode == SD_SCHED_GLOBAL_ARGMAX) nstar = bn;
      else if (mode == SD_SCHED_THRESHOLD) nstar = s_above;
      else nstar = sdv::clampi(*cap_k, 0, N);
      s_nstar = nstar;
      if (batch_out) *batch_out = R + nstar;
      if (n_sel_out) *n_sel_out = nstar;
      if (theta_out && nstar == 0) *theta_out = 0.0;
    }
  }
  __syncthreads();
  const int nstar = s_nstar;

  // 5. Theta_{n*} from its owner; l_r = largest selected position of request
  //    r (the selected set is prefix-closed), gathered through LDS.
  if (theta_out && nstar > 0 && nstar - 1 >= i0 && nstar - 1 < i0 + E) {
    uint64_t Ti = T0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (i0 + e <= nstar - 1) Ti += key_fixed_point(key[e]);
    *theta_out = (double)Ti * 0x1p-32 * (double)sps[R + nstar - 1];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (i0 + e < nstar) {
      const uint32_t lo = (uint32_t)key[e];
      atomicMax(&ell_lds[lo >> 8], (int)(lo & 0xFF));
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) ell[r] = ell_lds[r];
}

size_t sched_ws_bytes(int R, int gmax) {
  return sdv_align256((size_t)(R * gmax > 0 ? R * gmax : 1) * sizeof(uint64_t));
}

}  // namespace

extern "C" size_t sd_schedule_workspace_size(int R, int gamma_max) {
  if (R < 0 || gamma_max < 0) return 0;
  return sched_ws_bytes(R, gamma_max);
}

extern "C" int sd_schedule(hipStream_t stream, int R, int gamma_max, const int32_t* gamma_r,
                           const float* conf, const float* sts_temp, const float* sps, int sps_len,
                           int mode, const int32_t* cap_k, float threshold, int32_t* ell,
                           int32_t* batch, int32_t* n_sel, double* theta, float* surv,
                           void* workspace, size_t workspace_bytes) {
  if (R < 0 || gamma_max < 0) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA) return SD_EUNSUPPORTED;
  if ((long long)R * gamma_max > SD_MAX_SCHED_SLOTS) return SD_EUNSUPPORTED;
  if (mode != SD_SCHED_EARLY_STOP && mode != SD_SCHED_GLOBAL_ARGMAX &&
      mode != SD_SCHED_CAPPED_TOPK && mode != SD_SCHED_THRESHOLD)
    return SD_EINVAL;
  if (mode == SD_SCHED_CAPPED_TOPK && !cap_k) return SD_EINVAL;
  if (mode == SD_SCHED_THRESHOLD && threshold != threshold) return SD_EINVAL;  // NaN
  if (R > 0 && (!ell || !sps || (gamma_max > 0 && !conf))) return SD_EINVAL;
  if ((long long)sps_len < (long long)R * (1 + gamma_max)) return SD_ERANGE;
  if (!workspace || workspace_bytes < sched_ws_bytes(R, gamma_max)) return SD_ERANGE;
  if (((uintptr_t)workspace & 7) != 0) return SD_EINVAL;
  uint64_t* sorted = (uint64_t*)workspace;
  const int nslots = R * gamma_max;
  if (nslots > 0) {
    const size_t lds = (size_t)gamma_max * (R + 1) * sizeof(uint64_t);  // the padded key table
    if (lds > 64 * 1024)
      SDV_TRY_LAUNCH(hipFuncSetAttribute((const void*)k_sched_rank,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    SDV_TRY_LAUNCH(sdv::launch(k_sched_rank, dim3((nslots + kRankCand - 1) / kRankCand),
                               dim3(kRankThreads), lds, stream, R, gamma_max, gamma_r, conf,
                               sts_temp, surv, sorted));
  }
  int npad = 1;
  while (npad < nslots) npad <<= 1;
  const int E = npad > kThreads ? npad / kThreads : 1;
#define SDV_SELECT_LAUNCH(EV)                                                                   \
  SDV_TRY_LAUNCH(sdv::launch(k_sched_select<EV>, dim3(1), dim3(kThreads), 0, stream, R, gamma_max, \
                             gamma_r, sps, mode, cap_k, threshold, (const uint64_t*)sorted, ell,   \
                             batch, n_sel,                                                       \
                             theta))
  switch (E) {
    case 1: SDV_SELECT_LAUNCH(1); break;
    case 2: SDV_SELECT_LAUNCH(2); break;
    case 4: SDV_SELECT_LAUNCH(4); break;
    case 8: SDV_SELECT_LAUNCH(8); break;
    default: SDV_SELECT_LAUNCH(16); break;
  }
#undef SDV_SELECT_LAUNCH
  return SD_OK;
}
