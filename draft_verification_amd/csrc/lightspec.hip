// Training-free two-stage budget planner (LightSpec article): runtime
// statistics kept as exponential moving averages, interpolated across draft
// positions where samples are missing, then a verify budget (stage 1) and the
// next round's draft length with the drafting cost in the objective (stage 2).
//
// Readings: one EMA per draft position of the acceptance probability
// alpha = sum_v min(p, q) that sd_verify reports (the DSpark summary's
// confidence label, "2.1"); stage 1 is the prefix scheduler's global argmax on
// the interpolated EMA values, the same for every request; stage 2 maximises
// Phi(d) = (R + tau*(d)) / (draft_cost[d-1] + 1 / SPS(B*(d))) over d.
//
//   k_ls_update   one workgroup, one thread per position: the step's mean
//                 alpha over the requests that verified it (request order,
//                 fp64, requests staged through LDS), folded into the EMA
//                 with unfused fp64 arithmetic
//   k_ls_conf     one workgroup: interpolated confidences, and the same row
//                 broadcast to every request for the stage-1 scheduler
//   k_ls_draft    one workgroup: Theta_n for every n of the uniform-draft
//                 candidate order, a workgroup prefix argmax, Phi(d) and the
//                 smallest maximising d
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;        // k_ls_update, k_ls_conf
constexpr int kDraftThreads = 1024;  // k_ls_draft
constexpr int kDraftWaves = kDraftThreads / 64;
constexpr int kMaxPer = SD_MAX_SCHED_SLOTS / kDraftThreads;  // candidates per thread

// fp64 expressions evaluated without contraction into fused multiply-adds, so
// that every rounding is the one the definition states.
__device__ __forceinline__ double ema_step(double e, double lam, double mean) {
#pragma clang fp contract(off)
  return (1.0 - lam) * e + lam * mean;
}
__device__ __forceinline__ double lerp_at(double lo, double hi, double t) {
#pragma clang fp contract(off)
  return lo + (hi - lo) * t;
}
__device__ __forceinline__ double phi_of(int R, double tau, double cost, double sps) {
#pragma clang fp contract(off)
  return ((double)R + tau) / (cost + 1.0 / sps);
}

// One workgroup; thread t owns positions j = t+1, t+1+kThreads, ...  The
// requests are staged through LDS in chunks (coalesced loads), each thread
// then sums its column in request order.
constexpr int kUpdChunkFloats = 8192;
__global__ __launch_bounds__(kThreads) void k_ls_update(int R, int G, const float* __restrict__ alpha,
                                                        const int32_t* __restrict__ ell,
                                                        const int32_t* __restrict__ status,
                                                        double lam, double* __restrict__ ema,
                                                        int64_t* __restrict__ count) {
  __shared__ float s_alpha[kUpdChunkFloats];
  __shared__ int s_len[kUpdChunkFloats];  // verified length of a request that did not fail, else 0
  constexpr int kPer = (SD_MAX_GAMMA + kThreads - 1) / kThreads;
  double total[kPer];
  int64_t n[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    total[q] = 0.0;
    n[q] = 0;
  }
  const int chunk = kUpdChunkFloats / G;  // requests per chunk (G <= SD_MAX_GAMMA < 8192)
  for (int r0 = 0; r0 < R; r0 += chunk) {
    const int rc = min(chunk, R - r0);
    __syncthreads();  // the previous chunk is consumed
    for (int i = threadIdx.x; i < rc * G; i += kThreads) s_alpha[i] = alpha[(size_t)r0 * G + i];
    for (int r = threadIdx.x; r < rc; r += kThreads)
      s_len[r] = (status[r0 + r] & (SD_ST_NONFINITE | SD_ST_ZERO_Z)) ? 0 : sdv::clampi(ell[r0 + r], 0, G);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int j = threadIdx.x + q * kThreads + 1;
      if (j > G) continue;
      int r = 0;
      for (; r + 8 <= rc; r += 8) {  // loads of 8 requests in flight, adds in request order
        int len[8];
        float a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          len[u] = s_len[r + u];
          a[u] = s_alpha[(r + u) * G + (j - 1)];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (len[u] >= j) {
            total[q] += (double)a[u];
            ++n[q];
          }
        }
      }
      for (; r < rc; ++r) {
        if (s_len[r] >= j) {
          total[q] += (double)s_alpha[r * G + (j - 1)];
          ++n[q];
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int j = threadIdx.x + q * kThreads + 1;
    if (j > G || n[q] == 0) continue;
    const double mean = total[q] / (double)n[q];
    const int64_t c = count[j - 1];
    ema[j - 1] = c == 0 ? mean : ema_step(ema[j - 1], lam, mean);
    count[j - 1] = c + n[q];
  }
}

// Planning confidences: observed positions keep their EMA, unobserved ones
// are interpolated linearly between the nearest observed neighbours (held
// constant past the ends); nothing observed: the table as given.  Clamped to
// [0, 1], rounded to fp32, broadcast to conf_rows[R][G].
__global__ __launch_bounds__(kThreads) void k_ls_conf(int R, int G, const double* __restrict__ ema,
                                                      const int64_t* __restrict__ count,
                                                      float* __restrict__ conf_hat,
                                                      float* __restrict__ conf_rows) {
  __shared__ float s_c[SD_MAX_GAMMA];
  __shared__ int s_seen;
  if (threadIdx.x == 0) s_seen = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < G; j += kThreads)
    if (count[j] > 0) atomicOr(&s_seen, 1);
  __syncthreads();
  for (int j = threadIdx.x; j < G; j += kThreads) {
    double v;
    if (!s_seen || count[j] > 0) {
      v = ema[j];
    } else {
      int lo = -1, hi = -1;
      for (int i = j - 1; i >= 0; --i)
        if (count[i] > 0) { lo = i; break; }
      for (int i = j + 1; i < G; ++i)
        if (count[i] > 0) { hi = i; break; }
      if (lo < 0) v = ema[hi];
      else if (hi < 0) v = ema[lo];
      else v = lerp_at(ema[lo], ema[hi], (double)(j - lo) / (double)(hi - lo));
    }
    v = v < 0.0 ? 0.0 : (v > 1.0 ? 1.0 : v);
    const float c = (float)v;
    s_c[j] = c;
    if (conf_hat) conf_hat[j] = c;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * G; i += kThreads) conf_rows[i] = s_c[i % G];
}

// (value, index) maximum that keeps the smaller index on ties; `a` precedes `b`.
struct Best {
  double v;
  int n;
};
__device__ __forceinline__ Best better(Best a, Best b) { return b.v > a.v ? b : a; }

__global__ __launch_bounds__(kDraftThreads) void k_ls_draft(int R, int G, const float* __restrict__ conf_rows,
                                                            const float* __restrict__ sps,
                                                            const float* __restrict__ draft_cost,
                                                            double* __restrict__ phi,
                                                            int32_t* __restrict__ d_next,
                                                            int32_t* __restrict__ b_next) {
  __shared__ uint64_t s_q[SD_MAX_GAMMA];
  __shared__ uint64_t s_pref[SD_MAX_GAMMA + 1];  // s_pref[k] = q_1 + ... + q_k
  __shared__ Best s_wave[kDraftWaves];
  __shared__ double s_phi[SD_MAX_GAMMA];
  __shared__ int s_nbest[SD_MAX_GAMMA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {  // survivals of the shared confidence row, fp32 left to right
    float a = 1.0f;
    uint64_t p = 0;
    s_pref[0] = 0;
    for (int j = 0; j < G; ++j) {
      a = a * conf_rows[j];
      const uint64_t q = (uint64_t)__builtin_rint((double)a * 4294967296.0);
      s_q[j] = q;
      p += q;
      s_pref[j + 1] = p;
    }
  }
  __syncthreads();

  // Candidate n (1-based) of the order a_1 x R, a_2 x R, ... sits at position
  // k = (n-1)/R + 1; T_n = R * (q_1 + .. + q_{k-1}) + (n - R(k-1)) * q_k.
  const int N = R * G;
  const int per = (N + kDraftThreads - 1) / kDraftThreads;
  const int n0 = tid * per + 1;
  Best local[kMaxPer];
  Best run = {0.0, 0};  // Theta_0 = 0 at n = 0 for thread 0's prefix
  const Best none = {-__builtin_huge_val(), 0x7FFFFFFF};
  Best mine = none;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    const int n = n0 + e;
    Best b = none;
    if (e < per && n <= N) {
      const int k = (n - 1) / R + 1;
      const uint64_t T = (uint64_t)R * s_pref[k - 1] + (uint64_t)(n - R * (k - 1)) * s_q[k - 1];
      b.v = (double)T * 0x1p-32 * (double)sps[R + n - 1];
      b.n = n;
    }
    mine = better(mine, b);
    local[e] = mine;  // prefix best within this thread's range
  }
  // exclusive scan of the per-thread bests over the workgroup
  Best incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    Best t;
    t.v = __shfl_up(incl.v, o, 64);
    t.n = __shfl_up(incl.n, o, 64);
    if (lane >= o) incl = better(t, incl);
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  Best before = run;
  for (int w = 0; w < wave; ++w) before = better(before, s_wave[w]);
  Best up;
  up.v = __shfl_up(incl.v, 1, 64);
  up.n = __shfl_up(incl.n, 1, 64);
  if (lane > 0) before = better(before, up);
  // the prefix best at n = R*d, for every d whose boundary falls in this range
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    const int n = n0 + e;
    if (e < per && n <= N && n % R == 0) {
      const Best b = better(before, local[e]);
      const int d = n / R;
      const uint64_t T = b.n == 0 ? 0 : ((uint64_t)R * s_pref[(b.n - 1) / R] +
                                         (uint64_t)(b.n - R * ((b.n - 1) / R)) * s_q[(b.n - 1) / R]);
      s_phi[d - 1] = phi_of(R, (double)T * 0x1p-32, (double)draft_cost[d - 1], (double)sps[R + b.n - 1]);
      s_nbest[d - 1] = b.n;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int best = 1;
    for (int d = 2; d <= G; ++d)
      if (s_phi[d - 1] > s_phi[best - 1]) best = d;
    *d_next = best;
    *b_next = R + s_nbest[best - 1];
  }
  if (phi)
    for (int d = tid + 1; d <= G; d += kDraftThreads) phi[d - 1] = s_phi[d - 1];
}

size_t plan_ws_bytes(int R, int G) {
  return sdv_align256((size_t)(R * G > 0 ? R * G : 1) * sizeof(float)) +
         sd_schedule_workspace_size(R, G);
}

}  // namespace

extern "C" int sd_lightspec_update(hipStream_t stream, int R, int gamma_max, const float* alpha,
                                   const int32_t* ell, const int32_t* status, double lambda,
                                   double* ema, int64_t* count) {
  if (R < 0 || gamma_max < 0) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA) return SD_EUNSUPPORTED;
  if (!(lambda >= 0.0 && lambda <= 1.0)) return SD_EINVAL;
  if (R == 0 || gamma_max == 0) return SD_OK;
  if (!alpha || !ell || !status || !ema || !count) return SD_EINVAL;
  SDV_TRY_LAUNCH(sdv::launch(k_ls_update, dim3(1), dim3(kThreads), 0, stream, R, gamma_max, alpha, ell,
                             status, lambda, ema, count));
  return SD_OK;
}

extern "C" size_t sd_lightspec_plan_workspace_size(int R, int gamma_max) {
  if (R < 0 || gamma_max < 0) return 0;
  return plan_ws_bytes(R, gamma_max);
}

extern "C" int sd_lightspec_plan(hipStream_t stream, int R, int gamma_max, const double* ema,
                                 const int64_t* count, const int32_t* d_prev, const float* sps,
                                 int sps_len, const float* draft_cost, float* conf_hat,
                                 int32_t* ell, int32_t* batch, int32_t* n_sel, double* theta,
                                 int32_t* d_next, int32_t* b_next, double* phi, void* workspace,
                                 size_t workspace_bytes) {
  if (R < 0 || gamma_max < 0) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA) return SD_EUNSUPPORTED;
  if ((long long)R * gamma_max > SD_MAX_SCHED_SLOTS) return SD_EUNSUPPORTED;
  if (R == 0 || gamma_max == 0) return SD_OK;
  if (!ema || !count || !sps || !draft_cost || !ell || !d_next || !b_next) return SD_EINVAL;
  if ((long long)sps_len < (long long)R * (1 + gamma_max)) return SD_ERANGE;
  if (!workspace || workspace_bytes < plan_ws_bytes(R, gamma_max)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  float* rows = (float*)workspace;
  char* sched_ws = (char*)workspace + sdv_align256((size_t)R * gamma_max * sizeof(float));
  SDV_TRY_LAUNCH(sdv::launch(k_ls_conf, dim3(1), dim3(kThreads), 0, stream, R, gamma_max, ema, count,
                             conf_hat, rows));
  const int rc = sd_schedule(stream, R, gamma_max, d_prev, rows, nullptr, sps, sps_len,
                             SD_SCHED_GLOBAL_ARGMAX, nullptr, 0.0f, ell, batch, n_sel, theta, nullptr,
                             sched_ws, sd_schedule_workspace_size(R, gamma_max));
  if (rc != SD_OK) return rc;
  SDV_TRY_LAUNCH(sdv::launch(k_ls_draft, dim3(1), dim3(kDraftThreads), 0, stream, R, gamma_max,
                             (const float*)rows, sps, draft_cost, phi, d_next, b_next));
  return SD_OK;
}
