// sd_verify: lossless rejection-sampling verification over full vocabulary rows.
//
// Speculative-decoding history page, "1.1 mechanism": the target scores every
// drafted position in one pass, draft x is accepted outright when p(x) >= q(x)
// and otherwise with probability p(x)/q(x), everything after the first
// rejection is discarded and the target supplies one more token; the output
// law is exactly the target's.  The replacement law max(0, p - q) normalised
// is the one that losslessness forces; after a fully accepted block the extra
// token comes from the target row past the last draft (the verify batch holds
// 1 + l_r target rows per request, DSpark summary "2.2").
//
// Kernels (one stream, no host synchronisation):
//   k_row_partials    the bandwidth pass: every needed target and draft row is
//                     streamed once with 16-byte loads; each wave leaves a
//                     partial (max, sum 2^(x*c - ref)) per 16384-element chunk
//   k_accept          one workgroup per request: combine partials into (m, Z),
//                     run the accept tests for all positions at once, find the
//                     first rejection, write accepted tokens, plan the draw
//   k_residual_sums   per (request, chunk): sum of max(0, p - q) over the
//                     rejected position's row pair (skipped for bonus draws)
//   k_sample          one workgroup per request: locate the chunk where the
//                     inverse CDF crosses u * sum(w), rescan that chunk only
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kChunk = 16384;                 // elements per work item
constexpr float kNegInf = -__builtin_huge_valf();

struct Plan {
  int kind;        // 0: nothing to draw (failed request), 1: residual, 2: bonus / from p
  int n_acc;
  int st;          // status bits so far
  int tslot;       // target slot of the draw
  int64_t trow;    // target row index
  int64_t drow;    // draft row index (kind 1)
  float mct, mcd;  // exponent references of the two rows (fp32(max * c))
  double zt, zd;   // sums of 2^(x*c - ref) of the two rows
  double u;        // correction uniform
};

// 16-byte vector of logits -> floats.  bf16: 8 values, fp32: 4 values.
template <bool BF16>
struct Vec;
template <>
struct Vec<true> {
  static constexpr int kElems = 8;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  __device__ __forceinline__ static void unpack(const uint4& v, float* x) {
    x[0] = sdv::bf16lo(v.x); x[1] = sdv::bf16hi(v.x);
    x[2] = sdv::bf16lo(v.y); x[3] = sdv::bf16hi(v.y);
    x[4] = sdv::bf16lo(v.z); x[5] = sdv::bf16hi(v.z);
    x[6] = sdv::bf16lo(v.w); x[7] = sdv::bf16hi(v.w);
  }
  __device__ __forceinline__ static float at(const char* row, int v) {
    return sdv::bf16_to_f32(((const uint16_t*)row)[v]);
  }
};
template <>
struct Vec<false> {
  static constexpr int kElems = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  __device__ __forceinline__ static void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static float at(const char* row, int v) {
    return ((const float*)row)[v];
  }
};

// Reference exponent for a max m: fp32(m * c); 0 when nothing finite was seen
// (then every contribution is 2^-inf = 0, or NaN if a NaN was present).
__device__ __forceinline__ float exp_ref(float m, float c) { return m == kNegInf ? 0.0f : m * c; }

// slot -> row pointer for request r, or nullptr if the slot is outside the batch.
__device__ __forceinline__ const char* slot_row(int slot, int r, int L, int gmax, const char* tgt,
                                                const int32_t* tgt_row0, const char* drf,
                                                const int32_t* drf_row0, int64_t ld_bytes,
                                                int64_t* row_index) {
  if (slot <= gmax) {
    if (slot > L) return nullptr;
    const int64_t row = (int64_t)tgt_row0[r] + slot;
    if (row_index) *row_index = row;
    return tgt + row * ld_bytes;
  }
  const int j = slot - gmax;
  if (j > L) return nullptr;
  const int64_t row = (int64_t)drf_row0[r] + (j - 1);
  if (row_index) *row_index = row;
  return drf + row * ld_bytes;
}

// ---------------------------------------------------------------------------
// The bandwidth pass.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_row_partials(
    const char* __restrict__ tgt, const int32_t* __restrict__ tgt_row0,
    const char* __restrict__ drf, const int32_t* __restrict__ drf_row0,
    const int32_t* __restrict__ ell, int gmax, int V, int64_t ld_bytes, float c, int n_ch,
    float2* __restrict__ partial) {
  using VT = Vec<BF16>;
  constexpr int kVecPerThread = kChunk / VT::kElems / kThreads;
  const int item = blockIdx.x;
  const int S = 2 * gmax + 1;
  const int ch = item % n_ch;
  const int rs = item / n_ch;
  const int slot = rs % S, r = rs / S;
  const int L = sdv::clampi(ell[r], 0, gmax);
  const char* row = slot_row(slot, r, L, gmax, tgt, tgt_row0, drf, drf_row0, ld_bytes, nullptr);
  if (!row) return;

  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, V - e0) / VT::kElems;
  const uint4* p = (const uint4*)(row + (int64_t)e0 * (BF16 ? 2 : 4));
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);

  uint4 buf[kVecPerThread];
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    const int v = threadIdx.x + k * kThreads;
    buf[k] = v < nvec ? sdv::ld_nt(p + v) : ninf;
  }
  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    float x[VT::kElems];
    VT::unpack(buf[k], x);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) m = fmaxf(m, x[e]);
  }
  const float ref = exp_ref(m, c);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    float x[VT::kElems];
    VT::unpack(buf[k], x);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) s += sdv::fast_exp2(fmaf(x[e], c, -ref));
  }
  // wave partial: rescale every lane to the wave max
  const float wm = sdv::wave_max(m);
  const float wref = exp_ref(wm, c);
  const float contrib = (s == 0.0f) ? 0.0f : s * sdv::fast_exp2(ref - wref);
  const float ws = sdv::wave_sum(contrib);
  if ((threadIdx.x & 63) == 0) {
    const int wave = threadIdx.x >> 6;
    partial[((size_t)rs * n_ch + ch) * kWavesPerBlock + wave] = make_float2(wm, ws);
  }
}

// Combine the partials of one row: M = max, ref = fp32(M * c),
// Z = sum s_w 2^(ref_w - ref) in fp64.
__device__ void combine_row(const float2* __restrict__ pp, int nparts, float c, float* M_out,
                            float* ref_out, double* Z_out) {
  float M = kNegInf;
  for (int q = 0; q < nparts; ++q) M = fmaxf(M, pp[q].x);
  const float ref = exp_ref(M, c);
  double Z = 0.0;
  for (int q = 0; q < nparts; ++q) {
    const float s = pp[q].y;
    if (s != 0.0f) Z += (double)s * exp2((double)exp_ref(pp[q].x, c) - (double)ref);
  }
  *M_out = M;
  *ref_out = ref;
  *Z_out = Z;
}

__device__ __forceinline__ int row_status(float M, double Z) {
  if (isnan(M) || isnan(Z) || M == __builtin_huge_valf()) return SD_ST_NONFINITE;
  if (M == kNegInf) return SD_ST_ZERO_Z;
  return 0;
}

// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_accept(
    int gmax, int V, int64_t ld_bytes, float c, float inv_t, uint64_t seed,
    const int64_t* __restrict__ pos0, const char* __restrict__ tgt,
    const int32_t* __restrict__ tgt_row0, const char* __restrict__ drf,
    const int32_t* __restrict__ drf_row0, const int32_t* __restrict__ draft_tokens,
    const int32_t* __restrict__ ell, int n_ch, const float2* __restrict__ partial,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ status, float* __restrict__ probe_probs, float* __restrict__ row_stats,
    Plan* __restrict__ plans) {
  using VT = Vec<BF16>;
  __shared__ float sM[2 * SD_MAX_GAMMA + 1];
  __shared__ float sRef[2 * SD_MAX_GAMMA + 1];
  __shared__ double sZ[2 * SD_MAX_GAMMA + 1];
  __shared__ int s_st, s_jstar, s_zero_q_upto;

  const int r = blockIdx.x, tid = threadIdx.x;
  const int S = 2 * gmax + 1;
  const int L = sdv::clampi(ell[r], 0, gmax);
  const int nparts = n_ch * kWavesPerBlock;
  if (tid == 0) { s_st = 0; s_jstar = L + 1; s_zero_q_upto = 0x7FFFFFFF; }
  __syncthreads();

  for (int slot = tid; slot < S; slot += kThreads) {
    const bool in_batch = slot <= gmax ? slot <= L : slot - gmax <= L;
    if (!in_batch) continue;
    float M, ref;
    double Z;
    combine_row(partial + (size_t)(r * S + slot) * nparts, nparts, c, &M, &ref, &Z);
    sM[slot] = M;
    sRef[slot] = ref;
    sZ[slot] = Z;
    const int st = row_status(M, Z);
    if (st) atomicOr(&s_st, st);
    if (row_stats) {
      // report m = max(x)/T and Z = sum exp(x/T - m): shift Z from the fp32
      // reference to the exact one.
      const double zrep = Z * exp2((double)ref - (double)M * (double)c);
      row_stats[((size_t)r * S + slot) * 2 + 0] = M * inv_t;
      row_stats[((size_t)r * S + slot) * 2 + 1] = (float)zrep;
    }
  }
  __syncthreads();

  const int64_t pbase = pos0 ? pos0[r] : 0;
  Plan* plan = plans + r;
  if (s_st) {  // a needed row is unusable: the request fails
    for (int t = tid; t <= gmax; t += kThreads) out_tokens[(size_t)r * (gmax + 1) + t] = -1;
    if (tid == 0) {
      n_accepted[r] = 0;
      status[r] = s_st;
      plan->kind = 0;
    }
    return;
  }

  // all accept tests in parallel; the chain stops at the first rejection
  for (int j = tid + 1; j <= L; j += kThreads) {
    const int x = draft_tokens[(size_t)r * gmax + (j - 1)];
    bool reject;
    if (x < 0 || x >= V) {
      reject = true;
    } else {
      const char* trow = tgt + ((int64_t)tgt_row0[r] + (j - 1)) * ld_bytes;
      const char* drow = drf + ((int64_t)drf_row0[r] + (j - 1)) * ld_bytes;
      const int ts = j - 1, ds = gmax + j;
      const double p = exp2((double)VT::at(trow, x) * (double)c - (double)sRef[ts]) / sZ[ts];
      const double q = exp2((double)VT::at(drow, x) * (double)c - (double)sRef[ds]) / sZ[ds];
      if (probe_probs) {
        probe_probs[((size_t)r * gmax + (j - 1)) * 2 + 0] = (float)p;
        probe_probs[((size_t)r * gmax + (j - 1)) * 2 + 1] = (float)q;
      }
      const double u = sdv::uniform24(seed, (uint64_t)r, (uint64_t)(pbase + j), 1);
      if (q == 0.0) {
        atomicMin(&s_zero_q_upto, j);
        reject = !(p > 0.0);
      } else {
        reject = !(u * q < p);
      }
    }
    if (reject) atomicMin(&s_jstar, j);
  }
  __syncthreads();

  const int jstar = s_jstar;
  const bool rejected = jstar <= L;
  const int n = rejected ? jstar - 1 : L;
  for (int t = tid; t <= gmax; t += kThreads) {
    int v = -1;
    if (t < n) v = draft_tokens[(size_t)r * gmax + t];
    out_tokens[(size_t)r * (gmax + 1) + t] = v;
  }
  if (tid == 0) {
    int st = 0;
    if (s_zero_q_upto <= (rejected ? jstar : L)) st |= SD_ST_ZERO_Q;
    if (rejected) {
      const int x = draft_tokens[(size_t)r * gmax + (jstar - 1)];
      if (x < 0 || x >= V) st |= SD_ST_BAD_TOKEN;
    }
    n_accepted[r] = n;
    status[r] = st;
    Plan pl;
    pl.n_acc = n;
    pl.st = st;
    const int pos = rejected ? jstar : L + 1;
    pl.u = sdv::uniform24(seed, (uint64_t)r, (uint64_t)(pbase + pos), 2);
    pl.tslot = pos - 1;
    pl.trow = (int64_t)tgt_row0[r] + (pos - 1);
    pl.mct = sRef[pos - 1];
    pl.zt = sZ[pos - 1];
    if (rejected) {
      pl.kind = 1;
      pl.drow = (int64_t)drf_row0[r] + (jstar - 1);
      pl.mcd = sRef[gmax + jstar];
      pl.zd = sZ[gmax + jstar];
    } else {
      pl.kind = 2;
      pl.drow = -1;
      pl.mcd = 0.0f;
      pl.zd = 1.0;
    }
    *plan = pl;
  }
}

// ---------------------------------------------------------------------------
// Residual weights w = max(0, p - q), in fp64 from fp32 exponentials.  Thread t
// always owns the same elements of a chunk (vectors t, t + 256, ...), summed in
// the same order, so k_sample can rescan one chunk consistently.
template <bool BF16>
__device__ __forceinline__ double thread_chunk_weights(const char* trow, const char* drow,
                                                       int e0, int nvec, float c, float mct,
                                                       double izt, float mcd, double izd,
                                                       int kind, double* w_out) {
  using VT = Vec<BF16>;
  constexpr int kVecPerThread = kChunk / VT::kElems / kThreads;
  const uint4* tp = (const uint4*)(trow + (int64_t)e0 * (BF16 ? 2 : 4));
  const uint4* dp = drow ? (const uint4*)(drow + (int64_t)e0 * (BF16 ? 2 : 4)) : nullptr;
  double sum = 0.0;
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    const int v = threadIdx.x + k * kThreads;
    if (v < nvec) {
      float xt[VT::kElems], xd[VT::kElems];
      VT::unpack(tp[v], xt);
      if (kind == 1) VT::unpack(dp[v], xd);
#pragma unroll
      for (int e = 0; e < VT::kElems; ++e) {
        double w;
        const double et = (double)sdv::fast_exp2(fmaf(xt[e], c, -mct));
        if (kind == 1) {
          const double ed = (double)sdv::fast_exp2(fmaf(xd[e], c, -mcd));
          w = fmax(0.0, et * izt - ed * izd);
        } else {
          w = et;
        }
        if (w_out) w_out[k * VT::kElems + e] = w;
        sum += w;
      }
    } else if (w_out) {
#pragma unroll
      for (int e = 0; e < VT::kElems; ++e) w_out[k * VT::kElems + e] = 0.0;
    }
  }
  return sum;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_residual_sums(
    const char* __restrict__ tgt, const char* __restrict__ drf, int V, int64_t ld_bytes, float c,
    int n_ch, const Plan* __restrict__ plans, double* __restrict__ rsum) {
  using VT = Vec<BF16>;
  const int r = blockIdx.x / n_ch, ch = blockIdx.x % n_ch;
  const Plan pl = plans[r];
  if (pl.kind != 1) return;
  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, V - e0) / VT::kElems;
  const double s = thread_chunk_weights<BF16>(tgt + pl.trow * ld_bytes, drf + pl.drow * ld_bytes,
                                              e0, nvec, c, pl.mct, 1.0 / pl.zt, pl.mcd,
                                              1.0 / pl.zd, 1, nullptr);
  __shared__ double ws[kWavesPerBlock];
  const double t = sdv::wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < kWavesPerBlock; ++w) tot += ws[w];
    rsum[(size_t)r * n_ch + ch] = tot;
  }
}

// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_sample(
    const char* __restrict__ tgt, const char* __restrict__ drf, int gmax, int V, int64_t ld_bytes,
    float c, int n_ch, const float2* __restrict__ partial, const Plan* __restrict__ plans,
    const double* __restrict__ rsum, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ status) {
  using VT = Vec<BF16>;
  constexpr int kVecPerThread = kChunk / VT::kElems / kThreads;
  constexpr int kPerThread = kVecPerThread * VT::kElems;
  __shared__ double s_chunk[SD_MAX_VOCAB / kChunk];
  __shared__ int s_ch, s_last_pos;
  __shared__ double s_target;

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Plan pl = plans[r];
  if (pl.kind == 0) return;
  const int S = 2 * gmax + 1;
  int kind = pl.kind;
  int st = pl.st;

  // chunk sums of the weights
  if (kind == 1) {
    for (int ch = tid; ch < n_ch; ch += kThreads) s_chunk[ch] = rsum[(size_t)r * n_ch + ch];
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int ch = 0; ch < n_ch; ++ch) tot += s_chunk[ch];
      s_target = tot;
    }
    __syncthreads();
    if (!(s_target > 0.0)) {  // empty residual: draw from p instead
      kind = 2;
      st |= SD_ST_ZERO_RESIDUAL;
    }
    __syncthreads();
  }
  if (kind == 2) {
    // sum over chunk ch of 2^(x*c - mct), from the first pass's wave partials
    const float2* pp = partial + (size_t)(r * S + pl.tslot) * n_ch * kWavesPerBlock;
    for (int ch = tid; ch < n_ch; ch += kThreads) {
      double s = 0.0;
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const float2 q = pp[ch * kWavesPerBlock + w];
        if (q.y != 0.0f) s += (double)q.y * exp2((double)exp_ref(q.x, c) - (double)pl.mct);
      }
      s_chunk[ch] = s;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int ch = 0; ch < n_ch; ++ch) tot += s_chunk[ch];
    const double target = pl.u * tot;
    double base = 0.0;
    int found = -1, last_pos = -1;
    for (int ch = 0; ch < n_ch; ++ch) {
      if (s_chunk[ch] > 0.0) last_pos = ch;
      if (found < 0 && base + s_chunk[ch] > target) found = ch;
      if (found < 0) base += s_chunk[ch];
    }
    if (found < 0) {  // rounding put the target past the end: take the last mass
      found = last_pos;
      s_target = __builtin_huge_val();
    } else {
      s_target = target - base;
    }
    s_ch = found;
    s_last_pos = -1;
  }
  __syncthreads();
  const int ch = s_ch;
  const double target = s_target;
  if (ch < 0) {  // no mass anywhere (cannot happen for a finite row)
    if (tid == 0) {
      out_tokens[(size_t)r * (gmax + 1) + pl.n_acc] = -1;
      status[r] = st;
    }
    return;
  }

  // Rescan the located chunk.  Vocabulary order inside a chunk is
  // (vector column k, thread, element): thread t owns vectors t, t+256, ...,
  // so the cumulative sum is built column by column.
  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, V - e0) / VT::kElems;
  double w[kPerThread];
  const char* trow = tgt + pl.trow * ld_bytes;
  const char* drow = kind == 1 ? drf + pl.drow * ld_bytes : nullptr;
  thread_chunk_weights<BF16>(trow, drow, e0, nvec, c, pl.mct, 1.0 / pl.zt, pl.mcd, 1.0 / pl.zd,
                             kind, w);
  __shared__ double s_col_tot[kWavesPerBlock];
  __shared__ int s_found;
  int last = -1;
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k)
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e)
      if (w[k * VT::kElems + e] > 0.0) last = e0 + (tid + k * kThreads) * VT::kElems + e;
  if (tid == 0) s_found = 0x7FFFFFFF;
  __syncthreads();
  double run = 0.0;  // mass of all earlier columns
  for (int k = 0; k < kVecPerThread; ++k) {
    double vs = 0.0;
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) vs += w[k * VT::kElems + e];
    const double vincl = sdv::wave_incl_scan_d(vs, lane);
    if (lane == 63) s_col_tot[wave] = vincl;
    __syncthreads();
    double vexcl = vincl - vs;
    double coltot = 0.0;
    for (int ww = 0; ww < kWavesPerBlock; ++ww) {
      if (ww < wave) vexcl += s_col_tot[ww];
      coltot += s_col_tot[ww];
    }
    const double c0 = run + vexcl;
    if (c0 <= target && c0 + vs > target) {
      double cc = c0;
      for (int e = 0; e < VT::kElems; ++e) {
        cc += w[k * VT::kElems + e];
        if (cc > target) {
          atomicMin(&s_found, e0 + (tid + k * kThreads) * VT::kElems + e);
          break;
        }
      }
    }
    run += coltot;
    __syncthreads();
  }
  if (last >= 0) atomicMax(&s_last_pos, last);
  __syncthreads();
  if (tid == 0) {
    int token = s_found;
    if (token == 0x7FFFFFFF) token = s_last_pos;  // rounding: last element with mass
    out_tokens[(size_t)r * (gmax + 1) + pl.n_acc] = token;
    status[r] = st;
  }
}

template <bool BF16>
int run_verify(hipStream_t stream, int R, int gmax, int V, int ld, float temperature,
               uint64_t seed, const int64_t* pos0, const void* tgt, const int32_t* tgt_row0,
               const void* drf, const int32_t* drf_row0, const int32_t* draft_tokens,
               const int32_t* ell, int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
               float* probe_probs, float* row_stats, void* ws, hipEvent_t ev0, hipEvent_t ev1) {
  const int n_ch = (V + kChunk - 1) / kChunk;
  const int S = 2 * gmax + 1;
  const int64_t ld_bytes = (int64_t)ld * (BF16 ? 2 : 4);
  const float c = sdv::kLog2e / temperature;
  const float inv_t = 1.0f / temperature;
  char* p = (char*)ws;
  float2* partial = (float2*)p;
  p += sdv_align256((size_t)R * S * n_ch * kWavesPerBlock * sizeof(float2));
  Plan* plans = (Plan*)p;
  p += sdv_align256((size_t)R * sizeof(Plan));
  double* rsum = (double*)p;

  const long long items = (long long)R * S * n_ch;
  const bool timed = ev0 && ev1;
  if (timed) SDV_TRY_LAUNCH(hipEventRecord(ev0, stream));
  SDV_TRY_LAUNCH(sdv::launch(k_row_partials<BF16>, dim3((unsigned)items), dim3(kThreads), 0,
                             stream, (const char*)tgt, tgt_row0, (const char*)drf, drf_row0, ell,
                             gmax, V, ld_bytes, c, n_ch, partial));
  if (timed) SDV_TRY_LAUNCH(hipEventRecord(ev1, stream));
  SDV_TRY_LAUNCH(sdv::launch(k_accept<BF16>, dim3(R), dim3(kThreads), 0, stream, gmax, V,
                             ld_bytes, c, inv_t, seed, pos0, (const char*)tgt, tgt_row0,
                             (const char*)drf, drf_row0, draft_tokens, ell, n_ch,
                             (const float2*)partial, n_accepted, out_tokens, status, probe_probs,
                             row_stats, plans));
  SDV_TRY_LAUNCH(sdv::launch(k_residual_sums<BF16>, dim3((unsigned)(R * n_ch)), dim3(kThreads),
                             0, stream, (const char*)tgt, (const char*)drf, V, ld_bytes, c, n_ch,
                             (const Plan*)plans, rsum));
  SDV_TRY_LAUNCH(sdv::launch(k_sample<BF16>, dim3(R), dim3(kThreads), 0, stream,
                             (const char*)tgt, (const char*)drf, gmax, V, ld_bytes, c, n_ch,
                             (const float2*)partial, (const Plan*)plans, (const double*)rsum,
                             out_tokens, status));
  return SD_OK;
}

size_t verify_ws_bytes(int R, int gmax, int V) {
  const size_t n_ch = ((size_t)V + kChunk - 1) / kChunk;
  const size_t S = 2 * (size_t)gmax + 1;
  return sdv_align256((size_t)R * S * n_ch * kWavesPerBlock * sizeof(float2)) +
         sdv_align256((size_t)R * sizeof(Plan)) + sdv_align256((size_t)R * n_ch * sizeof(double));
}

}  // namespace

extern "C" size_t sd_verify_workspace_size(int R, int gamma_max, int V) {
  if (R < 0 || gamma_max < 0 || V <= 0) return 0;
  return verify_ws_bytes(R, gamma_max, V);
}

extern "C" int sd_verify(hipStream_t stream, int R, int gamma_max, int V, int ld, int dtype,
                         float temperature, uint64_t seed, const int64_t* pos0,
                         const void* tgt_logits, const int32_t* tgt_row0, const void* drf_logits,
                         const int32_t* drf_row0, const int32_t* draft_tokens,
                         const int32_t* ell, int32_t* n_accepted, int32_t* out_tokens,
                         int32_t* status, float* probe_probs, float* row_stats, void* workspace,
                         size_t workspace_bytes, hipEvent_t prof_start, hipEvent_t prof_stop) {
  if (R < 0 || gamma_max < 0 || V < 8 || (V % 8) != 0 || ld < V || (ld % 8) != 0) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA || V > SD_MAX_VOCAB) return SD_EUNSUPPORTED;
  if (dtype != SD_DTYPE_F32 && dtype != SD_DTYPE_BF16) return SD_EINVAL;
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf())) return SD_EINVAL;
  if (R == 0) return SD_OK;
  if (!tgt_logits || !tgt_row0 || !drf_row0 || !ell || !n_accepted || !out_tokens || !status)
    return SD_EINVAL;
  if (gamma_max > 0 && (!drf_logits || !draft_tokens)) return SD_EINVAL;
  if (!workspace || workspace_bytes < verify_ws_bytes(R, gamma_max, V)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  if ((((uintptr_t)tgt_logits) & 15) != 0 || (drf_logits && (((uintptr_t)drf_logits) & 15) != 0))
    return SD_EINVAL;
  const long long items = (long long)R * (2 * gamma_max + 1) * ((V + kChunk - 1) / kChunk);
  if (items > 0x7FFFFFFFLL) return SD_EUNSUPPORTED;
  if (dtype == SD_DTYPE_BF16)
    return run_verify<true>(stream, R, gamma_max, V, ld, temperature, seed, pos0, tgt_logits,
                            tgt_row0, drf_logits, drf_row0, draft_tokens, ell, n_accepted,
                            out_tokens, status, probe_probs, row_stats, workspace, prof_start,
                            prof_stop);
  return run_verify<false>(stream, R, gamma_max, V, ld, temperature, seed, pos0, tgt_logits,
                           tgt_row0, drf_logits, drf_row0, draft_tokens, ell, n_accepted,
                           out_tokens, status, probe_probs, row_stats, workspace, prof_start,
                           prof_stop);
}
