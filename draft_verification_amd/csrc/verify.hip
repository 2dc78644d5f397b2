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
//                     streamed once with 16-byte non-temporal loads; each wave
//                     leaves a partial (max, sum 2^(x*c - ref)) per
//                     16384-element chunk.  No LDS, no barrier.
//   k_accept          one workgroup per request: combine the partials into
//                     (m, Z) per row, run every accept test at once, find the
//                     first rejection, write the accepted tokens, plan the draw
//   k_residual_sums   per (request, chunk) of a rejected request: sums of
//                     max(0, p - q) over the rejected position's row pair
//   k_sample          one workgroup per request: locate the chunk where the
//                     inverse CDF crosses u * sum(w) (bonus draws take their
//                     chunk sums straight from the first pass), rescan it
//   k_alpha_sums      only when the acceptance rates are asked for: per
//                     (request, position, chunk), sums of min(p, q) - the
//                     probability that the position is accepted, which is
//                     1 - TV(p, q), the confidence label of the DSpark summary
//                     ("2.1"); k_sample finishes the per-row totals
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 16384;  // elements per work item
constexpr int kMaxChunks = SD_MAX_VOCAB / kChunk;
constexpr int kMaxSlots = 2 * SD_MAX_GAMMA + 1;
constexpr int kStagedParts = 4096;  // partials of one request staged in LDS
constexpr float kNegInf = -__builtin_huge_valf();

struct Plan {
  int kind;        // 0: nothing to draw (failed request), 1: residual, 2: from p
  int n_acc;
  int st;          // status bits so far
  int tslot;       // target slot of the draw
  int64_t trow;    // target row index
  int64_t drow;    // draft row index (kind 1)
  float mct, mcd;  // exponent references of the two rows (fp32(max * c))
  double zt, zd;   // sums of 2^(x*c - ref) of the two rows
  double u;        // correction uniform
};

struct VerifyArgs {
  const char* tgt;
  const int32_t* tgt_row0;
  const char* drf;
  const int32_t* drf_row0;
  const int32_t* draft_tokens;
  const int32_t* ell;
  const int64_t* pos0;
  int32_t* n_accepted;
  int32_t* out_tokens;
  int32_t* status;
  float* probe_probs;
  float* row_stats;
  float* accept_prob;  // [R][gmax] or null
  float2* partial;  // [R][S][n_ch][kWaves]
  float* row_ref;   // [R][S] fp32(max * c) of every batch row
  double* row_z;    // [R][S] sum 2^(x*c - ref)
  double* asum;     // [R][gmax][n_ch][kWaves] chunk sums of min(p, q)
  Plan* plans;      // [R]
  double* rsum;     // [R][n_ch][kWaves]
  int64_t ld_bytes;
  uint64_t seed;
  float c;          // log2(e) / T
  float inv_t;
  int gmax;
  int V;
  int n_ch;
};

// 16-byte vector of logits -> floats.  bf16: 8 values, fp32: 4 values.
template <bool BF16>
struct Vec;
template <>
struct Vec<true> {
  static constexpr int kElems = 8;
  static constexpr int kBytes = 2;
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
  static constexpr int kBytes = 4;
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

__device__ __forceinline__ int row_status(float M, double Z) {
  if (isnan(M) || isnan(Z) || M == __builtin_huge_valf()) return SD_ST_NONFINITE;
  if (M == kNegInf) return SD_ST_ZERO_Z;
  return 0;
}

__device__ __forceinline__ bool slot_in_batch(int slot, int gmax, int L) {
  return slot <= gmax ? slot <= L : slot - gmax <= L;
}

// ---------------------------------------------------------------------------
// The bandwidth pass.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_row_partials(VerifyArgs a) {
  using VT = Vec<BF16>;
  constexpr int kVec = kChunk / VT::kElems / kThreads;
  const int item = blockIdx.x;
  const int S = 2 * a.gmax + 1;
  const int ch = item % a.n_ch;
  const int rs = item / a.n_ch;
  const int slot = rs % S, r = rs / S;
  const int L = sdv::clampi(a.ell[r], 0, a.gmax);
  if (!slot_in_batch(slot, a.gmax, L)) return;
  const char* row = slot <= a.gmax
                        ? a.tgt + ((int64_t)a.tgt_row0[r] + slot) * a.ld_bytes
                        : a.drf + ((int64_t)a.drf_row0[r] + (slot - a.gmax - 1)) * a.ld_bytes;
  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, a.V - e0) / VT::kElems;
  const uint4* p = (const uint4*)(row + (int64_t)e0 * VT::kBytes);
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  const float c = a.c;

  uint4 buf[kVec];
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    const int v = threadIdx.x + k * kThreads;
    buf[k] = v < nvec ? sdv::ld_nt(p + v) : ninf;
  }
  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    float x[VT::kElems];
    VT::unpack(buf[k], x);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) m = fmaxf(m, x[e]);
  }
  const float ref = exp_ref(m, c);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    float x[VT::kElems];
    VT::unpack(buf[k], x);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) s += sdv::fast_exp2(fmaf(x[e], c, -ref));
  }
  // wave partial: rescale every lane to the wave max
  const float wm = sdv::wave_max(m);
  const float wref = exp_ref(wm, c);
  const float ws = sdv::wave_sum((s == 0.0f) ? 0.0f : s * sdv::fast_exp2(ref - wref));
  if ((threadIdx.x & 63) == 0)
    a.partial[((size_t)rs * a.n_ch + ch) * kWaves + (threadIdx.x >> 6)] = make_float2(wm, ws);
}

// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_accept(VerifyArgs a) {
  using VT = Vec<BF16>;
  __shared__ float sM[kMaxSlots];
  __shared__ float sRef[kMaxSlots];
  __shared__ double sZ[kMaxSlots];
  __shared__ float2 sPart[kStagedParts];
  __shared__ int s_st, s_jstar, s_zero_q_upto;

  const int r = blockIdx.x, tid = threadIdx.x;
  const int gmax = a.gmax, S = 2 * gmax + 1, V = a.V;
  const int L = sdv::clampi(a.ell[r], 0, gmax);
  const int nparts = a.n_ch * kWaves;
  const float c = a.c;
  if (tid == 0) { s_st = 0; s_jstar = L + 1; s_zero_q_upto = 0x7FFFFFFF; }

  // Stage the partials of the batch rows (target slots 0..L, then draft slots
  // gmax+1..gmax+L, i.e. local row b) in LDS when they fit: one load each.
  const int nrows = 2 * L + 1;
  const bool staged = (long long)nrows * nparts <= kStagedParts;
  const float2* base = a.partial + (size_t)r * S * nparts;
  if (staged) {
    for (int i = tid; i < nrows * nparts; i += kThreads) {
      const int b = i / nparts, q = i % nparts;
      const int slot = b <= L ? b : gmax + (b - L);
      sPart[i] = base[(size_t)slot * nparts + q];
    }
  }
  __syncthreads();

  // (m, Z) per row: 16 groups of 16 lanes, one row per group at a time
  const int grp = tid >> 4, gl = tid & 15;
  for (int b = grp; b < nrows; b += kThreads / 16) {
    const int slot = b <= L ? b : gmax + (b - L);
    const float2* pp = staged ? sPart + b * nparts : base + (size_t)slot * nparts;
    float M = kNegInf;
    for (int q = gl; q < nparts; q += 16) M = fmaxf(M, pp[q].x);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
    const float ref = exp_ref(M, c);
    double Z = 0.0;
    for (int q = gl; q < nparts; q += 16) {
      const float2 v = pp[q];
      if (v.y != 0.0f) Z += (double)v.y * (double)sdv::fast_exp2(exp_ref(v.x, c) - ref);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) Z += __shfl_xor(Z, o, 16);
    if (gl == 0) {
      sM[slot] = M;
      sRef[slot] = ref;
      sZ[slot] = Z;
      a.row_ref[(size_t)r * S + slot] = ref;
      a.row_z[(size_t)r * S + slot] = Z;
      const int st = row_status(M, Z);
      if (st) atomicOr(&s_st, st);
      if (a.row_stats) {
        // report m = max(x)/T and Z = sum exp(x/T - m): move Z from the fp32
        // reference to the exact one
        const double zrep = Z * exp2((double)ref - (double)M * (double)c);
        a.row_stats[((size_t)r * S + slot) * 2 + 0] = M * a.inv_t;
        a.row_stats[((size_t)r * S + slot) * 2 + 1] = (float)zrep;
      }
    }
  }
  __syncthreads();

  Plan* plan = a.plans + r;
  int32_t* out_tok = a.out_tokens + (size_t)r * (gmax + 1);
  if (s_st) {  // a needed row is unusable: the request fails
    for (int t = tid; t <= gmax; t += kThreads) out_tok[t] = -1;
    if (tid == 0) {
      a.n_accepted[r] = 0;
      a.status[r] = s_st;
      plan->kind = 0;
    }
    return;
  }

  // every accept test at once; the chain stops at the first rejection
  const int64_t pbase = a.pos0 ? a.pos0[r] : 0;
  const int32_t* drafts = a.draft_tokens + (size_t)r * gmax;
  for (int j = tid + 1; j <= L; j += kThreads) {
    const int x = drafts[j - 1];
    bool reject;
    if (x < 0 || x >= V) {
      reject = true;
    } else {
      const char* trow = a.tgt + ((int64_t)a.tgt_row0[r] + (j - 1)) * a.ld_bytes;
      const char* drow = a.drf + ((int64_t)a.drf_row0[r] + (j - 1)) * a.ld_bytes;
      const int ts = j - 1, ds = gmax + j;
      const double p = exp2((double)VT::at(trow, x) * (double)c - (double)sRef[ts]) / sZ[ts];
      const double q = exp2((double)VT::at(drow, x) * (double)c - (double)sRef[ds]) / sZ[ds];
      if (a.probe_probs) {
        a.probe_probs[((size_t)r * gmax + (j - 1)) * 2 + 0] = (float)p;
        a.probe_probs[((size_t)r * gmax + (j - 1)) * 2 + 1] = (float)q;
      }
      const double u = sdv::uniform24(a.seed, (uint64_t)r, (uint64_t)(pbase + j), 1);
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
  for (int t = tid; t <= gmax; t += kThreads) out_tok[t] = (t < n) ? drafts[t] : -1;
  if (tid == 0) {
    int st = 0;
    if (s_zero_q_upto <= (rejected ? jstar : L)) st |= SD_ST_ZERO_Q;
    if (rejected) {
      const int x = drafts[jstar - 1];
      if (x < 0 || x >= V) st |= SD_ST_BAD_TOKEN;
    }
    a.n_accepted[r] = n;
    a.status[r] = st;
    Plan pl;
    pl.n_acc = n;
    pl.st = st;
    const int pos = rejected ? jstar : L + 1;
    pl.u = sdv::uniform24(a.seed, (uint64_t)r, (uint64_t)(pbase + pos), 2);
    pl.tslot = pos - 1;
    pl.trow = (int64_t)a.tgt_row0[r] + (pos - 1);
    pl.mct = sRef[pos - 1];
    pl.zt = sZ[pos - 1];
    if (rejected) {
      pl.kind = 1;
      pl.drow = (int64_t)a.drf_row0[r] + (jstar - 1);
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
// Weight of element e of the correction draw: residual max(0, p - q)
// (kind 1) or the unnormalised target law 2^(x*c - ref) (kind 2); fp64 from
// fp32 exponentials.
__device__ __forceinline__ double draw_weight(float xt, float xd, int kind, float c, float mct,
                                              double izt, float mcd, double izd) {
  const double et = (double)sdv::fast_exp2(fmaf(xt, c, -mct));
  if (kind != 1) return et;
  const double ed = (double)sdv::fast_exp2(fmaf(xd, c, -mcd));
  return fmax(0.0, et * izt - ed * izd);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_residual_sums(VerifyArgs a) {
  using VT = Vec<BF16>;
  constexpr int kVec = kChunk / VT::kElems / kThreads;
  const int r = blockIdx.x / a.n_ch, ch = blockIdx.x % a.n_ch;
  const Plan pl = a.plans[r];
  if (pl.kind != 1) return;
  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, a.V - e0) / VT::kElems;
  const uint4* tp = (const uint4*)(a.tgt + pl.trow * a.ld_bytes + (int64_t)e0 * VT::kBytes);
  const uint4* dp = (const uint4*)(a.drf + pl.drow * a.ld_bytes + (int64_t)e0 * VT::kBytes);
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  const double izt = 1.0 / pl.zt, izd = 1.0 / pl.zd;
  double acc = 0.0;
  // two halves of the thread's vectors keep the kernel within 64 VGPRs
  constexpr int kHalf = kVec / 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 tv[kHalf], dv[kHalf];
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      const int v = threadIdx.x + (h * kHalf + k) * kThreads;
      tv[k] = v < nvec ? sdv::ld_nt(tp + v) : ninf;
      dv[k] = v < nvec ? sdv::ld_nt(dp + v) : ninf;
    }
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      float xt[VT::kElems], xd[VT::kElems];
      VT::unpack(tv[k], xt);
      VT::unpack(dv[k], xd);
#pragma unroll
      for (int e = 0; e < VT::kElems; ++e)
        acc += draw_weight(xt[e], xd[e], 1, a.c, pl.mct, izt, pl.mcd, izd);
    }
  }
  acc = sdv::wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0) a.rsum[((size_t)r * a.n_ch + ch) * kWaves + (threadIdx.x >> 6)] = acc;
}

// ---------------------------------------------------------------------------
// Acceptance rate of position j: sum over the vocabulary of min(p_j, q_j).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_alpha_sums(VerifyArgs a) {
  using VT = Vec<BF16>;
  constexpr int kVec = kChunk / VT::kElems / kThreads;
  const int gmax = a.gmax, S = 2 * gmax + 1;
  const int ch = blockIdx.x % a.n_ch;
  const int rj = blockIdx.x / a.n_ch;
  const int j = rj % gmax + 1, r = rj / gmax;
  const int L = sdv::clampi(a.ell[r], 0, gmax);
  if (j > L || a.plans[r].kind == 0) return;
  const float mct = a.row_ref[(size_t)r * S + (j - 1)];
  const float mcd = a.row_ref[(size_t)r * S + gmax + j];
  const double izt = 1.0 / a.row_z[(size_t)r * S + (j - 1)];
  const double izd = 1.0 / a.row_z[(size_t)r * S + gmax + j];
  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, a.V - e0) / VT::kElems;
  const uint4* tp = (const uint4*)(a.tgt + ((int64_t)a.tgt_row0[r] + (j - 1)) * a.ld_bytes + (int64_t)e0 * VT::kBytes);
  const uint4* dp = (const uint4*)(a.drf + ((int64_t)a.drf_row0[r] + (j - 1)) * a.ld_bytes + (int64_t)e0 * VT::kBytes);
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  double acc = 0.0;
  constexpr int kHalf = kVec / 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 tv[kHalf], dv[kHalf];
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      const int v = threadIdx.x + (h * kHalf + k) * kThreads;
      tv[k] = v < nvec ? sdv::ld_nt(tp + v) : ninf;
      dv[k] = v < nvec ? sdv::ld_nt(dp + v) : ninf;
    }
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      float xt[VT::kElems], xd[VT::kElems];
      VT::unpack(tv[k], xt);
      VT::unpack(dv[k], xd);
#pragma unroll
      for (int e = 0; e < VT::kElems; ++e) {
        const double pt = (double)sdv::fast_exp2(fmaf(xt[e], a.c, -mct)) * izt;
        const double qd = (double)sdv::fast_exp2(fmaf(xd[e], a.c, -mcd)) * izd;
        acc += fmin(pt, qd);
      }
    }
  }
  acc = sdv::wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0)
    a.asum[(((size_t)r * gmax + (j - 1)) * a.n_ch + ch) * kWaves + (threadIdx.x >> 6)] = acc;
}

// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_sample(VerifyArgs a) {
  using VT = Vec<BF16>;
  constexpr int kQuarterVec = kChunk / VT::kElems / kWaves;  // vectors per wave
  constexpr int kPerLane = kQuarterVec / 64;                  // vectors per lane
  __shared__ double s_chunk[kMaxChunks];
  __shared__ double s_wave_tot[kWaves];
  __shared__ int s_ch, s_found, s_last, s_kind;
  __shared__ double s_target;

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Plan pl = a.plans[r];
  if (pl.kind == 0) return;
  const int S = 2 * a.gmax + 1, n_ch = a.n_ch, V = a.V;
  if (a.accept_prob) {  // per-row totals of the min(p, q) chunk sums
    const int L = sdv::clampi(a.ell[r], 0, a.gmax);
    for (int j = tid + 1; j <= a.gmax; j += kThreads) {
      double t = 0.0;
      if (j <= L) {
        const double* q = a.asum + ((size_t)r * a.gmax + (j - 1)) * n_ch * kWaves;
        for (int i = 0; i < n_ch * kWaves; ++i) t += q[i];
      }
      a.accept_prob[(size_t)r * a.gmax + (j - 1)] = (float)t;
    }
  }
  const float c = a.c;
  int st = pl.st;

  // chunk sums of the weights
  if (pl.kind == 1) {
    for (int ch = tid; ch < n_ch; ch += kThreads) {
      const double* q = a.rsum + ((size_t)r * n_ch + ch) * kWaves;
      s_chunk[ch] = (q[0] + q[1]) + (q[2] + q[3]);
    }
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int ch = 0; ch < n_ch; ++ch) tot += s_chunk[ch];
      s_kind = (tot > 0.0) ? 1 : 2;  // empty residual: draw from p_j* instead
    }
  } else if (tid == 0) {
    s_kind = 2;
  }
  __syncthreads();
  const int kind = s_kind;
  if (pl.kind == 1 && kind == 2) st |= SD_ST_ZERO_RESIDUAL;
  if (kind == 2) {  // sum over chunk ch of 2^(x*c - mct), from the first pass
    const float2* pp = a.partial + ((size_t)r * S + pl.tslot) * n_ch * kWaves;
    for (int ch = tid; ch < n_ch; ch += kThreads) {
      double sum = 0.0;
      for (int w = 0; w < kWaves; ++w) {
        const float2 q = pp[ch * kWaves + w];
        if (q.y != 0.0f) sum += (double)q.y * exp2((double)exp_ref(q.x, c) - (double)pl.mct);
      }
      s_chunk[ch] = sum;
    }
    __syncthreads();
  }
  if (tid == 0) {
    double tot = 0.0;
    for (int ch = 0; ch < n_ch; ++ch) tot += s_chunk[ch];
    const double target = pl.u * tot;
    double acc = 0.0;
    int found = -1, last_pos = -1;
    for (int ch = 0; ch < n_ch; ++ch) {
      if (s_chunk[ch] > 0.0) last_pos = ch;
      if (found < 0 && acc + s_chunk[ch] > target) found = ch;
      if (found < 0) acc += s_chunk[ch];
    }
    if (found < 0) {  // rounding put the target past the end: take the last mass
      found = last_pos;
      s_target = __builtin_huge_val();
    } else {
      s_target = target - acc;
    }
    s_ch = found;
    s_found = 0x7FFFFFFF;
    s_last = -1;
  }
  __syncthreads();
  const int ch = s_ch;
  int32_t* out_tok = a.out_tokens + (size_t)r * (a.gmax + 1);
  if (ch < 0) {  // no mass anywhere (not reachable for a finite row)
    if (tid == 0) {
      out_tok[pl.n_acc] = -1;
      a.status[r] = st;
    }
    return;
  }

  // Rescan the chunk: wave w owns the contiguous quarter
  // [w*kQuarterVec, (w+1)*kQuarterVec) of its vectors, lane l the vectors
  // w*kQuarterVec + k*64 + l; vocabulary order is (k, lane, element).
  const double target = s_target;
  const int e0 = ch * kChunk;
  const int nvec = min(kChunk, V - e0) / VT::kElems;
  const uint4* tp = (const uint4*)(a.tgt + pl.trow * a.ld_bytes + (int64_t)e0 * VT::kBytes);
  const uint4* dp = kind == 1 ? (const uint4*)(a.drf + pl.drow * a.ld_bytes + (int64_t)e0 * VT::kBytes)
                              : nullptr;
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  const double izt = 1.0 / pl.zt, izd = 1.0 / pl.zd;
  uint4 tv[kPerLane], dv[kPerLane];
#pragma unroll
  for (int k = 0; k < kPerLane; ++k) {
    const int v = wave * kQuarterVec + k * 64 + lane;
    tv[k] = v < nvec ? tp[v] : ninf;
    dv[k] = (v < nvec && dp) ? dp[v] : ninf;
  }
  double col[kPerLane];
  double my_tot = 0.0;
  int last = -1;
#pragma unroll
  for (int k = 0; k < kPerLane; ++k) {
    float xt[VT::kElems], xd[VT::kElems];
    VT::unpack(tv[k], xt);
    VT::unpack(dv[k], xd);
    double vs = 0.0;
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) {
      const double w = draw_weight(xt[e], xd[e], kind, c, pl.mct, izt, pl.mcd, izd);
      vs += w;
      if (w > 0.0) last = e0 + (wave * kQuarterVec + k * 64 + lane) * VT::kElems + e;
    }
    col[k] = vs;
    my_tot += vs;
  }
  const double wtot = sdv::wave_sum_d(my_tot);
  if (lane == 0) s_wave_tot[wave] = wtot;
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  double run = 0.0;
  for (int w = 0; w < wave; ++w) run += s_wave_tot[w];
  if (run <= target && run + s_wave_tot[wave] > target) {
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const double incl = sdv::wave_incl_scan_d(col[k], lane);
      const double c0 = run + (incl - col[k]);
      int hit = 0x7FFFFFFF;
      if (c0 <= target && c0 + col[k] > target) {
        float xt[VT::kElems], xd[VT::kElems];
        VT::unpack(tv[k], xt);
        VT::unpack(dv[k], xd);
        double cc = c0;
        for (int e = 0; e < VT::kElems; ++e) {
          cc += draw_weight(xt[e], xd[e], kind, c, pl.mct, izt, pl.mcd, izd);
          if (cc > target) {
            hit = e0 + (wave * kQuarterVec + k * 64 + lane) * VT::kElems + e;
            break;
          }
        }
      }
      hit = sdv::wave_min_i(hit);
      if (hit != 0x7FFFFFFF) {
        if (lane == 0) atomicMin(&s_found, hit);
        break;
      }
      run += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int token = s_found;
    if (token == 0x7FFFFFFF) token = s_last;  // rounding: last element with mass
    out_tok[pl.n_acc] = token;
    a.status[r] = st;
  }
}

size_t partial_bytes(int R, int gmax, int V) {
  const size_t n_ch = ((size_t)V + kChunk - 1) / kChunk;
  return sdv_align256((size_t)R * (2 * (size_t)gmax + 1) * n_ch * kWaves * sizeof(float2));
}

size_t verify_ws_bytes(int R, int gmax, int V) {
  const size_t n_ch = ((size_t)V + kChunk - 1) / kChunk;
  const size_t S = 2 * (size_t)gmax + 1;
  return partial_bytes(R, gmax, V) + sdv_align256((size_t)R * sizeof(Plan)) +
         sdv_align256((size_t)R * n_ch * kWaves * sizeof(double)) +
         sdv_align256((size_t)R * S * sizeof(float)) + sdv_align256((size_t)R * S * sizeof(double)) +
         sdv_align256((size_t)R * gmax * n_ch * kWaves * sizeof(double));
}

template <bool BF16>
int launch_verify(hipStream_t stream, int R, const VerifyArgs& a, long long items,
                  hipEvent_t ev0, hipEvent_t ev1) {
  const bool timed = ev0 && ev1;
  if (timed) SDV_TRY_LAUNCH(hipEventRecord(ev0, stream));
  SDV_TRY_LAUNCH(sdv::launch(k_row_partials<BF16>, dim3((unsigned)items), dim3(kThreads), 0, stream, a));
  if (timed) SDV_TRY_LAUNCH(hipEventRecord(ev1, stream));
  SDV_TRY_LAUNCH(sdv::launch(k_accept<BF16>, dim3(R), dim3(kThreads), 0, stream, a));
  SDV_TRY_LAUNCH(sdv::launch(k_residual_sums<BF16>, dim3((unsigned)(R * a.n_ch)), dim3(kThreads), 0,
                             stream, a));
  if (a.accept_prob && a.gmax > 0)
    SDV_TRY_LAUNCH(sdv::launch(k_alpha_sums<BF16>, dim3((unsigned)((long long)R * a.gmax * a.n_ch)),
                               dim3(kThreads), 0, stream, a));
  SDV_TRY_LAUNCH(sdv::launch(k_sample<BF16>, dim3(R), dim3(kThreads), 0, stream, a));
  return SD_OK;
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
                         int32_t* status, float* probe_probs, float* row_stats,
                         float* accept_prob, void* workspace, size_t workspace_bytes,
                         hipEvent_t prof_start, hipEvent_t prof_stop) {
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
  const int n_ch = (V + kChunk - 1) / kChunk;
  const long long items = (long long)R * (2 * gamma_max + 1) * n_ch;
  if (items > 0x7FFFFFFFLL) return SD_EUNSUPPORTED;

  VerifyArgs a;
  a.tgt = (const char*)tgt_logits;
  a.tgt_row0 = tgt_row0;
  a.drf = (const char*)(drf_logits ? drf_logits : tgt_logits);
  a.drf_row0 = drf_row0;
  a.draft_tokens = draft_tokens;
  a.ell = ell;
  a.pos0 = pos0;
  a.n_accepted = n_accepted;
  a.out_tokens = out_tokens;
  a.status = status;
  a.probe_probs = probe_probs;
  a.row_stats = row_stats;
  a.accept_prob = accept_prob;
  const size_t S = 2 * (size_t)gamma_max + 1;
  char* p = (char*)workspace;
  a.partial = (float2*)p;
  p += partial_bytes(R, gamma_max, V);
  a.plans = (Plan*)p;
  p += sdv_align256((size_t)R * sizeof(Plan));
  a.rsum = (double*)p;
  p += sdv_align256((size_t)R * n_ch * kWaves * sizeof(double));
  a.row_ref = (float*)p;
  p += sdv_align256((size_t)R * S * sizeof(float));
  a.row_z = (double*)p;
  p += sdv_align256((size_t)R * S * sizeof(double));
  a.asum = (double*)p;
  a.ld_bytes = (int64_t)ld * (dtype == SD_DTYPE_BF16 ? 2 : 4);
  a.seed = seed;
  a.c = sdv::kLog2e / temperature;
  a.inv_t = 1.0f / temperature;
  a.gmax = gamma_max;
  a.V = V;
  a.n_ch = n_ch;
  if (dtype == SD_DTYPE_BF16) return launch_verify<true>(stream, R, a, items, prof_start, prof_stop);
  return launch_verify<false>(stream, R, a, items, prof_start, prof_stop);
}
