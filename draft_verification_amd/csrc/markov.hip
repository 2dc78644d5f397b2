// sd_markov_draft: the semi-autoregressive Markov drafting head and the
// confidence head.
//
// DSpark summary, "innovation one": a parallel backbone gives base logits U_k
// and hidden states h_k for the whole block in one pass; a light sequential
// head then injects the previous drafted token into each position,
// P_k = softmax(U_k + B_k(x_{k-1})), with the V x V transition table B_k
// stored low-rank (speculative-decoding history page, DSpark "move one").
// "2.1 confidence head": c_k = sigmoid(w . [h_k ; E[x_{k-1}]]).
//
// Per step k (sequential over the block):
//   k_markov_bias    the only dense contraction: G = A_k[x_{k-1}] . C_k as a
//                    bf16 MFMA GEMM (M = requests, N = vocabulary, K = rank),
//                    fused with + U_k, bf16 rounding, the q_logits store and a
//                    per-(row, 128-column tile) partial (max, sum 2^(L*c - ref));
//                    the rows A_k[x_{k-1}] arrive pre-gathered, so every load
//                    of a workgroup is issued before its first wait
//   k_markov_select  one workgroup per request: confidence of position k,
//                    combine tile partials, locate the inverse-CDF tile,
//                    rescan 128 logits, emit x_k, and gather A_{k+1}[x_k]
//                    for the next step
// plus, up front, one k_hidden_dot launch for w_h . h_k of every position and
// one k_gather_a launch for A_1[x_0].
#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 128;  // vocabulary columns per workgroup (4 waves x 32)
constexpr int kTileM = 128;  // requests per workgroup
constexpr int kMaxRank = 256;
constexpr int kApad = 8;     // bf16 padding per LDS row of the gathered A rows
constexpr int kGpad = 4;     // fp32 padding per LDS row of the output tile
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Reductions over each 16-lane DPP row; every lane of the row gets the result.
// Partners: xor 1, xor 2 (quad permutes), then the half-row and row mirrors.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}
__device__ __forceinline__ float exp_ref(float m, float c) { return m == kNegInf ? 0.0f : m * c; }

// ---------------------------------------------------------------------------
// hdot[r][k] = w[0:H] . h[r][k]   (one wave per (r, k))
__global__ __launch_bounds__(kThreads) void k_hidden_dot(const uint16_t* __restrict__ h, int H,
                                                         const float* __restrict__ w, int rows,
                                                         float* __restrict__ hdot) {
  const int wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= rows) return;
  const uint4* hp = (const uint4*)(h + (size_t)wave * H);
  float acc = 0.0f;
  for (int v = lane; v < H / 8; v += 64) {
    const uint4 q = hp[v];
    const float4 w0 = ((const float4*)w)[2 * v];
    const float4 w1 = ((const float4*)w)[2 * v + 1];
    acc += sdv::bf16lo(q.x) * w0.x + sdv::bf16hi(q.x) * w0.y + sdv::bf16lo(q.y) * w0.z +
           sdv::bf16hi(q.y) * w0.w + sdv::bf16lo(q.z) * w1.x + sdv::bf16hi(q.z) * w1.y +
           sdv::bf16lo(q.w) * w1.z + sdv::bf16hi(q.w) * w1.w;
  }
  acc = sdv::wave_sum(acc);
  if (lane == 0) hdot[wave] = acc;
}

// ---------------------------------------------------------------------------
// Ag[r] = A_k[x_prev[r]] (rank bf16), zeros when x_prev is outside [0, V): the
// anchor contributes no Markov bias.  Used for step 1; k_markov_select does it
// for the following steps.
__global__ __launch_bounds__(64) void k_gather_a(int R, int V, int rank, const uint16_t* __restrict__ Ak,
                                                 const int32_t* __restrict__ xprev,
                                                 uint16_t* __restrict__ Ag) {
  const int r = blockIdx.x;
  const int xp = xprev[r];
  const bool valid = xp >= 0 && xp < V;
  for (int v = threadIdx.x; v < rank / 8; v += 64)
    ((uint4*)(Ag + (size_t)r * rank))[v] =
        valid ? ((const uint4*)(Ak + (size_t)xp * rank))[v] : make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// G tile = A rows (128 x kdim) . Ct_k[n0..n0+127]^T (kdim x 128) with
// v_mfma_f32_16x16x32_bf16: wave w owns columns [32w, 32w+32) of the tile, all
// 128 rows: 8 row blocks x 2 column blocks of 16 x 16 accumulators.
// NSPLIT = 1: Ag[r] holds A_k[x_{k-1}] (the Markov head).  NSPLIT = 2: Ag[r]
// holds the RNN state as two bf16 terms, hi = bf16(s) then lo = bf16(s - hi),
// and both are multiplied by the same C fragments, so the product carries the
// fp32 state to within 2^-17 of each element.
template <int NSPLIT>
__global__ __launch_bounds__(kThreads, 2) void k_markov_bias(
    int R, int gamma, int k, int V, int kdim, float c, const uint16_t* __restrict__ U,
    const uint16_t* __restrict__ Ct, size_t ct_stride, const uint16_t* __restrict__ Ag,
    uint16_t* __restrict__ q_logits, float2* __restrict__ partial, int n_tiles) {
  // LDS: the A rows during the GEMM, then the fp32 output tile.
  constexpr int kAbytes = kTileM * (kMaxRank + kApad) * 2;
  constexpr int kGbytes = kTileM * (kTileN + kGpad) * 4;
  constexpr int kEpiPasses = kTileM / 16;
  constexpr int kAPerThread = kTileM * (kMaxRank / 8) / kThreads;
  __shared__ __align__(16) unsigned char lds[kAbytes > kGbytes ? kAbytes : kGbytes];
  uint16_t* sA = (uint16_t*)lds;
  float* sG = (float*)lds;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int n0 = tile * kTileN;
  const int m0 = blockIdx.y * kTileM;
  const int arow = NSPLIT * kdim;  // bf16 per A row
  const int lda = arow + kApad;
  const int kb = kdim / 32;        // K steps of the C fragments
  const uint16_t* Ck = Ct + (size_t)(k - 1) * ct_stride;

  // Every HBM read of the workgroup is issued before the first wait: the A
  // rows (needed first), the B fragments, then the U tile for the epilogue.
  const int vec_per_row = arow / 8;
  const int total = kTileM * vec_per_row;
  uint4 gat[kAPerThread];
#pragma unroll
  for (int i = 0; i < kAPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int row = idx / vec_per_row;
    gat[i] = (idx < total && m0 + row < R)
                 ? *(const uint4*)(Ag + (size_t)(m0 + row) * arow + (idx % vec_per_row) * 8)
                 : make_uint4(0, 0, 0, 0);
  }
  // B fragments: lane l holds column (l % 16) of its 16-column block,
  // K values [32*ks + 8*(l/16), +8).
  uint4 bfrag[2][kMaxRank / 32];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int col = n0 + wave * 32 + nb * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < kMaxRank / 32; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ks < kb && col < V) v = sdv::ld_nt(Ck + (size_t)col * kdim + ks * 32 + (lane >> 4) * 8);
      bfrag[nb][ks] = v;
    }
  }
  // U for the epilogue: 16 threads per row, 8 columns each, 16 rows per pass
  const int seg = tid & 15;
  const int ecol = n0 + seg * 8;
  uint4 upre[kEpiPasses];
#pragma unroll
  for (int pass = 0; pass < kEpiPasses; ++pass) {
    const int r = m0 + pass * 16 + (tid >> 4);
    upre[pass] = (r < R && ecol < V) ? sdv::ld_nt(U + ((size_t)r * gamma + (k - 1)) * V + ecol)
                                     : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kAPerThread; ++i) {
    const int idx = tid + i * kThreads;
    if (idx < total) *(uint4*)(sA + (idx / vec_per_row) * lda + (idx % vec_per_row) * 8) = gat[i];
  }
  __syncthreads();

  floatx4 acc[8][2];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int ks = 0; ks < kMaxRank / 32; ++ks) {
    if (ks < kb) {
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          const uint4 av = *(const uint4*)(sA + (mb * 16 + (lane & 15)) * lda + (sp * kb + ks) * 32 +
                                           (lane >> 4) * 8);
          const bf16x8 a = as_bf16x8(av);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(bfrag[nb][ks]),
                                                                  acc[mb][nb], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // A rows no longer needed: reuse LDS for the output tile

  // accumulator (mb, nb), register i: row mb*16 + 4*(lane/16) + i, column lane%16
  const int ldg = kTileN + kGpad;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sG[(mb * 16 + (lane >> 4) * 4 + i) * ldg + wave * 32 + nb * 16 + (lane & 15)] = acc[mb][nb][i];
  __syncthreads();

  // Epilogue: L = bf16(U + G), stored; per-(row, tile) partial (max, sum).
  // The 16 threads of a row are one DPP row of the wave.
#pragma unroll
  for (int pass = 0; pass < kEpiPasses; ++pass) {
    const int mr = pass * 16 + (tid >> 4);
    const int r = m0 + mr;
    const bool live = (r < R) && (ecol < V);
    const uint4 u = upre[pass];
    const float4 g0 = *(const float4*)(sG + mr * ldg + seg * 8);
    const float4 g1 = *(const float4*)(sG + mr * ldg + seg * 8 + 4);
    uint4 o;
    o.x = pack_bf16_rne(sdv::bf16lo(u.x) + g0.x, sdv::bf16hi(u.x) + g0.y);
    o.y = pack_bf16_rne(sdv::bf16lo(u.y) + g0.z, sdv::bf16hi(u.y) + g0.w);
    o.z = pack_bf16_rne(sdv::bf16lo(u.z) + g1.x, sdv::bf16hi(u.z) + g1.y);
    o.w = pack_bf16_rne(sdv::bf16lo(u.w) + g1.z, sdv::bf16hi(u.w) + g1.w);
    const float vals[8] = {sdv::bf16lo(o.x), sdv::bf16hi(o.x), sdv::bf16lo(o.y), sdv::bf16hi(o.y),
                           sdv::bf16lo(o.z), sdv::bf16hi(o.z), sdv::bf16lo(o.w), sdv::bf16hi(o.w)};
    float m = kNegInf;
    if (live) {
      sdv::st_nt(q_logits + ((size_t)r * gamma + (k - 1)) * V + ecol, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, vals[e]);
    }
    // row partial over the 16 lanes of this row: max, then sum relative to it
    m = row16_max(m);
    const float ref = exp_ref(m, c);
    float s = 0.0f;
    if (live) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s += sdv::fast_exp2(fmaf(vals[e], c, -ref));
    }
    s = row16_sum(s);
    if (seg == 0 && r < R) partial[(size_t)r * n_tiles + tile] = make_float2(m, s);
  }
}

// ---------------------------------------------------------------------------
// The rows the next step's bias multiplies, once x_k is known (every thread
// calls).  Markov: Ag[r] = A_{k+1}[x_k], zeros for an invalid token.  RNN:
// s_{k+1} = tanh(W s_k + E_s[x_k]) in fp32 (no embedding term for an invalid
// token), kept in state[r] and written to Ag[r] as its two bf16 terms.
struct NextRows {
  int rank;                 // Markov: A row length; RNN: state size d
  const uint16_t* A;        // Markov: A [gamma][V][rank]
  const uint16_t* W;        // RNN: W [d][d]
  const uint16_t* Es;       // RNN: E_s [V][d]
  float* state;             // RNN: [R][d]
  uint16_t* Ag;             // [R][rank] (Markov) or [R][2d] (RNN)
};

template <bool RNN>
__device__ void next_rows(const NextRows& nr, int r, int k, int V, int tok, float* s_s) {
  const int tid = threadIdx.x;
  const bool valid = tok >= 0 && tok < V;
  if constexpr (!RNN) {
    const uint16_t* Anext = nr.A + (size_t)k * V * nr.rank;
    for (int v = tid; v < nr.rank / 8; v += kThreads)
      ((uint4*)(nr.Ag + (size_t)r * nr.rank))[v] =
          valid ? ((const uint4*)(Anext + (size_t)tok * nr.rank))[v] : make_uint4(0, 0, 0, 0);
  } else {
    const int d = nr.rank;
    for (int i = tid; i < d; i += kThreads) s_s[i] = nr.state[(size_t)r * d + i];
    __syncthreads();
    for (int o = tid; o < d; o += kThreads) {
      const uint16_t* wr = nr.W + (size_t)o * d;
      float acc = 0.0f;
      for (int i = 0; i < d; i += 8) {
        const uint4 q = *(const uint4*)(wr + i);
        acc += sdv::bf16lo(q.x) * s_s[i] + sdv::bf16hi(q.x) * s_s[i + 1] +
               sdv::bf16lo(q.y) * s_s[i + 2] + sdv::bf16hi(q.y) * s_s[i + 3] +
               sdv::bf16lo(q.z) * s_s[i + 4] + sdv::bf16hi(q.z) * s_s[i + 5] +
               sdv::bf16lo(q.w) * s_s[i + 6] + sdv::bf16hi(q.w) * s_s[i + 7];
      }
      if (valid) acc += sdv::bf16_to_f32(nr.Es[(size_t)tok * d + o]);
      const float sn = tanhf(acc);
      nr.state[(size_t)r * d + o] = sn;
      const uint16_t hi = sdv::f32_to_bf16_rne(sn);
      nr.Ag[(size_t)r * 2 * d + o] = hi;
      nr.Ag[(size_t)r * 2 * d + d + o] = sdv::f32_to_bf16_rne(sn - sdv::bf16_to_f32(hi));
    }
  }
}

template <bool RNN>
__global__ __launch_bounds__(kThreads) void k_markov_select(
    int gamma, int k, int V, int H, int rank_e, float c, uint64_t seed,
    const int64_t* __restrict__ pos0, const int32_t* __restrict__ x0,
    const uint16_t* __restrict__ E, const float* __restrict__ w,
    const float* __restrict__ hdot, const float2* __restrict__ partial, int n_tiles,
    const uint16_t* __restrict__ q_logits, NextRows nr, int32_t* __restrict__ tokens,
    float* __restrict__ conf, int32_t* __restrict__ status) {
  __shared__ float s_s[kMaxRank];
  __shared__ float s_red[kThreads / 64];
  __shared__ double s_redd[kThreads / 64];
  __shared__ int s_tile;
  __shared__ double s_tgt;
  __shared__ int s_tok, s_claim;

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xp = (k == 1) ? x0[r] : tokens[(size_t)r * gamma + (k - 2)];
  // this thread's run of tile partials, requested before the confidence work
  const float2* pp = partial + (size_t)r * n_tiles;
  const int per = (n_tiles + kThreads - 1) / kThreads;
  const int t0 = tid * per;
  constexpr int kPre = 4;
  float2 pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i)
    pre[i] = (i < per && t0 + i < n_tiles) ? pp[t0 + i] : make_float2(kNegInf, 0.0f);
  auto part = [&](int i) { return i < kPre ? pre[i] : pp[t0 + i]; };
  const bool xvalid = xp >= 0 && xp < V;
  int st = (k == 1) ? 0 : status[r];
  if (!xvalid) st |= SD_ST_BAD_TOKEN;

  // confidence of position k: sigmoid(w_h . h_k + w_e . E[x_{k-1}])
  float e = 0.0f;
  if (xvalid)
    for (int i = tid; i < rank_e; i += kThreads) e += w[H + i] * sdv::bf16_to_f32(E[(size_t)xp * rank_e + i]);
  e = sdv::wave_sum(e);
  if (lane == 0) s_red[wave] = e;
  __syncthreads();
  if (tid == 0) {
    float z = hdot[(size_t)r * gamma + (k - 1)];
    for (int ww = 0; ww < kThreads / 64; ++ww) z += s_red[ww];
    conf[(size_t)r * gamma + (k - 1)] = 1.0f / (1.0f + expf(-z));
  }
  __syncthreads();

  // Combine the tile partials.  Thread t owns a contiguous run of tiles.
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < kPre; ++i) M = fmaxf(M, pre[i].x);
  for (int i = kPre; i < per; ++i)
    if (t0 + i < n_tiles) M = fmaxf(M, pp[t0 + i].x);
  M = sdv::wave_max(M);
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float REF = exp_ref(M, c);
  double own = 0.0;
  for (int i = 0; i < per; ++i) {
    if (t0 + i < n_tiles) {
      const float2 q = part(i);
      if (q.y != 0.0f) own += (double)q.y * exp2((double)exp_ref(q.x, c) - (double)REF);
    }
  }
  const double incl = sdv::wave_incl_scan_d(own, lane);
  if (lane == 63) s_redd[wave] = incl;
  __syncthreads();
  double excl = incl - own;
  double Z = 0.0;
  for (int ww = 0; ww < kThreads / 64; ++ww) {
    if (ww < wave) excl += s_redd[ww];
    Z += s_redd[ww];
  }
  if (tid == 0) { s_tile = -1; s_tok = -1; s_claim = 0x7FFFFFFF; }
  __syncthreads();

  int bad = 0;
  if (isnan(M) || isnan(Z) || M == __builtin_huge_valf()) bad = SD_ST_NONFINITE;
  else if (M == kNegInf) bad = SD_ST_ZERO_Z;
  if (bad) {
    if (tid == 0) {
      tokens[(size_t)r * gamma + (k - 1)] = -1;
      status[r] = st | bad;
    }
    if (k < gamma) next_rows<RNN>(nr, r, k, V, -1, s_s);  // no valid token to carry forward
    return;
  }

  const int64_t pbase = pos0 ? pos0[r] : 0;
  const double u = sdv::uniform24(seed, (uint64_t)r, (uint64_t)(pbase + k), 0);
  const double target = u * Z;
  // the thread whose tile run contains the crossing walks its tiles (the
  // lowest such thread, should rounding make two runs claim it)
  const bool claims = excl <= target && excl + own > target;
  if (claims) atomicMin(&s_claim, tid);
  __syncthreads();
  if (tid == s_claim) {
    double cum = excl;
    for (int i = 0; i < per && t0 + i < n_tiles; ++i) {
      const float2 q = pp[t0 + i];
      const double s = q.y != 0.0f ? (double)q.y * exp2((double)exp_ref(q.x, c) - (double)REF) : 0.0;
      if (cum + s > target && s > 0.0) {
        s_tile = t0 + i;
        s_tgt = target - cum;
        break;
      }
      cum += s;
    }
  }
  __syncthreads();
  int tile = s_tile;
  double tgt_in = s_tgt;
  if (tile < 0) {  // rounding pushed the target past the end: last tile with mass
    if (tid == 0) {
      for (int t = n_tiles - 1; t >= 0; --t)
        if (pp[t].y > 0.0f) { s_tile = t; break; }
      s_tgt = __builtin_huge_val();
    }
    __syncthreads();
    tile = s_tile;
    tgt_in = s_tgt;
  }

  // rescan the tile's 128 logits with wave 0: 2 per lane, weights relative to
  // the tile's own reference, scaled into the global frame.
  if (wave == 0 && tile >= 0) {
    const float2 q = pp[tile];
    const float tref = exp_ref(q.x, c);
    const double scale = exp2((double)tref - (double)REF);
    const int n0 = tile * kTileN;
    const size_t rowoff = ((size_t)r * gamma + (k - 1)) * V;
    double wv[2];
    int idx[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      idx[e2] = n0 + lane * 2 + e2;
      wv[e2] = 0.0;
      if (idx[e2] < V) {
        const float L = sdv::bf16_to_f32(q_logits[rowoff + idx[e2]]);
        wv[e2] = (double)sdv::fast_exp2(fmaf(L, c, -tref)) * scale;
      }
    }
    const double lsum = wv[0] + wv[1];
    const double li = sdv::wave_incl_scan_d(lsum, lane);
    double cum = li - lsum;
    int found = 0x7FFFFFFF, last = -1;
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      if (wv[e2] > 0.0) last = idx[e2];
      cum += wv[e2];
      if (found == 0x7FFFFFFF && cum > tgt_in && wv[e2] > 0.0) found = idx[e2];
    }
    found = sdv::wave_min_i(found);
    int lastm = last;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lastm = max(lastm, __shfl_xor(lastm, o, 64));
    if (lane == 0) s_tok = (found != 0x7FFFFFFF) ? found : lastm;
  }
  __syncthreads();
  const int tok = s_tok;
  if (tid == 0) {
    tokens[(size_t)r * gamma + (k - 1)] = tok;
    status[r] = st;
  }
  if (k < gamma) next_rows<RNN>(nr, r, k, V, tok, s_s);
}

// s_1 = tanh(W s_0 + E_s[x_0]) = tanh(E_s[x_0]) (s_0 = 0; no embedding term for
// an anchor outside [0, V)), kept in state[r] and written to Ag[r] split.
__global__ __launch_bounds__(kThreads) void k_rnn_init(int R, int V, int d, const uint16_t* __restrict__ Es,
                                                       const int32_t* __restrict__ x0,
                                                       float* __restrict__ state,
                                                       uint16_t* __restrict__ Ag) {
  const int r = blockIdx.x;
  const int x = x0[r];
  const bool valid = x >= 0 && x < V;
  for (int o = threadIdx.x; o < d; o += kThreads) {
    const float sn = tanhf(valid ? sdv::bf16_to_f32(Es[(size_t)x * d + o]) : 0.0f);
    state[(size_t)r * d + o] = sn;
    const uint16_t hi = sdv::f32_to_bf16_rne(sn);
    Ag[(size_t)r * 2 * d + o] = hi;
    Ag[(size_t)r * 2 * d + d + o] = sdv::f32_to_bf16_rne(sn - sdv::bf16_to_f32(hi));
  }
}

// Workspace: hdot [R][gamma] fp32, tile partials [R][n_tiles] float2, the next
// step's A rows [R][arow] bf16, RNN state [R][d] fp32 (d = 0 for Markov).
size_t head_ws_bytes(int R, int gamma, int V, int arow, int d) {
  const size_t n_tiles = ((size_t)V + kTileN - 1) / kTileN;
  return sdv_align256((size_t)R * gamma * sizeof(float)) +
         sdv_align256((size_t)R * n_tiles * sizeof(float2)) +
         sdv_align256((size_t)R * arow * sizeof(uint16_t)) +
         sdv_align256((size_t)R * d * sizeof(float));
}
size_t markov_ws_bytes(int R, int gamma, int V, int rank) { return head_ws_bytes(R, gamma, V, rank, 0); }
size_t rnn_ws_bytes(int R, int gamma, int V, int d) { return head_ws_bytes(R, gamma, V, 2 * d, d); }

// Checks shared by both heads (everything but the head's own tables).
int check_head_args(int R, int gamma, int V, int H, int rank_e, float temperature) {
  if (R < 0 || gamma < 0 || V < 8 || (V % 8) != 0 || H < 0 || (H % 8) != 0 || rank_e < 0 ||
      (rank_e % 8) != 0)
    return SD_EINVAL;
  if (gamma > SD_MAX_GAMMA || V > SD_MAX_VOCAB) return SD_EUNSUPPORTED;
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf())) return SD_EINVAL;
  return SD_OK;
}

// The sequential loop shared by both heads: per step the bias GEMM + epilogue,
// then the select kernel (which also prepares the next step's rows).
template <int NSPLIT>
int run_head(hipStream_t stream, int R, int gamma, int V, int kdim, size_t ct_stride, float c,
             uint64_t seed, const int64_t* pos0, const uint16_t* U, const uint16_t* Ct,
             const int32_t* x0, int H, const uint16_t* E, int rank_e, const float* w,
             const float* hdot, float2* partial, const NextRows& nr, int32_t* tokens,
             uint16_t* q_logits, float* conf, int32_t* status) {
  const int n_tiles = (V + kTileN - 1) / kTileN;
  const dim3 grid_bias(n_tiles, (R + kTileM - 1) / kTileM);
  for (int k = 1; k <= gamma; ++k) {
    SDV_TRY_LAUNCH(sdv::launch(k_markov_bias<NSPLIT>, grid_bias, dim3(kThreads), 0, stream, R, gamma,
                               k, V, kdim, c, U, Ct, ct_stride, (const uint16_t*)nr.Ag, q_logits,
                               partial, n_tiles));
    SDV_TRY_LAUNCH(sdv::launch(k_markov_select<NSPLIT == 2>, dim3(R), dim3(kThreads), 0, stream, gamma,
                               k, V, H, rank_e, c, seed, pos0, x0, E, w, hdot,
                               (const float2*)partial, n_tiles, (const uint16_t*)q_logits, nr, tokens,
                               conf, status));
  }
  return SD_OK;
}

}  // namespace

extern "C" size_t sd_markov_draft_workspace_size(int R, int gamma, int V, int rank) {
  if (R < 0 || gamma < 0 || V <= 0 || rank < 0) return 0;
  return markov_ws_bytes(R, gamma, V, rank);
}

extern "C" int sd_markov_draft(hipStream_t stream, int R, int gamma, int V, int rank,
                               float temperature, uint64_t seed, const int64_t* pos0,
                               const uint16_t* U, const uint16_t* A, const uint16_t* Ct,
                               const int32_t* x0, const uint16_t* h, int H, const uint16_t* E,
                               int rank_e, const float* w, int32_t* tokens, uint16_t* q_logits,
                               float* conf, int32_t* status, void* workspace,
                               size_t workspace_bytes) {
  const int rc = check_head_args(R, gamma, V, H, rank_e, temperature);
  if (rc != SD_OK) return rc;
  if (rank < 32 || (rank % 32) != 0) return SD_EINVAL;
  if (rank > kMaxRank) return SD_EUNSUPPORTED;
  if (R == 0 || gamma == 0) return SD_OK;
  if (!U || !A || !Ct || !x0 || !w || !tokens || !q_logits || !conf || !status) return SD_EINVAL;
  if ((H > 0 && !h) || (rank_e > 0 && !E)) return SD_EINVAL;
  if (H == 0) return SD_EINVAL;  // the confidence head needs a hidden state
  if (!workspace || workspace_bytes < markov_ws_bytes(R, gamma, V, rank)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  if ((((uintptr_t)U | (uintptr_t)A | (uintptr_t)Ct | (uintptr_t)q_logits | (uintptr_t)h |
        (uintptr_t)w) & 15) != 0)
    return SD_EINVAL;

  const int n_tiles = (V + kTileN - 1) / kTileN;
  char* p = (char*)workspace;
  float* hdot = (float*)p;
  p += sdv_align256((size_t)R * gamma * sizeof(float));
  float2* partial = (float2*)p;
  p += sdv_align256((size_t)R * n_tiles * sizeof(float2));
  NextRows nr{rank, A, nullptr, nullptr, nullptr, (uint16_t*)p};

  const int rows = R * gamma;
  SDV_TRY_LAUNCH(sdv::launch(k_hidden_dot, dim3((rows + 3) / 4), dim3(kThreads), 0, stream, h, H, w,
                             rows, hdot));
  SDV_TRY_LAUNCH(sdv::launch(k_gather_a, dim3(R), dim3(64), 0, stream, R, V, rank, A, x0, nr.Ag));
  return run_head<1>(stream, R, gamma, V, rank, (size_t)V * rank, sdv::kLog2e / temperature, seed,
                     pos0, U, Ct, x0, H, E, rank_e, w, hdot, partial, nr, tokens, q_logits, conf,
                     status);
}

extern "C" size_t sd_rnn_draft_workspace_size(int R, int gamma, int V, int d) {
  if (R < 0 || gamma < 0 || V <= 0 || d < 0) return 0;
  return rnn_ws_bytes(R, gamma, V, d);
}

extern "C" int sd_rnn_draft(hipStream_t stream, int R, int gamma, int V, int d, float temperature,
                            uint64_t seed, const int64_t* pos0, const uint16_t* U,
                            const uint16_t* W, const uint16_t* Es, const uint16_t* Ct,
                            const int32_t* x0, const uint16_t* h, int H, const uint16_t* E,
                            int rank_e, const float* w, int32_t* tokens, uint16_t* q_logits,
                            float* conf, int32_t* status, void* workspace,
                            size_t workspace_bytes) {
  const int rc = check_head_args(R, gamma, V, H, rank_e, temperature);
  if (rc != SD_OK) return rc;
  if (d < 32 || (d % 32) != 0) return SD_EINVAL;
  if (2 * d > kMaxRank) return SD_EUNSUPPORTED;
  if (R == 0 || gamma == 0) return SD_OK;
  if (!U || !W || !Es || !Ct || !x0 || !w || !tokens || !q_logits || !conf || !status)
    return SD_EINVAL;
  if ((H > 0 && !h) || (rank_e > 0 && !E)) return SD_EINVAL;
  if (H == 0) return SD_EINVAL;  // the confidence head needs a hidden state
  if (!workspace || workspace_bytes < rnn_ws_bytes(R, gamma, V, d)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  if ((((uintptr_t)U | (uintptr_t)W | (uintptr_t)Ct | (uintptr_t)q_logits | (uintptr_t)h |
        (uintptr_t)w) & 15) != 0)
    return SD_EINVAL;

  const int n_tiles = (V + kTileN - 1) / kTileN;
  char* p = (char*)workspace;
  float* hdot = (float*)p;
  p += sdv_align256((size_t)R * gamma * sizeof(float));
  float2* partial = (float2*)p;
  p += sdv_align256((size_t)R * n_tiles * sizeof(float2));
  uint16_t* Ag = (uint16_t*)p;
  p += sdv_align256((size_t)R * 2 * d * sizeof(uint16_t));
  NextRows nr{d, nullptr, W, Es, (float*)p, Ag};

  const int rows = R * gamma;
  SDV_TRY_LAUNCH(sdv::launch(k_hidden_dot, dim3((rows + 3) / 4), dim3(kThreads), 0, stream, h, H, w,
                             rows, hdot));
  SDV_TRY_LAUNCH(sdv::launch(k_rnn_init, dim3(R), dim3(kThreads), 0, stream, R, V, d, Es, x0, nr.state,
                             nr.Ag));
  return run_head<2>(stream, R, gamma, V, d, 0, sdv::kLog2e / temperature, seed, pos0, U, Ct, x0, H,
                     E, rank_e, w, hdot, partial, nr, tokens, q_logits, conf, status);
}
