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
// G tile = Ag[m0..m0+127] (128 x rank) . Ct_k[n0..n0+127]^T (rank x 128)
// with v_mfma_f32_16x16x32_bf16: wave w owns columns [32w, 32w+32) of the tile,
// all 128 rows: 8 row blocks x 2 column blocks of 16 x 16 accumulators.
__global__ __launch_bounds__(kThreads) void k_markov_bias(
    int R, int gamma, int k, int V, int rank, float c, const uint16_t* __restrict__ U,
    const uint16_t* __restrict__ Ct, const uint16_t* __restrict__ Ag,
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
  const int lda = rank + kApad;
  const int ksteps = rank / 32;
  const uint16_t* Ck = Ct + (size_t)(k - 1) * V * rank;

  // Every HBM read of the workgroup is issued before the first wait: the A
  // rows (needed first), the B fragments, then the U tile for the epilogue.
  const int vec_per_row = rank / 8;
  const int total = kTileM * vec_per_row;
  uint4 gat[kAPerThread];
#pragma unroll
  for (int i = 0; i < kAPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int row = idx / vec_per_row;
    gat[i] = (idx < total && m0 + row < R)
                 ? *(const uint4*)(Ag + (size_t)(m0 + row) * rank + (idx % vec_per_row) * 8)
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
      if (ks < ksteps && col < V) v = sdv::ld_nt(Ck + (size_t)col * rank + ks * 32 + (lane >> 4) * 8);
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
    if (ks < ksteps) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const uint4 av =
            *(const uint4*)(sA + (mb * 16 + (lane & 15)) * lda + ks * 32 + (lane >> 4) * 8);
        const bf16x8 a = as_bf16x8(av);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(bfrag[nb][ks]), acc[mb][nb], 0, 0, 0);
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
__global__ __launch_bounds__(kThreads) void k_markov_select(
    int gamma, int k, int V, int H, int rank_e, float c, uint64_t seed,
    const int64_t* __restrict__ pos0, const int32_t* __restrict__ x0,
    const uint16_t* __restrict__ E, const float* __restrict__ w,
    const float* __restrict__ hdot, const float2* __restrict__ partial, int n_tiles,
    const uint16_t* __restrict__ q_logits, int rank, const uint16_t* __restrict__ A,
    uint16_t* __restrict__ Ag, int32_t* __restrict__ tokens, float* __restrict__ conf,
    int32_t* __restrict__ status) {
  __shared__ float s_red[kThreads / 64];
  __shared__ double s_redd[kThreads / 64];
  __shared__ int s_tile;
  __shared__ double s_tgt;
  __shared__ int s_tok, s_claim;

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xp = (k == 1) ? x0[r] : tokens[(size_t)r * gamma + (k - 2)];
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
  const float2* pp = partial + (size_t)r * n_tiles;
  const int per = (n_tiles + kThreads - 1) / kThreads;
  const int t0 = tid * per;
  float M = kNegInf;
  for (int i = 0; i < per; ++i)
    if (t0 + i < n_tiles) M = fmaxf(M, pp[t0 + i].x);
  M = sdv::wave_max(M);
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float REF = exp_ref(M, c);
  double own = 0.0;
  for (int i = 0; i < per; ++i) {
    if (t0 + i < n_tiles) {
      const float2 q = pp[t0 + i];
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
    if (k < gamma)  // no anchor for the next step: no Markov bias
      for (int v = tid; v < rank / 8; v += kThreads)
        ((uint4*)(Ag + (size_t)r * rank))[v] = make_uint4(0, 0, 0, 0);
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
  if (k < gamma) {  // the next step's Markov rows: A_{k+1}[x_k]
    const bool valid = tok >= 0 && tok < V;
    const uint16_t* Anext = A + (size_t)k * V * rank;
    for (int v = tid; v < rank / 8; v += kThreads)
      ((uint4*)(Ag + (size_t)r * rank))[v] =
          valid ? ((const uint4*)(Anext + (size_t)tok * rank))[v] : make_uint4(0, 0, 0, 0);
  }
}

size_t markov_ws_bytes(int R, int gamma, int V, int rank) {
  const size_t n_tiles = ((size_t)V + kTileN - 1) / kTileN;
  return sdv_align256((size_t)R * gamma * sizeof(float)) +
         sdv_align256((size_t)R * n_tiles * sizeof(float2)) +
         sdv_align256((size_t)R * rank * sizeof(uint16_t));
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
  if (R < 0 || gamma < 0 || V < 8 || (V % 8) != 0 || H < 0 || (H % 8) != 0 || rank_e < 0 ||
      (rank_e % 8) != 0)
    return SD_EINVAL;
  if (rank < 32 || (rank % 32) != 0) return SD_EINVAL;
  if (rank > kMaxRank || gamma > SD_MAX_GAMMA || V > SD_MAX_VOCAB) return SD_EUNSUPPORTED;
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf())) return SD_EINVAL;
  const int n_tiles = (V + kTileN - 1) / kTileN;
  if (R == 0 || gamma == 0) return SD_OK;
  if (!U || !A || !Ct || !x0 || !w || !tokens || !q_logits || !conf || !status) return SD_EINVAL;
  if ((H > 0 && !h) || (rank_e > 0 && !E)) return SD_EINVAL;
  if (!workspace || workspace_bytes < markov_ws_bytes(R, gamma, V, rank)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  if ((((uintptr_t)U | (uintptr_t)A | (uintptr_t)Ct | (uintptr_t)q_logits | (uintptr_t)h |
        (uintptr_t)w) & 15) != 0)
    return SD_EINVAL;

  const float c = sdv::kLog2e / temperature;
  char* p = (char*)workspace;
  float* hdot = (float*)p;
  p += sdv_align256((size_t)R * gamma * sizeof(float));
  float2* partial = (float2*)p;
  p += sdv_align256((size_t)R * n_tiles * sizeof(float2));
  uint16_t* Ag = (uint16_t*)p;

  const int rows = R * gamma;
  if (H > 0) {
    SDV_TRY_LAUNCH(sdv::launch(k_hidden_dot, dim3((rows + 3) / 4), dim3(kThreads), 0, stream, h, H,
                               w, rows, hdot));
  } else {
    return SD_EINVAL;  // the confidence head needs a hidden state
  }
  SDV_TRY_LAUNCH(sdv::launch(k_gather_a, dim3(R), dim3(64), 0, stream, R, V, rank, A, x0, Ag));
  const dim3 grid_bias(n_tiles, (R + kTileM - 1) / kTileM);
  for (int k = 1; k <= gamma; ++k) {
    SDV_TRY_LAUNCH(sdv::launch(k_markov_bias, grid_bias, dim3(kThreads), 0, stream, R, gamma, k, V,
                               rank, c, U, Ct, (const uint16_t*)Ag, q_logits, partial, n_tiles));
    SDV_TRY_LAUNCH(sdv::launch(k_markov_select, dim3(R), dim3(kThreads), 0, stream, gamma, k, V, H,
                               rank_e, c, seed, pos0, x0, E, w, (const float*)hdot,
                               (const float2*)partial, n_tiles, (const uint16_t*)q_logits, rank, A,
                               Ag, tokens, conf, status));
  }
  return SD_OK;
}
