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
//                    per-(row, 128-column tile) partial (max, sum 2^(L*c - ref))
//   k_markov_select  one workgroup per request: confidence of position k,
//                    combine tile partials, locate the inverse-CDF tile,
//                    rescan 128 logits, emit x_k
// plus one k_hidden_dot launch up front for w_h . h_k of every position.
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

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
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
// G tile = A_k[x_prev[m0..m0+127]] (128 x rank) . Ct_k[n0..n0+127]^T (rank x 128)
// with v_mfma_f32_16x16x32_bf16: wave w owns columns [32w, 32w+32) of the tile,
// all 128 rows: 8 row blocks x 2 column blocks of 16 x 16 accumulators.
__global__ __launch_bounds__(kThreads) void k_markov_bias(
    int R, int gamma, int k, int V, int rank, float c, const uint16_t* __restrict__ U,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Ct,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ tokens,
    uint16_t* __restrict__ q_logits, float2* __restrict__ partial, int n_tiles) {
  // LDS: gathered A rows during the GEMM, then the fp32 output tile.
  constexpr int kAbytes = kTileM * (kMaxRank + kApad) * 2;
  constexpr int kGbytes = kTileM * (kTileN + kGpad) * 4;
  constexpr int kEpiPasses = kTileM / 16;
  constexpr int kGatherPerThread = kTileM * (kMaxRank / 8) / kThreads;
  __shared__ __align__(16) unsigned char lds[kAbytes > kGbytes ? kAbytes : kGbytes];
  __shared__ int s_xp[kTileM];
  uint16_t* sA = (uint16_t*)lds;
  float* sG = (float*)lds;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int n0 = tile * kTileN;
  const int m0 = blockIdx.y * kTileM;
  const int lda = rank + kApad;
  const int ksteps = rank / 32;
  const size_t vr = (size_t)V * rank;
  const uint16_t* Ak = A + (size_t)(k - 1) * vr;
  const uint16_t* Ck = Ct + (size_t)(k - 1) * vr;

  // Every HBM read of the workgroup is issued up front so that their
  // latencies overlap: previous tokens, B fragments, the U tile, the A rows.
  if (tid < kTileM) {
    const int r = m0 + tid;
    int xp = -1;
    if (r < R) xp = (k == 1) ? x0[r] : tokens[(size_t)r * gamma + (k - 2)];
    s_xp[tid] = (xp >= 0 && xp < V) ? xp : -1;  // out of range: no Markov bias
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
  __syncthreads();  // s_xp
  const int vec_per_row = rank / 8;
  const int total = kTileM * vec_per_row;
  uint4 gat[kGatherPerThread];
#pragma unroll
  for (int i = 0; i < kGatherPerThread; ++i) {
    const int idx = tid + i * kThreads;
    gat[i] = make_uint4(0, 0, 0, 0);
    if (idx < total) {
      const int xp = s_xp[idx / vec_per_row];
      if (xp >= 0) gat[i] = *(const uint4*)(Ak + (size_t)xp * rank + (idx % vec_per_row) * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < kGatherPerThread; ++i) {
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
#pragma unroll
  for (int pass = 0; pass < kEpiPasses; ++pass) {
    const int mr = pass * 16 + (tid >> 4);
    const int r = m0 + mr;
    float m = kNegInf, s = 0.0f;
    float vals[8];
    const bool live = (r < R) && (ecol < V);
    if (live) {
      const size_t off = ((size_t)r * gamma + (k - 1)) * V + ecol;
      const uint4 u = upre[pass];
      const float* g = sG + mr * ldg + seg * 8;
      const float uu[8] = {sdv::bf16lo(u.x), sdv::bf16hi(u.x), sdv::bf16lo(u.y), sdv::bf16hi(u.y),
                           sdv::bf16lo(u.z), sdv::bf16hi(u.z), sdv::bf16lo(u.w), sdv::bf16hi(u.w)};
      uint16_t ob[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ob[e] = sdv::f32_to_bf16_rne(uu[e] + g[e]);
        vals[e] = sdv::bf16_to_f32(ob[e]);
        m = fmaxf(m, vals[e]);
      }
      uint4 o;
      o.x = (uint32_t)ob[0] | ((uint32_t)ob[1] << 16);
      o.y = (uint32_t)ob[2] | ((uint32_t)ob[3] << 16);
      o.z = (uint32_t)ob[4] | ((uint32_t)ob[5] << 16);
      o.w = (uint32_t)ob[6] | ((uint32_t)ob[7] << 16);
      sdv::st_nt(q_logits + off, o);
    }
    // row partial over the 16 lanes of this row: max, then sum relative to it
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    const float ref = exp_ref(m, c);
    if (live) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s += sdv::fast_exp2(fmaf(vals[e], c, -ref));
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 16);
    if (seg == 0 && r < R) partial[(size_t)r * n_tiles + tile] = make_float2(m, s);
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_markov_select(
    int gamma, int k, int V, int H, int rank_e, float c, uint64_t seed,
    const int64_t* __restrict__ pos0, const int32_t* __restrict__ x0,
    const uint16_t* __restrict__ E, const float* __restrict__ w,
    const float* __restrict__ hdot, const float2* __restrict__ partial, int n_tiles,
    const uint16_t* __restrict__ q_logits, int32_t* __restrict__ tokens,
    float* __restrict__ conf, int32_t* __restrict__ status) {
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
  if (tid == 0) {
    tokens[(size_t)r * gamma + (k - 1)] = s_tok;
    status[r] = st;
  }
}

size_t markov_ws_bytes(int R, int gamma, int V) {
  const size_t n_tiles = ((size_t)V + kTileN - 1) / kTileN;
  return sdv_align256((size_t)R * gamma * sizeof(float)) +
         sdv_align256((size_t)R * n_tiles * sizeof(float2));
}

}  // namespace

extern "C" size_t sd_markov_draft_workspace_size(int R, int gamma, int V, int rank) {
  (void)rank;
  if (R < 0 || gamma < 0 || V <= 0) return 0;
  return markov_ws_bytes(R, gamma, V);
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
  if (!workspace || workspace_bytes < markov_ws_bytes(R, gamma, V)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  if ((((uintptr_t)U | (uintptr_t)A | (uintptr_t)Ct | (uintptr_t)q_logits | (uintptr_t)h |
        (uintptr_t)w) & 15) != 0)
    return SD_EINVAL;

  const float c = sdv::kLog2e / temperature;
  char* p = (char*)workspace;
  float* hdot = (float*)p;
  p += sdv_align256((size_t)R * gamma * sizeof(float));
  float2* partial = (float2*)p;

  const int rows = R * gamma;
  if (H > 0) {
    SDV_TRY_LAUNCH(sdv::launch(k_hidden_dot, dim3((rows + 3) / 4), dim3(kThreads), 0, stream, h, H,
                               w, rows, hdot));
  } else {
    return SD_EINVAL;  // the confidence head needs a hidden state
  }
  const dim3 grid_bias(n_tiles, (R + kTileM - 1) / kTileM);
  for (int k = 1; k <= gamma; ++k) {
    SDV_TRY_LAUNCH(sdv::launch(k_markov_bias, grid_bias, dim3(kThreads), 0, stream, R, gamma, k, V,
                               rank, c, U, A, Ct, x0, (const int32_t*)tokens, q_logits, partial,
                               n_tiles));
    SDV_TRY_LAUNCH(sdv::launch(k_markov_select, dim3(R), dim3(kThreads), 0, stream, gamma, k, V, H,
                               rank_e, c, seed, pos0, x0, E, w, (const float*)hdot,
                               (const float2*)partial, n_tiles, (const uint16_t*)q_logits, tokens,
                               conf, status));
  }
  return SD_OK;
}
