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
//   k_head_bias      the only dense contraction: G = A_k[x_{k-1}] . C_k as a
//                    bf16 MFMA GEMM (M = requests, N = vocabulary, K = rank),
//                    fused with + U_k, bf16 rounding, the q_logits store and a
//                    per-(row, 128-column tile) partial (max, sum 2^(L*c - ref));
//                    loader waves stream C_k into LDS ahead of the MFMA
//                    waves, which gather their rows A_k[x_{k-1}] while the
//                    first stage loads, load their own U_k vectors into
//                    registers and store L through a small LDS buffer as
//                    whole cache lines
//   k_markov_select  one workgroup per request: combine tile partials,
//                    locate the inverse-CDF tile, rescan 128 logits, emit x_k
//                    (and, when asked, the row's (m, Z), which spares the
//                    verifier a pass over the row)
// plus, after the block, one k_confidence launch for the confidence of every
// drafted position (it needs x_{k-1}, never anything later in the loop).
//
// sd_rnn_draft runs the same loop for the RNN head: k_rnn_init computes s_1,
// the bias kernel takes the state's three bf16 terms as its A rows against
// the shared readout C, and the select kernel also advances the state.
#include <algorithm>

#include "sdv_common.h"
#include "sdv_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 128;  // vocabulary columns per tile (two 64-column stages)
constexpr int kTileM = 128;  // requests per bias workgroup (8 compute waves x 16)
constexpr int kMaxRank = 256;
static_assert(kMaxRank / 2 <= kThreads, "an RNN state of d <= kMaxRank / 2: one element per thread");
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

__device__ __forceinline__ float exp_ref(float m, float c) { return m == kNegInf ? 0.0f : m * c; }

// ---------------------------------------------------------------------------
// The bias product G = A . C_k (M = requests, N = vocabulary, K = kdim) with
// v_mfma_f32_16x16x32_bf16, fused with + U_k, the bf16 rounding, the q_logits
// store and one partial (max, sum 2^(L*c - ref)) per (request, 128-column
// tile).  NSPLIT = 1, the Markov head: row r of A is A_k[x_{k-1}], gathered
// from the table at the start (zeros for an invalid token).  NSPLIT = 3, the
// RNN head: Ag[r] holds the state as three bf16 terms, hi = bf16(s),
// mid = bf16(s - hi), lo = bf16(s - hi - mid), all multiplied by the same C
// fragments; each term holds the next 8 bits of the fp32 significand, so the
// three carry the state exactly (normal values).
//
// The loads are pipelined by specialised waves.  One workgroup per CU takes
// one 128-column tile per round i, tile i * G + (blockIdx.x + i) % G (G =
// gridDim.x), in 64-column stages: a round sweeps one contiguous stretch of
// C_k and U_k, and the offset that grows with i moves each XCD's tiles
// across the memory.  (Measured: with tile i * G + blockIdx.x, the
// workgroups of two of the eight XCDs ended 3 to 5 us after the others on
// every call, and the call took 6 % longer.)
// Four loader waves copy each stage's 64 C rows from HBM straight into LDS
// (global_load_lds, 16 bytes per lane, no registers) three stages ahead of
// eight compute waves, in a ring of four, and every wave meets once per
// stage at a barrier.  A loader wave issues only these copies, so its vmcnt
// counts them in order and "all but the newest two stages done" is an exact
// wait.  Compute wave w owns requests [m0 + 16w, m0 + 16w + 16) and keeps
// their A rows (the B operand) in registers for the whole step; it loads its
// own part of each U tile straight into registers two stages ahead (U is
// read once, by the lane that adds it).  The product is taken transposed,
// G^T = C rows . A^T, with the C rows of a stage assigned to the four 16-row
// MFMA blocks so that lane l holds, in its 16 accumulators, the vocabulary
// columns [8q, 8q + 8) and [32 + 8q, 32 + 8q + 8) of the stage for request
// l % 16 (q = l / 16): each lane reads U as two 16-byte vectors (four lanes
// cover 64 contiguous bytes of a request).  L goes out through a 2 KB
// wave-private LDS buffer: the lanes put their vectors in, then read them
// back so that each store instruction writes eight requests' 128 contiguous
// bytes (whole cache lines), non-temporal.  (Measured per call: stores of
// 64-byte pieces straight from the accumulator layout, 0.601-0.606 ms
// Markov and 0.556 ms RNN; whole lines through the caches 0.588-0.590 and
// 0.556-0.558; whole lines non-temporal 0.586 and 0.534-0.535.)
//
// LDS per stage: C rows [64][kdim] bf16 with the 16-byte chunks of row j
// XOR-swizzled (c_swz) so that the sixteen rows one fragment read touches
// land on distinct chunk columns.  The L staging rows are padded to 144
// bytes.
constexpr int kWsCompute = 8;
constexpr int kWsLoaders = 4;
constexpr int kWsThreads = (kWsCompute + kWsLoaders) * 64;
constexpr int kSubN = 64;
constexpr int kStages = 4;                       // LDS ring of C stages
constexpr int kAhead = kStages - 1;              // stages in flight ahead of the one consumed
constexpr int kStageC = kSubN * kMaxRank * 2;    // 32 KB at the largest rank
constexpr int kStRow = 144;                      // L staging row: 128 bytes + 16 of padding
constexpr int kStLds = kWsCompute * 16 * kStRow;  // one 16-row buffer per compute wave
constexpr int kWsLds = kStages * kStageC + kStLds;
static_assert(kWsLds <= 160 * 1024, "one bias workgroup per CU: the LDS of a CU");
static_assert(kWsCompute * 16 == kTileM, "one 16-request block per compute wave");
static_assert(kSubN == 64, "four 16-row MFMA blocks per stage");

typedef __attribute__((address_space(3))) void lds_void_t;

// Cache-policy operand of global_load_lds on gfx950: the nt bit.
constexpr int kCPolNonTemporal = 2;

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// vmcnt(n) for n = copies a loader wave may leave outstanding: a multiple of
// kb = kdim / 32 (1..8) copies per stage, at most kAhead - 1 stages.
template <int N>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n == N) wait_vmcnt<N>();
    else wait_vmcnt_upto<N - 1>(n);
  }
}
__device__ __forceinline__ void wait_vmcnt_rt(int n) { wait_vmcnt_upto<8 * (kAhead - 1)>(n); }

// Stage row of the C fragment that lane rl of MFMA block mb supplies: the
// block's output row 4q + i then holds vocabulary column
// 32 (mb / 2) + 8q + 4 (mb % 2) + i of the stage.
__device__ __forceinline__ int c_row(int mb, int rl) {
  return 32 * (mb >> 1) + 8 * (rl >> 2) + 4 * (mb & 1) + (rl & 3);
}

// Chunk swizzle of the C rows: XOR with bits 0-1 and 3-4 of the row (the
// bits that tell apart the sixteen rows of one fragment read), limited to
// the largest power of two (at most 16) that divides the chunks per row.
__device__ __forceinline__ int c_swz(int row, int cpr) {
  const int p2 = cpr & -cpr;
  return ((row & 3) | (((row >> 3) & 3) << 2)) & ((p2 < 16 ? p2 : 16) - 1);
}

// 32-element K slices of the A rows a compute wave keeps: rank <= kMaxRank
// (Markov), state d <= kMaxRank / 2 (RNN).
template <int NSPLIT>
constexpr int kHeadKs = NSPLIT == 1 ? kMaxRank / 32 : kMaxRank / 64;

template <int NSPLIT>
__global__ __launch_bounds__(kWsThreads) void k_head_bias(
    int R, int gamma, int k, int V, int kdim, float c, const uint16_t* __restrict__ U,
    const uint16_t* __restrict__ Ct, size_t ct_stride, const uint16_t* __restrict__ Ag,
    const uint16_t* __restrict__ A, const int32_t* __restrict__ x0,
    const int32_t* __restrict__ tokens, uint16_t* __restrict__ q_logits,
    float2* __restrict__ partial, int n_tiles) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * kTileM;
  const int kb = kdim / 32;
  const int cpr = kdim / 8;  // 16-byte chunks per C row
  const uint16_t* Ck = Ct + (size_t)(k - 1) * ct_stride;
  // the tile of round i; rounds 0 .. last - 1 are whole, round `last` holds
  // the n_tiles - last * G tiles left (gridDim.x <= n_tiles)
  const int G = gridDim.x;
  auto tile_at = [&](int i) { return i * G + ((int)blockIdx.x + i) % G; };
  const int last = (n_tiles - 1) / G;
  const int my_tiles = last + (tile_at(last) < n_tiles ? 1 : 0);
  const int H = 2 * my_tiles;  // two stages per tile
  auto stage_col = [&](int h) {  // first vocabulary column of stage h
    return tile_at(h >> 1) * kTileN + (h & 1) * kSubN;
  };

  // Cache policy of the C copies: the Markov head's C_k serves one step, so
  // it streams past the caches (non-temporal); the RNN head's readout C is
  // the same at every step and keeps the default policy, under which
  // repeated steps find it in the last-level cache.  U is read once: always
  // non-temporal.
  constexpr int kCPolicy = NSPLIT == 1 ? kCPolNonTemporal : 0;

  if (wave >= kWsCompute) {
    // ---------------- loader waves ----------------
    // Stage h is copied kAhead stages ahead of its use into ring slot
    // h % kStages; "stage h+1 landed" is "at most the copies of the stages
    // issued after it outstanding", since a loader wave issues nothing else.
    // A stage is kb * 4 regions of 1 KB (64 lanes x 16 bytes); loader wave
    // lw copies regions lw, lw + 4, ... .  The stage row and swizzled chunk
    // of each of its copies are the same in every stage: worked out once.
    const int lw = wave - kWsCompute;
    int cp_row[kMaxRank / 32], cp_off[kMaxRank / 32];
#pragma unroll
    for (int ic = 0; ic < kMaxRank / 32; ++ic) {
      const int sid = (ic * kWsLoaders + lw) * 64 + lane;
      const int row = sid / cpr;
      cp_row[ic] = row;
      cp_off[ic] = ((sid % cpr) ^ c_swz(row, cpr)) * 8;
    }
    auto issue = [&](int h) {
      const int v0 = stage_col(h);
      unsigned char* st = lds + (h % kStages) * kStageC;
#pragma unroll
      for (int ic = 0; ic < kMaxRank / 32; ++ic) {  // C rows v0 .. v0+63
        if (ic < kb) {
          const int v = min(v0 + cp_row[ic], V - 1);
          __builtin_amdgcn_global_load_lds((const void*)(Ck + (size_t)v * kdim + cp_off[ic]),
                                           (lds_void_t*)(st + (ic * kWsLoaders + lw) * 1024), 16, 0,
                                           kCPolicy);
        }
      }
    };
    const int first = H < kAhead ? H : kAhead;
    for (int h = 0; h < first; ++h) issue(h);
    wait_vmcnt_rt((first - 1 > 0 ? first - 1 : 0) * kb);  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    for (int h = 0; h < H; ++h) {
      if (h + kAhead < H) issue(h + kAhead);
      // stage h+1 landed: the stages issued after it may be outstanding
      const int last = (h + kAhead < H ? h + kAhead : H - 1);
      const int after = last - (h + 1);
      wait_vmcnt_rt(after > 0 ? after * kb : 0);
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  // ---------------- compute waves ----------------
  const int rl = lane & 15, q = lane >> 4;
  const int req = wave * 16 + rl;
  const int r = m0 + req;
  const bool rvalid = r < R;
  const size_t urow = ((size_t)(rvalid ? r : 0) * gamma + (k - 1)) * V;
  // this lane's U vectors of stage h: columns [8q, 8q+8) and [32+8q, 32+8q+8)
  auto load_u = [&](int h, uint4 (&u)[2]) {
    const int v0 = stage_col(h);
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const int col = v0 + 32 * hv + 8 * q;
      u[hv] = (rvalid && col < V) ? sdv::ld_nt(U + urow + col) : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 ua[2], ub[2], uc[2];  // U of three consecutive stages
  constexpr int kKs = kHeadKs<NSPLIT>;
  uint4 agf[NSPLIT][kKs];
  if (A != nullptr) {  // Markov: gather A_k[x_{k-1}] here, under the first stages' loads
    const int x = rvalid ? (k == 1 ? x0[r] : tokens[(size_t)r * gamma + (k - 2)]) : -1;
    const bool xv = x >= 0 && x < V;  // no bias for an invalid token
    const uint16_t* arow = A + ((size_t)(k - 1) * V + (xv ? x : 0)) * kdim;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
      agf[0][ks] = (xv && ks < kb) ? *(const uint4*)(arow + ks * 32 + q * 8) : make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp)
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
        agf[sp][ks] = (rvalid && ks < kb)
                          ? *(const uint4*)(Ag + (size_t)r * NSPLIT * kdim + (sp * kb + ks) * 32 + q * 8)
                          : make_uint4(0, 0, 0, 0);
  }
  // The A rows are in before any U load is issued: every later wait for
  // vector memory is then for U alone, counted exactly across the loop.
  wait_vmcnt<0>();
  if (H > 0) load_u(0, ua);
  if (H > 1) load_u(1, ub);
  // The compute waves meet the loaders at plain barriers: the loaders have
  // waited for their copies before arriving, and a compute wave's LDS reads
  // of a stage are complete once its MFMAs have consumed them, so no memory
  // fence is needed (one would also wait for the U loads still in flight).
  __builtin_amdgcn_s_barrier();  // stage 0 landed
  float pm = kNegInf, ps = 0.0f;  // the first half's partial of the current tile

  // Stage h: the product from the C rows in LDS, then the epilogue from the
  // lane's U vectors u; ends at the barrier that frees the stage's slot.
  auto stage = [&](int h, const uint4 (&u)[2]) {
    const int t = tile_at(h >> 1);
    const int v0 = stage_col(h);
    const unsigned char* st = lds + (h % kStages) * kStageC;
    unsigned char* stg = lds + kStages * kStageC + wave * 16 * kStRow;
    floatx4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      if (ks < kb) {
        uint4 a[4];  // the four row blocks' fragments, read together
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int row = c_row(mb, rl);
          const int ch = (ks * 4 + q) ^ c_swz(row, cpr);
          a[mb] = *(const uint4*)(st + (row * cpr + ch) * 16);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int sp = 0; sp < NSPLIT; ++sp)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[mb]), as_bf16x8(agf[sp][ks]),
                                                              acc[mb], 0, 0, 0);
      }
    }
    // epilogue: L = bf16(U + G); vector hv holds blocks 2hv (columns +0..3)
    // and 2hv + 1 (columns +4..7) of columns v0 + 32hv + 8q
    float m = kNegInf;
    float vals[2][8];
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const int col = v0 + 32 * hv + 8 * q;
      const floatx4 g0 = acc[2 * hv], g1 = acc[2 * hv + 1];
      const uint4 uu = u[hv];
      uint4 o;
      o.x = pack_bf16_rne(sdv::bf16lo(uu.x) + g0[0], sdv::bf16hi(uu.x) + g0[1]);
      o.y = pack_bf16_rne(sdv::bf16lo(uu.y) + g0[2], sdv::bf16hi(uu.y) + g0[3]);
      o.z = pack_bf16_rne(sdv::bf16lo(uu.z) + g1[0], sdv::bf16hi(uu.z) + g1[1]);
      o.w = pack_bf16_rne(sdv::bf16lo(uu.w) + g1[2], sdv::bf16hi(uu.w) + g1[3]);
      vals[hv][0] = sdv::bf16lo(o.x);
      vals[hv][1] = sdv::bf16hi(o.x);
      vals[hv][2] = sdv::bf16lo(o.y);
      vals[hv][3] = sdv::bf16hi(o.y);
      vals[hv][4] = sdv::bf16lo(o.z);
      vals[hv][5] = sdv::bf16hi(o.z);
      vals[hv][6] = sdv::bf16lo(o.w);
      vals[hv][7] = sdv::bf16hi(o.w);
      *(uint4*)(stg + rl * kStRow + 16 * (4 * hv + q)) = o;  // chunk 4hv + q of row rl
      if (rvalid && col < V) {  // V % 8 == 0: a vector is all in or all out
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, vals[hv][i]);
      }
    }
    // A wave's LDS accesses are performed in order, so the reads below see
    // the writes above, and the next stage's writes come after these reads.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {  // rows 8 s2 .. 8 s2 + 7, eight lanes per row
      const int row = 8 * s2 + (lane >> 3), ch = lane & 7;
      const uint4 w = *(const uint4*)(stg + row * kStRow + 16 * ch);
      const int rr = m0 + wave * 16 + row;
      const int col = v0 + 8 * ch;
      if (rr < R && col < V) sdv::st_nt(q_logits + ((size_t)rr * gamma + (k - 1)) * V + col, w);
    }
    __builtin_amdgcn_wave_barrier();
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const float ref = exp_ref(m, c);
    float s = 0.0f;
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      if (rvalid && v0 + 32 * hv + 8 * q < V) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s += sdv::fast_exp2(fmaf(vals[hv][i], c, -ref));
      }
    }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if ((h & 1) == 0) {
      pm = m;
      ps = s;
    } else if (q == 0 && rvalid) {  // both halves of tile t: one partial
      const float M = fmaxf(pm, m);
      const float REF = exp_ref(M, c);
      float S = 0.0f;
      if (ps != 0.0f) S += ps * sdv::fast_exp2(exp_ref(pm, c) - REF);
      if (s != 0.0f) S += s * sdv::fast_exp2(ref - REF);
      partial[(size_t)r * n_tiles + t] = make_float2(M, S);
    }
    __builtin_amdgcn_s_barrier();  // this stage is consumed; the loaders may refill its slot
  };

  // three stages per trip, so that the U vectors rotate through named
  // registers (each loaded two stages before its use)
  for (int h = 0; h < H; h += 3) {
    if (h + 2 < H) load_u(h + 2, uc);
    stage(h, ua);
    if (h + 1 < H) {
      if (h + 3 < H) load_u(h + 3, ua);
      stage(h + 1, ub);
    }
    if (h + 2 < H) {
      if (h + 4 < H) load_u(h + 4, ub);
      stage(h + 2, uc);
    }
  }
}

// ---------------------------------------------------------------------------
// The RNN head's tables and the state the next step's bias multiplies.
struct NextRows {
  int rank;                 // state size d
  const uint16_t* W;        // W [d][d]
  const uint16_t* Es;       // E_s [V][d]
  float* state;             // [R][d]
  uint16_t* Ag;             // [R][3d]: the state as three bf16 terms
};

// RNN: row o = threadIdx.x of W times the state s_k in LDS (0 for o >= d).
// It does not depend on x_k, so the select kernel takes it early.
__device__ float rnn_w_times_state(const NextRows& nr, const float* s_s) {
  const int o = threadIdx.x, d = nr.rank;
  float acc = 0.0f;
  if (o < d) {
    const uint16_t* wr = nr.W + (size_t)o * d;
    for (int i = 0; i < d; i += 8) {
      const uint4 q = *(const uint4*)(wr + i);
      acc += sdv::bf16lo(q.x) * s_s[i] + sdv::bf16hi(q.x) * s_s[i + 1] +
             sdv::bf16lo(q.y) * s_s[i + 2] + sdv::bf16hi(q.y) * s_s[i + 3] +
             sdv::bf16lo(q.z) * s_s[i + 4] + sdv::bf16hi(q.z) * s_s[i + 5] +
             sdv::bf16lo(q.w) * s_s[i + 6] + sdv::bf16hi(q.w) * s_s[i + 7];
    }
  }
  return acc;
}

// Element o of a state as the three bf16 terms the bias kernel multiplies:
// hi = bf16(s), mid = bf16(s - hi), lo = bf16(s - hi - mid) at row offsets
// 0, d and 2d (each subtraction is exact in fp32).
__device__ __forceinline__ void split_state(uint16_t* row, int d, int o, float s) {
  const uint16_t hi = sdv::f32_to_bf16_rne(s);
  const float r1 = s - sdv::bf16_to_f32(hi);
  const uint16_t mid = sdv::f32_to_bf16_rne(r1);
  row[o] = hi;
  row[d + o] = mid;
  row[2 * d + o] = sdv::f32_to_bf16_rne(r1 - sdv::bf16_to_f32(mid));
}

// RNN, once x_k is known: s_{k+1} = tanh(W s_k + E_s[x_k]) in fp32 (no
// embedding term for an invalid token), kept in state[r] and written to Ag[r]
// as its three bf16 terms; ws = (W s_k)[threadIdx.x].
__device__ void rnn_next_state(const NextRows& nr, int r, int V, int tok, float ws) {
  const int d = nr.rank, o = threadIdx.x;  // d <= kThreads
  if (o < d) {
    float acc = ws;
    if (tok >= 0 && tok < V) acc += sdv::bf16_to_f32(nr.Es[(size_t)tok * d + o]);
    const float sn = tanhf(acc);
    nr.state[(size_t)r * d + o] = sn;
    split_state(nr.Ag + (size_t)r * 3 * d, d, o, sn);
  }
}

// Critical path: the tile partials and x_{k-1} (one round trip), the
// crossing tile's logits (a second), and for the RNN head the next state (a
// third); W s_k is computed while the tile's logits are in flight.  Tile
// masses are taken as the verifier combines its partials: fp32 exponentials
// of fp32 exponent differences, summed in fp64.  The confidences wait for
// the end of the block (k_confidence): nothing in the loop needs them.
template <bool RNN>
__global__ __launch_bounds__(kThreads) void k_markov_select(
    int gamma, int k, int V, float c, float inv_t, uint64_t seed, const int64_t* __restrict__ pos0,
    const int32_t* __restrict__ x0, const float2* __restrict__ partial, int n_tiles,
    const uint16_t* __restrict__ q_logits, NextRows nr, int32_t* __restrict__ tokens,
    float2* __restrict__ q_stats, int32_t* __restrict__ status) {
  __shared__ float s_s[kMaxRank];
  __shared__ float s_red[kThreads / 64];
  __shared__ double s_redd[kThreads / 64];
  __shared__ int s_tile;
  __shared__ double s_tgt;
  __shared__ float s_tref;
  __shared__ int s_tok, s_claim;

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xp = (k == 1) ? x0[r] : tokens[(size_t)r * gamma + (k - 2)];
  // this thread's run of tile partials
  const float2* pp = partial + (size_t)r * n_tiles;
  const int per = (n_tiles + kThreads - 1) / kThreads;
  const int t0 = tid * per;
  constexpr int kPre = 4;
  float2 pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i)
    pre[i] = (i < per && t0 + i < n_tiles) ? pp[t0 + i] : make_float2(kNegInf, 0.0f);
  if constexpr (RNN) {  // the state the next step advances
    for (int i = tid; i < nr.rank; i += kThreads) s_s[i] = nr.state[(size_t)r * nr.rank + i];
  }
  int st = (k == 1) ? 0 : status[r];
  if (!(xp >= 0 && xp < V)) st |= SD_ST_BAD_TOKEN;

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
  auto tile_mass = [&](float2 q) {
    return q.y != 0.0f ? (double)q.y * (double)sdv::fast_exp2(exp_ref(q.x, c) - REF) : 0.0;
  };
  double mass[kPre];  // the preloaded tiles' masses, kept for the walk
  double own = 0.0;
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    mass[i] = tile_mass(pre[i]);  // 0 for the padding entries
    own += mass[i];
  }
  for (int i = kPre; i < per; ++i)
    if (t0 + i < n_tiles) own += tile_mass(pp[t0 + i]);
  const double incl = sdv::wave_incl_scan_d(own, lane);
  if (lane == 63) s_redd[wave] = incl;
  if (tid == 0) { s_tile = -1; s_tok = -1; s_claim = 0x7FFFFFFF; }
  __syncthreads();
  double excl = incl - own;
  double Z = 0.0;
  for (int ww = 0; ww < kThreads / 64; ++ww) {
    if (ww < wave) excl += s_redd[ww];
    Z += s_redd[ww];
  }

  int bad = 0;
  if (isnan(M) || isnan(Z) || M == __builtin_huge_valf()) bad = SD_ST_NONFINITE;
  else if (M == kNegInf) bad = SD_ST_ZERO_Z;
  // the row's normaliser, for the verifier
  if (q_stats && tid == 0) q_stats[(size_t)r * gamma + (k - 1)] = sdv::stats_report(M, REF, Z, inv_t);
  const int64_t pbase = pos0 ? pos0[r] : 0;
  const double u = sdv::uniform24(seed, (uint64_t)r, (uint64_t)(pbase + k), 0);
  const double target = u * Z;
  if (!bad) {
    // the thread whose tile run contains the crossing walks its tiles (the
    // lowest such thread, should rounding make two runs claim it)
    const bool claims = excl <= target && excl + own > target;
    if (claims) atomicMin(&s_claim, tid);
    __syncthreads();
    if (tid == s_claim) {
      double cum = excl;
      bool done = false;
#pragma unroll
      for (int i = 0; i < kPre; ++i) {
        if (!done && i < per && t0 + i < n_tiles) {
          const double s = mass[i];
          if (cum + s > target && s > 0.0) {
            s_tile = t0 + i;
            s_tgt = target - cum;
            s_tref = exp_ref(pre[i].x, c);
            done = true;
          } else {
            cum += s;
          }
        }
      }
      for (int i = kPre; !done && i < per && t0 + i < n_tiles; ++i) {
        const float2 q = pp[t0 + i];
        const double s = tile_mass(q);
        if (cum + s > target && s > 0.0) {
          s_tile = t0 + i;
          s_tgt = target - cum;
          s_tref = exp_ref(q.x, c);
          done = true;
        } else {
          cum += s;
        }
      }
    }
    __syncthreads();
    // every thread reads the claim's result before thread 0 may rewrite it
    // below, so the branch (and its barriers) is taken by all or by none
    const bool missed = s_tile < 0;
    if (missed) {  // rounding pushed the target past the end: last tile with mass
      __syncthreads();
      if (tid == 0) {
        for (int t = n_tiles - 1; t >= 0; --t)
          if (pp[t].y > 0.0f) {
            s_tile = t;
            s_tref = exp_ref(pp[t].x, c);
            break;
          }
        s_tgt = __builtin_huge_val();
      }
      __syncthreads();
    }
  }
  const int tile = bad ? -1 : s_tile;

  // wave 0 requests the tile's 128 logits (2 per lane) ...
  const size_t rowoff = ((size_t)r * gamma + (k - 1)) * V;
  const int n0 = tile * kTileN;
  float lg[2] = {0.0f, 0.0f};
  if (wave == 0 && tile >= 0) {
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int idx = n0 + lane * 2 + e2;
      if (idx < V) lg[e2] = sdv::bf16_to_f32(q_logits[rowoff + idx]);
    }
  }
  // ... while the RNN head multiplies its state
  float ws = 0.0f;
  if constexpr (RNN) ws = rnn_w_times_state(nr, s_s);
  if (bad) {
    if (tid == 0) {
      tokens[(size_t)r * gamma + (k - 1)] = -1;
      status[r] = st | bad;
    }
    if (RNN && k < gamma) rnn_next_state(nr, r, V, -1, ws);  // no valid token to carry forward
    return;
  }

  // rescan the tile's logits: weights relative to the tile's own reference,
  // scaled into the global frame by the factor its mass was taken with
  if (wave == 0 && tile >= 0) {
    const float tref = s_tref;
    const double scale = (double)sdv::fast_exp2(tref - REF);
    const double tgt_in = s_tgt;
    double wv[2];
    int idx[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      idx[e2] = n0 + lane * 2 + e2;
      wv[e2] = idx[e2] < V ? (double)sdv::fast_exp2(fmaf(lg[e2], c, -tref)) * scale : 0.0;
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
  if (RNN && k < gamma) rnn_next_state(nr, r, V, tok, ws);
}

// Confidence head for every drafted position once the block's tokens are
// known: conf[r][k-1] = sigmoid(w[0:H] . h[r][k-1] + w[H:] . E[x_{k-1}]), with
// x_0 the anchor and no embedding term for a token outside [0, V) (a
// position after a failed row).  One wave per (r, k).
__global__ __launch_bounds__(kThreads) void k_confidence(int rows, int gamma, int V, int H, int rank_e,
                                                         const uint16_t* __restrict__ h,
                                                         const uint16_t* __restrict__ E,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ x0,
                                                         const int32_t* __restrict__ tokens,
                                                         float* __restrict__ conf) {
  const int row = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int r = row / gamma, k = row % gamma + 1;
  const int xp = k == 1 ? x0[r] : tokens[(size_t)r * gamma + (k - 2)];
  const uint4* hp = (const uint4*)(h + (size_t)row * H);
  const float4* w4 = (const float4*)w;
  auto dot8 = [](uint4 q, float4 w0, float4 w1) {
    return sdv::bf16lo(q.x) * w0.x + sdv::bf16hi(q.x) * w0.y + sdv::bf16lo(q.y) * w0.z +
           sdv::bf16hi(q.y) * w0.w + sdv::bf16lo(q.z) * w1.x + sdv::bf16hi(q.z) * w1.y +
           sdv::bf16lo(q.w) * w1.z + sdv::bf16hi(q.w) * w1.w;
  };
  // lane sums vectors lane, lane + 64, ... in that order, four loads at a time
  float acc = 0.0f;
  int v = lane;
  for (; v + 3 * 64 < H / 8; v += 4 * 64) {
    uint4 q[4];
    float4 wa[4], wb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      q[u] = hp[v + 64 * u];
      wa[u] = w4[2 * (v + 64 * u)];
      wb[u] = w4[2 * (v + 64 * u) + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += dot8(q[u], wa[u], wb[u]);
  }
  for (; v < H / 8; v += 64) acc += dot8(hp[v], w4[2 * v], w4[2 * v + 1]);
  float e = 0.0f;
  if (xp >= 0 && xp < V) {
    const uint16_t* er = E + (size_t)xp * rank_e;
    int i = lane;
    for (; i + 3 * 64 < rank_e; i += 4 * 64) {
      uint16_t x[4];
      float wx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = er[i + 64 * u];
        wx[u] = w[H + i + 64 * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) e += wx[u] * sdv::bf16_to_f32(x[u]);
    }
    for (; i < rank_e; i += 64) e += w[H + i] * sdv::bf16_to_f32(er[i]);
  }
  const float z = sdv::wave_sum(acc) + sdv::wave_sum(e);
  if (lane == 0) conf[row] = 1.0f / (1.0f + expf(-z));
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
    split_state(Ag + (size_t)r * 3 * d, d, o, sn);
  }
}

// Workspace: tile partials [R][n_tiles] float2, and for the RNN head the
// split state [R][arow = 3d] bf16 and the state [R][d] fp32.
size_t head_ws_bytes(int R, int, int V, int arow, int d) {
  const size_t n_tiles = ((size_t)V + kTileN - 1) / kTileN;
  return sdv_align256((size_t)R * n_tiles * sizeof(float2)) +
         sdv_align256((size_t)R * arow * sizeof(uint16_t)) +
         sdv_align256((size_t)R * d * sizeof(float));
}
size_t markov_ws_bytes(int R, int gamma, int V, int) { return head_ws_bytes(R, gamma, V, 0, 0); }
size_t rnn_ws_bytes(int R, int gamma, int V, int d) { return head_ws_bytes(R, gamma, V, 3 * d, d); }

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
// then the select kernel (which also prepares the next step's rows); then
// the confidences of the whole block.
template <int NSPLIT>
int run_head(hipStream_t stream, int R, int gamma, int V, int kdim, size_t ct_stride,
             float temperature, uint64_t seed, const int64_t* pos0, const uint16_t* U,
             const uint16_t* A, const uint16_t* Ct, const int32_t* x0, const uint16_t* h, int H,
             const uint16_t* E, int rank_e, const float* w, float2* partial, const NextRows& nr,
             int32_t* tokens, uint16_t* q_logits, float* q_stats, float* conf, int32_t* status) {
  const float c = sdv::kLog2e / temperature, inv_t = 1.0f / temperature;
  const int n_tiles = (V + kTileN - 1) / kTileN;
  int dev = 0, n_cu = 0;
  SDV_TRY_LAUNCH(hipGetDevice(&dev));
  SDV_TRY_LAUNCH(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  SDV_TRY_LAUNCH(hipFuncSetAttribute((const void*)k_head_bias<NSPLIT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kWsLds));
  const dim3 grid_bias(std::min(n_tiles, std::max(n_cu, 1)), (R + kTileM - 1) / kTileM);
  for (int k = 1; k <= gamma; ++k) {
    SDV_TRY_LAUNCH(sdv::launch(k_head_bias<NSPLIT>, grid_bias, dim3(kWsThreads), kWsLds, stream, R,
                               gamma, k, V, kdim, c, U, Ct, ct_stride, (const uint16_t*)nr.Ag, A, x0,
                               (const int32_t*)tokens, q_logits, partial, n_tiles));
    SDV_TRY_LAUNCH(sdv::launch(k_markov_select<NSPLIT != 1>, dim3(R), dim3(kThreads), 0, stream, gamma,
                               k, V, c, inv_t, seed, pos0, x0, (const float2*)partial, n_tiles,
                               (const uint16_t*)q_logits, nr, tokens, (float2*)q_stats, status));
  }
  const int rows = R * gamma;
  SDV_TRY_LAUNCH(sdv::launch(k_confidence, dim3((rows + kThreads / 64 - 1) / (kThreads / 64)),
                             dim3(kThreads), 0, stream, rows, gamma, V, H, rank_e, h, E, w, x0,
                             (const int32_t*)tokens, conf));
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
                               float* q_stats, float* conf, int32_t* status, void* workspace,
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
        (uintptr_t)w) & 15) != 0 || ((uintptr_t)q_stats & 7) != 0)
    return SD_EINVAL;

  float2* partial = (float2*)workspace;
  const NextRows nr{rank, nullptr, nullptr, nullptr, nullptr};  // unused: no recurrent state
  return run_head<1>(stream, R, gamma, V, rank, (size_t)V * rank, temperature, seed, pos0, U, A, Ct,
                     x0, h, H, E, rank_e, w, partial, nr, tokens, q_logits, q_stats, conf, status);
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
                            float* q_stats, float* conf, int32_t* status, void* workspace,
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
        (uintptr_t)w) & 15) != 0 || ((uintptr_t)q_stats & 7) != 0)
    return SD_EINVAL;

  const int n_tiles = (V + kTileN - 1) / kTileN;
  char* p = (char*)workspace;
  float2* partial = (float2*)p;
  p += sdv_align256((size_t)R * n_tiles * sizeof(float2));
  uint16_t* Ag = (uint16_t*)p;
  p += sdv_align256((size_t)R * 3 * d * sizeof(uint16_t));
  const NextRows nr{d, W, Es, (float*)p, Ag};

  SDV_TRY_LAUNCH(sdv::launch(k_rnn_init, dim3(R), dim3(kThreads), 0, stream, R, V, d, Es, x0, nr.state,
                             nr.Ag));
  return run_head<3>(stream, R, gamma, V, d, 0, temperature, seed, pos0, U, nullptr, Ct, x0, h, H, E,
                     rank_e, w, partial, nr, tokens, q_logits, q_stats, conf, status);
}
