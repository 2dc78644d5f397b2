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
//   k_row_partials  (row_partials.hip) the bandwidth pass: one partial
//                   (max, sum 2^(x*c - ref)) per wave and 16384-element chunk
//                   of every batch row (of every target row when the drafter
//                   supplied its rows' (m, Z): it normalised q when it drew)
//   k_finish        one 1024-thread workgroup per request does the rest:
//                   combine the partials into (m, Z) per row, run every accept
//                   test at once, find the first rejection, write the accepted
//                   tokens; then the correction draw.  A rejection streams the
//                   rejected row pair once (16 waves, next block's loads in
//                   flight) for the sums of max(0, p - q) per 1024-element
//                   block, locates the block where the inverse CDF crosses
//                   u * sum(w) within one wave (a ballot over the lanes'
//                   running sums), and that wave scans the block.  A bonus
//                   draw locates its chunk from the first pass's partials and
//                   rescans only that chunk.
//   k_draw_sums     small batches of long rows only (too few requests to fill
//                   the CUs): k_finish records the draws, this kernel takes
//                   the block sums with many workgroups per rejected row
//                   pair, and a last k_finish launch locates and scans as
//                   above
//
// Verification that stops at each request's first rejection runs the
// bandwidth pass and the deciding half of k_finish in rounds of positions
// (up to 2, 6, 14, ...): a round decides the requests that rejected, failed
// or reached their bonus row and lists the others for the next round; the
// last round's k_finish decides the requests still listed and makes every
// draw at once.
//   k_alpha_sums,   only when the acceptance rates are asked for: sums of
//   k_alpha_total   min(p, q) per (request, position, chunk), then per row -
//                   the probability that the position is accepted, which is
//                   1 - TV(p, q), the confidence label of the DSpark summary
//                   ("2.1")
#include <algorithm>
#include <atomic>
#include <mutex>

#include "sdv_host.h"
#include "verify_common.h"

namespace {

using sdv::kChunk;
using sdv::kNegInf;
using sdv::kRowWaves;

constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kBlk = 1024;                          // elements per residual block
constexpr int kChunkBlocks = kChunk / kBlk;         // = kFinWaves: one block per wave
constexpr int kMaxSlots = 2 * SD_MAX_GAMMA + 1;
constexpr int kStagedParts = 4096;                  // partials of one request staged in LDS
constexpr int kLdsBlocks = 2048;                    // residual block sums kept in LDS (V <= 2M)
constexpr int kAlphaThreads = 256;
constexpr int kNone = 0x7FFFFFFF;
constexpr int kMaxRounds = 8;          // position rounds 2, 6, 14, ..., 510 > SD_MAX_GAMMA + 1
constexpr unsigned kListGrid = 4096;   // workgroups of a listed round's bandwidth pass
static_assert(kChunkBlocks == kFinWaves, "a bonus chunk is rescanned one block per wave");
static_assert(sdv::kMaxChunks <= kFinThreads, "chunk locate assumes one chunk per thread");
static_assert(SD_MAX_GAMMA < kFinThreads, "one accept test per thread");

// The correction draw a request was decided on.
struct DrawRec {
  int kind;              // 0: nothing to draw (the request failed), 1: residual, 2: target row,
                         // 3: not decided yet (listed for the next round)
  int n;                 // drafts accepted
  int st;                // status bits so far
  int pos;               // position of the drawn token
  float mct, izt, mcd, izd;  // the rows' references and fp32(1 / Z) (draft row: kind 1)
};

struct VerifyArgs {
  const char* tgt;
  const int32_t* tgt_row0;
  const char* drf;
  const int32_t* drf_row0;
  const float2* drf_stats;  // [R][gmax] (m, Z) of the draft rows, or null
  const int32_t* draft_tokens;
  const int32_t* ell;
  const int64_t* pos0;
  int32_t* n_accepted;
  int32_t* out_tokens;
  int32_t* status;
  float* probe_probs;
  float* row_stats;
  float* accept_prob;     // [R][gmax] or null
  const float2* partial;  // [R][S][n_ch][kRowWaves] from the bandwidth pass
  float* row_ref;         // [R][S] fp32(max * c) of every batch row
  double* row_z;          // [R][S] sum 2^(x*c - ref)
  double* bsum;           // [R][n_blk] residual mass per 1024-element block
  double* asum;           // [R][gmax][n_ch][kRowWaves] chunk sums of min(p, q)
  // Rounds (verification that stops at each request's first rejection): the
  // rows read so far are the target slots < cover and the draft positions
  // <= cover; `list`/`count` name the requests of this round (null: all),
  // and an undecided request is appended to next_list/next_count.
  const int32_t* list;
  const int32_t* count;
  int32_t* next_list;
  int32_t* next_count;
  int cover;              // gmax + 1 covers every row
  int stop_at_rejection;  // rows past the first rejection are not needed
  DrawRec* recs;          // [R] decided draws, when the draws run in a kernel of their own
  int64_t ld_bytes;
  uint64_t seed;
  float c;                // log2(e) / T
  float inv_t;
  int gmax;
  int V;
  int n_ch;
  int n_blk;
};

__device__ __forceinline__ int row_status(float M, double Z) {
  if (isnan(M) || isnan(Z) || M == __builtin_huge_valf()) return SD_ST_NONFINITE;
  if (M == kNegInf) return SD_ST_ZERO_Z;
  return 0;
}

// Weight of one element of the correction draw: residual max(0, p - q)
// (kind 1) or the unnormalised target law 2^(x*c - ref) (kind 2), in fp32
// from fp32 exponentials (their rounding already bounds the accuracy); every
// sum of weights is taken in fp64.
__device__ __forceinline__ float draw_weight(float xt, float xd, int kind, float c, float mct,
                                             float izt, float mcd, float izd) {
  const float et = sdv::fast_exp2(fmaf(xt, c, -mct));
  if (kind != 1) return et;
  const float ed = sdv::fast_exp2(fmaf(xd, c, -mcd));
  return fmaxf(0.0f, fmaf(et, izt, -(ed * izd)));
}

struct DrawParams {
  int kind;
  float c, mct, mcd;
  float izt, izd;  // fp32(1 / Z) of the target and draft rows (kind 1)
};

// One wave scans one 1024-element block held in registers (lane l holds
// vectors k*64 + l of the block, vocabulary order (k, lane, element)) for the
// first element whose running sum of weights exceeds `rem`.  Returns that
// element's row index, or kNone; *last gets the block's last index with
// positive weight (or -1).  Wave-uniform results.
template <bool BF16, int VL>
__device__ int wave_block_scan(const uint4 (&tv)[VL], const uint4 (&dv)[VL], int vbase,
                               const DrawParams& dp, double rem, int lane, int* last) {
  using VT = sdv::Vec<BF16>;
  double col[VL];
  int lst = -1;
#pragma unroll
  for (int k = 0; k < VL; ++k) {
    float xt[VT::kElems], xd[VT::kElems];
    VT::unpack(tv[k], xt);
    VT::unpack(dv[k], xd);
    double vs = 0.0;
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) {
      const double w = (double)draw_weight(xt[e], xd[e], dp.kind, dp.c, dp.mct, dp.izt, dp.mcd, dp.izd);
      vs += w;
      if (w > 0.0) lst = (vbase + k * 64 + lane) * VT::kElems + e;
    }
    col[k] = vs;
  }
  *last = -sdv::wave_min_i(-lst);
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < VL; ++k) {  // unrolled: the arrays stay in registers
    const double incl = sdv::wave_incl_scan_d(col[k], lane);
    const double c0 = run + (incl - col[k]);
    int hit = kNone;
    if (c0 <= rem && c0 + col[k] > rem) {
      float xt[VT::kElems], xd[VT::kElems];
      VT::unpack(tv[k], xt);
      VT::unpack(dv[k], xd);
      double cc = c0;
      for (int e = 0; e < VT::kElems; ++e) {
        cc += (double)draw_weight(xt[e], xd[e], dp.kind, dp.c, dp.mct, dp.izt, dp.mcd, dp.izd);
        if (cc > rem) {
          hit = (vbase + k * 64 + lane) * VT::kElems + e;
          break;
        }
      }
    }
    hit = sdv::wave_min_i(hit);
    if (hit != kNone) return hit;
    run += __shfl(incl, 63, 64);
  }
  return kNone;
}

// Inclusive prefix sum over the workgroup in thread order (every thread calls).
__device__ __forceinline__ double block_incl_scan(double v, int lane, int wave, double* s_w) {
  const double incl = sdv::wave_incl_scan_d(v, lane);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wave; ++w) off += s_w[w];
  __syncthreads();
  return off + incl;
}

// ---------------------------------------------------------------------------
// Request r, up to its correction draw: the rows' (m, Z), the accept tests
// and the decision, recorded in *rec: the draw to make (kind 1 or 2), a
// failure (kind 0, its outputs written) or no decision yet (kind 3, listed
// for the next round).
template <bool BF16>
__device__ __forceinline__ void finish_decide(const VerifyArgs& a, int r, DrawRec* rec) {
  using VT = sdv::Vec<BF16>;
  __shared__ float sRef[kMaxSlots];
  __shared__ double sZ[kMaxSlots];
  __shared__ float2 sPart[kStagedParts];
  __shared__ int s_rst[kMaxSlots];  // status bits of each unusable row
  __shared__ int s_st, s_jb, s_jstar, s_zero_q_upto;

  const int tid = threadIdx.x;
  const int gmax = a.gmax, S = 2 * gmax + 1, V = a.V;
  const int L = sdv::clampi(a.ell[r], 0, gmax);
  const int nparts = a.n_ch * kRowWaves;
  const float c = a.c;
  // rows read so far: target slots 0..nT-1, draft positions 1..Lt (the
  // positions tested in this round)
  const int Lt = min(L, a.cover);
  const int nT = min(L, a.cover - 1) + 1;
  const bool lazy = a.stop_at_rejection != 0;
  for (int i = tid; i < kMaxSlots; i += kFinThreads) s_rst[i] = 0;
  if (tid == 0) {
    s_st = 0;
    s_jb = kNone;
    s_jstar = Lt + 1;
    s_zero_q_upto = kNone;
  }

  // The accept tests' operands (thread j-1 tests position j: the drafted
  // token, its two logits and, when the drafter supplied it, the draft row's
  // (m, Z)) are requested first, then the partials.
  const int32_t* drafts = a.draft_tokens + (size_t)r * gmax;
  const int jt = tid + 1;
  int xj = -1;
  float ltj = 0.0f, ldj = 0.0f;
  float2 mzj = make_float2(0.0f, 0.0f);
  if (jt <= Lt) {
    xj = drafts[jt - 1];
    if (a.drf_stats) mzj = a.drf_stats[(size_t)r * gmax + (jt - 1)];
    if (xj >= 0 && xj < V) {
      ltj = VT::at(a.tgt + ((int64_t)a.tgt_row0[r] + (jt - 1)) * a.ld_bytes, xj);
      ldj = VT::at(a.drf + ((int64_t)a.drf_row0[r] + (jt - 1)) * a.ld_bytes, xj);
    }
  }

  // Stage the partials of the rows read (target slots 0..nT-1, then draft
  // slots gmax+1..gmax+Lt unless their statistics were supplied, i.e. local
  // row b) in LDS when they fit: one load each.
  const int nrows = a.drf_stats ? nT : nT + Lt;
  const bool staged = (long long)nrows * nparts <= kStagedParts;
  const float2* base = a.partial + (size_t)r * S * nparts;
  if (staged) {
    for (int i = tid; i < nrows * nparts; i += kFinThreads) {
      const int b = i / nparts, q = i % nparts;
      const int slot = b < nT ? b : gmax + 1 + (b - nT);
      sPart[i] = base[(size_t)slot * nparts + q];
    }
  }
  __syncthreads();

  // An unusable row fails the request: any row of the batch, or, when rows
  // past the first rejection are not needed, a row at or before it (the
  // first position whose target or draft row is unusable, s_jb, is kept;
  // target slot s serves position s + 1, the bonus row position L + 1).
  auto unusable = [&](int slot, int st) {
    if (!lazy) {
      atomicOr(&s_st, st);
    } else {
      s_rst[slot] = st;
      atomicMin(&s_jb, slot <= gmax ? slot + 1 : slot - gmax);
    }
  };

  // (m, Z) per row: groups of 16 lanes, one row per group at a time
  const int grp = tid >> 4, gl = tid & 15;
  for (int b = grp; b < nrows; b += kFinThreads / 16) {
    const int slot = b < nT ? b : gmax + 1 + (b - nT);
    const float2* pp = staged ? sPart + b * nparts : base + (size_t)slot * nparts;
    float M = kNegInf;
    for (int q = gl; q < nparts; q += 16) M = fmaxf(M, pp[q].x);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
    const float ref = sdv::exp_ref(M, c);
    double Z = 0.0;
    for (int q = gl; q < nparts; q += 16) {
      const float2 v = pp[q];
      if (v.y != 0.0f) Z += (double)v.y * (double)sdv::fast_exp2(sdv::exp_ref(v.x, c) - ref);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) Z += __shfl_xor(Z, o, 16);
    if (gl == 0) {
      sRef[slot] = ref;
      sZ[slot] = Z;
      a.row_ref[(size_t)r * S + slot] = ref;
      a.row_z[(size_t)r * S + slot] = Z;
      const int st = row_status(M, Z);
      if (st) unusable(slot, st);
      if (a.row_stats)
        ((float2*)a.row_stats)[(size_t)r * S + slot] = sdv::stats_report(M, ref, Z, a.inv_t);
    }
  }
  if (a.drf_stats && jt <= Lt) {  // the drafter's statistics of draft row jt
    const int slot = gmax + jt;
    float ref;
    double Z;
    const int st = sdv::stats_read(mzj, &ref, &Z);
    if (st) unusable(slot, st);
    sRef[slot] = ref;
    sZ[slot] = Z;
    a.row_ref[(size_t)r * S + slot] = ref;
    a.row_z[(size_t)r * S + slot] = Z;
    if (a.row_stats) ((float2*)a.row_stats)[(size_t)r * S + slot] = mzj;
  }
  __syncthreads();

  int32_t* out_tok = a.out_tokens + (size_t)r * (gmax + 1);
  auto fail = [&](int st) {  // the request fails: no token
    for (int t = tid; t <= gmax; t += kFinThreads) out_tok[t] = -1;
    if (tid == 0) {
      a.n_accepted[r] = 0;
      a.status[r] = st;
    }
  };
  if (s_st) {  // a needed row is unusable
    fail(s_st);
    rec->kind = 0;
    return;
  }
  const int jb = s_jb;  // kNone unless rows past the first rejection are not needed

  // every accept test at once (before the first unusable row); the chain
  // stops at the first rejection
  const int64_t pbase = a.pos0 ? a.pos0[r] : 0;
  if (jt <= Lt && jt < jb) {
    const int j = jt, x = xj;
    bool reject;
    if (x < 0 || x >= V) {
      reject = true;
    } else {
      const int ts = j - 1, ds = gmax + j;
      const double p = exp2((double)ltj * (double)c - (double)sRef[ts]) / sZ[ts];
      const double q = exp2((double)ldj * (double)c - (double)sRef[ds]) / sZ[ds];
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
  const bool rejected = jstar <= Lt;
  if (jb != kNone && !rejected) {  // an unusable row before any rejection
    fail(s_rst[jb - 1] | (jb <= gmax ? s_rst[gmax + jb] : 0));
    rec->kind = 0;
    return;
  }
  if (!rejected && L >= a.cover) {  // all accepted so far; the rest is not read yet
    if (tid == 0) a.next_list[atomicAdd(a.next_count, 1)] = r;
    rec->kind = 3;
    return;
  }
  const int n = rejected ? jstar - 1 : L;
  for (int t = tid; t <= gmax; t += kFinThreads) out_tok[t] = (t < n) ? drafts[t] : -1;
  int st = 0;
  if (s_zero_q_upto <= (rejected ? jstar : L)) st |= SD_ST_ZERO_Q;
  if (rejected) {
    const int x = drafts[jstar - 1];
    if (x < 0 || x >= V) st |= SD_ST_BAD_TOKEN;
  }

  const int pos = rejected ? jstar : L + 1;
  rec->kind = rejected ? 1 : 2;
  rec->n = n;
  rec->st = st;
  rec->pos = pos;
  rec->mct = sRef[pos - 1];
  rec->izt = (float)(1.0 / sZ[pos - 1]);
  rec->mcd = rejected ? sRef[gmax + jstar] : 0.0f;
  rec->izd = rejected ? (float)(1.0 / sZ[gmax + jstar]) : 1.0f;
}

// Per-lane part of one 1024-element block's residual mass, the block's two
// rows held in registers (lane l holds vectors k*64 + l): fp32 weights, fp64
// sum.
template <bool BF16, int VL>
__device__ __forceinline__ double block_lane_mass(const uint4 (&t)[VL], const uint4 (&d)[VL],
                                                  const DrawParams& dp) {
  using VT = sdv::Vec<BF16>;
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < VL; ++k) {
    float xt[VT::kElems], xd[VT::kElems];
    VT::unpack(t[k], xt);
    VT::unpack(d[k], xd);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e)
      acc += (double)draw_weight(xt[e], xd[e], 1, dp.c, dp.mct, dp.izt, dp.mcd, dp.izd);
  }
  return acc;
}

// The correction draw of request r (every thread of the workgroup): the
// residual max(0, p - q) of the rejected position or the target row after
// the last draft, by inverse CDF; writes the token, n_accepted and status.
// SUMS_READY: the residual's block sums are already in a.bsum (k_draw_sums).
template <bool BF16, bool SUMS_READY>
__device__ __forceinline__ void finish_draw(const VerifyArgs& a, int r, DrawRec rec) {
  using VT = sdv::Vec<BF16>;
  constexpr int VL = kBlk / VT::kElems / 64;  // vectors per lane per row of a block
  constexpr int kBlkVec = kBlk / VT::kElems;
  __shared__ double s_incl[kFinThreads];
  __shared__ double s_bs[kLdsBlocks];
  __shared__ double s_w[kFinWaves];
  __shared__ int s_owner, s_tok, s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gmax = a.gmax, S = 2 * gmax + 1, V = a.V;
  const int nparts = a.n_ch * kRowWaves;
  const float c = a.c;
  const int64_t pbase = a.pos0 ? a.pos0[r] : 0;
  int32_t* out_tok = a.out_tokens + (size_t)r * (gmax + 1);
  const int n = rec.n, pos = rec.pos;
  int st = rec.st;
  if (tid == 0) s_owner = kNone;  // read after the first prefix sum's barriers

  const double u = sdv::uniform24(a.seed, (uint64_t)r, (uint64_t)(pbase + pos), 2);
  const int tslot = pos - 1;
  const char* trow = a.tgt + ((int64_t)a.tgt_row0[r] + (pos - 1)) * a.ld_bytes;
  const char* drow = rec.kind == 1 ? a.drf + ((int64_t)a.drf_row0[r] + (pos - 1)) * a.ld_bytes : trow;
  DrawParams dp;
  dp.kind = rec.kind;
  dp.c = c;
  dp.mct = rec.mct;
  dp.izt = rec.izt;
  dp.mcd = rec.mcd;
  dp.izd = rec.izd;
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  const int nvec = V / VT::kElems;
  const uint4* tp = (const uint4*)trow;
  const uint4* dq = (const uint4*)drow;
  double* bsum = a.bsum + (size_t)r * a.n_blk;
  const int n_blk = a.n_blk;

  double target = 0.0;
  if (dp.kind == 1) {
    // Residual mass per block (unless k_draw_sums took it): wave w streams
    // blocks w, w + 16, ... with the next block's loads issued before the
    // current block is summed.  The block sums stay in LDS when they fit.
    double* bs = bsum;
    if constexpr (!SUMS_READY) {
      if (n_blk <= kLdsBlocks) bs = s_bs;
      // Blocks wholly inside the row stream through two register buffers in
      // turn, each block's loads issued before the previous block is
      // summed.  Their loads are never skipped (a prefetch past the wave's
      // last block reads the row's first 16 bytes, every lane the same, and
      // is not used), so the compiler counts the loads in flight exactly and
      // waits only for the block about to be summed.  The row's last block,
      // if partial, follows with bounds-checked loads.
      const int n_full = nvec / kBlkVec;
      auto load_full = [&](int b, bool use, uint4 (&t)[VL], uint4 (&d)[VL]) {
#pragma unroll
        for (int k = 0; k < VL; ++k) {
          const int v = use ? b * kBlkVec + k * 64 + lane : 0;
          t[k] = sdv::ld_nt(tp + v);
          d[k] = sdv::ld_nt(dq + v);
        }
      };
      auto sum_block = [&](int b, const uint4 (&t)[VL], const uint4 (&d)[VL]) {
        const double acc = sdv::wave_sum_d(block_lane_mass<BF16, VL>(t, d, dp));
        if (lane == 0) bs[b] = acc;
      };
      uint4 at[VL], ad[VL], bt[VL], bd[VL];
      load_full(wave, wave < n_full, at, ad);
      for (int b = wave; b < n_full; b += 2 * kFinWaves) {
        const int b1 = b + kFinWaves, b2 = b1 + kFinWaves;
        load_full(b1, b1 < n_full, bt, bd);
        sum_block(b, at, ad);
        if (b1 >= n_full) break;
        load_full(b2, b2 < n_full, at, ad);
        sum_block(b1, bt, bd);
      }
      if (n_blk > n_full && wave == n_full % kFinWaves) {  // the partial last block
#pragma unroll
        for (int k = 0; k < VL; ++k) {
          const int v = n_full * kBlkVec + k * 64 + lane;
          at[k] = v < nvec ? sdv::ld_nt(tp + v) : ninf;
          ad[k] = v < nvec ? sdv::ld_nt(dq + v) : ninf;
        }
        sum_block(n_full, at, ad);
      }
      __syncthreads();  // block sums of every wave visible to the workgroup
    }

    // Locate the block where the inverse CDF crosses u * sum(w) within one
    // wave: lane l owns the contiguous run of blocks [l*per, (l+1)*per).
    // Every wave takes the same sums in the same order, so all agree on the
    // total; with mass present wave 0 locates and scans alone, and without
    // it all waves go on to the draw from p below.
    const int per = (n_blk + 63) / 64;
    const int b0 = min(lane * per, n_blk), b1 = min(b0 + per, n_blk);
    double tot = 0.0;
    for (int b = b0; b < b1; ++b) tot += bs[b];
    const double incl = sdv::wave_incl_scan_d(tot, lane);
    const double total = __shfl(incl, 63, 64);
    if (total > 0.0) {
      if (wave != 0) return;
      target = u * total;
      // the first lane whose running sum passes the target (lane 63's is the
      // total, which u < 1 keeps above it) walks its run
      const unsigned long long passed = __ballot(incl > target);
      const int owner = passed ? __ffsll((long long)passed) - 1 : 63;
      const double before = __shfl_up(incl, 1, 64);
      int blk = -1;
      double rem = __builtin_huge_val();
      if (lane == owner) {
        double acc = lane == 0 ? 0.0 : before;
        int lastpos = -1;
        for (int b = b0; b < b1; ++b) {
          const double w = bs[b];
          if (w > 0.0) lastpos = b;
          if (acc + w > target) {
            blk = b;
            rem = target - acc;
            break;
          }
          acc += w;
        }
        if (blk < 0) blk = lastpos;  // rounding: last block with mass, its last element
      }
      blk = __shfl(blk, owner, 64);
      rem = __shfl(rem, owner, 64);
      if (blk < 0) {  // no block with mass (not reachable when total > 0)
        if (lane == 0) {
          out_tok[n] = -1;
          a.n_accepted[r] = n;
          a.status[r] = st;
        }
        return;
      }
      uint4 tv[VL], dv[VL];
#pragma unroll
      for (int k = 0; k < VL; ++k) {
        const int v = blk * kBlkVec + k * 64 + lane;
        tv[k] = v < nvec ? tp[v] : ninf;
        dv[k] = v < nvec ? dq[v] : ninf;
      }
      int last;
      int tok = wave_block_scan<BF16, VL>(tv, dv, blk * kBlkVec, dp, rem, lane, &last);
      if (tok == kNone) tok = last;
      if (lane == 0) {
        out_tok[n] = tok;
        a.n_accepted[r] = n;
        a.status[r] = st;
      }
      return;
    }
    // empty residual: draw from p_j* instead
    st |= SD_ST_ZERO_RESIDUAL;
    dp.kind = 2;
    dp.mcd = 0.0f;
    dp.izd = 1.0f;
    drow = trow;
    dq = tp;
  }

  // Draw from the target law of slot tslot: chunk sums from the first pass
  // (thread t = chunk t), the crossing chunk by a workgroup prefix sum, then
  // each wave sums one 1024-element block of that chunk and the wave holding
  // the crossing scans its block.
  const int n_ch = a.n_ch;
  double tot = 0.0;
  if (tid < n_ch) {
    const float2* pp = a.partial + ((size_t)r * S + tslot) * nparts + (size_t)tid * kRowWaves;
    for (int w = 0; w < kRowWaves; ++w) {
      const float2 q = pp[w];
      if (q.y != 0.0f) tot += (double)q.y * exp2((double)sdv::exp_ref(q.x, c) - (double)dp.mct);
    }
  }
  const double incl = block_incl_scan(tot, lane, wave, s_w);
  s_incl[tid] = incl;
  __syncthreads();
  target = u * s_incl[kFinThreads - 1];
  if (incl > target && tid < n_ch) atomicMin(&s_owner, tid);
  if (tid == 0) {
    s_last = -1;
    s_tok = kNone;
  }
  __syncthreads();
  int ch = s_owner;
  double rem;
  if (ch == kNone) {  // rounding put the target past the end: last chunk with mass
    int lp = -1;
    for (int t = 0; t < n_ch; ++t)
      if (s_incl[t] > (t == 0 ? 0.0 : s_incl[t - 1])) lp = t;
    ch = lp;
    rem = __builtin_huge_val();
  } else {
    rem = target - (ch == 0 ? 0.0 : s_incl[ch - 1]);
  }
  if (ch < 0) {  // no mass anywhere (not reachable for a finite row)
    if (tid == 0) {
      out_tok[n] = -1;
      a.n_accepted[r] = n;
      a.status[r] = st;
    }
    return;
  }
  const int blk = ch * kChunkBlocks + wave;
  uint4 tv[VL], dv[VL];
#pragma unroll
  for (int k = 0; k < VL; ++k) {
    const int v = blk * kBlkVec + k * 64 + lane;
    tv[k] = v < nvec ? tp[v] : ninf;
    dv[k] = ninf;
  }
  double wsum = 0.0;
#pragma unroll
  for (int k = 0; k < VL; ++k) {
    float xt[VT::kElems];
    VT::unpack(tv[k], xt);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) wsum += (double)sdv::fast_exp2(fmaf(xt[e], c, -dp.mct));
  }
  wsum = sdv::wave_sum_d(wsum);
  if (lane == 0) s_w[wave] = wsum;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += s_w[w];
  // the waves' intervals [before, before + wsum) partition the chunk's mass
  const bool mine = before <= rem && before + wsum > rem;
  int last;
  // every wave scans (for its last positive element); only the owner's hit counts
  const int tok = wave_block_scan<BF16, VL>(tv, dv, blk * kBlkVec, dp, mine ? rem - before : -1.0,
                                            lane, &last);
  if (lane == 0) {
    if (mine && tok != kNone) s_tok = tok;
    if (last >= 0) atomicMax(&s_last, last);
  }
  __syncthreads();
  if (tid == 0) {
    out_tok[n] = s_tok != kNone ? s_tok : s_last;  // rounding: last element with mass
    a.n_accepted[r] = n;
    a.status[r] = st;
  }
}

// The finishing kernel, one workgroup per request: decide and draw at once
// (every row read in one pass), or in rounds: decide only, recording the
// draws, in every round but the last; the last decides the requests still
// listed and makes every draw at once.  For small batches the draws are
// spread over the chip instead: the deciding phases record every draw
// (kDecide over all requests, kFinalRec), k_draw_sums takes the residuals'
// block sums with many workgroups per request, and kPick makes the draws.
enum { kFused = 0, kDecide = 1, kFinal = 2, kFinalRec = 3, kPick = 4 };

template <bool BF16, int PHASE>
__global__ __launch_bounds__(kFinThreads) void k_finish(VerifyArgs a) {
  DrawRec rec;
  int r;
  if constexpr (PHASE == kPick) {
    r = (int)blockIdx.x;
    rec = a.recs[r];
    if (rec.kind == 1 || rec.kind == 2) finish_draw<BF16, true>(a, r, rec);
    return;
  } else if constexpr (PHASE == kFinal || PHASE == kFinalRec) {
    r = (int)blockIdx.x;
    rec = a.recs[r];
    if (rec.kind == 3) {  // listed for this round
      finish_decide<BF16>(a, r, &rec);
      if constexpr (PHASE == kFinalRec) {
        if (threadIdx.x == 0) a.recs[r] = rec;
      }
    }
    if constexpr (PHASE == kFinalRec) return;
  } else {
    if (a.list && (int)blockIdx.x >= *a.count) return;
    r = a.list ? a.list[blockIdx.x] : (int)blockIdx.x;
    finish_decide<BF16>(a, r, &rec);
    if constexpr (PHASE == kDecide) {
      if (threadIdx.x == 0) a.recs[r] = rec;
      return;
    }
  }
  if (rec.kind == 1 || rec.kind == 2) finish_draw<BF16, false>(a, r, rec);
}

// Block sums of the residual draws recorded in a.recs: workgroup
// (r, part) sums blocks [8 part, 8 part + 8) of request r's rejected row pair
// into a.bsum, two blocks per wave, both loaded before either is summed.
constexpr int kSumThreads = 256;
constexpr int kSumWaves = kSumThreads / 64;
constexpr int kSumBlocks = 2 * kSumWaves;  // residual blocks per workgroup

template <bool BF16>
__global__ __launch_bounds__(kSumThreads) void k_draw_sums(VerifyArgs a, int parts) {
  using VT = sdv::Vec<BF16>;
  constexpr int VL = kBlk / VT::kElems / 64;
  constexpr int kBlkVec = kBlk / VT::kElems;
  const int r = (int)(blockIdx.x / (unsigned)parts), part = (int)(blockIdx.x % (unsigned)parts);
  const DrawRec rec = a.recs[r];
  if (rec.kind != 1) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pos = rec.pos;
  const uint4* tp = (const uint4*)(a.tgt + ((int64_t)a.tgt_row0[r] + (pos - 1)) * a.ld_bytes);
  const uint4* dq = (const uint4*)(a.drf + ((int64_t)a.drf_row0[r] + (pos - 1)) * a.ld_bytes);
  DrawParams dp;
  dp.kind = 1;
  dp.c = a.c;
  dp.mct = rec.mct;
  dp.izt = rec.izt;
  dp.mcd = rec.mcd;
  dp.izd = rec.izd;
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  const int nvec = a.V / VT::kElems;
  uint4 t[2][VL], d[2][VL];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = part * kSumBlocks + wave + i * kSumWaves;
#pragma unroll
    for (int k = 0; k < VL; ++k) {
      const int v = b * kBlkVec + k * 64 + lane;  // v < nvec implies b < n_blk
      t[i][k] = v < nvec ? sdv::ld_nt(tp + v) : ninf;
      d[i][k] = v < nvec ? sdv::ld_nt(dq + v) : ninf;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = part * kSumBlocks + wave + i * kSumWaves;
    const double acc = sdv::wave_sum_d(block_lane_mass<BF16, VL>(t[i], d[i], dp));
    if (lane == 0 && b < a.n_blk) a.bsum[(size_t)r * a.n_blk + b] = acc;
  }
}

// ---------------------------------------------------------------------------
// Acceptance rate of position j: sum over the vocabulary of min(p_j, q_j).
template <bool BF16>
__global__ __launch_bounds__(sdv::kRowThreads) void k_alpha_sums(VerifyArgs a) {
  using VT = sdv::Vec<BF16>;
  constexpr int kThreads = sdv::kRowThreads;
  constexpr int kVec = kChunk / VT::kElems / kThreads;
  const int gmax = a.gmax, S = 2 * gmax + 1;
  const int ch = blockIdx.x % a.n_ch;
  const int rj = blockIdx.x / a.n_ch;
  const int j = rj % gmax + 1, r = rj / gmax;
  const int L = sdv::clampi(a.ell[r], 0, gmax);
  if (j > L || (a.status[r] & (SD_ST_NONFINITE | SD_ST_ZERO_Z))) return;
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
    a.asum[(((size_t)r * gmax + (j - 1)) * a.n_ch + ch) * kRowWaves + (threadIdx.x >> 6)] = acc;
}

// Per-row totals of the min(p, q) chunk sums; 0 past l_r and for a failed
// request.
__global__ __launch_bounds__(kAlphaThreads) void k_alpha_total(VerifyArgs a, int R) {
  const int i = blockIdx.x * kAlphaThreads + threadIdx.x;
  if (i >= R * a.gmax) return;
  const int r = i / a.gmax, j = i % a.gmax + 1;
  const int L = sdv::clampi(a.ell[r], 0, a.gmax);
  double t = 0.0;
  if (j <= L && !(a.status[r] & (SD_ST_NONFINITE | SD_ST_ZERO_Z))) {
    const double* q = a.asum + ((size_t)r * a.gmax + (j - 1)) * a.n_ch * kRowWaves;
    for (int k = 0; k < a.n_ch * kRowWaves; ++k) t += q[k];
  }
  a.accept_prob[i] = (float)t;
}

size_t partial_bytes(int R, int gmax, int V) {
  const size_t n_ch = ((size_t)V + kChunk - 1) / kChunk;
  return sdv_align256((size_t)R * (2 * (size_t)gmax + 1) * n_ch * kRowWaves * sizeof(float2));
}

size_t verify_ws_bytes(int R, int gmax, int V) {
  const size_t n_ch = ((size_t)V + kChunk - 1) / kChunk;
  const size_t n_blk = ((size_t)V + kBlk - 1) / kBlk;
  const size_t S = 2 * (size_t)gmax + 1;
  return partial_bytes(R, gmax, V) + sdv_align256((size_t)R * S * sizeof(float)) +
         sdv_align256((size_t)R * S * sizeof(double)) +
         sdv_align256((size_t)R * n_blk * sizeof(double)) +
         sdv_align256((size_t)R * gmax * n_ch * kRowWaves * sizeof(double)) +
         sdv_align256((size_t)kMaxRounds * (R + 1) * sizeof(int32_t)) +
         sdv_align256((size_t)R * sizeof(DrawRec));
}

// Rounds of positions when verification stops at the first rejection: the
// rows of positions up to 2, 6, 14, ... are read in turn, each round only
// for the requests that accepted every position so far.
int next_cover(int cover) { return 2 * cover + 2; }

// Full-pass items (request x slot x chunk) from which a bf16 pass takes two
// chunks per workgroup.
#ifndef SDV_PAIRED_PASS_MIN_ITEMS
#define SDV_PAIRED_PASS_MIN_ITEMS 16384
#endif
constexpr long long kPairedPassMinItems = SDV_PAIRED_PASS_MIN_ITEMS;

// Draws spread over the chip: at most this many requests (measured: the two
// extra launches cost more than they save once the requests fill the CUs),
// and rows of at least this many residual blocks (measured, graph-replayed
// steps: V = 1024 fp32 at R = 4, 37.4 us spread against 32.8 us in the
// request's workgroup; V = 32000 bf16 (32 blocks) at R = 64, 40.4 against
// 36.9 us; V = 151936 (149 blocks) is faster spread at every R up to 128).
constexpr int kWideDrawMaxR = 128;
constexpr int kWideDrawMinBlk = 64;

// The finishing launches of the last round: PHASE is kFused (one round) or
// kFinal.
template <bool BF16, int PHASE>
int launch_finish(hipStream_t stream, int R, const VerifyArgs& a) {
  if (R <= kWideDrawMaxR && a.n_blk >= kWideDrawMinBlk && (PHASE == kFused || PHASE == kFinal)) {
    constexpr int kRec = PHASE == kFused ? kDecide : kFinalRec;
    SDV_TRY_LAUNCH(sdv::launch(k_finish<BF16, kRec>, dim3(R), dim3(kFinThreads), 0, stream, a));
    const int parts = (a.n_blk + kSumBlocks - 1) / kSumBlocks;
    SDV_TRY_LAUNCH(sdv::launch(k_draw_sums<BF16>, dim3((unsigned)((long long)R * parts)),
                               dim3(kSumThreads), 0, stream, a, parts));
    SDV_TRY_LAUNCH(sdv::launch(k_finish<BF16, kPick>, dim3(R), dim3(kFinThreads), 0, stream, a));
  } else {
    SDV_TRY_LAUNCH(sdv::launch(k_finish<BF16, PHASE>, dim3(R), dim3(kFinThreads), 0, stream, a));
  }
  if (a.accept_prob && a.gmax > 0) {
    SDV_TRY_LAUNCH(sdv::launch(k_alpha_sums<BF16>, dim3((unsigned)((long long)R * a.gmax * a.n_ch)),
                               dim3(sdv::kRowThreads), 0, stream, a));
    const unsigned g = (unsigned)(((long long)R * a.gmax + kAlphaThreads - 1) / kAlphaThreads);
    SDV_TRY_LAUNCH(sdv::launch(k_alpha_total, dim3(g), dim3(kAlphaThreads), 0, stream, a, R));
  }
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
                         const int32_t* drf_row0, const float* drf_stats, const int32_t* draft_tokens,
                         const int32_t* ell, int32_t* n_accepted, int32_t* out_tokens,
                         int32_t* status, float* probe_probs, float* row_stats,
                         float* accept_prob, int options, void* workspace, size_t workspace_bytes,
                         hipEvent_t prof_start, hipEvent_t prof_stop) {
  if (R < 0 || gamma_max < 0 || V < 8 || (V % 8) != 0 || ld < V || (ld % 8) != 0) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA || V > SD_MAX_VOCAB) return SD_EUNSUPPORTED;
  if (dtype != SD_DTYPE_F32 && dtype != SD_DTYPE_BF16) return SD_EINVAL;
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf())) return SD_EINVAL;
  if ((prof_start == nullptr) != (prof_stop == nullptr)) return SD_EINVAL;
  if ((options & ~SD_VERIFY_STOP_AT_REJECTION) != 0) return SD_EINVAL;
  const bool lazy = (options & SD_VERIFY_STOP_AT_REJECTION) != 0;
  if (lazy && accept_prob) return SD_EINVAL;  // acceptance rates need every row
  if (R == 0) return SD_OK;
  if (!tgt_logits || !tgt_row0 || !drf_row0 || !ell || !n_accepted || !out_tokens || !status)
    return SD_EINVAL;
  if (gamma_max > 0 && (!drf_logits || !draft_tokens)) return SD_EINVAL;
  if (!workspace || workspace_bytes < verify_ws_bytes(R, gamma_max, V)) return SD_ERANGE;
  if (((uintptr_t)workspace & 255) != 0) return SD_EINVAL;
  if ((((uintptr_t)tgt_logits) & 15) != 0 || (drf_logits && (((uintptr_t)drf_logits) & 15) != 0))
    return SD_EINVAL;
  if ((((uintptr_t)drf_stats) & 7) != 0 || (((uintptr_t)row_stats) & 7) != 0) return SD_EINVAL;
  const int n_ch = (V + kChunk - 1) / kChunk;
  const long long items = (long long)R * (2 * gamma_max + 1) * n_ch;  // the largest pass
  if (items > 0xFFFFFFFFLL / sdv::kRowThreads) return SD_EUNSUPPORTED;  // work-items of one launch
  const int64_t ld_bytes = (int64_t)ld * (dtype == SD_DTYPE_BF16 ? 2 : 4);
  const float c = sdv::kLog2e / temperature;
  const char* drf = (const char*)(drf_logits ? drf_logits : tgt_logits);
  const size_t S = 2 * (size_t)gamma_max + 1;
  const int n_blk = (V + kBlk - 1) / kBlk;

  char* p = (char*)workspace;
  float2* partial = (float2*)p;
  p += partial_bytes(R, gamma_max, V);

  sdv::RowPassArgs ra;
  ra.tgt = (const char*)tgt_logits;
  ra.tgt_row0 = tgt_row0;
  ra.drf = drf;
  ra.drf_row0 = drf_row0;
  ra.ell = ell;
  ra.partial = partial;
  ra.ld_bytes = ld_bytes;
  ra.c = c;
  ra.gmax = gamma_max;
  ra.V = V;
  ra.n_ch = n_ch;
  ra.list = nullptr;
  ra.count = nullptr;
  ra.clear = nullptr;
  // Two chunks of a bf16 row per workgroup once the full pass has many items
  // (measured at the headline size: 249 against 258 us per pass; with the
  // 2176 items of R = 64, gamma = 8, V = 32000, two chunks were slower).
  ra.chunks = (dtype == SD_DTYPE_BF16 && items >= kPairedPassMinItems) ? 2 : 1;
  // target slots [t_lo, t_hi) and draft positions [d_lo, d_hi] of one pass
  auto set_range = [&](int t_lo, int t_hi, int d_lo, int d_hi) {
    if (drf_stats) d_hi = d_lo - 1;  // the drafter's statistics replace the draft rows
    ra.t_lo = t_lo;
    ra.t_hi = t_hi;
    ra.d_lo = d_lo;
    ra.d_hi = d_hi;
    ra.slots = (t_hi - t_lo) + (d_hi >= d_lo ? d_hi - d_lo + 1 : 0);
  };

  VerifyArgs a;
  a.tgt = (const char*)tgt_logits;
  a.tgt_row0 = tgt_row0;
  a.drf = drf;
  a.drf_row0 = drf_row0;
  a.drf_stats = (const float2*)drf_stats;
  a.draft_tokens = draft_tokens;
  a.ell = ell;
  a.pos0 = pos0;
  a.n_accepted = n_accepted;
  a.out_tokens = out_tokens;
  a.status = status;
  a.probe_probs = probe_probs;
  a.row_stats = row_stats;
  a.accept_prob = accept_prob;
  a.partial = partial;
  a.row_ref = (float*)p;
  p += sdv_align256((size_t)R * S * sizeof(float));
  a.row_z = (double*)p;
  p += sdv_align256((size_t)R * S * sizeof(double));
  a.bsum = (double*)p;
  p += sdv_align256((size_t)R * n_blk * sizeof(double));
  a.asum = (double*)p;
  p += sdv_align256((size_t)R * gamma_max * n_ch * kRowWaves * sizeof(double));
  int32_t* lists = (int32_t*)p;                          // [kMaxRounds][R]
  int32_t* counts = lists + (size_t)kMaxRounds * R;      // [kMaxRounds]
  p += sdv_align256((size_t)kMaxRounds * (R + 1) * sizeof(int32_t));
  a.recs = (DrawRec*)p;                                  // [R]
  a.list = nullptr;
  a.count = nullptr;
  a.next_list = nullptr;
  a.next_count = nullptr;
  a.cover = gamma_max + 1;
  a.stop_at_rejection = lazy ? 1 : 0;
  a.ld_bytes = ld_bytes;
  a.seed = seed;
  a.c = c;
  a.inv_t = 1.0f / temperature;
  a.gmax = gamma_max;
  a.V = V;
  a.n_ch = n_ch;
  a.n_blk = n_blk;

  const bool bf16 = dtype == SD_DTYPE_BF16;
  if (!lazy) {  // every row of the batch in one pass
    set_range(0, gamma_max + 1, 1, gamma_max);
    if (prof_start) SDV_TRY_LAUNCH(hipEventRecord(prof_start, stream));
    SDV_TRY_LAUNCH(sdv::launch_row_partials(bf16, ra, (unsigned)((long long)R * ra.slots * sdv::pass_groups(n_ch, ra.chunks)),
                                            stream));
    if (prof_stop) SDV_TRY_LAUNCH(hipEventRecord(prof_stop, stream));
    return bf16 ? launch_finish<true, kFused>(stream, R, a) : launch_finish<false, kFused>(stream, R, a);
  }
  // Rounds of positions: round k reads target slots [prev, cover) and draft
  // positions (prev, cover] of the requests still undecided (every request
  // in round 0), then decides those that rejected, failed, or reached their
  // bonus row, and lists the others for round k + 1.  The last round decides
  // the requests still listed and makes the draws of all at once (with one
  // round, the one-pass kernel).
  int prev = 0;
  for (int k = 0; prev < gamma_max + 1; ++k) {
    const int cover = std::min(next_cover(prev), gamma_max + 1);
    const bool last = cover == gamma_max + 1;
    set_range(prev, cover, prev + 1, std::min(cover, gamma_max));
    ra.list = k ? lists + (size_t)k * R : nullptr;
    ra.count = k ? counts + k : nullptr;
    ra.clear = last ? nullptr : counts + k + 1;
    // the listed rounds cover a fraction of the requests: one chunk each
    ra.chunks = (bf16 && k == 0 && (long long)R * ra.slots * n_ch >= kPairedPassMinItems) ? 2 : 1;
    const long long n_items = (long long)R * ra.slots * sdv::pass_groups(n_ch, ra.chunks);
    const unsigned grid = k ? (unsigned)std::min<long long>(n_items, kListGrid) : (unsigned)n_items;
    if (k == 0 && prof_start) SDV_TRY_LAUNCH(hipEventRecord(prof_start, stream));
    if (grid > 0) SDV_TRY_LAUNCH(sdv::launch_row_partials(bf16, ra, grid, stream));
    if (k == 0 && prof_stop) SDV_TRY_LAUNCH(hipEventRecord(prof_stop, stream));
    a.cover = cover;
    a.list = ra.list;
    a.count = ra.count;
    a.next_list = last ? nullptr : lists + (size_t)(k + 1) * R;
    a.next_count = last ? nullptr : counts + k + 1;
    int rc;
    if (!last)
      rc = bf16 ? launch_finish<true, kDecide>(stream, R, a) : launch_finish<false, kDecide>(stream, R, a);
    else if (k == 0)
      rc = bf16 ? launch_finish<true, kFused>(stream, R, a) : launch_finish<false, kFused>(stream, R, a);
    else
      rc = bf16 ? launch_finish<true, kFinal>(stream, R, a) : launch_finish<false, kFinal>(stream, R, a);
    if (rc != SD_OK) return rc;
    prev = cover;
  }
  return SD_OK;
}

// ---------------------------------------------------------------------------
// sd_verify_noalloc: sd_verify with its workspace held by the library, for
// callers that cannot allocate (code under graph capture, serving loops that
// forbid allocation).  The workspace is one file-scope device array; each GPU
// holds its own copy at its own address, looked up once per device with that
// device current.  Every workspace word a call reads is first written by the
// same call's kernels (the round counters are zeroed by a kernel of the round
// before), so no call depends on what an earlier one left there; calls that
// overlap on one GPU share the array and race.
namespace {

constexpr size_t kNoAllocScratchBytes = SD_VERIFY_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kNoAllocMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kNoAllocMaxDevices];
std::mutex g_scratch_mu;

// The scratch array's device address on the current device (null on error).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int sd_verify_noalloc(hipStream_t stream, int R, int gamma_max, int V, int ld, int dtype,
                                 float temperature, uint64_t seed, const int64_t* pos0,
                                 const void* tgt_logits, const int32_t* tgt_row0, const void* drf_logits,
                                 const int32_t* drf_row0, const float* drf_stats,
                                 const int32_t* draft_tokens, const int32_t* ell, int32_t* n_accepted,
                                 int32_t* out_tokens, int32_t* status, float* probe_probs,
                                 float* row_stats, float* accept_prob, int options) {
  if (R < 0 || gamma_max < 0 || V < 8) return SD_EINVAL;
  if (gamma_max > SD_MAX_GAMMA || V > SD_MAX_VOCAB) return SD_EUNSUPPORTED;
  if (R == 0) return SD_OK;
  if (verify_ws_bytes(R, gamma_max, V) > kNoAllocScratchBytes) return SD_ERANGE;
  void* ws = scratch_on_current_device();
  if (!ws) return SD_ELAUNCH;
  return sd_verify(stream, R, gamma_max, V, ld, dtype, temperature, seed, pos0, tgt_logits, tgt_row0,
                   drf_logits, drf_row0, drf_stats, draft_tokens, ell, n_accepted, out_tokens, status,
                   probe_probs, row_stats, accept_prob, options, ws, kNoAllocScratchBytes, nullptr,
                   nullptr);
}
