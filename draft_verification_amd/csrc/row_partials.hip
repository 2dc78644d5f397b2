// The bandwidth pass of sd_verify: row statistics of every verify-batch row.
//
// Verification needs p = softmax(target row / T) and q = softmax(draft row / T)
// at the drafted tokens (speculative-decoding history page, "1.1 mechanism"),
// so the normaliser of every target and draft row in the batch is required;
// this is the one pass over the whole batch and it is bound by HBM.
//
// One 256-thread workgroup per (batch row, chunk group: one 16384-element
// chunk, or two consecutive ones of a bf16 row in a pass of many
// workgroups): each thread issues all of its 16-byte non-temporal loads
// together, then per chunk takes the max and sum 2^(x*c - fp32(max*c)) in
// registers, and each wave leaves one partial (max, sum) per chunk.  No
// LDS, no barrier.  Workgroups of rows outside the
// scheduled batch exit at once.  When the drafter hands over its rows'
// statistics the pass covers the target rows alone; when verification stops
// at each request's first rejection it runs once per round of positions,
// the later rounds over the list of requests still undecided.
#include "sdv_host.h"
#include "verify_common.h"

namespace {

using sdv::kChunk;
using sdv::kNegInf;
using sdv::kRowThreads;
using sdv::kRowWaves;

// One chunk held in registers: the partials of its four waves.
template <bool BF16>
__device__ __forceinline__ void chunk_partial(const sdv::RowPassArgs& a, const uint4* buf, int rs, int ch) {
  using VT = sdv::Vec<BF16>;
  constexpr int kVec = kChunk / VT::kElems / kRowThreads;
  const float c = a.c;
  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    float x[VT::kElems];
    VT::unpack(buf[k], x);
#pragma unroll
    for (int e = 0; e < VT::kElems; ++e) m = fmaxf(m, x[e]);
  }
  const float ref = sdv::exp_ref(m, c);
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
  const float wref = sdv::exp_ref(wm, c);
  const float ws = sdv::wave_sum((s == 0.0f) ? 0.0f : s * sdv::fast_exp2(ref - wref));
  if ((threadIdx.x & 63) == 0)
    a.partial[((size_t)rs * a.n_ch + ch) * kRowWaves + (threadIdx.x >> 6)] = make_float2(wm, ws);
}

// Chunk group g of one row: chunks NCH * g, ... (those inside the row).
template <bool BF16, int NCH>
__device__ __forceinline__ void row_chunks(const sdv::RowPassArgs& a, int r, int slot, int g) {
  using VT = sdv::Vec<BF16>;
  constexpr int kVec = kChunk / VT::kElems / kRowThreads;
  constexpr int kPassChunks = NCH;
  // the row's first index is requested with the request's length (one
  // round trip for both: the exit test reads it too, so it is not deferred
  // past the test); a negative one names no row and is skipped
  const int row0 = slot <= a.gmax ? a.tgt_row0[r] : a.drf_row0[r];
  const int L = sdv::clampi(a.ell[r], 0, a.gmax);
  if (!sdv::slot_in_batch(slot, a.gmax, L) || row0 < 0) return;
  const int rs = r * (2 * a.gmax + 1) + slot;  // row of the partials' layout
  const char* row = slot <= a.gmax ? a.tgt + ((int64_t)row0 + slot) * a.ld_bytes
                                   : a.drf + ((int64_t)row0 + (slot - a.gmax - 1)) * a.ld_bytes;
  const int ch0 = kPassChunks * g;
  const uint4 ninf = make_uint4(VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord, VT::kNegInfWord);
  uint4 buf[kPassChunks][kVec];
#pragma unroll
  for (int h = 0; h < kPassChunks; ++h) {
    const int e0 = (ch0 + h) * kChunk;
    const int nvec = ch0 + h < a.n_ch ? min(kChunk, a.V - e0) / VT::kElems : 0;
    const uint4* p = (const uint4*)(row + (int64_t)e0 * VT::kBytes);
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int v = threadIdx.x + k * kRowThreads;
      buf[h][k] = v < nvec ? sdv::ld_nt(p + v) : ninf;
    }
  }
  chunk_partial<BF16>(a, buf[0], rs, ch0);
  // Where the request's whole reserved block is in the batch, the next
  // chunk's reduction waits until this partial is stored (all of the wave's
  // loads are in by now): with every workgroup streaming, the pass runs
  // faster with that pause, which holds back new loads (measured: 249 us per
  // headline pass with it, 257 us without).  Where slots of the block are
  // outside the batch, their workgroups exit at once and the pass wants
  // every load in flight it can get (ragged step: 403 us without the pause
  // there, 416 us with it).
  if (kPassChunks > 1 && L == a.gmax) __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
#pragma unroll
  for (int h = 1; h < kPassChunks; ++h)
    if (ch0 + h < a.n_ch) chunk_partial<BF16>(a, buf[h], rs, ch0 + h);
}

// Item -> (request index, slot, chunk group) in the pass's ranges.
template <int NCH>
__device__ __forceinline__ void item_slot(const sdv::RowPassArgs& a, int item, int* ri, int* slot, int* g) {
  const int ng = sdv::pass_groups(a.n_ch, NCH);
  *g = item % ng;
  const int rl = item / ng;
  const int sl = rl % a.slots, nt = a.t_hi - a.t_lo;
  *ri = rl / a.slots;
  *slot = sl < nt ? a.t_lo + sl : a.gmax + a.d_lo + (sl - nt);
}

template <bool BF16, bool LIST, int NCH>
__global__ __launch_bounds__(kRowThreads) void k_row_partials(sdv::RowPassArgs a) {
  if (a.clear && blockIdx.x == 0 && threadIdx.x == 0) *a.clear = 0;
  int ri, slot, g;
  if constexpr (!LIST) {
    item_slot<NCH>(a, blockIdx.x, &ri, &slot, &g);
    row_chunks<BF16, NCH>(a, ri, slot, g);
  } else {  // the listed requests' items, strided over the grid
    const int n_items = *a.count * a.slots * sdv::pass_groups(a.n_ch, NCH);
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
      item_slot<NCH>(a, item, &ri, &slot, &g);
      row_chunks<BF16, NCH>(a, a.list[ri], slot, g);
    }
  }
}

}  // namespace

namespace sdv {

hipError_t launch_row_partials(bool bf16, const RowPassArgs& a, unsigned grid, hipStream_t stream) {
  const dim3 g(grid), b(kRowThreads);
  if (!bf16) {
    if (a.list) return launch(k_row_partials<false, true, 1>, g, b, 0, stream, a);
    return launch(k_row_partials<false, false, 1>, g, b, 0, stream, a);
  }
  if (a.chunks == 2) {
    if (a.list) return launch(k_row_partials<true, true, 2>, g, b, 0, stream, a);
    return launch(k_row_partials<true, false, 2>, g, b, 0, stream, a);
  }
  if (a.list) return launch(k_row_partials<true, true, 1>, g, b, 0, stream, a);
  return launch(k_row_partials<true, false, 1>, g, b, 0, stream, a);
}

}  // namespace sdv
