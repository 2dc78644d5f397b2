// Definitions shared by the two halves of sd_verify: the bandwidth pass over
// every batch row (row_partials.hip) and the per-request finishing kernels
// (verify.hip).
#pragma once

#include "sdv_common.h"

namespace sdv {

constexpr int kRowThreads = 256;                   // bandwidth-pass workgroup
constexpr int kRowWaves = kRowThreads / 64;        // partials per (row, chunk)
constexpr int kChunk = 16384;                      // elements per chunk of a row
// Chunks of one row per bandwidth-pass workgroup (1 or 2), all their loads
// issued together: the items of a pass are (request, slot, chunk group).
__host__ __device__ inline int pass_groups(int n_ch, int chunks) { return (n_ch + chunks - 1) / chunks; }
constexpr int kMaxChunks = SD_MAX_VOCAB / kChunk;
constexpr float kNegInf = -__builtin_huge_valf();

// 16-byte vector of logits -> floats.  bf16: 8 values, fp32: 4 values.
template <bool BF16>
struct Vec;
template <>
struct Vec<true> {
  static constexpr int kElems = 8;
  static constexpr int kBytes = 2;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  SDV_DEV static void unpack(const uint4& v, float* x) {
    x[0] = bf16lo(v.x); x[1] = bf16hi(v.x);
    x[2] = bf16lo(v.y); x[3] = bf16hi(v.y);
    x[4] = bf16lo(v.z); x[5] = bf16hi(v.z);
    x[6] = bf16lo(v.w); x[7] = bf16hi(v.w);
  }
  SDV_DEV static float at(const char* row, int v) { return bf16_to_f32(((const uint16_t*)row)[v]); }
};
template <>
struct Vec<false> {
  static constexpr int kElems = 4;
  static constexpr int kBytes = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  SDV_DEV static void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  SDV_DEV static float at(const char* row, int v) { return ((const float*)row)[v]; }
};

// Reference exponent for a max m: fp32(m * c); 0 when nothing finite was seen
// (then every contribution is 2^-inf = 0, or NaN if a NaN was present).
SDV_DEV float exp_ref(float m, float c) { return m == kNegInf ? 0.0f : m * c; }

// Batch slots of request r: target slots 0..gmax, draft slots gmax+1..2*gmax;
// with l drafts scheduled the batch holds target 0..l and draft 1..l.
SDV_DEV bool slot_in_batch(int slot, int gmax, int L) {
  return slot <= gmax ? slot <= L : slot - gmax <= L;
}

// Arguments of the bandwidth pass.  One pass covers, of every listed request,
// the target slots [t_lo, t_hi) and the draft positions [d_lo, d_hi] (draft
// position j is slot gmax + j of the partials' layout), within the scheduled
// batch: all of them in one pass, or a range of positions per round when
// verification stops at each request's first rejection.
struct RowPassArgs {
  const char* tgt;
  const int32_t* tgt_row0;
  const char* drf;
  const int32_t* drf_row0;
  const int32_t* ell;
  float2* partial;  // [R][2*gmax+1][n_ch][kRowWaves]: (max, sum 2^(x*c - fp32(max*c)))
  int64_t ld_bytes;
  float c;          // log2(e) / T
  int gmax;
  int V;
  int n_ch;
  int t_lo, t_hi;   // target slots [t_lo, t_hi)
  int d_lo, d_hi;   // draft positions [d_lo, d_hi]; none when d_lo > d_hi (the
                    // drafter's statistics replace the draft rows)
  int slots;        // (t_hi - t_lo) + number of draft positions
  const int32_t* list;   // the requests of this pass (null: every request) ...
  const int32_t* count;  // ... and their number
  int32_t* clear;        // counter the next round appends to, zeroed here (or null)
  int chunks;            // consecutive chunks per workgroup: 1, or 2 (bf16 only)
};

// Launch the bandwidth pass: one workgroup per (request, slot, chunk group) item
// without a list, else `grid` workgroups striding over the listed items.
hipError_t launch_row_partials(bool bf16, const RowPassArgs& a, unsigned grid, hipStream_t stream);

}  // namespace sdv
