// Internal declarations shared by the HIP translation units of libring_attn.
// Not part of the public ABI (that is include/ring_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "ring_attn.h"

namespace ra {

// Segment of global positions for a run of local rows: pos = start + i * stride.
struct Seg {
  int64_t start;
  int64_t len;
  int64_t stride;
};

// Everything a step kernel needs, passed by value.
struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;          // fp32 state [B, Hq, q_len, D]
  float* m;          // [B, Hq, q_len]
  float* l;          // [B, Hq, q_len]
  void* out;         // fused finalize: output in the input dtype, else nullptr
  float* lse;        // fused finalize: natural-log LSE (may be nullptr)
  int64_t q_len;
  int64_t kv_len;
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t group;     // heads_q / heads_kv
  float scale_log2;  // softmax scale * log2(e)
  int32_t causal;
  int32_t init;      // ignore the incoming state
  int32_t final_;    // write out/lse instead of the state
  int32_t n_q_seg;
  int32_t n_kv_seg;
  Seg qs[2];
  Seg ks[2];
  // Fused receive (bf16 step only): while it computes, the launch also
  // copies rx_bytes of each of two tensors, rx_src[i] -> rx_dst[i] (the next
  // K/V block into its receive slot). Work items whose query tile is at or
  // after rx_tile_lo take rx_share bytes of both tensors each, in the order
  // of their dense rank. rx_bytes == 0: no receive in this launch.
  const void* rx_src[2];
  void* rx_dst[2];
  int64_t rx_bytes;
  int64_t rx_share;
  int32_t rx_tile_lo;
  // Key split (bf16 step only): split > 1 runs every query tile as `split`
  // work items, item j over its share of the tile's key tiles, each starting
  // from the empty state and writing a partial state j ([split][rows][D] in
  // po, [split][rows] in pm and pl; rows = batch * heads_q * q_len). A fold
  // launched after the step merges the incoming state (unless init) with the
  // partials in order and writes the state, or the output when final_.
  int32_t split;
  float* po;
  float* pm;
  float* pl;
};

// The lazy-rescale threshold in base-2 exponent units: the reference m is
// only raised when the running maximum exceeds it by more than this, so every
// weight 2^(t - m) stays <= 2^32. Sums of such weights over any block stay far
// inside fp32 range (2^32 per weight, below 2^63 for 2^31 keys), and bf16 P
// carries fp32's exponent range, so a higher threshold costs no precision; it
// only makes the rescales rarer on rows whose maximum keeps climbing.
constexpr float kRescaleThreshold = 32.0f;

// Launchers (each returns hipGetLastError() of its launch).
hipError_t launch_step_bf16(const StepArgs& a, int head_dim, hipStream_t s);
hipError_t launch_step_f32(const StepArgs& a, int head_dim, hipStream_t s);
hipError_t launch_merge(float* o_a, float* m_a, float* l_a, const float* o_b, const float* m_b,
                        const float* l_b, int64_t rows, int head_dim, hipStream_t s);
hipError_t launch_finalize(const float* o, const float* m, const float* l, void* out, float* lse,
                           int64_t rows, int head_dim, int dtype, hipStream_t s);
hipError_t launch_init_state(float* o, float* m, float* l, int64_t rows, int head_dim,
                             hipStream_t s);
// The fold after a split step (see StepArgs::split).
hipError_t launch_fold(const StepArgs& a, int64_t rows, int head_dim, int dtype, hipStream_t s);


// ---- device helpers shared by the finalize kernel and the fused finalize of
// the step kernels (so both produce bit-identical results). ----------------

// 1 / l for a finished row (0 when the row saw no key).
__device__ __forceinline__ float finalize_inv(float l) { return l > 0.0f ? 1.0f / l : 0.0f; }

// Natural-log LSE of a base-2 state row: ln(2) * (m + log2(l)); -inf if empty.
__device__ __forceinline__ float finalize_lse(float m, float l) {
  return l > 0.0f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  // round to nearest even; inputs here are finite
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// ---- causal tile planning shared by the step kernels ----------------------
//
// Positions inside a segment grow with the local row, so "keys with position
// <= x" is always a prefix of each K/V segment. A query tile with positions
// in [qmin, qmax] therefore sees, in K/V segment s, the local key range
// [koff_s, koff_s + count_s(qmax)); its first count_s(qmin) keys are visible
// to every row of the tile (no mask), the rest need the per-element test.
// Blocks above the causal diagonal are never visited (the skipping of fully
// masked blocks in "Ring Attention and Sequence Parallelism", section 6 and
// lecture 30, section 3.2).

__device__ __forceinline__ int64_t seg_position(const Seg* segs, int n, int64_t row) {
  if (n <= 0) return row;
  if (row < segs[0].len || n == 1) return segs[0].start + row * segs[0].stride;
  return segs[1].start + (row - segs[0].len) * segs[1].stride;
}

// Number of entries of `s` whose position is <= x.
__host__ __device__ __forceinline__ int64_t seg_count_le(const Seg& s, int64_t x) {
  if (x < s.start) return 0;
  const int64_t c = (x - s.start) / s.stride + 1;
  return c < s.len ? c : s.len;
}

// Position range of local rows [r0, r1) (r1 > r0) under the segments.
__host__ __device__ __forceinline__ void seg_range(const Seg* segs, int n, int64_t r0, int64_t r1, int64_t* lo,
                                          int64_t* hi) {
  if (n <= 0) {
    *lo = r0;
    *hi = r1 - 1;
    return;
  }
  int64_t mn = INT64_MAX, mx = INT64_MIN;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i < n) {
      const int64_t off = i == 0 ? 0 : segs[0].len;
      const int64_t a = r0 > off ? r0 : off;
      const int64_t b = r1 < off + segs[i].len ? r1 : off + segs[i].len;
      if (a < b) {
        const int64_t p0 = segs[i].start + (a - off) * segs[i].stride;
        const int64_t p1 = segs[i].start + (b - 1 - off) * segs[i].stride;
        mn = p0 < mn ? p0 : mn;
        mx = p1 > mx ? p1 : mx;
      }
    }
  }
  *lo = mn;
  *hi = mx;
}

// One run of local keys a query tile visits: [begin, end); keys below `full`
// are visible to every row of the tile. `seg` is the K/V segment (-1: all
// keys, not causal), `koff` the local index where that segment starts.
struct KeyRange {
  int32_t begin;
  int32_t end;
  int32_t full;
  int32_t koff;
  int32_t ntiles;
  int32_t seg;
};

// The ranges of one query tile (0, 1 or 2 of them). Kept as named members and
// selected with conditionals so that nothing is indexed at run time (which
// would push the plan out of registers).
struct TilePlan {
  KeyRange r0;
  KeyRange r1;
  int32_t n;
  __host__ __device__ __forceinline__ int32_t total_tiles() const {
    return (n > 0 ? r0.ntiles : 0) + (n > 1 ? r1.ntiles : 0);
  }
  // range of tile t and the tile's first local key
  __device__ __forceinline__ KeyRange range_of(int t) const { return t < r0.ntiles ? r0 : r1; }
};

template <int BN>
__host__ __device__ __forceinline__ KeyRange make_range(const Seg& g, int32_t seg, int64_t off, int64_t qmin, int64_t qmax) {
  const int64_t vis = seg_count_le(g, qmax);
  const int64_t full = seg_count_le(g, qmin);
  KeyRange r;
  r.koff = (int32_t)off;
  r.begin = (int32_t)off;
  r.end = (int32_t)(off + vis);
  r.full = (int32_t)(off + full);
  r.ntiles = (int32_t)((vis + BN - 1) / BN);
  r.seg = seg;
  return r;
}

template <int BN>
__host__ __device__ __forceinline__ TilePlan plan_tiles(const StepArgs& a, int64_t qmin, int64_t qmax) {
  TilePlan p;
  p.n = 0;
  p.r0 = KeyRange{0, 0, 0, 0, 0, -1};
  p.r1 = p.r0;
  if (a.kv_len == 0) return p;
  if (!a.causal || a.n_kv_seg <= 0) {
    p.n = 1;
    p.r0 = KeyRange{0, (int32_t)a.kv_len, (int32_t)a.kv_len, 0, (int32_t)((a.kv_len + BN - 1) / BN), -1};
    return p;
  }
  const KeyRange x = make_range<BN>(a.ks[0], 0, 0, qmin, qmax);
  const bool has_x = x.end > x.begin;
  if (a.n_kv_seg < 2) {
    p.n = has_x ? 1 : 0;
    p.r0 = x;
    return p;
  }
  const KeyRange y = make_range<BN>(a.ks[1], 1, a.ks[0].len, qmin, qmax);
  const bool has_y = y.end > y.begin;
  p.n = (has_x ? 1 : 0) + (has_y ? 1 : 0);
  p.r0 = has_x ? x : y;
  p.r1 = y;
  return p;
}

// The tiles [t0, t1) of a plan (in its order), as a plan of their own.
template <int BN>
__host__ __device__ __forceinline__ TilePlan restrict_plan(const TilePlan& p, int32_t t0, int32_t t1) {
  const int32_t n0 = p.n > 0 ? p.r0.ntiles : 0;
  const int32_t a0 = t0 < n0 ? t0 : n0, b0 = t1 < n0 ? t1 : n0;
  const int32_t a1 = (t0 > n0 ? t0 : n0) - n0, b1 = (t1 > n0 ? t1 : n0) - n0;
  KeyRange x = p.r0;
  x.begin += a0 * BN;
  x.ntiles = b0 - a0;
  KeyRange y = p.r1;
  y.begin += a1 * BN;
  y.ntiles = p.n > 1 ? b1 - a1 : 0;
  const bool has_x = x.ntiles > 0, has_y = y.ntiles > 0;
  TilePlan q;
  q.n = (has_x ? 1 : 0) + (has_y ? 1 : 0);
  q.r0 = has_x ? x : y;
  q.r1 = y;
  return q;
}

// Exclusive end (local key index) of the keys of range r visible to a query
// at position qpos: every key of the range when not causal.
__device__ __forceinline__ int32_t row_visible_end(const StepArgs& a, const KeyRange& r, int64_t qpos) {
  if (r.seg < 0) return r.end;
  const Seg g = r.seg == 0 ? a.ks[0] : a.ks[1];
  return r.koff + (int32_t)seg_count_le(g, qpos);
}

}  // namespace ra
