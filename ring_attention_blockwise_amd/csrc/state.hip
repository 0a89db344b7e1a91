// State kernels of the ring step: merge of two (O, m, l) states, finalize
// (O / l and LSE), the empty-state fill, and the fold of the partial states
// of a step whose query tiles were split over their keys.
//
// Merge is the online-softmax fold of "distributed training hands-on code",
// section 6.2 (block_attention: M' = max(M, M_b), L' = L e^(M-M') + ...,
// O' = O e^(M-M') + ...) applied to two partial states; finalize is that
// page's closing O / L plus the log-sum-exp. All three are HBM-bound
// streaming passes: one workgroup of 256 threads handles 16 rows, 16 threads
// per row, each thread moving 16-byte vectors along head_dim. Every element
// of O is touched once, so its loads and stores carry the non-temporal hint
// (measured: merge 5.5 -> 6.5 TB/s, finalize 5.9 -> 6.5 TB/s at the 128K/8
// share's shapes, the level of the D2D copy).
#include <type_traits>

#include "common.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 stream_load(const float4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void stream_store(float4* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

constexpr int kThreads = 256;
constexpr int kThreadsPerRow = 16;
constexpr int kRowsPerBlock = kThreads / kThreadsPerRow;

// Scale factor 2^(m_x - m) of one side of a merge, 0 for an empty side.
__device__ __forceinline__ float side_weight(float mx, float m) {
  return mx == -INFINITY ? 0.0f : exp2f(mx - m);
}

template <int D>
__global__ void __launch_bounds__(kThreads) merge_kernel(float* __restrict__ o_a, float* __restrict__ m_a,
                                                         float* __restrict__ l_a, const float* __restrict__ o_b,
                                                         const float* __restrict__ m_b,
                                                         const float* __restrict__ l_b, int64_t rows) {
  // Both products are rounded before the single add (no FMA contraction), so
  // the result is bitwise symmetric in (a, b).
#pragma clang fp contract(off)
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  const int sub = threadIdx.x % kThreadsPerRow;
  if (row >= rows) return;
  const float ma = m_a[row], mb = m_b[row];
  const float m = fmaxf(ma, mb);
  if (m == -INFINITY) return;  // both sides empty: a stays empty
  const float wa = side_weight(ma, m), wb = side_weight(mb, m);
  float4* oa = reinterpret_cast<float4*>(o_a + row * D);
  const float4* ob = reinterpret_cast<const float4*>(o_b + row * D);
#pragma unroll
  for (int i = sub; i < D / 4; i += kThreadsPerRow) {
    const f32x4 x = stream_load(oa + i), y = stream_load(ob + i);
    stream_store(oa + i, wa * x + wb * y);
  }
  if (sub == 0) {
    l_a[row] = wa * l_a[row] + wb * l_b[row];
    m_a[row] = m;
  }
}

template <int D, bool BF16>
__global__ void __launch_bounds__(kThreads) finalize_kernel(const float* __restrict__ o, const float* __restrict__ m,
                                                            const float* __restrict__ l, void* __restrict__ out,
                                                            float* __restrict__ lse, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  const int sub = threadIdx.x % kThreadsPerRow;
  if (row >= rows) return;
  const float lr = l[row];
  const float inv = finalize_inv(lr);
  const float4* src = reinterpret_cast<const float4*>(o + row * D);
#pragma unroll
  for (int i = sub; i < D / 4; i += kThreadsPerRow) {
    const f32x4 x = stream_load(src + i) * inv;
    if constexpr (BF16) {
      const u32x2 packed = {(uint32_t)f32_to_bf16_bits(x.x) | ((uint32_t)f32_to_bf16_bits(x.y) << 16),
                            (uint32_t)f32_to_bf16_bits(x.z) | ((uint32_t)f32_to_bf16_bits(x.w) << 16)};
      __builtin_nontemporal_store(packed, reinterpret_cast<u32x2*>(static_cast<unsigned short*>(out) + row * D) + i);
    } else {
      stream_store(reinterpret_cast<float4*>(static_cast<float*>(out) + row * D) + i, x);
    }
  }
  if (sub == 0 && lse != nullptr) lse[row] = finalize_lse(m[row], lr);
}

template <int D>
__global__ void __launch_bounds__(kThreads) init_state_kernel(float* __restrict__ o, float* __restrict__ m,
                                                              float* __restrict__ l, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  const int sub = threadIdx.x % kThreadsPerRow;
  if (row >= rows) return;
  float4* dst = reinterpret_cast<float4*>(o + row * D);
#pragma unroll
  for (int i = sub; i < D / 4; i += kThreadsPerRow) stream_store(dst + i, f32x4{0.f, 0.f, 0.f, 0.f});
  if (sub == 0) {
    m[row] = -INFINITY;
    l[row] = 0.0f;
  }
}

// The fold after a split step: the incoming state (unless init) and the
// partial states 0 .. parts-1, in that order, merged with one common
// reference M (the largest m; each side scaled by 2^(m_x - M), an empty side
// skipped), then written as the state or, when final_, as the output and LSE.
// Rows whose sides are all empty keep an empty state (written only with
// init). The fold is bound by memory latency, not bandwidth: every m is
// requested at once, then every O row of a non-empty side (P >= parts is the
// compile-time bound), and only then added up.
template <int D, bool BF16, int P>
__global__ void __launch_bounds__(kThreads) fold_kernel(float* __restrict__ o, float* __restrict__ m,
                                                        float* __restrict__ l, const float* __restrict__ po,
                                                        const float* __restrict__ pm, const float* __restrict__ pl,
                                                        int32_t parts, int64_t rows, int32_t init, int32_t final_,
                                                        void* __restrict__ out, float* __restrict__ lse) {
  constexpr int kV = D / 4 / kThreadsPerRow;  // 16-byte vectors per thread
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  const int sub = threadIdx.x % kThreadsPerRow;
  if (row >= rows) return;
  float mj[P + 1], lj[P + 1];  // side 0: the incoming state; side j + 1: partial j
  mj[0] = init ? -INFINITY : m[row];
#pragma unroll
  for (int j = 0; j < P; ++j) mj[j + 1] = j < parts ? pm[(size_t)j * rows + row] : -INFINITY;
  float mx = mj[0];
#pragma unroll
  for (int j = 1; j <= P; ++j) mx = fmaxf(mx, mj[j]);
  f32x4 x[P + 1][kV];
  if (mx != -INFINITY) {
#pragma unroll
    for (int j = 0; j <= P; ++j) {
      const bool live = mj[j] != -INFINITY;
      const size_t pj = j - 1 < parts ? (size_t)(j - 1) : 0;  // an address inside the partials for every j
      const float* src = j == 0 ? o + row * D : po + (pj * rows + row) * D;
      lj[j] = live ? (j == 0 ? l[row] : pl[pj * rows + row]) : 0.0f;
#pragma unroll
      for (int i = 0; i < kV; ++i)
        x[j][i] = live ? stream_load(reinterpret_cast<const float4*>(src) + sub + i * kThreadsPerRow)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  f32x4 acc[kV];
#pragma unroll
  for (int i = 0; i < kV; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.0f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int j = 0; j <= P; ++j) {
      const float w = side_weight(mj[j], mx);
#pragma unroll
      for (int i = 0; i < kV; ++i) acc[i] += w * x[j][i];
      lsum += w * lj[j];
    }
  }
  if (final_) {
    const float inv = finalize_inv(lsum);
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const f32x4 y = acc[i] * inv;
      const int v = sub + i * kThreadsPerRow;
      if constexpr (BF16) {
        const u32x2 packed = {(uint32_t)f32_to_bf16_bits(y.x) | ((uint32_t)f32_to_bf16_bits(y.y) << 16),
                              (uint32_t)f32_to_bf16_bits(y.z) | ((uint32_t)f32_to_bf16_bits(y.w) << 16)};
        __builtin_nontemporal_store(packed, reinterpret_cast<u32x2*>(static_cast<unsigned short*>(out) + row * D) + v);
      } else {
        stream_store(reinterpret_cast<float4*>(static_cast<float*>(out) + row * D) + v, y);
      }
    }
    if (sub == 0 && lse != nullptr) lse[row] = finalize_lse(mx, lsum);
    return;
  }
  if (mx == -INFINITY && !init) return;  // empty before and after
  float4* dst = reinterpret_cast<float4*>(o + row * D);
#pragma unroll
  for (int i = 0; i < kV; ++i) stream_store(dst + sub + i * kThreadsPerRow, acc[i]);
  if (sub == 0) {
    m[row] = mx;
    l[row] = lsum;
  }
}

inline dim3 grid_for(int64_t rows) { return dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)); }

}  // namespace

hipError_t launch_merge(float* o_a, float* m_a, float* l_a, const float* o_b, const float* m_b,
                        const float* l_b, int64_t rows, int head_dim, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (head_dim == 128)
    merge_kernel<128><<<grid_for(rows), kThreads, 0, s>>>(o_a, m_a, l_a, o_b, m_b, l_b, rows);
  else
    merge_kernel<64><<<grid_for(rows), kThreads, 0, s>>>(o_a, m_a, l_a, o_b, m_b, l_b, rows);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* o, const float* m, const float* l, void* out, float* lse,
                           int64_t rows, int head_dim, int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 g = grid_for(rows);
  if (head_dim == 128) {
    if (dtype == RA_BF16)
      finalize_kernel<128, true><<<g, kThreads, 0, s>>>(o, m, l, out, lse, rows);
    else
      finalize_kernel<128, false><<<g, kThreads, 0, s>>>(o, m, l, out, lse, rows);
  } else {
    if (dtype == RA_BF16)
      finalize_kernel<64, true><<<g, kThreads, 0, s>>>(o, m, l, out, lse, rows);
    else
      finalize_kernel<64, false><<<g, kThreads, 0, s>>>(o, m, l, out, lse, rows);
  }
  return hipGetLastError();
}

hipError_t launch_fold(const StepArgs& a, int64_t rows, int head_dim, int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (a.split < 1 || a.split > 16) return hipErrorInvalidValue;
  const dim3 g = grid_for(rows);
  auto go = [&](auto kernel) {
    kernel<<<g, kThreads, 0, s>>>(a.o, a.m, a.l, a.po, a.pm, a.pl, a.split, rows, a.init, a.final_, a.out, a.lse);
  };
  // the kernel for the smallest bound P >= split
  auto by_parts = [&](auto d_tag, auto bf_tag) {
    constexpr int D = decltype(d_tag)::value;
    constexpr bool B = decltype(bf_tag)::value;
    if (a.split <= 2)
      go(fold_kernel<D, B, 2>);
    else if (a.split <= 4)
      go(fold_kernel<D, B, 4>);
    else if (a.split <= 8)
      go(fold_kernel<D, B, 8>);
    else
      go(fold_kernel<D, B, 16>);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  if (head_dim == 128)
    dtype == RA_BF16 ? by_parts(D128{}, std::true_type{}) : by_parts(D128{}, std::false_type{});
  else
    dtype == RA_BF16 ? by_parts(D64{}, std::true_type{}) : by_parts(D64{}, std::false_type{});
  return hipGetLastError();
}

hipError_t launch_init_state(float* o, float* m, float* l, int64_t rows, int head_dim, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (head_dim == 128)
    init_state_kernel<128><<<grid_for(rows), kThreads, 0, s>>>(o, m, l, rows);
  else
    init_state_kernel<64><<<grid_for(rows), kThreads, 0, s>>>(o, m, l, rows);
  return hipGetLastError();
}

}  // namespace ra
