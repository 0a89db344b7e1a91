// fp32 ring step: the block step of "distributed training hands-on code",
// section 6.2 (S = Q K^T / sqrt(d); M' = max(M, rowmax S);
// L' = L e^(M - M') + rowsum e^(S - M'); O' = O e^(M - M') + e^(S - M') V),
// computed entirely in fp32 on the vector ALUs — no reduced-precision
// operand anywhere, for inputs that are fp32 end to end.
//
// Work split: a workgroup owns 64 query rows of one (batch, head); each row is
// held by D/64 threads (64 head_dim elements of q and of the accumulator per
// thread). K/V tiles of 32 keys are staged in LDS and read as broadcasts.
// The online softmax is computed in base 2 with the exact running maximum.
#include "common.h"

namespace ra {
namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKeys = 32;   // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(kRows * (D / 64)) step_f32_kernel(StepArgs a) {
  constexpr int TPR = D / 64;        // threads per query row
  constexpr int NT = kRows * TPR;    // threads per workgroup
  __shared__ float4 ks[kKeys * D / 4];
  __shared__ float4 vs[kKeys * D / 4];

  const int tid = threadIdx.x;
  const int r = tid / TPR;
  const int part = tid % TPR;
  const int64_t tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = h / a.group;
  const int64_t row0 = tile * kRows;
  const int64_t row = row0 + r;
  const bool valid = row < a.q_len;
  const int64_t rowc = valid ? row : a.q_len - 1;
  const int64_t r1 = (row0 + kRows < a.q_len) ? row0 + kRows : a.q_len;

  int64_t qmin, qmax;
  seg_range(a.qs, a.n_q_seg, row0, r1, &qmin, &qmax);
  const TilePlan plan = plan_tiles<kKeys>(a, qmin, qmax);
  const int ntiles = plan.total_tiles();
  if (ntiles == 0 && !a.init && !a.final_) return;  // no key of this block is visible

  const int64_t bh = (int64_t)b * a.heads_q + h;
  const size_t srow = (size_t)(bh * a.q_len + rowc);
  const float* qp = static_cast<const float*>(a.q) + srow * D + part * 64;
  const float* kbase = static_cast<const float*>(a.k) + ((int64_t)b * a.heads_kv + kvh) * a.kv_len * D;
  const float* vbase = static_cast<const float*>(a.v) + ((int64_t)b * a.heads_kv + kvh) * a.kv_len * D;

  float q[64], o[64];
#pragma unroll
  for (int e = 0; e < 64; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qp + e);
    q[e] = x.x; q[e + 1] = x.y; q[e + 2] = x.z; q[e + 3] = x.w;
  }
  float m_run, l_run;
  if (a.init) {
#pragma unroll
    for (int e = 0; e < 64; ++e) o[e] = 0.0f;
    m_run = -INFINITY;
    l_run = 0.0f;
  } else {
    const float* op = a.o + srow * D + part * 64;
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(op + e);
      o[e] = x.x; o[e + 1] = x.y; o[e + 2] = x.z; o[e + 3] = x.w;
    }
    m_run = a.m[srow];
    l_run = a.l[srow];
  }

  const int64_t qpos = seg_position(a.qs, a.n_q_seg, rowc);
  const int32_t vend0 = row_visible_end(a, plan.r0, qpos);
  const int32_t vend1 = row_visible_end(a, plan.r1, qpos);

  for (int t = 0; t < ntiles; ++t) {
    const bool first_range = t < plan.r0.ntiles;
    const int32_t start =
        first_range ? plan.r0.begin + t * kKeys : plan.r1.begin + (t - plan.r0.ntiles) * kKeys;
    const int32_t full = first_range ? plan.r0.full : plan.r1.full;
    const int32_t vend = first_range ? vend0 : vend1;
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < kKeys * D / 4; i += NT) {
      const int kr = i / (D / 4), c4 = i % (D / 4);
      int64_t key = start + kr;
      key = key < a.kv_len ? key : a.kv_len - 1;
      ks[i] = reinterpret_cast<const float4*>(kbase + key * D)[c4];
      vs[i] = reinterpret_cast<const float4*>(vbase + key * D)[c4];
    }
    __syncthreads();
    const bool masked = start + kKeys > full;
    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float4* kr = ks + j * (D / 4) + part * 16;
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float4 kv4 = kr[e];
        acc = fmaf(q[4 * e], kv4.x, acc);
        acc = fmaf(q[4 * e + 1], kv4.y, acc);
        acc = fmaf(q[4 * e + 2], kv4.z, acc);
        acc = fmaf(q[4 * e + 3], kv4.w, acc);
      }
      if constexpr (TPR == 2) acc += __shfl_xor(acc, 1);
      float tj = acc * a.scale_log2;
      if (masked && start + j >= vend) tj = -INFINITY;
      s[j] = tj;
      mx = fmaxf(mx, tj);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == m_run) ? 1.0f : exp2f(m_run - m_new);
    const float msub = (m_new == -INFINITY) ? 0.0f : m_new;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      s[j] = exp2f(s[j] - msub);
      psum += s[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < 64; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float4* vr = vs + j * (D / 4) + part * 16;
      const float pj = s[j];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float4 v4 = vr[e];
        o[4 * e] = fmaf(pj, v4.x, o[4 * e]);
        o[4 * e + 1] = fmaf(pj, v4.y, o[4 * e + 1]);
        o[4 * e + 2] = fmaf(pj, v4.z, o[4 * e + 2]);
        o[4 * e + 3] = fmaf(pj, v4.w, o[4 * e + 3]);
      }
    }
  }

  if (!valid) return;
  if (a.final_) {
    const float inv = finalize_inv(l_run);
    float* dst = static_cast<float*>(a.out) + srow * D + part * 64;
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
      float4 x = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      x.x *= inv; x.y *= inv; x.z *= inv; x.w *= inv;
      *reinterpret_cast<float4*>(dst + e) = x;
    }
    if (part == 0 && a.lse != nullptr) a.lse[srow] = finalize_lse(m_run, l_run);
  } else {
    float* op = a.o + srow * D + part * 64;
#pragma unroll
    for (int e = 0; e < 64; e += 4)
      *reinterpret_cast<float4*>(op + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    if (part == 0) {
      a.m[srow] = m_run;
      a.l[srow] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_step_f32(const StepArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid((unsigned)((a.q_len + kRows - 1) / kRows), (unsigned)a.heads_q, (unsigned)a.batch);
  if (head_dim == 128)
    step_f32_kernel<128><<<grid, kRows * 2, 0, s>>>(a);
  else
    step_f32_kernel<64><<<grid, kRows, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ra
