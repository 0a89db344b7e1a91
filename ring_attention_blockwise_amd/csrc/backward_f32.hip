// fp32 backward ring step: the same gradients as the bf16 path (dQ, dK, dV of
// one K/V block, from the forward's LSE and D = dO . O), computed entirely in
// fp32 on the vector ALUs for inputs that are fp32 end to end.
//
// bwd_f32_dq_kernel: a workgroup owns 64 query rows of one (batch, head), D/64
// threads per row; K/V tiles of 32 keys are staged in LDS and read as
// broadcasts (the fp32 forward's layout). Per key: s = q.k, dp = dO.v,
// p = 2^(s scale log2 e - LSE log2 e), dS = p (dp - D), dQ += dS k.
// bwd_f32_dkdv_kernel: a workgroup owns 64 keys of one (batch, KV head), D/64
// threads per key; tiles of 32 query rows (Q, dO and the two row terms) of
// every query head of the GQA group are staged in LDS. Per row:
// dV += p dO, dK += dS q. Both add scale to dQ and dK on the way out.
#include "backward.h"

namespace ra {
namespace {

constexpr int kRows = 64;  // query rows (dQ kernel) or keys (dK/dV kernel) per workgroup
constexpr int kTile = 32;  // keys (dQ kernel) or query rows (dK/dV kernel) per LDS tile

// Dot product of this thread's 64 elements with a 64-float LDS slice; with two
// threads per row the partial sums are combined across the lane pair.
template <int TPR>
__device__ __forceinline__ float dot64(const float* x, const float4* y) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float4 v = y[e];
    acc = fmaf(x[4 * e], v.x, acc);
    acc = fmaf(x[4 * e + 1], v.y, acc);
    acc = fmaf(x[4 * e + 2], v.z, acc);
    acc = fmaf(x[4 * e + 3], v.w, acc);
  }
  if constexpr (TPR == 2) acc += __shfl_xor(acc, 1);
  return acc;
}

__device__ __forceinline__ void axpy64(float* acc, float a, const float4* y) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float4 v = y[e];
    acc[4 * e] = fmaf(a, v.x, acc[4 * e]);
    acc[4 * e + 1] = fmaf(a, v.y, acc[4 * e + 1]);
    acc[4 * e + 2] = fmaf(a, v.z, acc[4 * e + 2]);
    acc[4 * e + 3] = fmaf(a, v.w, acc[4 * e + 3]);
  }
}

__device__ __forceinline__ void load64(float* dst, const float* src) {
#pragma unroll
  for (int e = 0; e < 64; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(src + e);
    dst[e] = x.x;
    dst[e + 1] = x.y;
    dst[e + 2] = x.z;
    dst[e + 3] = x.w;
  }
}

template <int D>
__global__ void __launch_bounds__(kRows * (D / 64)) bwd_f32_dq_kernel(BwdArgs a) {
  constexpr int TPR = D / 64;
  constexpr int NT = kRows * TPR;
  __shared__ float4 ks[kTile * D / 4];
  __shared__ float4 vs[kTile * D / 4];
  const StepArgs& s = a.s;
  const int tid = threadIdx.x;
  const int r = tid / TPR;
  const int part = tid % TPR;
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = h / s.group;
  const int64_t row = row0 + r;
  const bool valid = row < s.q_len;
  const int64_t rowc = valid ? row : s.q_len - 1;
  const int64_t r1 = (row0 + kRows < s.q_len) ? row0 + kRows : s.q_len;
  int64_t qmin, qmax;
  seg_range(s.qs, s.n_q_seg, row0, r1, &qmin, &qmax);
  const TilePlan plan = plan_tiles<kTile>(s, qmin, qmax);
  const int ntiles = plan.total_tiles();
  if (ntiles == 0 && !a.init_dq) return;

  const int64_t n_rows = (int64_t)s.batch * s.heads_q * s.q_len;
  const size_t srow = (size_t)(((int64_t)b * s.heads_q + h) * s.q_len + rowc);
  const float* kbase = static_cast<const float*>(s.k) + ((int64_t)b * s.heads_kv + kvh) * s.kv_len * D;
  const float* vbase = static_cast<const float*>(s.v) + ((int64_t)b * s.heads_kv + kvh) * s.kv_len * D;
  float q[64], g[64], dq[64];
  load64(q, static_cast<const float*>(s.q) + srow * D + part * 64);
  load64(g, static_cast<const float*>(a.dout) + srow * D + part * 64);
#pragma unroll
  for (int e = 0; e < 64; ++e) dq[e] = 0.0f;
  const float sl2 = s.scale_log2;
  const float c2 = a.terms[srow] * sl2;  // -LSE log2(e), or -inf
  const float e_row = a.terms[n_rows + srow];
  const int64_t qpos = seg_position(s.qs, s.n_q_seg, rowc);
  const int32_t vend0 = row_visible_end(s, plan.r0, qpos);
  const int32_t vend1 = row_visible_end(s, plan.r1, qpos);

  for (int t = 0; t < ntiles; ++t) {
    const bool first_range = t < plan.r0.ntiles;
    const int32_t start = first_range ? plan.r0.begin + t * kTile : plan.r1.begin + (t - plan.r0.ntiles) * kTile;
    const int32_t full = first_range ? plan.r0.full : plan.r1.full;
    const int32_t vend = first_range ? vend0 : vend1;
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < kTile * D / 4; i += NT) {
      const int kr = i / (D / 4), c4 = i % (D / 4);
      int64_t key = start + kr;
      key = key < s.kv_len ? key : s.kv_len - 1;
      ks[i] = reinterpret_cast<const float4*>(kbase + key * D)[c4];
      vs[i] = reinterpret_cast<const float4*>(vbase + key * D)[c4];
    }
    __syncthreads();
    const bool masked = start + kTile > full;
    for (int j = 0; j < kTile; ++j) {
      const float4* kr = ks + j * (D / 4) + part * 16;
      const float4* vr = vs + j * (D / 4) + part * 16;
      const float sj = dot64<TPR>(q, kr);
      const float dpj = dot64<TPR>(g, vr);
      float p = exp2f(fmaf(sj, sl2, c2));
      if (masked && start + j >= vend) p = 0.0f;
      axpy64(dq, p * (dpj + e_row), kr);
    }
  }
  if (!valid) return;
  float* dst = a.dq + srow * D + part * 64;
#pragma unroll
  for (int e = 0; e < 64; e += 4) {
    float4 x = make_float4(dq[e] * a.scale, dq[e + 1] * a.scale, dq[e + 2] * a.scale, dq[e + 3] * a.scale);
    if (!a.init_dq) {
      const float4 y = *reinterpret_cast<const float4*>(dst + e);
      x.x += y.x;
      x.y += y.y;
      x.z += y.z;
      x.w += y.w;
    }
    *reinterpret_cast<float4*>(dst + e) = x;
  }
}

// Query rows [begin, end) of one query segment that see a key of the tile.
struct F32Range {
  int64_t begin, end, off;
  int32_t ntiles;
};

__device__ __forceinline__ F32Range f32_range(const StepArgs& s, int seg, bool causal, int64_t kmin) {
  F32Range r;
  if (!causal) {
    r.off = 0;
    r.begin = 0;
    r.end = s.q_len;
  } else {
    const Seg g = seg == 0 ? s.qs[0] : s.qs[1];
    r.off = seg == 0 ? 0 : s.qs[0].len;
    r.begin = r.off + seg_count_le(g, kmin - 1);
    r.end = r.off + g.len;
  }
  r.ntiles = r.end > r.begin ? (int32_t)((r.end - r.begin + kTile - 1) / kTile) : 0;
  return r;
}

template <int D>
__global__ void __launch_bounds__(kRows * (D / 64)) bwd_f32_dkdv_kernel(BwdArgs a) {
  constexpr int TPR = D / 64;
  constexpr int NT = kRows * TPR;
  __shared__ float4 qs[kTile * D / 4];
  __shared__ float4 gs[kTile * D / 4];
  __shared__ float cs[kTile], es[kTile];
  const StepArgs& s = a.s;
  const int tid = threadIdx.x;
  const int r = tid / TPR;
  const int part = tid % TPR;
  const int64_t key0 = (int64_t)blockIdx.x * kRows;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t key = key0 + r;
  const bool valid = key < s.kv_len;
  const int64_t keyc = valid ? key : s.kv_len - 1;
  const int64_t k1 = (key0 + kRows < s.kv_len) ? key0 + kRows : s.kv_len;
  int64_t kmin, kmax;
  seg_range(s.ks, s.n_kv_seg, key0, k1, &kmin, &kmax);
  const bool causal = s.causal && s.n_q_seg > 0 && s.n_kv_seg > 0;
  const F32Range ra0 = f32_range(s, 0, causal, kmin);
  const F32Range ra1 = (causal && s.n_q_seg > 1) ? f32_range(s, 1, true, kmin) : F32Range{0, 0, 0, 0};
  const int32_t nq = ra0.ntiles + ra1.ntiles;
  if (nq == 0) return;

  const size_t kvrow = (size_t)(((int64_t)b * s.heads_kv + kvh) * s.kv_len + keyc);
  float k[64], v[64], dk[64], dv[64];
  load64(k, static_cast<const float*>(s.k) + kvrow * D + part * 64);
  load64(v, static_cast<const float*>(s.v) + kvrow * D + part * 64);
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  // first local query row of each range that sees this thread's key
  int64_t fv0 = ra0.begin, fv1 = ra1.begin;
  if (causal) {
    const int64_t kpos = seg_position(s.ks, s.n_kv_seg, keyc);
    fv0 = ra0.off + seg_count_le(s.qs[0], kpos - 1);
    if (s.n_q_seg > 1) fv1 = ra1.off + seg_count_le(s.qs[1], kpos - 1);
  }
  const int64_t n_rows = (int64_t)s.batch * s.heads_q * s.q_len;
  const float sl2 = s.scale_log2;

  for (int g = 0; g < s.group; ++g) {
    const int h = kvh * s.group + g;
    const int64_t head_row0 = ((int64_t)b * s.heads_q + h) * s.q_len;
    const float* qbase = static_cast<const float*>(s.q) + head_row0 * D;
    const float* gbase = static_cast<const float*>(a.dout) + head_row0 * D;
    for (int t = 0; t < nq; ++t) {
      const bool first = t < ra0.ntiles;
      const F32Range& rr = first ? ra0 : ra1;
      const int64_t rs = rr.begin + (int64_t)(first ? t : t - ra0.ntiles) * kTile;
      const int nrows = (int)(rr.end - rs < kTile ? rr.end - rs : kTile);
      const int64_t fv = first ? fv0 : fv1;
      __syncthreads();  // previous tile fully consumed
      for (int i = tid; i < kTile * D / 4; i += NT) {
        const int qr = i / (D / 4), c4 = i % (D / 4);
        const int64_t qrow = rs + (qr < nrows ? qr : nrows - 1);
        qs[i] = reinterpret_cast<const float4*>(qbase + qrow * D)[c4];
        gs[i] = reinterpret_cast<const float4*>(gbase + qrow * D)[c4];
      }
      for (int i = tid; i < kTile; i += NT) {
        const int64_t qrow = rs + (i < nrows ? i : nrows - 1);
        cs[i] = a.terms[head_row0 + qrow] * sl2;
        es[i] = a.terms[n_rows + head_row0 + qrow];
      }
      __syncthreads();
      for (int i = 0; i < nrows; ++i) {
        const float4* qr = qs + i * (D / 4) + part * 16;
        const float4* gr = gs + i * (D / 4) + part * 16;
        const float si = dot64<TPR>(k, qr);
        const float dpi = dot64<TPR>(v, gr);
        float p = exp2f(fmaf(si, sl2, cs[i]));
        if (causal && rs + i < fv) p = 0.0f;
        axpy64(dv, p, gr);
        axpy64(dk, p * (dpi + es[i]), qr);
      }
    }
  }
  if (!valid) return;
  float* dkp = a.dk + kvrow * D + part * 64;
  float* dvp = a.dv + kvrow * D + part * 64;
#pragma unroll
  for (int e = 0; e < 64; e += 4) {
    float4 xk = *reinterpret_cast<const float4*>(dkp + e);
    float4 xv = *reinterpret_cast<const float4*>(dvp + e);
    xk.x += dk[e] * a.scale;
    xk.y += dk[e + 1] * a.scale;
    xk.z += dk[e + 2] * a.scale;
    xk.w += dk[e + 3] * a.scale;
    xv.x += dv[e];
    xv.y += dv[e + 1];
    xv.z += dv[e + 2];
    xv.w += dv[e + 3];
    *reinterpret_cast<float4*>(dkp + e) = xk;
    *reinterpret_cast<float4*>(dvp + e) = xv;
  }
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, int head_dim, hipStream_t s) {
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  if (a.s.q_len == 0 || a.s.batch == 0) return hipSuccess;
  const dim3 gq((unsigned)((a.s.q_len + kRows - 1) / kRows), (unsigned)a.s.heads_q, (unsigned)a.s.batch);
  if (head_dim == 128)
    bwd_f32_dq_kernel<128><<<gq, kRows * 2, 0, s>>>(a);
  else
    bwd_f32_dq_kernel<64><<<gq, kRows, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.s.kv_len == 0) return e;
  const dim3 gk((unsigned)((a.s.kv_len + kRows - 1) / kRows), (unsigned)a.s.heads_kv, (unsigned)a.s.batch);
  if (head_dim == 128)
    bwd_f32_dkdv_kernel<128><<<gk, kRows * 2, 0, s>>>(a);
  else
    bwd_f32_dkdv_kernel<64><<<gk, kRows, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ra
