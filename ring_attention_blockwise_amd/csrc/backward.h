// Internal declarations of the backward ring step (gradients of the block
// step with respect to Q, K and V). Not part of the public ABI.
#pragma once

#include "common.h"

namespace ra {

// Arguments of one backward step, passed by value. `s` carries the shapes,
// segments, q/k/v pointers and scale_log2 of the forward step (its o, m, l,
// out and lse are unused).
struct BwdArgs {
  StepArgs s;
  const void* dout;    // [B, Hq, q_len, D] upstream gradient, input dtype
  const float* terms;  // [2, B, Hq, q_len]: c = -LSE/scale (-inf: no visible key), e = -D
  float* dq;           // [B, Hq, q_len, D] fp32, accumulated
  float* dk;           // [B, Hkv, kv_len, D] fp32, accumulated
  float* dv;           // [B, Hkv, kv_len, D] fp32, accumulated
  float scale;
  int32_t init_dq;     // dq starts at zero (it is not read)
};

// terms[r] = -lse[r] / scale (or -inf), terms[rows + r] = -(dout[r] . out[r]).
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* terms, int64_t rows,
                           int head_dim, int dtype, float scale, hipStream_t s);
// dq += ..., dk += ..., dv += ... for one K/V block (bf16, head_dim 64 or 128).
hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, hipStream_t s);
// The same for fp32 inputs (fp32 arithmetic throughout).
hipError_t launch_bwd_f32(const BwdArgs& a, int head_dim, hipStream_t s);
// y = x converted to dtype (RA_F32 copies), n a multiple of 4.
hipError_t launch_convert(const float* x, void* y, int64_t n, int dtype, hipStream_t s);
// Zero `bytes` (a multiple of 16) at p with a fill kernel (no memset node
// when the call is captured into a graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace ra
