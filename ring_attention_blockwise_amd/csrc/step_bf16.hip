// bf16 ring step on the CDNA4 matrix cores (gfx950).
//
// One launch folds one K/V block into the running (O, m, l) state of the local
// query block — the block step of "distributed training hands-on code",
// section 6.2 — with the causal skipping of "Ring Attention and Sequence
// Parallelism", sections 4/6 and lecture 30, section 3.2, and GQA head
// sharing (lecture 30, section 3.4).
//
// Mapping (all sizes for head_dim D in {64, 128}):
//  * A workgroup of 4 waves owns 128 query rows of one (batch, q head); each
//    wave owns 32 rows. Workgroups that read the same KV head are placed on
//    the same XCD (consecutive workgroup ids go round-robin over the 8 XCDs),
//    and heavy causal tiles are dispatched first.
//  * Keys are consumed in tiles of 64. K and V tiles are copied HBM -> LDS by
//    16-byte direct-to-LDS loads (no register staging), double-buffered, one
//    barrier per tile; an XOR swizzle of the 16-byte units of each row is
//    applied through the global address so the LDS reads below are free of
//    bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (A operand) is read with ds_read_b128, Q^T
//    (B operand) sits in VGPRs for the whole launch. In the accumulator every
//    lane then holds 32 keys of ONE query row, so the row max and row sum are
//    lane-local plus one v_permlane32_swap with the partner lane.
//  * P^T is converted to bf16 in registers and is directly the B operand of
//    O^T += V^T P^T: the 32x32 accumulator layout puts keys {0-3, 8-11}+4h of
//    each 16-key chunk in lane half h, and V^T (A operand) is fetched with the
//    same key order by ds_read_b64_tr_b16 from row-major V, so no LDS round
//    trip of P and no separate V transpose is needed.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score.
//    The reference maximum is raised lazily (only when a row's maximum grows
//    by more than 2^8); O and l are rescaled only then, for the whole wave.
#include "common.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile

template <int D>
struct Layout {
  static constexpr int kRowBytes = D * 2;                       // one K or V row in LDS
  static constexpr int kUnits = D / 8;                          // 16-byte units per row
  static constexpr int kTileBytes = kBN * kRowBytes;            // one K (or V) tile
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;  // 1 KB per wave load
  static constexpr int kSmemBytes = 4 * kTileBytes;             // 2 buffers x (K, V)
  static constexpr int kDChunks = D / 16;                       // K=16 steps of QK^T
  static constexpr int kDBlocks = D / 32;                       // 32-row blocks of O^T

  // Stored position of logical 16-byte unit c of row `row`.
  // K rows are read 16 lanes x 16 B at a time over 16 consecutive rows;
  // V rows are read by the transposing 8-byte reads over 4 consecutive rows.
  __device__ static __forceinline__ int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

__device__ __forceinline__ float max_with_partner(float x) {
  // v_permlane32_swap(x, x): lanes < 32 get (x[l], x[l+32]), lanes >= 32
  // get (x[l-32], x[l]); either way the pair max is max of the two.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 pack_p(const f32x16& s, int base) {
  f32x2 a = {s[base + 0], s[base + 1]};
  f32x2 b = {s[base + 2], s[base + 3]};
  f32x2 c = {s[base + 4], s[base + 5]};
  f32x2 d = {s[base + 6], s[base + 7]};
  const bf16x2 pa = __builtin_convertvector(a, bf16x2);
  const bf16x2 pb = __builtin_convertvector(b, bf16x2);
  const bf16x2 pc = __builtin_convertvector(c, bf16x2);
  const bf16x2 pd = __builtin_convertvector(d, bf16x2);
  const auto ab = __builtin_shufflevector(pa, pb, 0, 1, 2, 3);
  const auto cd = __builtin_shufflevector(pc, pd, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Copy one K or V tile (64 rows starting at local key `start`) into LDS.
// The wave's i-th load writes 1 KB of LDS at unit block (wave*L + i)*64; lane
// `lane` of it fills stored unit p of row `row`, fetching logical unit
// p ^ swz(row) from HBM. Rows past the end of the block are clamped to the
// last row (their scores are masked).
template <int D, bool IS_K>
__device__ __forceinline__ void load_tile(const unsigned short* __restrict__ src, int64_t kv_len, int32_t start,
                                          char* lds_tile, int wave, int lane) {
  using Ly = Layout<D>;
#pragma unroll
  for (int i = 0; i < Ly::kLoadsPerWave; ++i) {
    const int blk = wave * Ly::kLoadsPerWave + i;
    const int u = blk * 64 + lane;
    const int row = u / Ly::kUnits;
    const int p = u % Ly::kUnits;
    const int c = p ^ (IS_K ? Ly::k_swz(row) : Ly::v_swz(row));
    int64_t key = (int64_t)start + row;
    key = key < kv_len ? key : kv_len - 1;
    const unsigned short* g = src + key * D + c * 8;
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_tile + blk * 1024), 16, 0, 0);
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) step_bf16_kernel(StepArgs a, int32_t n_items, int32_t items_per_xcd,
                                                                int32_t q_tiles) {
  using Ly = Layout<D>;
  __shared__ __attribute__((aligned(1024))) char smem[Ly::kSmemBytes];

  // ---- work item: XCD-major so one XCD streams one KV head -----------------
  const int32_t item = (int32_t)(blockIdx.x % 8) * items_per_xcd + (int32_t)(blockIdx.x / 8);
  if (item >= n_items) return;
  const int32_t per_kv = q_tiles * a.group;
  const int32_t bk = item / per_kv;
  const int32_t rem = item % per_kv;
  const int32_t tile = q_tiles - 1 - rem / a.group;  // heavy (late) tiles first
  const int32_t kvh = bk % a.heads_kv;
  const int32_t b = bk / a.heads_kv;
  const int32_t h = kvh * a.group + rem % a.group;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int qcol = lane & 31;
  const int hh = lane >> 5;

  const int64_t row0 = (int64_t)tile * kBM;
  const int64_t r1 = (row0 + kBM < a.q_len) ? row0 + kBM : a.q_len;
  int64_t qmin, qmax;
  seg_range(a.qs, a.n_q_seg, row0, r1, &qmin, &qmax);
  const TilePlan plan = plan_tiles<kBN>(a, qmin, qmax);
  const int ntiles = plan.total_tiles();
  if (ntiles == 0 && !a.init && !a.final_) return;  // nothing visible, state untouched

  const int64_t row = row0 + wave * 32 + qcol;
  const bool valid = row < a.q_len;
  const int64_t rowc = valid ? row : a.q_len - 1;
  const int64_t bh = (int64_t)b * a.heads_q + h;
  const size_t srow = (size_t)(bh * a.q_len + rowc);
  const int64_t kv_off = ((int64_t)b * a.heads_kv + kvh) * a.kv_len * D;
  const unsigned short* kg = static_cast<const unsigned short*>(a.k) + kv_off;
  const unsigned short* vg = static_cast<const unsigned short*>(a.v) + kv_off;

  // ---- start the first tile's copy as early as possible ----------------------
  auto tile_start = [&](int t) -> int32_t {
    return t < plan.r0.ntiles ? plan.r0.begin + t * kBN : plan.r1.begin + (t - plan.r0.ntiles) * kBN;
  };
  if (ntiles > 0) {
    const int32_t st = tile_start(0);
    load_tile<D, true>(kg, a.kv_len, st, smem, wave, lane);
    load_tile<D, false>(vg, a.kv_len, st, smem + Ly::kTileBytes, wave, lane);
  }

  // ---- Q^T fragments (B operand of S^T = K Q^T) ------------------------------
  bf16x8 qf[Ly::kDChunks];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(a.q) + srow * D);
#pragma unroll
    for (int c = 0; c < Ly::kDChunks; ++c) qf[c] = qp[2 * c + hh];
  }

  // ---- running state: lane holds O^T rows d = 32*db + 8*(j/4) + 4*hh + j%4 ---
  f32x16 oacc[Ly::kDBlocks];
  float m_run, l_run;
  if (a.init) {
#pragma unroll
    for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
    m_run = -INFINITY;
    l_run = 0.0f;
  } else {
    const float* op = a.o + srow * D;
#pragma unroll
    for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 x = *reinterpret_cast<const float4*>(op + 32 * db + 8 * jj + 4 * hh);
        oacc[db][4 * jj + 0] = x.x;
        oacc[db][4 * jj + 1] = x.y;
        oacc[db][4 * jj + 2] = x.z;
        oacc[db][4 * jj + 3] = x.w;
      }
    m_run = a.m[srow];
    l_run = hh == 0 ? a.l[srow] : 0.0f;  // the pair's two partial sums add up to l
  }

  // ---- per-lane constants -----------------------------------------------------
  const int64_t qpos = seg_position(a.qs, a.n_q_seg, rowc);
  const int32_t vend0 = row_visible_end(a, plan.r0, qpos);
  const int32_t vend1 = row_visible_end(a, plan.r1, qpos);
  const float sl2 = a.scale_log2;

  // K read (A operand of S^T): row kb*32 + qcol, logical unit 2c + hh.
  const int k_swz = Ly::k_swz(qcol);
  // V^T read by ds_read_b64_tr_b16: within each 16-lane group, source lane
  // s = 4t + q points at row (4*hh + t) of the 8-row slice and at head_dim
  // offset 32*db + 16*(group & 1) + 4q; the instruction hands output lane j
  // element j%4 of source lane 4t + j/4, i.e. V[row t][d = ... + j].
  const int grp = lane >> 4;
  const int t4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  const int v_row = 4 * hh + t4;
  const int v_swz = Ly::v_swz(v_row);
  int v_off[Ly::kDBlocks];
#pragma unroll
  for (int db = 0; db < Ly::kDBlocks; ++db) {
    const int unit = 4 * db + 2 * (grp & 1) + (q4 >> 1);
    v_off[db] = v_row * Ly::kRowBytes + ((unit ^ v_swz) << 4) + ((q4 & 1) << 3);
  }

  for (int t = 0; t < ntiles; ++t) {
    const bool first_range = t < plan.r0.ntiles;
    const int32_t start = tile_start(t);
    char* kt = smem + (t & 1) * 2 * Ly::kTileBytes;
    char* vt = kt + Ly::kTileBytes;

    // tile t has landed in LDS for every wave
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) {
      // the other buffer was last read in iteration t-1, before the barrier
      char* kn = smem + ((t + 1) & 1) * 2 * Ly::kTileBytes;
      const int32_t sn = tile_start(t + 1);
      load_tile<D, true>(kg, a.kv_len, sn, kn, wave, lane);
      load_tile<D, false>(vg, a.kv_len, sn, kn + Ly::kTileBytes, wave, lane);
    }

    // ---- S^T = K Q^T for two 32-key blocks --------------------------------
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.0f;
      const char* krow = kt + (kb * 32 + qcol) * Ly::kRowBytes;
#pragma unroll
      for (int c = 0; c < Ly::kDChunks; ++c) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + (((2 * c + hh) ^ k_swz) << 4));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
      }
    }

    // ---- causal / ragged mask on partial tiles ---------------------------------
    if (start + kBN > (first_range ? plan.r0.full : plan.r1.full)) {
      const int32_t lim = (first_range ? vend0 : vend1) - start;  // keys [0, lim) of this tile are visible
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (key >= lim) sacc[kb][j] = -INFINITY;
        }
    }

    // ---- online softmax (base 2, lazy rescale) ------------------------------------
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
    mx = max_with_partner(mx) * sl2;
    const float cand = fmaxf(m_run, mx);
    const bool need = cand > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_upd = need ? cand : m_run;
      const float alpha = (m_upd == m_run) ? 1.0f : exp2f(m_run - m_upd);
#pragma unroll
      for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      l_run *= alpha;
      m_run = m_upd;
    }
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j], sl2, -msub));
        sacc[kb][j] = p;
        psum += p;
      }
    l_run += psum;

    // ---- O^T += V^T P^T ------------------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 pf = pack_p(sacc[kb], 8 * c);
        const char* vslice = vt + (kb * 32 + 16 * c) * Ly::kRowBytes;
#pragma unroll
        for (int db = 0; db < Ly::kDBlocks; ++db) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vslice + v_off[db]));
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vslice + 8 * Ly::kRowBytes + v_off[db]));
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf, oacc[db], 0, 0, 0);
        }
      }
  }

  // ---- write back ---------------------------------------------------------------
  const float l_tot = sum_with_partner(l_run);
  if (!valid) return;
  if (a.final_) {
    const float inv = finalize_inv(l_tot);
    unsigned short* dst = static_cast<unsigned short*>(a.out) + srow * D;
#pragma unroll
    for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float4 x = make_float4(oacc[db][4 * jj], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]);
        x.x *= inv;
        x.y *= inv;
        x.z *= inv;
        x.w *= inv;
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_bits(x.x) | ((uint32_t)f32_to_bf16_bits(x.y) << 16);
        packed.y = (uint32_t)f32_to_bf16_bits(x.z) | ((uint32_t)f32_to_bf16_bits(x.w) << 16);
        *reinterpret_cast<uint2*>(dst + 32 * db + 8 * jj + 4 * hh) = packed;
      }
    if (hh == 0 && a.lse != nullptr) a.lse[srow] = finalize_lse(m_run, l_tot);
  } else {
    float* op = a.o + srow * D;
#pragma unroll
    for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(op + 32 * db + 8 * jj + 4 * hh) =
            make_float4(oacc[db][4 * jj], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]);
    if (hh == 0) {
      a.m[srow] = m_run;
      a.l[srow] = l_tot;
    }
  }
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, int head_dim, hipStream_t s) {
  const int64_t q_tiles = (a.q_len + kBM - 1) / kBM;
  const int64_t items = q_tiles * a.heads_q * a.batch;
  const int64_t per_xcd = (items + 7) / 8;
  const dim3 grid((unsigned)(per_xcd * 8));
  if (head_dim == 128)
    step_bf16_kernel<128><<<grid, kThreads, 0, s>>>(a, (int32_t)items, (int32_t)per_xcd, (int32_t)q_tiles);
  else
    step_bf16_kernel<64><<<grid, kThreads, 0, s>>>(a, (int32_t)items, (int32_t)per_xcd, (int32_t)q_tiles);
  return hipGetLastError();
}

}  // namespace ra
