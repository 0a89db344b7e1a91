// Backward ring step on the CDNA4 matrix cores (gfx950), bf16, head_dim 64 or 128.
//
// The pages run the ring forward only ("distributed training hands-on code",
// section 6.2, has no backward pass); this is the plain extension of the same
// block step. With P_ij = exp(scale q_i.k_j - LSE_i) over the visible keys,
// D_i = dO_i . O_i and dS_ij = P_ij (dO_i . v_j - D_i):
//   dQ_i += scale sum_j dS_ij k_j,  dK_j += scale sum_i dS_ij q_i,
//   dV_j += sum_i P_ij dO_i,
// where i runs over the local query rows and j over the keys of one K/V
// block; dK_j and dV_j are the accumulators that travel with the block.
//
// Two kernels, both v_mfma_f32_32x32x16_bf16:
//  * bwd_dq_kernel: query-stationary like the forward step. 8 waves x 32
//    rows; Q^T and dO^T stay in VGPRs; K and V tiles of 64 keys go HBM -> LDS
//    by buffer-to-LDS copies into four stages. Per tile: S^T = K Q^T and
//    dP^T = V dO^T (K, V read row-wise), dS^T in registers (one row per
//    lane, so LSE and D are one value per lane), then dQ^T += K^T dS^T with
//    K^T read by ds_read_b64_tr_b16 and dS^T (bf16) as the B operand.
//  * bwd_dkdv_kernel: key-stationary. 4 waves x 32 keys, one wave per SIMD;
//    K^T and V^T stay in VGPRs; tiles of 64 query rows of Q, dO and the two
//    row terms are copied into four LDS stages, for every query head of the
//    GQA group. Per tile: S = Q K^T and dP = dO V^T with the accumulators
//    started at -LSE/scale and -D (so no per-element subtraction), P and dS
//    in registers (one key per lane), then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T, Q^T read transposed.
//  Every tile that is read both row-wise and transposed uses one XOR swizzle
//  of its 16-byte units, 4 (row mod 4) + (row / 4 mod 4), under which both
//  read patterns hit distinct banks.
//  Rows (keys) past a range read as zero through the buffer bounds; a zero
//  query row with zero dO and zero row terms contributes exactly nothing.
#include "backward.h"
#include "bf16_tiles.h"

namespace ra {
namespace {

using namespace bf16k;

typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef RA_BWD_SCHED
#define RA_BWD_SCHED 0
#endif
#ifndef RA_KV_AHEAD
#define RA_KV_AHEAD 3
#endif
#ifndef RA_DQ_AHEAD
#define RA_DQ_AHEAD 3
#endif
#ifndef RA_BWD_AHEAD
#define RA_BWD_AHEAD 8
#endif
constexpr int kSchedValu = 0x002;
constexpr int kSchedTrans = 0x400;

// Tile geometry for head_dim D (64 or 128): rows of D bf16, 64-row tiles.
template <int D>
struct BL {
  static constexpr int kRowB = D * 2;         // one bf16 row
  static constexpr int kUnits = D / 8;         // 16-byte units per row
  static constexpr int kTileB = 64 * kRowB;    // 64 rows
  static constexpr int kDC = D / 16;           // K=16 chunks of a head_dim contraction
  static constexpr int kDB = D / 32;           // 32-column blocks of head_dim
  // Stored unit of logical unit u in row r is u ^ swz(r). D = 128 (16 units,
  // one row per 256-byte bank window): 4 (r mod 4) + (r / 4 mod 4). D = 64
  // (8 units, two rows per window): 4 (r / 2 mod 2) + (r / 4 mod 4). Either
  // way the 16 rows of a row-wise b128 read and the 4 rows x 4 units of a
  // transposed half-wave read land on distinct banks.
  __device__ static __forceinline__ int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

// Row-wise read (A operand, lane = row qcol of a 32-row block, 8 consecutive
// elements of logical unit 2c + hh).
template <int D>
__device__ __forceinline__ uint32_t row_read_addr(uint32_t base, int qcol, int hh, int c) {
  return base + qcol * BL<D>::kRowB + (((2 * c + hh) ^ BL<D>::swz(qcol)) << 4);
}

// Transposed read for ds_read_b64_tr_b16: d block db, lower (e = 0) or upper
// (e = 1) 8-row half of a 16-row chunk. Within a 16-lane group, source lane
// 4t + q points at row 8e + 4hh + t and columns 32db + 16(group & 1) + 4q..;
// output lane l then holds column 32db + l % 32 at rows 8e + 4hh + 0..3.
template <int D>
__device__ __forceinline__ uint32_t tr_read_addr(uint32_t base, int lane, int db, int e) {
  const int hh = lane >> 5;
  const int grp16 = lane >> 4;
  const int t4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  const int row = 8 * e + 4 * hh + t4;
  const int unit = 4 * db + 2 * (grp16 & 1) + (q4 >> 1);
  return base + row * BL<D>::kRowB + ((unit ^ BL<D>::swz(row)) << 4) + ((q4 & 1) << 3);
}

// A operand of a product that contracts over the rows of a tile: columns
// 32db + lane % 32, rows {0-3, 8-11} + 4hh of the 16-row chunk at byte offset
// `off` — the row order of the B operands packed from accumulators.
template <int N>
__device__ __forceinline__ bf16x8 read_tr(const uint32_t (&lo)[N], const uint32_t (&hi)[N], int db, uint32_t off) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_ptr<s16x4>(lo[db] + off));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_ptr<s16x4>(hi[db] + off));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// This lane's byte offsets for a wave's NB consecutive 1 KB blocks of a
// 64-row tile, first block `first_block`, in the form dma16_blocks takes
// (block j's offset minus 1024 j); the lane fills stored unit p of row r and
// fetches logical unit p ^ swz(r).
template <int D, int NB>
__device__ __forceinline__ void tile_block_offsets(int first_block, int lane, int (&voff)[NB]) {
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int u = (first_block + i) * 64 + lane;
    const int r = u / BL<D>::kUnits;
    const int p = u % BL<D>::kUnits;
    voff[i] = r * BL<D>::kRowB + ((p ^ BL<D>::swz(r)) << 4) - i * 1024;
  }
}

// Scheduling shape of N MFMAs that take R LDS reads each, interleaved with
// vector work: the reads run AHEAD MFMAs ahead of their use, and V vector
// instructions and T transcendental ones follow every MFMA.
template <int N, int R, int AHEAD, int V, int T>
__device__ __forceinline__ void sched_mfma_reads_valu() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD * R, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, V, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedTrans, T, 0);
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, V, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedTrans, T, 0);
  }
}

// ============================================================================
// dQ: query-stationary
// ============================================================================
constexpr int kQWaves = 8;
constexpr int kQRows = kQWaves * 32;
constexpr int kQStages = 4;  // a tile is read row-wise in M_t and transposed in M_{t+1}
template <int D>
__global__ void __launch_bounds__(kQWaves * 64) bwd_dq_kernel(BwdArgs a, int32_t q_tiles) {
  using L = BL<D>;
  constexpr int kD = D, kRowB = L::kRowB, kTileB = L::kTileB, kDC = L::kDC, kDB = L::kDB;
  constexpr int kQStageB = 2 * kTileB;                    // K tile, then V tile
  constexpr int kQCopies = 2 * (kTileB / 1024) / kQWaves;  // 1 KB copies per wave per tile
  __shared__ __attribute__((aligned(1024))) char smem[kQStages * kQStageB];
  const StepArgs& s = a.s;
  // Workgroup i runs on XCD i % 8. When the (batch, KV head) pairs divide
  // evenly over the 8 XCDs, each XCD takes whole KV heads, so its L2 holds
  // the K/V their query tiles stream; heavy (late) causal tiles first.
  // Otherwise the heavy-first order is dealt round-robin over the XCDs.
  int32_t tile, b, h;
  {
    const int32_t n_items = q_tiles * s.batch * s.heads_q;
    const int32_t n_bk = s.batch * s.heads_kv;
    if (n_bk % 8 == 0) {
      const int32_t per_xcd = n_items / 8;
      const int32_t item = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
      const int32_t per_kv = q_tiles * s.group;
      const int32_t bk = item / per_kv;
      const int32_t rem = item % per_kv;
      tile = q_tiles - 1 - rem / s.group;
      b = bk / s.heads_kv;
      h = (bk % s.heads_kv) * s.group + rem % s.group;
    } else {
      const int32_t n_bh = s.batch * s.heads_q;
      const int32_t item = (int32_t)blockIdx.x;
      tile = q_tiles - 1 - item / n_bh;
      b = (item % n_bh) / s.heads_q;
      h = (item % n_bh) % s.heads_q;
    }
  }
  const int32_t kvh = h / s.group;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qcol = lane & 31;
  const int hh = lane >> 5;

  const int64_t row0 = (int64_t)tile * kQRows;
  const int64_t r1 = (row0 + kQRows < s.q_len) ? row0 + kQRows : s.q_len;
  int64_t qmin, qmax;
  seg_range(s.qs, s.n_q_seg, row0, r1, &qmin, &qmax);
  const TilePlan plan = plan_tiles<64>(s, qmin, qmax);
  const int ntiles = plan.total_tiles();
  if (ntiles == 0 && !a.init_dq) return;  // nothing to add

  const int64_t row = row0 + wave * 32 + qcol;
  const bool valid = row < s.q_len;
  const int64_t rowc = valid ? row : s.q_len - 1;
  const int64_t n_rows = (int64_t)s.batch * s.heads_q * s.q_len;
  const size_t srow = (size_t)(((int64_t)b * s.heads_q + h) * s.q_len + rowc);
  const int64_t kv_off = ((int64_t)b * s.heads_kv + kvh) * s.kv_len * kD;
  const char* kg = reinterpret_cast<const char*>(static_cast<const unsigned short*>(s.k) + kv_off);
  const char* vg = reinterpret_cast<const char*>(static_cast<const unsigned short*>(s.v) + kv_off);

  auto tile_start = [&](int t) -> int32_t {
    return t < plan.r0.ntiles ? plan.r0.begin + t * 64 : plan.r1.begin + (t - plan.r0.ntiles) * 64;
  };
  const uint32_t smem_base = lds_address(smem);
  // K and V tiles share the swizzle, so one set of per-lane offsets serves both
  constexpr int kNB = kQCopies / 2;
  int voff[kNB];
  tile_block_offsets<D, kNB>(wave * kNB, lane, voff);
  const uint64_t kbase = uniform_address(kg), vbase = uniform_address(vg);
  auto issue = [&](int t) {
    const int32_t start = tile_start(t);
    const int32_t left = (int32_t)s.kv_len - start;  // row counts are < 2^31
    const int nbytes = (left < 64 ? left : 64) * kRowB;
    const uint32_t dst = smem_base + (uint32_t)(t % kQStages) * kQStageB + (uint32_t)(wave * kNB * 1024);
    const uint64_t off = (uint64_t)start * kRowB;
    dma16_blocks<kNB>(resource_at(kbase, off, nbytes), dst, voff);
    dma16_blocks<kNB>(resource_at(vbase, off, nbytes), dst + kTileB, voff);
  };
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);

  // Q^T and dO^T fragments (B operands): row rowc, elements 16c + 8hh .. +7.
  bf16x8 qf[kDC], of[kDC];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(s.q) + srow * kD);
    const bf16x8* op = reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(a.dout) + srow * kD);
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      qf[c] = qp[2 * c + hh];
      of[c] = op[2 * c + hh];
    }
  }
  const float sl2 = s.scale_log2;
  const float c2 = a.terms[srow] * sl2;  // -LSE * log2(e), or -inf
  const float e_row = a.terms[n_rows + srow];  // -D
  const int64_t qpos = seg_position(s.qs, s.n_q_seg, rowc);
  const int32_t vend0 = row_visible_end(s, plan.r0, qpos);
  const int32_t vend1 = row_visible_end(s, plan.r1, qpos);

  uint32_t k_addr[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) k_addr[c] = row_read_addr<D>(smem_base, qcol, hh, c);
  uint32_t lo[kDB], hi[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    lo[db] = tr_read_addr<D>(smem_base, lane, db, 0);
    hi[db] = tr_read_addr<D>(smem_base, lane, db, 1);
  }

  f32x16 dqa[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqa[db][j] = 0.0f;
  f32x16 sacc[2], pacc[2];
  bf16x8 dsf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sacc[kb][j] = 0.0f;
      pacc[kb][j] = 0.0f;
    }
    dsf[kb][0] = bf16x8{};
    dsf[kb][1] = bf16x8{};
  }

  // Per wave the work is M_0 V_0 M_1 V_1 ... V_{n-1} M_n with M_v = (dQ of
  // tile v-1, S and dP of tile v) on the matrix cores and V_v the vector work
  // of tile v (mask, P, dS). Waves 0-3 (group 0) run item i in phase i, waves
  // 4-7 (group 1) in phase i+1, so while one wave of a SIMD issues MFMAs its
  // partner works on the vector ALUs. Only even phases start with a barrier
  // (every wave passes n+1 of them). Tile t sits in stage t % 4: it is read
  // row-wise in M_t and transposed in M_{t+1}, by group 1 as late as phase
  // 2t+3, and refilled with tile t+4 after the barrier of phase 2t+4: group 0
  // copies its half of tile v+2 after V_v (phase 2v+1), group 1 its half of
  // tile v+3 after V_v (phase 2v+2). At even phase 2u each wave waits for its
  // copies of tile u (those of tile u+1 may stay in flight) and the barrier
  // publishes it.
  const int group = wave >> 2;
  int ph = 0;
  auto next_phase = [&]() {
    const int u = ph >> 1;
    if ((ph & 1) == 0) {
      if (u < ntiles) {
        if (u + 1 < ntiles)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kQCopies) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_barrier" ::: "memory");
    }
    ++ph;
  };

  auto iteration = [&](int v) {
    const uint32_t so = (uint32_t)(v % kQStages) * kQStageB;
    const uint32_t sp = (uint32_t)((v + kQStages - 1) % kQStages) * kQStageB;
    next_phase();
    // ---- M_v: dQ^T += K^T dS^T (tile v-1), then S^T = K Q^T and dP^T = V dO^T
    // (tile v): dS of tile v-1 is dead before the accumulators of tile v are
    // live, which keeps the wave within its registers. On the last iteration
    // (v == ntiles) the S and dP products read a stage holding an older tile
    // and are never used.
    if constexpr (D == 128) {
      // One stream of products with their LDS operands read AH products
      // ahead, fenced per product: dQ of tile v-1 (if any), then S and dP of
      // tile v.
      constexpr int AH = RA_DQ_AHEAD;
      constexpr int NQ = 4 * kDB;   // dQ products
      constexpr int NS = 4 * kDC;   // S and dP products
      const int first = v > 0 ? 0 : NQ;
      constexpr int NT = NQ + NS;
      bf16x8 op[NT];
      auto rd = [&](int i) {
        if (i < NQ) {
          op[i] = read_tr(lo, hi, i % kDB, sp + (i / kDB) * 16 * kRowB);
        } else {
          const int j = i - NQ;  // j = 4 c + 2 kb + (0: K, 1: V)
          const int c = j >> 2, kb = (j >> 1) & 1, isv = j & 1;
          op[i] = *lds_ptr<bf16x8>(k_addr[c] + so + (isv ? kTileB : 0) + kb * 32 * kRowB);
        }
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sacc[kb][j] = 0.0f;
          pacc[kb][j] = 0.0f;
        }
#pragma unroll
      for (int i = 0; i < AH; ++i)
        if (first + i < NT) rd(first + i);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (i < first) continue;
        if (i + AH < NT) rd(i + AH);
        if (i < NQ) {
          const int kc = i / kDB, db = i % kDB;
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], dsf[kc >> 1][kc & 1], dqa[db], 0, 0, 0);
        } else {
          const int j = i - NQ;
          const int c = j >> 2, kb = (j >> 1) & 1, isv = j & 1;
          if (isv)
            pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], of[c], pacc[kb], 0, 0, 0);
          else
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], qf[c], sacc[kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {  // at head_dim 64 the compiler's own schedule is faster
      if (v > 0) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const bf16x8 kt = read_tr(lo, hi, db, sp + kc * 16 * kRowB);
            dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf[kc >> 1][kc & 1], dqa[db], 0, 0, 0);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sacc[kb][j] = 0.0f;
          pacc[kb][j] = 0.0f;
        }
#pragma unroll
      for (int c = 0; c < kDC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *lds_ptr<bf16x8>(k_addr[c] + so + kb * 32 * kRowB);
          const bf16x8 vf = *lds_ptr<bf16x8>(k_addr[c] + so + kTileB + kb * 32 * kRowB);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
          pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, of[c], pacc[kb], 0, 0, 0);
        }
    }
    if (v < ntiles) {
      next_phase();
      // ---- V_v: P and dS of tile v, packed as the B operand of dQ
      const bool first_range = v < plan.r0.ntiles;
      const int32_t start = tile_start(v);
      if (start + 64 > (first_range ? plan.r0.full : plan.r1.full)) {
        const int32_t lim = (first_range ? vend0 : vend1) - start;  // keys [0, lim) are visible
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            if (key >= lim) sacc[kb][j] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j], sl2, c2));
          sacc[kb][j] = p * (pacc[kb][j] + e_row);
        }
        dsf[kb][0] = pack_p(sacc[kb], 0);
        dsf[kb][1] = pack_p(sacc[kb], 8);
      }
      const int t = v + (group == 1 ? 3 : 2);
      if (t >= 2 && t < ntiles) issue(t);
    }
  };

  // Q, dO, the row terms and the first tiles are in registers / LDS before
  // the loop.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (group == 1) {  // group 1 starts one phase late
    next_phase();
    if (2 < ntiles) issue(2);
  }
  for (int v = 0; v <= ntiles; ++v) iteration(v);
  if (group == 0) next_phase();  // group 0 ends one phase early

  if (!valid) return;
  float* dst = a.dq + srow * kD;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4* p = reinterpret_cast<float4*>(dst + 32 * db + 8 * jj + 4 * hh);
      float4 x = make_float4(dqa[db][4 * jj] * a.scale, dqa[db][4 * jj + 1] * a.scale, dqa[db][4 * jj + 2] * a.scale,
                             dqa[db][4 * jj + 3] * a.scale);
      if (!a.init_dq) {
        const float4 y = *p;
        x.x += y.x;
        x.y += y.y;
        x.z += y.z;
        x.w += y.w;
      }
      *p = x;
    }
}

// ============================================================================
// dK, dV: key-stationary
// ============================================================================
constexpr int kKWaves = 4;
constexpr int kKKeys = kKWaves * 32;
constexpr int kKStages = 4;

// Query rows [begin, end) of one query segment that see a key of the tile;
// rows from `full` on see every key of it.
struct RowRange {
  int64_t begin, end, full, off;
  int32_t ntiles, seg;
};

__device__ __forceinline__ RowRange row_range(const StepArgs& s, int seg, int64_t kmin, int64_t kmax) {
  RowRange r;
  r.seg = seg;
  if (!s.causal || s.n_q_seg <= 0 || s.n_kv_seg <= 0) {
    r.off = 0;
    r.begin = 0;
    r.end = s.q_len;
    r.full = 0;
  } else {
    const Seg g = seg == 0 ? s.qs[0] : s.qs[1];
    r.off = seg == 0 ? 0 : s.qs[0].len;
    r.begin = r.off + seg_count_le(g, kmin - 1);
    r.end = r.off + g.len;
    r.full = r.off + seg_count_le(g, kmax - 1);
  }
  r.ntiles = r.end > r.begin ? (int32_t)((r.end - r.begin + 63) / 64) : 0;
  return r;
}

template <int D>
__global__ void __launch_bounds__(kKWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_kernel(BwdArgs a, int32_t k_tiles) {
  using L = BL<D>;
  constexpr int kD = D, kRowB = L::kRowB, kTileB = L::kTileB, kDC = L::kDC, kDB = L::kDB;
  // stage: Q tile, dO tile, 64 row terms c, 64 row terms e (1 KB regions:
  // their copies write 64 lanes x 16 B)
  constexpr int kKOffDo = kTileB;
  constexpr int kKOffC = 2 * kTileB;
  constexpr int kKOffE = 2 * kTileB + 1024;
  constexpr int kKStageB = 2 * kTileB + 2048;
  constexpr int kKCopies = (kTileB / 1024) / kKWaves;  // per tensor, per wave
  __shared__ __attribute__((aligned(1024))) char smem[kKStages * kKStageB];
  const StepArgs& s = a.s;
  const int32_t n_bk = s.batch * s.heads_kv;
  const int32_t item = (int32_t)blockIdx.x;
  const int32_t kt = item / n_bk;  // early keys (most query rows) first
  const int32_t b = (item % n_bk) / s.heads_kv;
  const int32_t kvh = (item % n_bk) % s.heads_kv;
  if (kt >= k_tiles) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qcol = lane & 31;
  const int hh = lane >> 5;

  const int64_t key0 = (int64_t)kt * kKKeys;
  const int64_t k1 = (key0 + kKKeys < s.kv_len) ? key0 + kKKeys : s.kv_len;
  int64_t kmin, kmax;
  seg_range(s.ks, s.n_kv_seg, key0, k1, &kmin, &kmax);
  const bool causal = s.causal && s.n_q_seg > 0 && s.n_kv_seg > 0;
  const RowRange ra0 = row_range(s, 0, kmin, kmax);
  const RowRange ra1 = (causal && s.n_q_seg > 1) ? row_range(s, 1, kmin, kmax) : RowRange{0, 0, 0, 0, 0, 1};
  const int32_t nq = ra0.ntiles + ra1.ntiles;
  const int32_t total = nq * s.group;
  if (total == 0) return;  // no query row sees this tile: nothing to add

  const int64_t key = key0 + wave * 32 + qcol;
  const bool valid = key < s.kv_len;
  const int64_t keyc = valid ? key : s.kv_len - 1;
  const size_t kvrow = (size_t)(((int64_t)b * s.heads_kv + kvh) * s.kv_len + keyc);

  // K^T and V^T fragments (B operands): key keyc, elements 16c + 8hh .. +7.
  bf16x8 kf[kDC], vf[kDC];
  {
    const bf16x8* kp = reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(s.k) + kvrow * kD);
    const bf16x8* vp = reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(s.v) + kvrow * kD);
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      kf[c] = kp[2 * c + hh];
      vf[c] = vp[2 * c + hh];
    }
  }
  // First query row of each range that sees this lane's key.
  int64_t fv0 = ra0.begin, fv1 = ra1.begin;
  if (causal) {
    const int64_t kpos = seg_position(s.ks, s.n_kv_seg, keyc);
    fv0 = ra0.off + seg_count_le(s.qs[0], kpos - 1);
    if (s.n_q_seg > 1) fv1 = ra1.off + seg_count_le(s.qs[1], kpos - 1);
  }

  const int64_t n_rows = (int64_t)s.batch * s.heads_q * s.q_len;
  const uint32_t smem_base = lds_address(smem);
  // iteration it -> (query head, range, tile): the last query tile first,
  // every head of the group per tile. The row ranges of all key tiles end at
  // the same row (and, in the contiguous and zigzag layouts, their tiles are
  // 64-row aligned), so the workgroups of one
  // KV head that run together on an XCD read the same Q and dO tiles at about
  // the same time and share them in its L2 (their reads per step: 1317 ->
  // 896 MiB against head-major order from each range's first row).
  auto decode = [&](int it, int32_t* h, const RowRange** r, int64_t* rs) {
    const int g = it % s.group;
    const int tt = nq - 1 - it / s.group;
    *h = kvh * s.group + g;
    *r = tt < ra0.ntiles ? &ra0 : &ra1;
    *rs = (*r)->begin + (int64_t)(tt < ra0.ntiles ? tt : tt - ra0.ntiles) * 64;
  };
  // Q and dO tiles share the swizzle, so one set of per-lane offsets serves both
  int voff[kKCopies];
  tile_block_offsets<D, kKCopies>(wave * kKCopies, lane, voff);
  const int toff[1] = {lane * 16};  // a block of 64 row terms
  const uint64_t qbase = uniform_address(s.q), obase = uniform_address(a.dout);
  const uint64_t tbase = uniform_address(a.terms);
  auto issue = [&](int it) {
    int32_t h;
    const RowRange* r;
    int64_t rs;
    decode(it, &h, &r, &rs);
    const int64_t left = r->end - rs;
    const int nrows = (int)(left < 64 ? left : 64);
    const int64_t first = ((int64_t)b * s.heads_q + h) * s.q_len + rs;
    const uint32_t dst = smem_base + (uint32_t)(it % kKStages) * kKStageB;
    const uint32_t wdst = dst + (uint32_t)(wave * kKCopies * 1024);
    const uint64_t off = (uint64_t)first * kRowB;
    dma16_blocks<kKCopies>(resource_at(qbase, off, nrows * kRowB), wdst, voff);
    dma16_blocks<kKCopies>(resource_at(obase, off, nrows * kRowB), wdst + kKOffDo, voff);
    if (wave == 0) dma16_blocks<1>(resource_at(tbase, (uint64_t)first * 4, nrows * 4), dst + kKOffC, toff);
    if (wave == 1)
      dma16_blocks<1>(resource_at(tbase, (uint64_t)(n_rows + first) * 4, nrows * 4), dst + kKOffE, toff);
  };
  issue(0);
  if (total > 1) issue(1);

  uint32_t q_addr[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) q_addr[c] = row_read_addr<D>(smem_base, qcol, hh, c);
  uint32_t lo[kDB], hi[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    lo[db] = tr_read_addr<D>(smem_base, lane, db, 0);
    hi[db] = tr_read_addr<D>(smem_base, lane, db, 1);
  }
  const float sl2 = s.scale_log2;

  f32x16 dka[kDB], dva[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      dka[db][j] = 0.0f;
      dva[db][j] = 0.0f;
    }

  // Tile `it` is published at the start of iteration it. Its S and dP
  // products run first; then the dV/dK products of tile it-1 (which need only
  // its packed P and dS and its LDS stage) are interleaved with the vector
  // work (mask, P, dS) of tile it, so the matrix cores keep busy while the
  // wave exponentiates. With four stages and copies issued two tiles ahead,
  // the stage refilled at iteration it held tile it-2, last read in
  // iteration it-1, before this iteration's barrier.
  bf16x8 pf[2][2], dsf[2][2];
  auto publish = [&](int it) {
    // Waves 0 and 1 also copy one block of row terms per tile.
    if (it + 1 < total) {
      if (wave < 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kKCopies + 1) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kKCopies) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    if (it + 2 < total) issue(it + 2);
  };
  // S = Q K^T and dP = dO V^T, accumulators started at the row terms
  // (S - LSE/scale and dP - D); then the causal mask of partial tiles.
  auto products = [&](int it, f32x16 (&sacc)[2], f32x16 (&pacc)[2]) {
    const uint32_t so = (uint32_t)(it % kKStages) * kKStageB;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t ro = (uint32_t)((32 * rb + 8 * jj + 4 * hh) * 4);
        const f32x4 c4 = *lds_ptr<f32x4>(smem_base + so + kKOffC + ro);
        const f32x4 e4 = *lds_ptr<f32x4>(smem_base + so + kKOffE + ro);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[rb][4 * jj + i] = c4[i];
          pacc[rb][4 * jj + i] = e4[i];
        }
      }
    if constexpr (D == 128) {
      {
        // the products in one fenced stream, LDS operands read AH ahead
        constexpr int AH = RA_KV_AHEAD;
        constexpr int N = 4 * kDC;  // i = 4 c + 2 rb + (0: S, 1: dP)
        bf16x8 op[N];
        auto rd = [&](int i) {
          const int c = i >> 2, rb = (i >> 1) & 1, isp = i & 1;
          op[i] = *lds_ptr<bf16x8>(q_addr[c] + so + (isp ? kKOffDo : 0) + rb * 32 * kRowB);
        };
#pragma unroll
        for (int i = 0; i < AH; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          if (i + AH < N) rd(i + AH);
          const int c = i >> 2, rb = (i >> 1) & 1;
          if (i & 1)
            pacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], vf[c], pacc[rb], 0, 0, 0);
          else
            sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], kf[c], sacc[rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {  // at head_dim 64 the compiler's own schedule is faster
#pragma unroll
      for (int c = 0; c < kDC; ++c)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const bf16x8 qa = *lds_ptr<bf16x8>(q_addr[c] + so + rb * 32 * kRowB);
          const bf16x8 oa = *lds_ptr<bf16x8>(q_addr[c] + so + kKOffDo + rb * 32 * kRowB);
          sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[c], sacc[rb], 0, 0, 0);
          pacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[c], pacc[rb], 0, 0, 0);
        }
    }
#if RA_BWD_SCHED
    // the 16 row-term reads first (they start the accumulators), then the
    // operand reads RA_BWD_AHEAD MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 16, 0);
    sched_mfma_reads_valu<32, 1, RA_BWD_AHEAD, 0, 0>();
#endif
    int32_t h;
    const RowRange* r;
    int64_t rs;
    decode(it, &h, &r, &rs);
    if (causal && rs < r->full) {
      // rows of the tile before this lane's first visible row see no key of it
      const int64_t fv = r == &ra0 ? fv0 : fv1;
      const int64_t d = fv - rs;
      const int32_t lim = d < 0 ? 0 : (d > 64 ? 64 : (int32_t)d);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * rb + 8 * (j >> 2) + 4 * hh + (j & 3) < lim) sacc[rb][j] = -INFINITY;
    }
  };
  auto softmax = [&](f32x16 (&sacc)[2], f32x16 (&pacc)[2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(sacc[rb][j] * sl2);
        sacc[rb][j] = p;
        pacc[rb][j] = p * pacc[rb][j];
      }
      pf[rb][0] = pack_p(sacc[rb], 0);
      pf[rb][1] = pack_p(sacc[rb], 8);
      dsf[rb][0] = pack_p(pacc[rb], 0);
      dsf[rb][1] = pack_p(pacc[rb], 8);
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS of tile `it` (P, dS given packed).
  auto grads = [&](int it, const bf16x8 (&p)[2][2], const bf16x8 (&ds)[2][2]) {
    const uint32_t so = (uint32_t)(it % kKStages) * kKStageB;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const uint32_t off = so + kc * 16 * kRowB;
        const bf16x8 ot = read_tr(lo, hi, db, off + kKOffDo);
        const bf16x8 qt = read_tr(lo, hi, db, off);
        dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot, p[kc >> 1][kc & 1], dva[db], 0, 0, 0);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, ds[kc >> 1][kc & 1], dka[db], 0, 0, 0);
      }
  };

  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  {
    publish(0);
    f32x16 sacc[2], pacc[2];
    products(0, sacc, pacc);
    softmax(sacc, pacc);
  }
  for (int it = 1; it < total; ++it) {
    publish(it);
    f32x16 sacc[2], pacc[2];
    products(it, sacc, pacc);
    bf16x8 pp[2][2], dp[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        pp[i][k] = pf[i][k];
        dp[i][k] = dsf[i][k];
      }
    grads(it - 1, pp, dp);
    softmax(sacc, pacc);
#if RA_BWD_SCHED
    sched_mfma_reads_valu<32, 2, RA_BWD_AHEAD, 3, 1>();
#endif
  }
  grads(total - 1, pf, dsf);

  if (!valid) return;
  float* dkp = a.dk + kvrow * kD;
  float* dvp = a.dv + kvrow * kD;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 32 * db + 8 * jj + 4 * hh;
      float4* pk = reinterpret_cast<float4*>(dkp + d);
      float4* pv = reinterpret_cast<float4*>(dvp + d);
      float4 xk = *pk, xv = *pv;
      xk.x += dka[db][4 * jj + 0] * a.scale;
      xk.y += dka[db][4 * jj + 1] * a.scale;
      xk.z += dka[db][4 * jj + 2] * a.scale;
      xk.w += dka[db][4 * jj + 3] * a.scale;
      xv.x += dva[db][4 * jj + 0];
      xv.y += dva[db][4 * jj + 1];
      xv.z += dva[db][4 * jj + 2];
      xv.w += dva[db][4 * jj + 3];
      *pk = xk;
      *pv = xv;
    }
}

// ============================================================================
// Row terms and conversion
// ============================================================================
template <int D, typename T>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const T* out, const T* dout, const float* lse, float* terms,
                                                       int64_t rows, float inv_scale) {
  constexpr int kPer = D / 16;  // elements per lane, 16 lanes per row
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < rows) {
    const T* o = out + row * D + sub * kPer;
    const T* g = dout + row * D + sub * kPer;
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc += (float)o[i] * (float)g[i];
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (sub == 0 && row < rows) {
    const float l = lse[row];
    terms[row] = l == -INFINITY ? -INFINITY : -l * inv_scale;
    terms[rows + row] = -acc;
  }
}

__global__ void __launch_bounds__(256) convert_kernel(const float* x, void* y, int64_t n4, int dtype) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(x)[i];
  if (dtype == RA_BF16) {
    uint2 p;
    p.x = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
    p.y = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
    reinterpret_cast<uint2*>(y)[i] = p;
  } else {
    reinterpret_cast<float4*>(y)[i] = v;
  }
}

__global__ void __launch_bounds__(256) zero_kernel(uint4* p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  zero_kernel<<<dim3((unsigned)((n16 + 255) / 256)), 256, 0, s>>>(static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* terms, int64_t rows,
                           int head_dim, int dtype, float scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows * 16 + 255) / 256));
  const float inv = 1.0f / scale;
  if (dtype == RA_BF16) {
    if (head_dim == 128)
      bwd_prep_kernel<128, __bf16><<<grid, 256, 0, s>>>(static_cast<const __bf16*>(out),
                                                        static_cast<const __bf16*>(dout), lse, terms, rows, inv);
    else
      bwd_prep_kernel<64, __bf16><<<grid, 256, 0, s>>>(static_cast<const __bf16*>(out),
                                                       static_cast<const __bf16*>(dout), lse, terms, rows, inv);
  } else {
    if (head_dim == 128)
      bwd_prep_kernel<128, float><<<grid, 256, 0, s>>>(static_cast<const float*>(out),
                                                       static_cast<const float*>(dout), lse, terms, rows, inv);
    else
      bwd_prep_kernel<64, float><<<grid, 256, 0, s>>>(static_cast<const float*>(out),
                                                      static_cast<const float*>(dout), lse, terms, rows, inv);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  const int32_t q_tiles = (int32_t)((a.s.q_len + kQRows - 1) / kQRows);
  const int64_t nq = (int64_t)q_tiles * a.s.batch * a.s.heads_q;
  bwd_dq_kernel<D><<<dim3((unsigned)nq), kQWaves * 64, 0, s>>>(a, q_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.s.kv_len == 0) return e;
  const int32_t k_tiles = (int32_t)((a.s.kv_len + kKKeys - 1) / kKKeys);
  const int64_t nk = (int64_t)k_tiles * a.s.batch * a.s.heads_kv;
  bwd_dkdv_kernel<D><<<dim3((unsigned)nk), kKWaves * 64, 0, s>>>(a, k_tiles);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, hipStream_t s) {
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  if (a.s.q_len == 0 || a.s.batch == 0) return hipSuccess;
  return head_dim == 128 ? launch_bwd_d<128>(a, s) : launch_bwd_d<64>(a, s);
}

hipError_t launch_convert(const float* x, void* y, int64_t n, int dtype, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  convert_kernel<<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, s>>>(x, y, n4, dtype);
  return hipGetLastError();
}

}  // namespace ra
