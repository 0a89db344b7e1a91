// bf16 ring step on the CDNA4 matrix cores (gfx950).
//
// One launch folds one K/V block into the running (O, m, l) state of the local
// query block — the block step of "distributed training hands-on code",
// section 6.2 — with the causal skipping of "Ring Attention and Sequence
// Parallelism", sections 4/6 and lecture 30, section 3.2, and GQA head
// sharing (lecture 30, section 3.4).
//
// Mapping (head_dim D in {64, 128}):
//  * A workgroup of 8 waves owns 256 query rows of one (batch, q head); each
//    wave owns 32 rows. Waves w and w+4 run on the same SIMD. The two groups
//    (waves 0-3 and 4-7) run one phase apart: in each tile interval group 0
//    issues its matrix instructions (P V of tile t-1 and S of tile t) and
//    then runs its softmax, group 1 the other way round, so while one wave of
//    a SIMD keeps the MFMA pipe busy its partner works on the vector ALUs
//    ("ping-pong"). The groups meet at a workgroup barrier once per tile,
//    where the next tile is published.
//  * Keys are consumed in tiles of 64. K and V tiles are copied HBM -> LDS by
//    16-byte buffer-to-LDS loads (bounds-checked by the buffer resource: rows
//    past the block read as zero and are masked), in a ring of four LDS
//    stages: a tile is requested four phases before its first use.
//  * The 16-byte units of each LDS row are XOR-swizzled through the global
//    offset, so the K reads (16 lanes x 16 B over 16 rows) and the V
//    transposed reads (4 rows x 4 units per half-wave) are free of bank
//    conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (A operand) is read with ds_read_b128, Q^T
//    (B operand) sits in VGPRs for the whole launch. In the accumulator every
//    lane holds 32 keys of ONE query row, so row max and row sum are
//    lane-local plus one v_permlane32_swap with the partner lane.
//  * P^T is converted to bf16 in registers and is directly the B operand of
//    O^T += V^T P^T: the 32x32 accumulator layout puts keys {0-3, 8-11}+4h of
//    each 16-key chunk in lane half h, and V^T (A operand) is fetched in the
//    same key order by ds_read_b64_tr_b16 from row-major V.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score.
//    The reference maximum is raised lazily (only when a row's maximum grows
//    by more than 8 in base-2 units); O and l are rescaled only then.
#include <type_traits>

#include "bf16_tiles.h"

namespace ra {
namespace {

using namespace bf16k;

constexpr int kWaves = 8;               // two groups of four; w and w+4 share a SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;        // query rows per workgroup
constexpr int kPrefetch = kStages - 2;  // tiles fetched ahead of the one in use
static_assert(kStages == 4, "the copy schedule below assumes four stages");
// 1 KB copies per wave, per tensor and half tile
template <int D>
constexpr int kLoadsPerWave = Layout<D>::kTileBytes / 1024 / kWaves;
#ifndef RA_LOOKAHEAD
#define RA_LOOKAHEAD 6
#endif
constexpr int kLookahead = RA_LOOKAHEAD;  // MFMAs whose LDS operands are in flight
#ifndef RA_PVS_AHEAD
#define RA_PVS_AHEAD 4
#endif
constexpr int kPvsAhead = RA_PVS_AHEAD;  // same, for the interleaved P-V / S phase
#ifndef RA_VPRE
#define RA_VPRE 2
#endif
// P-V MFMAs of a matrix phase whose V^T operands are read at the end of the
// wave's preceding softmax phase, before the barrier (the stage holding that
// V tile was published two phases earlier and is not refilled until later).
constexpr int kVPre = RA_VPRE;

// Copy the K and V tile of 64 rows starting at local key `start` into one LDS
// stage. The buffer resources bound the reads to the rows the block has: rows
// past kv_len read as zero (their scores are masked).
// One half of a tile: `half` picks the first or second half of the tile's 1 KB
// blocks, `slot` (0..3) this wave's quarter of that half.
template <int D>
__device__ __forceinline__ void issue_tile(const char* kg, const char* vg, int64_t kv_len, int32_t start,
                                           uint32_t k_dst, uint32_t v_dst, int half, int slot, int lane) {
  using Ly = Layout<D>;
  const int64_t left = kv_len - start;
  const int nbytes = (int)((left < kBN ? left : kBN) * Ly::kRowBytes);
  const i32x4 rk = buffer_resource(kg + (int64_t)start * Ly::kRowBytes, nbytes);
  const i32x4 rv = buffer_resource(vg + (int64_t)start * Ly::kRowBytes, nbytes);
#pragma unroll
  for (int i = 0; i < kLoadsPerWave<D>; ++i) {
    // lane fills stored unit p of row r and fetches logical unit p ^ swz(r)
    const int b = half * (Ly::kTileBytes / 2048) + slot * kLoadsPerWave<D> + i;  // 1 KB block of the tile
    const int u = b * 64 + lane;
    const int r = u / Ly::kUnits;
    const int p = u % Ly::kUnits;
    const uint32_t blk = (uint32_t)(b * 1024);
    dma16(rk, k_dst + blk, r * Ly::kRowBytes + ((p ^ Ly::k_swz(r)) << 4));
    dma16(rv, v_dst + blk, r * Ly::kRowBytes + ((p ^ Ly::v_swz(r)) << 4));
  }
}

// Scheduling shape of a block of N MFMAs that each take R LDS reads: the
// reads run four MFMAs ahead of their use (enough to cover LDS latency)
// instead of all being hoisted up front, which would exhaust the registers.
template <int N, int R, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma() {
  if constexpr (AHEAD <= 0) return;  // leave the order to the compiler
  constexpr int kAhead = AHEAD < N ? AHEAD : N - 1;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kAhead * R, 0);
#pragma unroll
  for (int i = 0; i < N - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAhead, 0);
}

template <int D>
__device__ __forceinline__ void pv_mfma(int i, const bf16x8& vt, const bf16x8 (&pf)[2][2], f32x16* oacc) {
  using Ly = Layout<D>;
  const int db = i % Ly::kDBlocks;
  const int kc = i / Ly::kDBlocks;
  oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf[kc / 2][kc % 2], oacc[db], 0, 0, 0);
}

// MFMA i of S^T = K Q^T for the tile in stage ST: key block kb = i % 2,
// head_dim chunk c = i / 2.
template <int D, int ST>
__device__ __forceinline__ void s_mfma(int i, const uint32_t* k_addr, const bf16x8* qf, f32x16 (&sacc)[2]) {
  using Ly = Layout<D>;
  const int kb = i % 2;
  const int c = i / 2;
  const bf16x8 kf = *lds_ptr<bf16x8>(k_addr[c] + ST * Ly::kTileBytes + kb * 32 * Ly::kRowBytes);
  sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
}

// LDS reads taken by MFMA k of the interleaved order P-V 0, S 0, P-V 1,
// S 1, ..., then the P-V MFMAs past NS: two per P-V MFMA (none for the first
// PRE, whose operands were read earlier), one per S MFMA.
constexpr int pvs_reads(int k, int NP, int NS, int PRE) {
  if (k >= NP + NS) return 0;
  if (k < 2 * NS) return (k & 1) ? 1 : ((k / 2) < PRE ? 0 : 2);
  return (NS + k - 2 * NS) < PRE ? 0 : 2;
}
constexpr int pvs_reads_before(int n, int NP, int NS, int PRE) {
  int r = 0;
  for (int k = 0; k < n; ++k) r += pvs_reads(k, NP, NS, PRE);
  return r;
}

// Scheduling shape of NP P-V MFMAs interleaved with NS S MFMAs: the operands
// of MFMA k + AHEAD are read right after MFMA k is issued.
template <int NP, int NS, int PRE, int AHEAD>
__device__ __forceinline__ void pipeline_pv_s() {
  static_assert(NS <= NP, "more S than P-V MFMAs");
  constexpr int kPro = pvs_reads_before(AHEAD, NP, NS, PRE);
  if constexpr (kPro > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPro, 0);
#pragma unroll
  for (int k = 0; k < NP + NS; ++k) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    const int r = pvs_reads(k + AHEAD, NP, NS, PRE);
    if (r == 1) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    if (r == 2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) step_bf16_kernel(StepArgs a, int32_t n_items, int32_t items_per_xcd,
                                                             int32_t q_tiles) {
  using Ly = Layout<D>;
  __shared__ __attribute__((aligned(1024))) char smem[Ly::kSmemBytes];

  // ---- work item ------------------------------------------------------------
  // Workgroup i runs on XCD i % 8. When the (batch, KV head) pairs divide
  // evenly over the 8 XCDs, each XCD takes whole KV heads (its L2 streams
  // their K/V), heavy (late) causal tiles first. Otherwise (e.g. one KV head)
  // that would hand the heavy tiles to some XCDs and the light ones to
  // others, so the heavy-first order is dealt round-robin over all XCDs.
  int32_t tile, b, h;
  {
    const int32_t n_bk = a.batch * a.heads_kv;
    if (n_bk % 8 == 0) {
      const int32_t item = (int32_t)(blockIdx.x % 8) * items_per_xcd + (int32_t)(blockIdx.x / 8);
      if (item >= n_items) return;
      const int32_t per_kv = q_tiles * a.group;
      const int32_t bk = item / per_kv;
      const int32_t rem = item % per_kv;
      tile = q_tiles - 1 - rem / a.group;
      b = bk / a.heads_kv;
      h = (bk % a.heads_kv) * a.group + rem % a.group;
    } else {
      const int32_t item = (int32_t)blockIdx.x;
      if (item >= n_items) return;
      const int32_t n_bh = a.batch * a.heads_q;
      tile = q_tiles - 1 - item / n_bh;
      b = (item % n_bh) / a.heads_q;
      h = (item % n_bh) % a.heads_q;
    }
  }
  const int32_t kvh = h / a.group;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qcol = lane & 31;
  const int hh = lane >> 5;
  const int group = wave >> 2;  // 0: first phase group, 1: one phase behind

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
  const char* kg = reinterpret_cast<const char*>(static_cast<const unsigned short*>(a.k) + kv_off);
  const char* vg = reinterpret_cast<const char*>(static_cast<const unsigned short*>(a.v) + kv_off);

  auto tile_start = [&](int t) -> int32_t {
    return t < plan.r0.ntiles ? plan.r0.begin + t * kBN : plan.r1.begin + (t - plan.r0.ntiles) * kBN;
  };

  const uint32_t smem_base = lds_address(smem);
  // Tile copies are issued by the waves that run a softmax phase, right after
  // their softmax, where they would otherwise wait at the barrier; the matrix
  // waves never stall on load issue. Group g copies half g of each tile.
  auto issue = [&](int t) {
    const uint32_t st = (uint32_t)(t % kStages) * Ly::kTileBytes;
    issue_tile<D>(kg, vg, a.kv_len, tile_start(t), smem_base + st, smem_base + Ly::kVBase + st, group, wave & 3,
                  lane);
  };
#pragma unroll
  for (int t = 0; t < kPrefetch; ++t)
    if (t < ntiles) issue(t);

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

  // Per-lane LDS addresses, fixed for the launch; every read below adds only a
  // compile-time offset (stage, key block, slice) that fits the 16-bit
  // offset field of the instruction.
  // K read (A operand of S^T): row kb*32 + qcol, logical unit 2c + hh.
  uint32_t k_addr[Ly::kDChunks];
#pragma unroll
  for (int c = 0; c < Ly::kDChunks; ++c) k_addr[c] = k_read_address<D>(smem_base, qcol, hh, c);
  uint32_t v_addr[Ly::kDBlocks];
#pragma unroll
  for (int db = 0; db < Ly::kDBlocks; ++db) v_addr[db] = v_read_address<D>(smem_base, lane, db);

  f32x16 sacc[2];
  bf16x8 pf[2][2];
  bf16x8 vpre[kVPre > 0 ? kVPre : 1];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c) pf[kb][c] = bf16x8{};

  // Per wave the work is the sequence M_0 S_0 M_1 S_1 ... S_{n-1} M_n with
  // M_v = (P V of tile v-1, S of tile v) on the matrix cores and S_t the
  // softmax of tile t. Group 0 runs item i in phase i, group 1 in phase i+1.
  // Only even phases start with a workgroup barrier (all waves pass n+1 of
  // them); within the two phases between barriers each wave runs one matrix
  // and one softmax phase at its own pace. The tile loop is unrolled by
  // kStages so the stage is a compile-time constant.
  int ph = 0;
  // Tile t lands in stage t % kStages (four stages). Group 1 copies its half
  // after its softmax of tile t-3 (phase 2t-4; its idle phase 0 for tile 2),
  // group 0 after its softmax of tile t-2 (phase 2t-3); the stage last held
  // tile t-4, read for the last time in phase 2t-5, so the barrier that
  // opens phase 2t-4 lies between its last read and the copies. At the start of even
  // phase 2u each wave waits until its copies of tile u have landed (its
  // copies of tile u+1 were issued after them and may still be in flight;
  // loads complete in order) and the barrier publishes tile u.
  auto next_phase = [&]() {
    const int u = ph >> 1;
    if ((ph & 1) == 0) {
      if (u < ntiles) {
        if (kPrefetch == 2 && u + 1 < ntiles)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLoadsPerWave<D>) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      // Execution barrier only: a fence here would make every wave wait for
      // all of its copies in flight, not just for the tile being published.
      // Every LDS read of a matrix phase feeds an MFMA of that phase, so it
      // has completed; reads issued at the end of a softmax phase (V^T
      // operands of a tile published earlier) may still be in flight and are
      // waited for at their first use.
      asm volatile("s_barrier" ::: "memory");
    }
    // Odd phase boundaries need no barrier: nothing is published there, and
    // every stage is refilled (after S_v: tile v+2 by group 0, tile v+3 by
    // group 1) at least one even barrier after the last read of the tile it
    // held.
    ++ph;
  };

  // One loop iteration: M_v (P V of tile v-1 from stage ST_PREV, S of tile v
  // from stage ST), then S_v.
  auto iteration = [&](auto st_tag, int v) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr int ST_PREV = (ST + kStages - 1) % kStages;
    next_phase();
    // ---- M_v: O^T += V^T P^T (tile v-1) interleaved with S^T = K Q^T (tile v).
    // The two products use different accumulators, so alternating them keeps
    // six independent MFMA chains in flight.
    // v == 0 has no P-V yet (it is peeled off below); on the last iteration
    // (v == ntiles) the S products read a stage holding an older tile and
    // are never used, which keeps a single code path.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.0f;
    if (v == 0) {
#pragma unroll
      for (int i = 0; i < 2 * Ly::kDChunks; ++i) s_mfma<D, ST>(i, k_addr, qf, sacc);
      pipeline_lds_mfma<2 * Ly::kDChunks, 1, kLookahead>();
    } else {
#pragma unroll
      for (int i = 0; i < 4 * Ly::kDBlocks; ++i) {
        if (i < kVPre)
          pv_mfma<D>(i, vpre[i < kVPre ? i : 0], pf, oacc);
        else
          pv_mfma<D>(i, read_vt<D, ST_PREV>(i, v_addr), pf, oacc);
        if (i < 2 * Ly::kDChunks) s_mfma<D, ST>(i, k_addr, qf, sacc);
      }
      pipeline_pv_s<4 * Ly::kDBlocks, 2 * Ly::kDChunks, kVPre, kPvsAhead>();
    }
    const bool do_s = v < ntiles;
    if (do_s) {
      next_phase();
      // ---- softmax of tile v -------------------------------------------------------
      const bool first_range = v < plan.r0.ntiles;
      const int32_t start = tile_start(v);
      if (start + kBN > (first_range ? plan.r0.full : plan.r1.full)) {
        const int32_t lim = (first_range ? vend0 : vend1) - start;  // keys [0, lim) are visible
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            if (key >= lim) sacc[kb][j] = -INFINITY;
          }
      }
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
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) pf[kb][c] = pack_p(sacc[kb], 8 * c);
      {
        const int t = v + (group == 1 ? 3 : 2);
        if (t >= kPrefetch && t < ntiles) issue(t);
      }
#pragma unroll
      for (int i = 0; i < kVPre; ++i) vpre[i] = read_vt<D, ST>(i, v_addr);
    }
  };

  // Everything loaded so far (Q, the incoming state, the first tiles) must
  // be in registers / LDS before the loop. The builtin (not asm) form lets
  // the compiler see it, so it inserts no load waits inside the loop, where
  // the hardware counter also counts the tile copies in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  if (group == 1) {  // group 1 starts one phase late
    next_phase();
    if (kPrefetch < ntiles) issue(kPrefetch);
  }
  for (int v = 0; v <= ntiles; v += kStages) {
    iteration(std::integral_constant<int, 0>{}, v);
    if (v + 1 > ntiles) break;
    iteration(std::integral_constant<int, 1>{}, v + 1);
    if (v + 2 > ntiles) break;
    iteration(std::integral_constant<int, 2>{}, v + 2);
    if constexpr (kStages == 4) {
      if (v + 3 > ntiles) break;
      iteration(std::integral_constant<int, 3 % kStages>{}, v + 3);
    }
  }
  if (group == 0) next_phase();  // group 0 ends one phase early

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
