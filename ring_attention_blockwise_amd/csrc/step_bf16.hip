// bf16 ring step on the CDNA4 matrix cores (gfx950), software-pipelined.
//
// One launch folds one K/V block into the running (O, m, l) state of the local
// query block — the block step of "distributed training hands-on code",
// section 6.2 — with the causal skipping of "Ring Attention and Sequence
// Parallelism", sections 4/6 and lecture 30, section 3.2, and GQA head
// sharing (lecture 30, section 3.4).
//
// Mapping (head_dim D in {64, 128}):
//  * A workgroup of 8 waves owns 256 query rows of one (batch, q head); each
//    wave owns 32 rows; two waves share each SIMD.
//  * Keys are consumed in tiles of 64. Every wave runs the same pipeline: in
//    iteration t it issues, interleaved in one instruction stream, the
//    matrix-core products O^T += V^T P^T of tile t-1 and S^T = K Q^T of tile
//    t+1, and the vector work of tile t (row maximum, exponentials, row sum,
//    bf16 packing of P). The products never wait for the vector work of the
//    same iteration, so the matrix pipe and the vector ALU of a SIMD run side
//    by side in both of its waves.
//  * The exponentials of tile t are taken against the current reference
//    maximum, and the tile's maximum is not computed on the main path: a
//    weight can exceed 2^32 only if the lane's sum of the tile's weights does,
//    so that sum (needed for l anyway) decides. Only then, or on a row's
//    first visible tile, the rare path recomputes the tile's scores, takes
//    their maximum, raises the reference where the maximum passes it by more
//    than 32 in base-2 units (so every weight stays <= 2^32), rescales O and l,
//    and recomputes the weights (identical ones where nothing was raised).
//  * K and V tiles are copied HBM -> LDS by 16-byte buffer-to-LDS loads into
//    two rings of four stages each: K of tile t+3 after the first few
//    products of iteration t (issued behind queued products rather than by
//    all eight waves at once right after the barrier, where they queue at
//    the compute unit's address unit), V of tile t+2 in its middle (every
//    wave copies one eighth of each), so a copy has about one and a half
//    iterations to land. One workgroup
//    barrier per iteration, at the end of iteration t, publishes K of tile
//    t+2 and V of tile t+1 (V of tile t+1 is first read at the end of
//    iteration t+1, for the first P-V products of the next iteration). Each
//    copy goes to a stage whose last reader ran before the previous barrier
//    (K of tile t is read by the products of iteration t-1 and by the rare
//    path of iteration t).
//  * LDS layout, swizzle, operand lane layouts and the transposed V reads are
//    those of bf16_tiles.h.
//  * Fused receive (optional): the launch also copies the next ring block
//    into its receive slot. Each work item takes a share of it, in pieces of
//    1 KB per wave, spread evenly over its iterations: in a receive
//    iteration every wave requests its next piece (buffer-to-LDS into a
//    private staging ring of three 1 KB slots) and stores the piece it
//    requested two receive iterations earlier from LDS to the slot. A
//    receive iteration leaves its fetch in flight at the barrier wait as
//    well; what the iterations do not cover is copied after the loop.
#include <type_traits>

#include "bf16_tiles.h"

namespace ra {
namespace {

using namespace bf16k;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per workgroup
static_assert(kStages == 4, "the K/V rings below have four stages each");
constexpr int kKAhead = 3;        // K of tile t + kKAhead is requested at the start of iteration t
constexpr int kVAhead = 2;        // V of tile t + kVAhead is requested in the middle of iteration t
constexpr int kKSlot = 6;         // the product slot of an iteration that requests K

#ifndef RA_PIPE_AHEAD
#define RA_PIPE_AHEAD 3
#endif
constexpr int kAhead = RA_PIPE_AHEAD;  // MFMAs whose LDS operands are in flight

// 1 KB copies per wave for one K (or V) tile
template <int D>
constexpr int kCopies = Layout<D>::kTileBytes / 1024 / kWaves;

// Fused receive: a piece is 1 KB per wave, 8 KB per workgroup; three staging
// slots per wave after the K/V rings.
constexpr int kRxPiece = kWaves * 1024;
constexpr int kRxSlots = 3;
constexpr int kRxStageBytes = kRxSlots * kRxPiece;

// A lane's speculative weights of one tile sum past this only if one of them
// may exceed 2^kRescaleThreshold (each is >= 0).
constexpr float kWeightCap = 4294967296.0f;  // 2^32
static_assert(kRescaleThreshold == 32.0f, "kWeightCap is 2^kRescaleThreshold");
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Copies of one tensor (K or V) of one head into the LDS rings. Set up once
// per work item: this lane's byte offsets for the wave's kCopies 1 KB blocks
// of a tile (dma16_blocks), and a cursor over the item's tiles in the order
// they are requested, so that a copy costs a few scalar instructions: the
// address of the next tile's first row and the bytes of the block from there
// to its end (kv_len rows), restarted at the second key range.
template <int D, bool IS_V>
struct TileCopier {
  using Ly = Layout<D>;
  int voff[kCopies<D>];
  uint64_t addr, addr1;  // next tile; start of the second range
  int32_t left, left1;   // bytes from there to the end of the block
  int32_t next, n0, ntiles;

  __device__ __forceinline__ void init(const char* g, int wave, int lane, const TilePlan& plan, int64_t kv_len) {
    const uint64_t base = uniform_address(g);
    addr = base + (uint64_t)plan.r0.begin * Ly::kRowBytes;
    left = ((int32_t)kv_len - plan.r0.begin) * Ly::kRowBytes;  // blocks are far below 2 GB
    addr1 = base + (uint64_t)plan.r1.begin * Ly::kRowBytes;
    left1 = ((int32_t)kv_len - plan.r1.begin) * Ly::kRowBytes;
    next = 0;
    n0 = plan.r0.ntiles;
    ntiles = plan.total_tiles();
#pragma unroll
    for (int i = 0; i < kCopies<D>; ++i) {
      // lane fills stored unit q of row r and fetches logical unit q ^ swz(r)
      const int u = (wave * kCopies<D> + i) * 64 + lane;
      const int r = u / Ly::kUnits;
      const int q = u % Ly::kUnits;
      const int swz = IS_V ? Ly::v_swz(r) : Ly::k_swz(r);
      voff[i] = r * Ly::kRowBytes + ((q ^ swz) << 4) - i * 1024;
    }
  }

  // This wave's blocks of the next tile (64 rows) into the LDS stage at
  // `stage`. The buffer resource bounds the reads to the rows the block has:
  // rows past kv_len read as zero. A tile past the last one reads an empty
  // range and fills its stage with zeros, which keeps the number of copies
  // per iteration fixed (the stage it lands in is not read again).
  __device__ __forceinline__ void copy_next(uint32_t stage, int wave) {
    if (next == n0) {
      addr = addr1;
      left = left1;
    }
    const int32_t nb = next < ntiles ? (left < Ly::kTileBytes ? left : Ly::kTileBytes) : 0;
    dma16_blocks<kCopies<D>>(resource_at(addr, 0, nb), stage + (uint32_t)(wave * kCopies<D> * 1024), voff);
    addr += Ly::kTileBytes;
    left -= Ly::kTileBytes;
    ++next;
  }
  // Zeros into the LDS stage at `stage` (an empty range).
  __device__ __forceinline__ void zero(uint32_t stage, int wave) const {
    dma16_blocks<kCopies<D>>(resource_at(addr, 0, 0), stage + (uint32_t)(wave * kCopies<D> * 1024), voff);
  }
};

// Product k of an iteration in the order P-V 0 .. P-V kPre-1, then S 0,
// P-V kPre, S 1, P-V kPre+1, ..., then whatever kind is left: is it a P-V
// product, and its index within its kind. The operands of the first kPre
// P-V products are read before the barrier that opens the iteration (their
// V tile was published one iteration earlier).
#ifndef RA_PIPE_PRE
#define RA_PIPE_PRE 2
#endif
constexpr int kPre = RA_PIPE_PRE;
template <int NP, int NS>
constexpr bool is_pv(int k) {
  if (k < kPre) return true;
  const int r = k - kPre;  // alternate S, P-V while both are left
  const int both = 2 * (NS < NP - kPre ? NS : NP - kPre);
  if (r < both) return (r % 2) == 1;
  return NS < NP - kPre;  // the longer kind finishes the iteration
}
template <int NP, int NS>
constexpr int kind_index(int k) {
  int n = 0;
  for (int j = 0; j < k; ++j)
    if (is_pv<NP, NS>(j) == is_pv<NP, NS>(k)) ++n;
  return n;
}

// SPLIT: the launch of a key-split step (parts and partial states); the
// unsplit instantiation carries none of that code.
template <int D, bool SPLIT>
__global__ void __launch_bounds__(kThreads) step_bf16_kernel(StepArgs a, int32_t n_items, int32_t items_per_xcd,
                                                             int32_t q_tiles) {
  using Ly = Layout<D>;
  constexpr int NP = 4 * Ly::kDBlocks;  // P-V products per tile
  constexpr int NS = 2 * Ly::kDChunks;  // S products per tile
  __shared__ __attribute__((aligned(1024))) char smem[Ly::kSmemBytes + kRxStageBytes];

  // ---- work item ------------------------------------------------------------
  // Workgroup i runs on XCD i % 8. When the (batch, KV head) pairs divide
  // evenly over the 8 XCDs, each XCD takes whole KV heads (its L2 streams
  // their K/V), heavy (late) causal tiles first. Otherwise (e.g. one KV head)
  // that would hand the heavy tiles to some XCDs and the light ones to
  // others, so the heavy-first order is dealt round-robin over all XCDs.
  // Items whose tile is at or after rx_tile_lo carry a share of the fused
  // receive; rx_rank is their dense rank (-1: no share).
  // With a key split, workgroup w runs part w % split of item w / split.
  const int32_t split = SPLIT ? a.split : 1;
  const int32_t vb = (int32_t)blockIdx.x / split;
  const int32_t part = (int32_t)blockIdx.x % split;
  int32_t tile, b, h;
  int64_t rx_rank = -1;
  {
    const int32_t n_bk = a.batch * a.heads_kv;
    const int32_t rx_tiles = q_tiles - a.rx_tile_lo;
    if (n_bk % 8 == 0) {
      const int32_t item = (vb % 8) * items_per_xcd + vb / 8;
      if (item >= n_items) return;
      const int32_t per_kv = q_tiles * a.group;
      const int32_t bk = item / per_kv;
      const int32_t rem = item % per_kv;
      tile = q_tiles - 1 - rem / a.group;
      b = bk / a.heads_kv;
      h = (bk % a.heads_kv) * a.group + rem % a.group;
      if (a.rx_bytes > 0 && rem < rx_tiles * a.group) rx_rank = (int64_t)bk * rx_tiles * a.group + rem;
    } else {
      const int32_t item = vb;
      if (item >= n_items) return;
      const int32_t n_bh = a.batch * a.heads_q;
      tile = q_tiles - 1 - item / n_bh;
      b = (item % n_bh) / a.heads_q;
      h = (item % n_bh) % a.heads_q;
      if (a.rx_bytes > 0 && item < rx_tiles * n_bh) rx_rank = item;
    }
    if (rx_rank >= 0) rx_rank = rx_rank * split + part;
  }
  const int32_t kvh = h / a.group;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qcol = lane & 31;
  const int hh = lane >> 5;

  // ---- fused receive: this item's share [rx_lo, rx_lo + rx_len) of each of
  // the two tensors, in pieces j = 0 .. n_rx-1 (tensor j % 2, 8 KB piece j / 2;
  // the wave moves its KB of each) ----------------------------------------------
  int64_t rx_lo = 0, rx_len = 0;
  if (rx_rank >= 0) {
    rx_lo = rx_rank * a.rx_share < a.rx_bytes ? rx_rank * a.rx_share : a.rx_bytes;
    rx_len = a.rx_bytes - rx_lo < a.rx_share ? a.rx_bytes - rx_lo : a.rx_share;
  }
  const int32_t n_rx = 2 * (int32_t)((rx_len + kRxPiece - 1) / kRxPiece);
  // Wave-uniform addresses of this wave's first KB of the share in each
  // source and destination tensor, and the share's bytes from there on (a
  // share is far below 2 GB).
  const uint64_t rx_wave = (uint64_t)(rx_lo + wave * 1024);
  const uint64_t rx_s0 = uniform_address(a.rx_src[0]) + rx_wave;
  const uint64_t rx_s1 = uniform_address(a.rx_src[1]) + rx_wave;
  const uint64_t rx_d0 = uniform_address(a.rx_dst[0]) + rx_wave;
  const uint64_t rx_d1 = uniform_address(a.rx_dst[1]) + rx_wave;
  const int32_t rx_left = (int32_t)rx_len - wave * 1024;
  // Piece j of this wave: byte offset from the wave's first KB and length
  // (0 outside the share).
  auto rx_piece = [&](int32_t j, int32_t& off, int32_t& nbytes) {
    const int32_t o = (j >> 1) * kRxPiece;
    const int32_t left = rx_left - o;
    const bool in = j >= 0 && j < n_rx && left > 0;
    off = in ? o : 0;
    nbytes = in ? (left < 1024 ? left : 1024) : 0;
  };
  // The pieces [j0, n_rx) with plain loads and stores (after the loop, or
  // for an item with no key tile).
  auto rx_direct = [&](int32_t j0) {
    for (int32_t j = j0 < 0 ? 0 : j0; j < n_rx; ++j) {
      int32_t off, nb;
      rx_piece(j, off, nb);
      const uint64_t src = ((j & 1) ? rx_s1 : rx_s0) + (uint64_t)(off + lane * 16);
      const uint64_t dst = ((j & 1) ? rx_d1 : rx_d0) + (uint64_t)(off + lane * 16);
      if (lane * 16 < nb) *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
  };

  const int64_t row0 = (int64_t)tile * kBM;
  const int64_t r1 = (row0 + kBM < a.q_len) ? row0 + kBM : a.q_len;
  int64_t qmin, qmax;
  seg_range(a.qs, a.n_q_seg, row0, r1, &qmin, &qmax);
  // A part of a split tile takes its share of the tile's key tiles, starts
  // from the empty state and writes partial state `part`; the fold after the
  // launch merges and finalizes.
  const TilePlan plan = [&] {
    const TilePlan p = plan_tiles<kBN>(a, qmin, qmax);
    if (split == 1) return p;
    const int32_t n = p.total_tiles();
    return restrict_plan<kBN>(p, part * n / split, (part + 1) * n / split);
  }();
  const int ntiles = plan.total_tiles();
  const bool init = a.init || split > 1;
  const bool fin = a.final_ && split == 1;
  if (ntiles == 0 && !init && !fin) {  // nothing visible, state untouched
    rx_direct(0);
    return;
  }

  const int64_t row = row0 + wave * 32 + qcol;
  const bool valid = row < a.q_len;
  const int64_t rowc = valid ? row : a.q_len - 1;
  const int64_t bh = (int64_t)b * a.heads_q + h;
  const size_t srow = (size_t)(bh * a.q_len + rowc);
  // where the state goes: the running state, or partial `part`
  const size_t prow = split > 1 ? (size_t)part * ((size_t)a.batch * a.heads_q * a.q_len) + srow : srow;
  float* const o_dst = split > 1 ? a.po : a.o;
  float* const m_dst = split > 1 ? a.pm : a.m;
  float* const l_dst = split > 1 ? a.pl : a.l;
  if (SPLIT && ntiles == 0) {  // an empty partial: the fold reads only its m
    if (valid && hh == 0) {
      m_dst[prow] = -INFINITY;
      l_dst[prow] = 0.0f;
    }
    rx_direct(0);
    return;
  }
  const int64_t kv_off = ((int64_t)b * a.heads_kv + kvh) * a.kv_len * D;
  const char* kg = reinterpret_cast<const char*>(static_cast<const unsigned short*>(a.k) + kv_off);
  const char* vg = reinterpret_cast<const char*>(static_cast<const unsigned short*>(a.v) + kv_off);

  auto tile_start = [&](int t) -> int32_t {
    return t < plan.r0.ntiles ? plan.r0.begin + t * kBN : plan.r1.begin + (t - plan.r0.ntiles) * kBN;
  };

  const uint32_t smem_base = lds_address(smem);
  TileCopier<D, false> kcopy;
  TileCopier<D, true> vcopy;
  kcopy.init(kg, wave, lane, plan, a.kv_len);
  vcopy.init(vg, wave, lane, plan, a.kv_len);
  // tiles are requested in order: K of t and V of t go to stage t % 4
  auto issue_k = [&](int t) {
    kcopy.copy_next(smem_base + (uint32_t)(t % kStages) * Ly::kTileBytes, wave);
  };
  auto issue_v = [&](int t) {
    vcopy.copy_next(smem_base + Ly::kVBase + (uint32_t)(t % kStages) * Ly::kTileBytes, wave);
  };
  // Piece j into staging slot `slot` (buffer-to-LDS), and the piece held in
  // staging out to the receive slot as piece j. Outside the share both use
  // empty buffer ranges: the fetch fills the staging slot with zeros, the
  // store writes nothing.
  const uint32_t rx_stage = smem_base + Ly::kSmemBytes + (uint32_t)wave * 1024u;
  const int rx_voff[1] = {lane * 16};
  auto rx_fetch = [&](int32_t j, uint32_t slot) {
    int32_t off, nb;
    rx_piece(j, off, nb);
    dma16_blocks<1>(resource_at((j & 1) ? rx_s1 : rx_s0, (uint64_t)off, nb), rx_stage + slot * kRxPiece, rx_voff);
  };
  auto rx_put = [&](int32_t j, const u32x4& x) {
    int32_t off, nb;
    rx_piece(j, off, nb);
    void* dst = reinterpret_cast<void*>(((j & 1) ? rx_d1 : rx_d0) + (uint64_t)off);
    __builtin_amdgcn_raw_buffer_store_b128(x, __builtin_amdgcn_make_buffer_rsrc(dst, 0, nb, kBufferWord3), lane * 16,
                                           0, 0);
  };

  // K of tiles 0 and 1 and V of tile 0 first (iteration 0 reads them), and
  // zeros into the V stage of "tile -1" (the stage of tile 3, requested in
  // iteration 1)
  issue_k(0);
  issue_k(1);
  issue_v(0);
  vcopy.zero(smem_base + Ly::kVBase + 3u * Ly::kTileBytes, wave);

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
  if (init) {
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

  uint32_t k_addr[Ly::kDChunks];
#pragma unroll
  for (int c = 0; c < Ly::kDChunks; ++c) k_addr[c] = k_read_address<D>(smem_base, qcol, hh, c);
  uint32_t v_addr[Ly::kDBlocks];
#pragma unroll
  for (int db = 0; db < Ly::kDBlocks; ++db) v_addr[db] = v_read_address<D>(smem_base, lane, db);

  f32x16 sacc[2][2];   // S^T of two tiles: [buffer][key block]
  bf16x8 vpre[kPre];   // V^T operands of an iteration's first P-V products
  bf16x8 pf[2][2][2];  // packed P^T of two tiles: [buffer][key block][16-key chunk]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c) pf[1][kb][c] = bf16x8{};  // the weights of "tile -1"

  // Everything loaded so far (Q, the incoming state, K of tiles 0 and 1) must
  // be in registers / LDS before the loop. The builtin (not asm) form lets
  // the compiler see it, so it inserts no load waits inside the loop, where
  // the hardware counter also counts the tile copies in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // the copies iteration -1 would make (K of 2, V of 1)
  issue_k(2);
  issue_v(1);
  asm volatile("s_barrier" ::: "memory");  // K of tiles 0 and 1, V of 0 visible to all waves

  // Tile t's softmax: mask (partial tiles only), then the speculative
  // exponentials against the current reference. Returns the row maximum
  // (in base-2 units, this lane's pair combined) and the lane's sum.
  // tiles of range r from index p_r on cross some row's causal boundary
  const int32_t part0 = (plan.r0.full - plan.r0.begin) / kBN;
  const int32_t part1 = plan.r0.ntiles + (plan.r1.full - plan.r1.begin) / kBN;
  auto mask_tile = [&](f32x16 (&s)[2], int t) {
    const bool first_range = t < plan.r0.ntiles;
    if (t >= (first_range ? part0 : part1)) {
      const int32_t start = tile_start(t);
      // keys [0, lim) are visible; this lane holds keys 4*hh + (a constant)
      const int32_t lim = (first_range ? vend0 : vend1) - start - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb * 32 + 8 * (j >> 2) + (j & 3);
          if (key >= lim) s[kb][j] = -INFINITY;
        }
    }
  };

  // Weights of a tile against reference msub, in place of its scores, packed
  // into pb; returns this lane's sum of the fp32 weights.
  auto weights = [&](f32x16 (&s)[2], float msub, bf16x8 (&pb)[2][2]) -> float {
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[kb][j] = __builtin_amdgcn_exp2f(fmaf(s[kb][j], sl2, -msub));
        part[j & 3] += s[kb][j];
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) pb[kb][c] = pack_p(s[kb], 8 * c);
    return (part[0] + part[1]) + (part[2] + part[3]);
  };

  // S^T of one tile from the K tile in stage ST into s.
  auto scores = [&](auto st_tag, f32x16 (&s)[2]) {
    constexpr int ST = decltype(st_tag)::value;
    const f32x16 zero = {};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int kb = i % 2;
      const int c = i / 2;
      const bf16x8 kf = *lds_ptr<bf16x8>(k_addr[c] + ST * Ly::kTileBytes + kb * 32 * Ly::kRowBytes);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], c == 0 ? zero : s[kb], 0, 0, 0);
    }
  };

  // The rare path after tile t's speculative weights (K of tile t still in
  // stage ST): raise the reference to the tile's maximum where it passed it
  // by more than the threshold, rescale O and l, and recompute the tile's
  // scores and weights. O must already hold the products of tile t-1 (the
  // compiler orders the rescale after them).
  auto settle = [&](auto st_tag, f32x16 (&s)[2], int t, float& psum, bf16x8 (&pb)[2][2]) {
    // Every speculative weight is <= 2^32 unless this lane's sum of them
    // passed 2^32 (or overflowed): only then, or while the row has no
    // reference yet (its first visible tile), is the tile's maximum needed.
    if (__builtin_amdgcn_ballot_w64(!(psum <= kWeightCap) || m_run == -INFINITY) != 0) {
      scores(st_tag, s);
      mask_tile(s, t);
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
      mx = max_with_partner(mx) * sl2;
      const float cand = fmaxf(m_run, mx);
      const bool need = cand > m_run + kRescaleThreshold;
      const float m_upd = need ? cand : m_run;
      const float alpha = (m_upd == m_run) ? 1.0f : exp2f(m_run - m_upd);
#pragma unroll
      for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      l_run *= alpha;
      m_run = m_upd;
      psum = weights(s, (m_run == -INFINITY) ? 0.0f : m_run, pb);
    }
    l_run += psum;
  };

  // End of iteration t: wait for this wave's copies of the tiles that
  // iteration t+1 reads, then publish them: K of t+2 (its S products,
  // requested at the start of iteration t-1) and V of t+1 (read at the end
  // of iteration t+1 for the first P-V products of iteration t+2, requested
  // in the middle of iteration t-1). The loads issued after V of t+1 may
  // stay in flight: K of t+3, in a receive iteration the fetch of one piece,
  // and V of t+2. The counter also counts stores, and a store may be
  // counted done before older loads, so stores are never part of the
  // allowance: a store still in flight only makes the wait stricter. The
  // receive fetches of earlier iterations are older than V of t+1, so they
  // have landed too.
  auto publish = [&](bool rx_on) {
    if (rx_on)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kCopies<D> + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kCopies<D>) : "memory");
    asm volatile("s_barrier" ::: "memory");
  };

  // Receive iterations: every rx_every-th iteration while pieces are left,
  // plus two to store the last two; only the first iteration of each group
  // of four (the unrolled loop body) can be one, so rx_every is a multiple
  // of 4 and the other three carry no receive code. rx_r counts them,
  // rx_slot is the staging slot of piece rx_r (rx_r mod 3).
  const int32_t rx_every = 4 * (4 * (n_rx + 2) <= ntiles ? ntiles / (4 * (n_rx + 2)) : 1);
  int32_t rx_r = 0, rx_next = 0;
  uint32_t rx_slot = 0;

  // One iteration t with K of tile t+1 in stage SK and V of tile t-1 in
  // stage SV; the softmax tile is sacc[BUF], the next S goes to
  // sacc[BUF^1], the new weights to pf[BUF], the P-V products read
  // pf[BUF^1]. Every iteration has the same shape: for t = 0 the weights of
  // "tile -1" are zero and its V stage holds zeros, so those products add
  // nothing; for the last tile the S products read a stage of zeros and are
  // never used.
  auto iteration = [&](auto sk_tag, auto sv_tag, auto buf_tag, auto rx_tag, int t) {
    constexpr int SK = decltype(sk_tag)::value;
    constexpr int SV = decltype(sv_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr int NM = NP + NS;      // products per iteration
    constexpr int EPS = 32 / NM;     // softmax elements per slot
    static_assert(kKSlot < NM / 2, "K is requested before V");
    // receive: fetch piece r, store piece r-2 (from the slot after r's)
    const bool rx_on = decltype(rx_tag)::value && t == rx_next && rx_r < n_rx + 2;
    const int32_t r = rx_r;
    const uint32_t slot_in = rx_slot;
    const uint32_t slot_out = rx_slot == kRxSlots - 1 ? 0u : rx_slot + 1;
    if (rx_on) rx_fetch(r, slot_in);
    mask_tile(sacc[BUF], t);
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
    f32x16(&sc)[2] = sacc[BUF];
    f32x16(&sn)[2] = sacc[BUF ^ 1];
    const f32x16 zero = {};

    // Slot k: product k, the operand read of product k + kAhead, and a fixed
    // share of tile t's vector work: the exponentials of elements
    // [k*EPS, (k+1)*EPS), the sums of the previous slot's elements (the
    // exponential's latency), the maximum of two more elements while any
    // are left, and one bf16 pair conversion two slots after both of its
    // exponentials. Slots are fenced so the compiler keeps this interleave.
    bf16x8 frag[NM];
#pragma unroll
    for (int k = 0; k < kPre; ++k) frag[k] = vpre[k];
    auto read_operand = [&](int k) {
      const int i = kind_index<NP, NS>(k);
      if (is_pv<NP, NS>(k)) {
        frag[k] = read_vt<D, SV>(i, v_addr);
      } else {
        const int kb = i % 2;
        const int c = i / 2;
        frag[k] = *lds_ptr<bf16x8>(k_addr[c] + SK * Ly::kTileBytes + kb * 32 * Ly::kRowBytes);
      }
    };
    float p[32];
    float part[4];
    u32x4 rx_x;
    bf16x2 pairs[16];
    auto elem = [&](int e) -> float { return sc[e / 16][e % 16]; };
#pragma unroll
    for (int k = kPre; k < kAhead; ++k) read_operand(k);
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      const int i = kind_index<NP, NS>(k);
      if (is_pv<NP, NS>(k)) {
        const int db = i % Ly::kDBlocks;
        const int kc = i / Ly::kDBlocks;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[k], pf[BUF ^ 1][kc / 2][kc % 2], oacc[db], 0, 0, 0);
      } else {
        const int kb = i % 2;
        const int c = i / 2;
        sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[k], qf[c], c == 0 ? zero : sn[kb], 0, 0, 0);
      }
      if (k + kAhead < NM) read_operand(k + kAhead);
      if (k == 0 && rx_on) rx_x = *lds_ptr<u32x4>(rx_stage + slot_out * kRxPiece + lane * 16);
      if (k == 2 && rx_on) rx_put(r - 2, rx_x);
#pragma unroll
      for (int e = k * EPS; e < (k + 1) * EPS; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(elem(e), sl2, -msub));
      if (k >= 1) {
#pragma unroll
        for (int e = (k - 1) * EPS; e < k * EPS; ++e) part[e & 3] = e < 4 ? p[e] : part[e & 3] + p[e];
      }
#pragma unroll
      for (int m = 0; m < 16; ++m)
        if ((2 * m + 1) / EPS + 2 == k) pairs[m] = __builtin_convertvector((f32x2){p[2 * m], p[2 * m + 1]}, bf16x2);
      // K of tile t+3 goes to the stage of K of tile t-1 (last read before
      // the previous barrier), V of tile t+2 to that of V of tile t-2
      if (k == kKSlot) issue_k(t + kKAhead);
      if (k == NM / 2) issue_v(t + kVAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = (NM - 1) * EPS; e < 32; ++e) part[e & 3] = e < 4 ? p[e] : part[e & 3] + p[e];
#pragma unroll
    for (int m = 0; m < 16; ++m)
      if ((2 * m + 1) / EPS + 2 >= NM) pairs[m] = __builtin_convertvector((f32x2){p[2 * m], p[2 * m + 1]}, bf16x2);
    // pairs m = 8 kb + 4 c + q hold keys 8 c + 2 q, +1 of key block kb
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int m0 = 8 * kb + 4 * c;
        const auto ab = __builtin_shufflevector(pairs[m0], pairs[m0 + 1], 0, 1, 2, 3);
        const auto cd = __builtin_shufflevector(pairs[m0 + 2], pairs[m0 + 3], 0, 1, 2, 3);
        pf[BUF][kb][c] = __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    float psum = (part[0] + part[1]) + (part[2] + part[3]);
    // The rare path below overwrites the speculative weights; without these
    // uses the compiler would sink their computation past the branch, out of
    // the interleaved slots.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) asm volatile("" ::"v"(__builtin_bit_cast(i32x4, pf[BUF][kb][c])));
    asm volatile("" ::"v"(psum));
    settle(std::integral_constant<int, (SK + 3) % 4>{}, sacc[BUF], t, psum, pf[BUF]);
    // operands of the next iteration's first P-V products: V of tile t, in
    // stage (SV + 1) % 4, published at the end of the previous iteration
    // (for t = 0, by the barrier before the loop)
#pragma unroll
    for (int k = 0; k < kPre; ++k) vpre[k] = read_vt<D, (SV + 1) % 4>(k, v_addr);
    publish(rx_on);
    if (rx_on) {
      ++rx_r;
      rx_next += rx_every;
      rx_slot = slot_out;
    }
  };

  // The P-V products of the last tile (V in stage SV, weights in pf[BUF]).
  auto last_pv = [&](auto sv_tag, auto buf_tag) {
    constexpr int SV = decltype(sv_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int db = i % Ly::kDBlocks;
      const int kc = i / Ly::kDBlocks;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_vt<D, SV>(i, v_addr), pf[BUF][kc / 2][kc % 2], oacc[db],
                                                         0, 0, 0);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  if (ntiles > 0) {
    scores(I0{}, sacc[0]);  // S of tile 0 (stage 0)
    // A row without a reference yet (an empty incoming state) takes tile 0's
    // maximum as its reference here, as the rare path of iteration 0 would
    // (same value), so iteration 0's speculative weights are final and its
    // rare path runs only for rows that see no key of tile 0.
    if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0) {
      mask_tile(sacc[0], 0);
      float mx = sacc[0][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[0][kb][j]);
      mx = max_with_partner(mx) * sl2;
      if (m_run == -INFINITY) m_run = mx;
    }
#pragma unroll
    for (int k = 0; k < kPre; ++k) vpre[k] = read_vt<D, 3>(k, v_addr);  // "tile -1": zeros
    // iteration t: K of t+1 in stage (t+1)%4, V of t-1 in (t-1)%4, buffer t%2
    for (int t = 0; t < ntiles; t += 4) {
      iteration(I1{}, I3{}, I0{}, std::true_type{}, t);
      if (t + 1 >= ntiles) break;
      iteration(I2{}, I0{}, I1{}, std::false_type{}, t + 1);
      if (t + 2 >= ntiles) break;
      iteration(I3{}, I1{}, I0{}, std::false_type{}, t + 2);
      if (t + 3 >= ntiles) break;
      iteration(I0{}, I2{}, I1{}, std::false_type{}, t + 3);
    }
    switch ((ntiles - 1) & 3) {  // P-V of the last tile
      case 0: last_pv(I0{}, I0{}); break;
      case 1: last_pv(I1{}, I1{}); break;
      case 2: last_pv(I2{}, I0{}); break;
      default: last_pv(I3{}, I1{}); break;
    }
  }

  // receive pieces the loop did not store (piece r-2 is stored in receive
  // iteration r)
  rx_direct(rx_r - 2);

  // ---- write back ---------------------------------------------------------------
  const float l_tot = sum_with_partner(l_run);
  if (!valid) return;
  if (fin) {
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
    float* op = o_dst + prow * D;
#pragma unroll
    for (int db = 0; db < Ly::kDBlocks; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(op + 32 * db + 8 * jj + 4 * hh) =
            make_float4(oacc[db][4 * jj], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]);
    if (hh == 0) {
      m_dst[prow] = m_run;
      l_dst[prow] = l_tot;
    }
  }
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& args, int head_dim, hipStream_t s) {
  const int64_t q_tiles = (args.q_len + kBM - 1) / kBM;
  const int64_t items = q_tiles * args.heads_q * args.batch;
  const int64_t per_xcd = (items + 7) / 8;
  const int64_t split = args.split > 1 ? args.split : 1;
  const dim3 grid((unsigned)(per_xcd * 8 * split));
  StepArgs a = args;
  a.split = (int32_t)split;
  if (a.rx_bytes > 0 && split > 1) {
    // every part of every item carries an equal share
    const int64_t carriers = items * split;
    const int64_t per = (a.rx_bytes + carriers - 1) / carriers;
    a.rx_tile_lo = 0;
    a.rx_share = (per + kRxPiece - 1) / kRxPiece * kRxPiece;
  } else if (a.rx_bytes > 0) {
    // Carriers of the receive: the items of query tiles lo .. q_tiles-1,
    // each taking rx_share bytes of both tensors, i.e. n = 2 * rx_share / 8 KB
    // pieces, moved in n + 2 receive iterations at most one in four
    // iterations apart. Take the lowest lo for which every carrier has
    // enough key tiles to move its pieces inside its loop (the late tiles
    // of the causal layouts see the most keys); failing that, every item
    // carries and the rest is copied after the loop.
    auto share_of = [&](int64_t lo) {
      const int64_t carriers = (q_tiles - lo) * a.heads_q * a.batch;
      const int64_t per = (a.rx_bytes + carriers - 1) / carriers;
      return (per + kRxPiece - 1) / kRxPiece * kRxPiece;
    };
    int64_t best = -1;
    int64_t min_tiles = INT64_MAX;
    for (int64_t lo = q_tiles - 1; lo >= 0 && min_tiles >= 16; --lo) {  // a carrier needs >= 16 tiles
      const int64_t r0 = lo * kBM;
      const int64_t r1 = r0 + kBM < a.q_len ? r0 + kBM : a.q_len;
      int64_t qmin, qmax;
      seg_range(a.qs, a.n_q_seg, r0, r1, &qmin, &qmax);
      const int64_t nt = plan_tiles<kBN>(a, qmin, qmax).total_tiles();
      min_tiles = nt < min_tiles ? nt : min_tiles;
      if (min_tiles >= 4 * (2 * (share_of(lo) / kRxPiece) + 2)) best = lo;
    }
    if (best < 0) best = 0;
    a.rx_tile_lo = (int32_t)best;
    a.rx_share = share_of(best);
  }
  const int32_t ni = (int32_t)items, px = (int32_t)per_xcd, qt = (int32_t)q_tiles;
  if (head_dim == 128) {
    if (split > 1)
      step_bf16_kernel<128, true><<<grid, kThreads, 0, s>>>(a, ni, px, qt);
    else
      step_bf16_kernel<128, false><<<grid, kThreads, 0, s>>>(a, ni, px, qt);
  } else {
    if (split > 1)
      step_bf16_kernel<64, true><<<grid, kThreads, 0, s>>>(a, ni, px, qt);
    else
      step_bf16_kernel<64, false><<<grid, kThreads, 0, s>>>(a, ni, px, qt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  return launch_fold(a, (int64_t)a.batch * a.heads_q * a.q_len, head_dim, RA_BF16, s);
}

}  // namespace ra
