/*
 * ring_attn.h — C ABI of the per-device blockwise ring-attention step for
 * AMD Instinct MI355X (gfx950).
 *
 * One device keeps a local query block Q_i and folds key/value blocks K_j, V_j
 * into a running online-softmax state (O, m, l), one ring step at a time; a
 * finalize pass turns the state into the attention output and its log-sum-exp.
 *
 * Sources (pages and sections):
 *   [HC]  "distributed training hands-on code" (LLM-101-CN), section 6.2
 *         (block_attention, ring_send_recv_kv, forward): S = Q K^T / sqrt(d),
 *         running max M, running sum L, unnormalised O; forward ends with O / L.
 *   [RS]  "Ring Attention and Sequence Parallelism" (airsota M4-051), sections 3
 *         and 4: K/V blocks travel around a ring of n devices while the local
 *         block computes (double buffering); causal blocks above the diagonal
 *         are skipped; zigzag gives device i its segment and its mirror.
 *   [L30] Lecture 30 "TP/PP/SP/CP", section 3.2 (ring walk-through, causal
 *         imbalance, zigzag/striped) and 3.4 (the ring carries the few GQA KV
 *         heads).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.    Every tensor is dense, row-major [batch, heads, rows, head_dim]
 *            ([HC] forward: bs, heads, q_len, d), 16-byte aligned. Row vectors
 *            m, l, lse are [batch, heads_q, q_len].
 * Memory.    Tensor arguments are DEVICE pointers; descriptors, segment and
 *            pointer arrays are HOST memory. The caller allocates and owns every
 *            buffer, including the workspace. The library allocates no device
 *            memory.
 * Streams.   `stream` arguments are hipStream_t handles passed as void*
 *            (NULL = the default stream). Calls only enqueue work and return;
 *            nothing synchronises the device.
 * Errors.    Every entry point returns an ra_status. All arguments are checked
 *            on the host before any work is enqueued, so on any error nothing
 *            is written. A failed HIP call returns RA_ERR_HIP.
 *            ring_attn_last_error() gives a message for the calling thread.
 * Sizes.     Row counts (q_len, kv_len, local_len, seq_len) are at most 2^30,
 *            and batch x heads x rows at most 2^34 on the query and on the
 *            key/value side, else RA_ERR_INVALID_ARG (every launch's grid then
 *            fits in 32 bits).
 * GQA.       Query head h reads KV head h / (heads_q / heads_kv) — contiguous
 *            groups ([L30] 3.4, 8.3: 8 Q heads per KV head per GPU).
 * Causality. A key is visible to a query iff pos_k <= pos_q (lower triangle,
 *            diagonal included; [L30] 3.2). Positions come from segments.
 * State.     (O, m, l) is kept in base 2: with t_j = log2(e) * scale * q.k_j,
 *            O = sum_j 2^(t_j - m) v_j and l = sum_j 2^(t_j - m) over the keys
 *            folded so far. m is a reference exponent no smaller than
 *            max_j t_j - 32 (it is raised lazily, which is exact: any reference
 *            gives the same O / l). The empty state is m = -inf, l = 0, O = 0.
 *            This is [HC]'s (M, L, O) with M expressed in base 2.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define RA_OK               0
#define RA_ERR_INVALID_ARG (-1)   /* bad size, pointer, segment or flag        */
#define RA_ERR_UNSUPPORTED (-2)   /* valid but not built: head_dim or dtype    */
#define RA_ERR_WORKSPACE   (-3)   /* workspace pointer NULL or too small        */
#define RA_ERR_HIP         (-4)   /* a HIP runtime call failed                  */

/* ---- element types ------------------------------------------------------ */
#define RA_F32  0                 /* float32 Q/K/V/out; fp32 arithmetic         */
#define RA_BF16 1                 /* bfloat16 Q/K/V/out; fp32 accumulation      */

/* ---- partitions of the global sequence over `world` devices --------------- */
#define RA_PART_CONTIGUOUS 0      /* device r: tokens [r*c, (r+1)*c)            */
#define RA_PART_ZIGZAG     1      /* device r: chunks r and 2w-1-r of c/2 ([RS] 4) */
#define RA_PART_STRIPED    2      /* device r: tokens r, r+w, r+2w, ... ([L30] 3.2) */

/* ---- ring_attn_step flags ------------------------------------------------ */
#define RA_STEP_INIT 1            /* ignore the incoming state: start empty     */

/* Global positions of a run of local rows: row i of the run has position
 * start + i * stride. */
typedef struct {
  int64_t start;
  int64_t len;
  int64_t stride;                 /* >= 1 */
} ra_segment;

/* One ring step: a local query block against one key/value block.
 * Local row r of Q lies in q_seg[0] if r < q_seg[0].len, else in q_seg[1];
 * likewise for K/V rows. The lens of a side's segments add up to its row count.
 * n_q_seg / n_kv_seg are 1 or 2 (0 is allowed only when causal == 0). */
typedef struct {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;               /* heads_q % heads_kv == 0 */
  int32_t head_dim;               /* 64 or 128 */
  int64_t q_len;                  /* local query rows (may be 0) */
  int64_t kv_len;                 /* rows of this K/V block (may be 0) */
  int32_t dtype;                  /* RA_F32 or RA_BF16 */
  int32_t causal;                 /* 0 or 1 */
  float   scale;                  /* softmax scale; <= 0 means 1/sqrt(head_dim) */
  int32_t n_q_seg;
  int32_t n_kv_seg;
  ra_segment q_seg[2];
  ra_segment kv_seg[2];
} ra_step_desc;

/* Fold one K/V block into the running state ([HC] 6.2 block_attention;
 * causal tile skipping per [RS] 4/6 and [L30] 3.2).
 *   q      [B, Hq,  q_len,  d]  dtype        read
 *   k, v   [B, Hkv, kv_len, d]  dtype        read
 *   o_acc  [B, Hq,  q_len,  d]  fp32         read (unless RA_STEP_INIT), written
 *   m, l   [B, Hq,  q_len]      fp32         read (unless RA_STEP_INIT), written
 *   flags  0 or RA_STEP_INIT.
 * Rows that see no key of this block are left untouched — or, with
 * RA_STEP_INIT, set to the empty state. */
int ring_attn_step(const ra_step_desc* desc, const void* q, const void* k, const void* v,
                   float* o_acc, float* m, float* l, int32_t flags, void* stream);

/* Combine two states over the same rows: (a) <- (a) (+) (b). The fold of [HC]
 * 6.2 written for two partial states; commutative and associative. Uses
 * batch, heads_q, q_len and head_dim of desc. */
int ring_attn_merge(const ra_step_desc* desc, float* o_a, float* m_a, float* l_a,
                    const float* o_b, const float* m_b, const float* l_b, void* stream);

/* Normalise a state ([HC] 6.2: O / L) and write LSE = ln(2) * (m + log2 l)
 * (natural log). A row with l == 0 gets out = 0 and lse = -inf.
 *   out [B, Hq, q_len, d] in desc->dtype; lse [B, Hq, q_len] fp32 (may be NULL). */
int ring_attn_finalize(const ra_step_desc* desc, const float* o_acc, const float* m,
                       const float* l, void* out, float* lse, void* stream);

/* One device's share of a simulated ring ([RS] 3-4, [HC] 6.2 forward). */
typedef struct {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  int64_t local_len;              /* c: rows per device, also rows per K/V block */
  int32_t dtype;
  int32_t causal;
  float   scale;                  /* <= 0 means 1/sqrt(head_dim) */
  int32_t world;                  /* n >= 1 simulated devices */
  int32_t rank;                   /* this device, 0 <= rank < world */
  int32_t partition;              /* RA_PART_* */
  int32_t reverse_order;          /* 0: step s uses block (rank - s) mod n (blocks
                                     are sent to rank + 1, as [HC]'s code does);
                                     1: block (rank + s) mod n ([HC]'s 6.1 text) */
  int32_t receive;                /* RA_RECV_*: how a block is copied into its
                                     receive slot (the result is the same) */
  int32_t key_split;              /* bf16 forward: ways to split each query
                                     tile's keys (0 = automatic, 1 = never,
                                     2..16 = that many; see below) */
} ra_ring_desc;

/* Key split of the bf16 forward (desc->key_split). A step kernel runs one
 * work item per 256-row query tile and head, one per compute unit at a time,
 * so a small share leaves most of the 256 compute units idle while each item
 * walks all of its key tiles. With a split of k every item runs as k parts,
 * part j over its j-th share of the item's 64-key tiles, each from the empty
 * state into a partial state of the workspace; a fold kernel after the step
 * merges the incoming state and the k partials in order with one common
 * reference (the block-combination rule of [HC] 6.2 applied k times) and
 * writes the state, or the output on the last step. Automatic: shares with at
 * most 128 work items get the largest power of two up to 8 that keeps items x
 * k <= 256 and at least two key tiles per part; larger shares are not split.
 * A given k is capped at the block's key tiles. The result is the same
 * attention up to rounding (not bit for bit the unsplit one: the partial
 * states are summed in a different order). fp32 forwards never split. */

/* Receive copy of the ring drivers (desc->receive).
 * RA_RECV_MEMCPY: hipMemcpyAsync of the K and V block on copy_stream (or on
 *   compute_stream when copy_stream is NULL).
 * RA_RECV_FUSED: the bf16 step kernel of step s copies the block of step
 *   s + 1 into its slot while it computes: the work items of the launch
 *   each move a share of it through a small LDS staging ring, one 1 KB
 *   piece per wave per key tile, so the copy runs on the compute units the
 *   step already holds (a separate copy kernel only gets compute units
 *   between step workgroups). A step that launches no kernel (no visible
 *   key) or computes in fp32 falls back to hipMemcpyAsync on
 *   compute_stream. copy_stream is not used. Same results bit for bit.
 * RA_RECV_AUTO: RA_RECV_FUSED for bf16, RA_RECV_MEMCPY for fp32.
 * ring_attn_backward always copies with hipMemcpyAsync. */
#define RA_RECV_AUTO   0
#define RA_RECV_MEMCPY 1
#define RA_RECV_FUSED  2

/* Bytes of workspace ring_attn_forward needs: two receive slots for one K/V
 * block each, the fp32 state, the partial states of a key split (k fp32
 * states; none without a split) and alignment padding. Returns 0 on a bad
 * desc. */
size_t ring_attn_forward_workspace_size(const ra_ring_desc* desc);

/* Run the whole ring for one device: n steps, then finalize.
 *   q_local        [B, Hq, c, d] dtype, rows in this device's partition order.
 *   k_blocks[j],
 *   v_blocks[j]    HOST arrays of `world` DEVICE pointers: the K/V block device j
 *                  holds, [B, Hkv, c, d], rows in device j's partition order.
 *                  Block rank is used in place; every other block is first
 *                  copied into a receive slot of the workspace on copy_stream
 *                  while the previous step computes on compute_stream (the
 *                  simulated receive; desc->receive picks the copy; events
 *                  order the two streams, two slots alternate).
 *   out, lse       as ring_attn_finalize.
 *   compute_stream, copy_stream  hipStream_t (distinct; copy_stream may be NULL
 *                  to copy on compute_stream, which serialises the receive).
 *   step_events    NULL, or a HOST array of 2*world hipEvent_t handles; the
 *                  driver records events[2s] / events[2s+1] on compute_stream
 *                  right before / after step s's kernel (both at the same point
 *                  when step s has no visible key and launches nothing).
 * Steps whose block has no key visible to any local row launch no kernel;
 * the block is still received. Step kernels never read a slot while it is
 * being filled. The two streams are ordered by four untimed hipEvent_t that
 * the library creates on first use per calling thread and device and reuses
 * on later calls from that thread (no other state survives a call). They are
 * destroyed only by ring_attn_release_thread_events(); a thread that ends
 * without calling it leaves them to the runtime, which frees them when the
 * process exits (four events per device the thread used). The copy stream
 * forks from and joins back into compute_stream through these events, so a
 * call can be captured into a HIP graph on compute_stream (pass
 * step_events = NULL while capturing). */
int ring_attn_forward(const ra_ring_desc* desc, const void* q_local,
                      const void* const* k_blocks, const void* const* v_blocks,
                      void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* compute_stream, void* copy_stream, void* const* step_events);

/* ---- forward without device allocation ------------------------------------ */

/* For callers that cannot allocate device memory or hand over a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same ring and same kernels as ring_attn_forward with
 * copy_stream = NULL (bit for bit the same out and lse): every receive copy
 * and step runs in order on `stream`. The receive slots and the running
 * state live in a device array owned by the library, RA_NOALLOC_SCRATCH_BYTES
 * long, one per GPU, held from the time the library's code is loaded on that
 * GPU until the process ends. The call allocates nothing (no hipMalloc,
 * hipFree, event or stream creation); the first call on a device looks up
 * that device's array address once.
 *   desc, q_local, k_blocks, v_blocks, out, lse   as ring_attn_forward.
 *   stream         hipStream_t (NULL: the default stream).
 * Errors: as ring_attn_forward; RA_ERR_WORKSPACE when the share needs more
 * than RA_NOALLOC_SCRATCH_BYTES (ring_attn_forward_workspace_size(desc) - 256
 * bytes), with nothing enqueued. Every call on a GPU uses that GPU's one
 * array and leaves its contents behind (nothing in it has to start at zero:
 * the first step of a ring ignores the old state): calls that overlap on one
 * GPU (on different streams or from different threads) race on it, so order
 * them, e.g. on one stream. */
#define RA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int ring_attn_forward_noalloc(const ra_ring_desc* desc, const void* q_local,
                              const void* const* k_blocks, const void* const* v_blocks,
                              void* out, float* lse, void* stream);

/* ---- Ulysses: sequence <-> head all-to-all around local attention --------- */

/* One device's share of DeepSpeed-Ulysses ([L30] section 3.3, and the
 * interview answer comparing it with the ring): the input is sharded along
 * the sequence over `world` devices; a first all-to-all gives every device
 * the whole sequence for heads_q/world query heads and heads_kv/world KV
 * heads, the device runs full attention on them, and a second all-to-all
 * restores the sequence sharding. Both head counts must be divisible by world
 * ([L30] 3.4: with 8 KV heads Ulysses cannot go past 8 devices). */
typedef struct {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  int64_t seq_len;                /* L, the global sequence; divisible by world */
  int32_t dtype;
  int32_t causal;                 /* positions are the global token indices */
  float   scale;                  /* <= 0 means 1/sqrt(head_dim) */
  int32_t world;                  /* >= 1; divides heads_q, heads_kv and seq_len */
  int32_t rank;                   /* this device, 0 <= rank < world */
} ra_ulysses_desc;

/* Bytes of workspace ring_attn_ulysses_forward needs: this device's
 * head-sharded Q, K, V, output and LSE over the whole sequence. 0 on a bad
 * desc. */
size_t ring_attn_ulysses_workspace_size(const ra_ulysses_desc* desc);

/* Device `rank`'s part of one Ulysses attention, simulated on one device:
 * the other devices' shards sit in this device's memory and each all-to-all
 * is this device's share of strided device-to-device copies.
 *   q_shards[j], out_shards[j]   [B, Hq,  L/world, d] dtype: device j's rows
 *                                j*L/world .. (j+1)*L/world - 1.
 *   k_shards[j], v_shards[j]     [B, Hkv, L/world, d] dtype.
 *   lse_shards[j]                [B, Hq,  L/world] fp32, 4-byte aligned; the array may be NULL.
 *   (HOST arrays of `world` DEVICE pointers.)
 * Reads query heads rank*Hq/world .. (rank+1)*Hq/world - 1 (and the matching
 * KV heads) of every shard and writes the same heads of every out (and lse)
 * shard; running every rank fills the outputs. All work is enqueued on
 * `stream`: gather (first all-to-all: one copy kernel per tensor), one
 * attention launch (init and finalize fused), scatter (second all-to-all).
 * Q/K/V/out shards must be 16-byte aligned (RA_ERR_INVALID_ARG otherwise). */
int ring_attn_ulysses_forward(const ra_ulysses_desc* desc, const void* const* q_shards,
                              const void* const* k_shards, const void* const* v_shards,
                              void* const* out_shards, float* const* lse_shards,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- backward ring step (gradients) --------------------------------------- */

/* The pages run the ring forward only ([HC] 6.2 has no backward pass). The
 * backward step is the plain extension of the same block step: with the
 * forward's LSE and P_ij = exp(scale q_i.k_j - LSE_i) over the visible keys,
 * D_i = dO_i . O_i and dS_ij = P_ij (dO_i . v_j - D_i),
 *   dQ_i += scale sum_j dS_ij k_j,   dK_j += scale sum_i dS_ij q_i,
 *   dV_j += sum_i P_ij dO_i,
 * i over the local query rows, j over the keys of one K/V block. dQ stays on
 * the device; dK and dV are accumulators that travel around the ring with
 * their K/V block and are back at the block's owner after a full turn.
 * Built for head_dim 64 and 128: bf16 on the matrix cores, fp32 on the vector
 * ALUs (fp32 arithmetic throughout). */

#define RA_BWD_INIT_DQ 1          /* ring_attn_backward_step: dq_acc starts at 0 */

/* Per-row terms every backward step reads, from the forward's output:
 *   out, d_out [B, Hq, q_len, d] desc->dtype (O and the upstream gradient dO)
 *   lse        [B, Hq, q_len]    fp32, natural log, as ring_attn_finalize writes
 *   terms      [2, B, Hq, q_len] fp32, written: terms[r] = -LSE_r / scale
 *              (-inf for a row with LSE = -inf), terms[R + r] = -(dO_r . O_r),
 *              R = B * Hq * q_len.
 * Uses batch, heads_q, q_len, head_dim, dtype and scale of desc (any dtype
 * and head_dim the forward supports). */
int ring_attn_backward_prep(const ra_step_desc* desc, const void* out, const void* d_out, const float* lse,
                            float* terms, void* stream);

/* One backward step: the gradient contributions of the local query rows
 * against one K/V block (same descriptor as the forward step).
 *   q          [B, Hq,  q_len,  d] dtype   read
 *   k, v       [B, Hkv, kv_len, d] dtype   read
 *   d_out      [B, Hq,  q_len,  d] dtype   read
 *   terms      as ring_attn_backward_prep wrote them               read
 *   dq_acc     [B, Hq,  q_len,  d] fp32    read (unless RA_BWD_INIT_DQ) and written
 *   dk_acc, dv_acc [B, Hkv, kv_len, d] fp32  read and written (accumulated)
 *   flags      0 or RA_BWD_INIT_DQ.
 * Keys that no local row sees are left untouched; so are rows that see no
 * key of the block (set to 0 with RA_BWD_INIT_DQ). */
int ring_attn_backward_step(const ra_step_desc* desc, const void* q, const void* k, const void* v,
                            const void* d_out, const float* terms, float* dq_acc, float* dk_acc, float* dv_acc,
                            int32_t flags, void* stream);

/* Bytes of workspace ring_attn_backward needs: two receive slots, the fp32
 * dQ accumulator and the row terms. 0 on a bad desc. */
size_t ring_attn_backward_workspace_size(const ra_ring_desc* desc);

/* The backward pass of one device's share of a simulated ring: the row
 * terms, then n backward steps in the forward's block order, then dQ in the
 * input dtype.
 *   q_local, k_blocks, v_blocks, step_events, streams  as ring_attn_forward
 *                  (K/V blocks are received into workspace slots the same way).
 *   out, lse       the forward's output [B, Hq, c, d] and LSE [B, Hq, c].
 *   d_out          [B, Hq, c, d] the upstream gradient of out.
 *   dq             [B, Hq, c, d] written, input dtype.
 *   dk_acc[j], dv_acc[j]  HOST arrays of `world` DEVICE pointers, fp32
 *                  [B, Hkv, c, d]: the accumulators travelling with block j;
 *                  this device adds its contribution to every block's pair.
 *                  Starting them at zero and running every rank leaves the
 *                  full dK_j, dV_j in them. */
int ring_attn_backward(const ra_ring_desc* desc, const void* q_local, const void* const* k_blocks,
                       const void* const* v_blocks, const void* out, const void* d_out, const float* lse, void* dq,
                       float* const* dk_acc, float* const* dv_acc, void* workspace, size_t workspace_bytes,
                       void* compute_stream, void* copy_stream, void* const* step_events);

/* ---- host-only helpers (no device work) ---------------------------------- */

/* Segments of device `rank`'s local rows under `partition` (RA_PART_*).
 * Writes up to 2 segments to segs and their count to n_segs. */
int ring_attn_partition_segments(int32_t partition, int32_t world, int32_t rank,
                                 int64_t local_len, ra_segment* segs, int32_t* n_segs);

/* Fill a step descriptor for ring step `step` of desc: the local rows of
 * desc->rank against the block of device block_owner(step). Writes the block
 * owner to *owner (may be NULL). */
int ring_attn_ring_step_desc(const ra_ring_desc* desc, int32_t step, ra_step_desc* out,
                             int32_t* owner);

/* Number of visible (query, key) pairs of one (batch, query head) of a step:
 * q_len * kv_len when not causal. Returns -1 on an invalid descriptor. */
int64_t ring_attn_visible_pairs(const ra_step_desc* desc);

/* Message of the last error on the calling thread ("" if none). */
const char* ring_attn_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t ring_attn_abi_version(void);

/* Timing helpers for callers without their own HIP bindings: create n
 * timing-enabled hipEvent_t into events[n]; elapsed ms between two recorded
 * events (after they completed); destroy. */
int ring_attn_events_create(int32_t n, void** events);
int ring_attn_event_elapsed_ms(void* start, void* stop, float* ms);
int ring_attn_events_destroy(int32_t n, void* const* events);
int ring_attn_synchronize(void* stream);

/* Destroy the ordering events that ring_attn_forward and ring_attn_backward
 * keep for the calling thread (every device it used); the next driver call on
 * this thread creates them again. Call it before a thread that used the
 * drivers ends, once the work it enqueued no longer needs ordering (e.g. after
 * synchronising both streams). Makes no HIP call when the thread holds none.
 * Returns RA_OK, or RA_ERR_HIP if a destroy fails (the rest are still
 * destroyed). */
int ring_attn_release_thread_events(void);

/* Measurement aid (not part of the attention path): the dense bf16 matrix-core
 * rate and shader clock of this device, with the instruction the step kernels
 * use. Enqueues `blocks` workgroups of 4 waves on `stream`; every wave issues
 * iters x 4 independent v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 products,
 * 32768 FLOP each) on register operands, so the launch performs
 * blocks * 4 * iters * 4 * 32768 FLOP. Caller-owned device buffers:
 *   sink   [blocks * 256] float — the accumulators (keeps every product live);
 *   stamps [blocks * 4] uint64 — per workgroup, wave 0's shader clock counter
 *          (s_memtime) at the start and end of its loop, then the constant
 *          reference counter (s_memrealtime) at the same two points; the ratio
 *          of the differences times the reference rate is the shader clock.
 * Returns RA_ERR_INVALID_ARG for blocks <= 0, iters <= 0 or a NULL buffer,
 * RA_ERR_HIP if the launch fails; nothing is enqueued on error. */
int ring_attn_mfma_probe(int32_t blocks, int32_t iters, float* sink, uint64_t* stamps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
