// C ABI of libring_attn: argument checks, kernel dispatch and the ring driver.
//
// Every entry point validates all of its arguments on the host before it
// enqueues anything, so an error leaves every buffer untouched.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "backward.h"
#include "common.h"
#include "ring_attn.h"
#include "ulysses_leg.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxRows = (int64_t)1 << 30;
constexpr int64_t kMaxStateRows = (int64_t)1 << 34;  // batch x heads x rows

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t count_le(const ra_segment& s, int64_t x) {
  if (x < s.start) return 0;
  const int64_t c = (x - s.start) / s.stride + 1;
  return c < s.len ? c : s.len;
}

// Shape/segment checks shared by step, merge and finalize.
int check_shape(const ra_step_desc* d, bool need_kv) {
  if (d == nullptr) return fail(RA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0 || d->heads_q <= 0 || d->heads_kv <= 0)
    return fail(RA_ERR_INVALID_ARG, "batch must be >= 0 and head counts > 0");
  if (d->heads_q % d->heads_kv != 0)
    return fail(RA_ERR_INVALID_ARG, "heads_q (%d) must be a multiple of heads_kv (%d)", d->heads_q, d->heads_kv);
  if (d->q_len < 0 || d->q_len > kMaxRows) return fail(RA_ERR_INVALID_ARG, "q_len out of range");
  if (need_kv && (d->kv_len < 0 || d->kv_len > kMaxRows)) return fail(RA_ERR_INVALID_ARG, "kv_len out of range");
  // rows of the state and of K/V over all (batch, head) pairs: bounded so that
  // every launch's work-item count and grid size stay within 32 bits
  if ((int64_t)d->batch * d->heads_q > kMaxStateRows / (d->q_len > 0 ? d->q_len : 1) ||
      (need_kv && (int64_t)d->batch * d->heads_kv > kMaxStateRows / (d->kv_len > 0 ? d->kv_len : 1)))
    return fail(RA_ERR_INVALID_ARG, "batch x heads x rows exceeds 2^34");
  if (d->dtype != RA_F32 && d->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (!std::isfinite(d->scale)) return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  return RA_OK;
}

int check_segments(const ra_segment* segs, int32_t n, int64_t rows, int causal, const char* side) {
  if (n < 0 || n > 2) return fail(RA_ERR_INVALID_ARG, "%s: segment count %d (0..2)", side, n);
  if (n == 0) {
    if (causal) return fail(RA_ERR_INVALID_ARG, "%s: causal steps need position segments", side);
    return RA_OK;
  }
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (segs[i].len < 0 || segs[i].stride < 1 || segs[i].start < 0)
      return fail(RA_ERR_INVALID_ARG, "%s: segment %d needs len >= 0, stride >= 1, start >= 0", side, i);
    if (segs[i].len > 0 && (segs[i].start > INT64_MAX / 4 - (segs[i].len - 1) * segs[i].stride))
      return fail(RA_ERR_INVALID_ARG, "%s: segment %d positions overflow", side, i);
    total += segs[i].len;
  }
  if (total != rows)
    return fail(RA_ERR_INVALID_ARG, "%s: segment lengths add up to %lld, rows are %lld", side, (long long)total,
                (long long)rows);
  return RA_OK;
}

int check_step_desc(const ra_step_desc* d) {
  int rc = check_shape(d, true);
  if (rc) return rc;
  if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  rc = check_segments(d->q_seg, d->n_q_seg, d->q_len, d->causal, "q");
  if (rc) return rc;
  return check_segments(d->kv_seg, d->n_kv_seg, d->kv_len, d->causal, "kv");
}

ra::StepArgs make_args(const ra_step_desc* d) {
  ra::StepArgs a{};
  a.q_len = d->q_len;
  a.kv_len = d->kv_len;
  a.batch = d->batch;
  a.heads_q = d->heads_q;
  a.heads_kv = d->heads_kv;
  a.group = d->heads_q / d->heads_kv;
  const double scale = d->scale > 0.0f ? (double)d->scale : 1.0 / std::sqrt((double)d->head_dim);
  a.scale_log2 = (float)(scale * 1.4426950408889634074);
  a.causal = d->causal;
  a.n_q_seg = d->n_q_seg;
  a.n_kv_seg = d->n_kv_seg;
  for (int i = 0; i < 2; ++i) {
    const bool qv = i < d->n_q_seg, kvv = i < d->n_kv_seg;
    a.qs[i] = {qv ? d->q_seg[i].start : 0, qv ? d->q_seg[i].len : 0, qv ? d->q_seg[i].stride : 1};
    a.ks[i] = {kvv ? d->kv_seg[i].start : 0, kvv ? d->kv_seg[i].len : 0, kvv ? d->kv_seg[i].stride : 1};
  }
  return a;
}

int64_t pairs_of(const ra_step_desc* d) {
  if (!d->causal) return d->q_len * d->kv_len;
  int64_t total = 0;
  for (int qi = 0; qi < d->n_q_seg; ++qi) {
    const ra_segment& q = d->q_seg[qi];
    for (int ki = 0; ki < d->n_kv_seg; ++ki) {
      const ra_segment& k = d->kv_seg[ki];
      if (q.len == 0 || k.len == 0) continue;
      if (q.stride == 1) {
        // rows whose count is clipped at 0, growing by one per row (stride-1
        // keys), or saturated at k.len: sum in closed form by splitting the
        // q range where count_le changes regime.
        int64_t i = 0;
        while (i < q.len) {
          const int64_t x = q.start + i;
          const int64_t c = count_le(k, x);
          if (c == 0) {  // jump to the first row that sees key 0
            const int64_t first = k.start - q.start;
            if (first >= q.len) break;
            i = first > i ? first : i + 1;
            continue;
          }
          if (c == k.len) {
            total += (q.len - i) * k.len;
            break;
          }
          if (k.stride == 1) {
            // c grows by 1 per row until it reaches k.len
            const int64_t n = std::min(q.len - i, k.len - c);
            total += n * c + n * (n - 1) / 2;
            i += n;
          } else {
            total += c;
            ++i;
          }
        }
      } else {
        for (int64_t i = 0; i < q.len; ++i) total += count_le(k, q.start + i * q.stride);
      }
    }
  }
  return total;
}

hipError_t launch_step(const ra::StepArgs& a, int head_dim, int dtype, hipStream_t s) {
  if (a.q_len == 0 || a.batch == 0) return hipSuccess;
  return dtype == RA_BF16 ? ra::launch_step_bf16(a, head_dim, s) : ra::launch_step_f32(a, head_dim, s);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of an MI355X; a step launches one workgroup per compute unit
// at a time (its LDS use), so a step with fewer work items than this leaves
// compute units idle.
constexpr int64_t kComputeUnits = 256;
constexpr int32_t kMaxKeySplit = 16;

// Ways the forward splits each query tile's keys (bf16 only): desc->key_split
// when given (capped so that every part gets a key tile), else, for shares
// with at most half as many 256-row work items as compute units, the largest
// power of two up to 8 that keeps items x split within the compute units and
// at least two 64-key tiles per part.
int32_t key_split_of(const ra_ring_desc* d) {
  if (d->dtype != RA_BF16 || d->key_split == 1) return 1;
  const int64_t kv_tiles = (d->local_len + 63) / 64;
  int64_t s = d->key_split;
  if (s == 0) {
    const int64_t items = (d->local_len + 255) / 256 * d->heads_q * (int64_t)d->batch;
    s = 1;
    while (s < 8 && items * s * 2 <= kComputeUnits && kv_tiles >= 4 * s) s *= 2;
  }
  if (s > kv_tiles) s = kv_tiles;
  return s > 1 ? (int32_t)s : 1;
}

struct RingLayout {
  size_t block_bytes;  // one K (or V) block
  size_t state_rows;
  int32_t split;       // key split of every step (1: none)
  size_t off_slot[2][2];
  size_t off_o, off_m, off_l;
  size_t off_po, off_pm, off_pl;  // partial states of a split step
  size_t total;
};

bool ring_layout(const ra_ring_desc* d, RingLayout* L) {
  const size_t es = d->dtype == RA_BF16 ? 2 : 4;
  L->block_bytes = (size_t)d->batch * d->heads_kv * (size_t)d->local_len * d->head_dim * es;
  L->state_rows = (size_t)d->batch * d->heads_q * (size_t)d->local_len;
  L->split = key_split_of(d);
  size_t off = 0;
  for (int s = 0; s < 2; ++s)
    for (int t = 0; t < 2; ++t) {
      L->off_slot[s][t] = off;
      off += align256(L->block_bytes);
    }
  L->off_o = off;
  off += align256(L->state_rows * d->head_dim * 4);
  L->off_m = off;
  off += align256(L->state_rows * 4);
  L->off_l = off;
  off += align256(L->state_rows * 4);
  const size_t parts = L->split > 1 ? (size_t)L->split : 0;
  L->off_po = off;
  off += align256(parts * L->state_rows * d->head_dim * 4);
  L->off_pm = off;
  off += align256(parts * L->state_rows * 4);
  L->off_pl = off;
  off += align256(parts * L->state_rows * 4);
  L->total = off + 256;  // room to align the caller's base pointer
  return true;
}

int check_ring_desc(const ra_ring_desc* d) {
  if (d == nullptr) return fail(RA_ERR_INVALID_ARG, "ring desc is NULL");
  if (d->world < 1) return fail(RA_ERR_INVALID_ARG, "world must be >= 1");
  if (d->rank < 0 || d->rank >= d->world) return fail(RA_ERR_INVALID_ARG, "rank out of range");
  if (d->partition < RA_PART_CONTIGUOUS || d->partition > RA_PART_STRIPED)
    return fail(RA_ERR_INVALID_ARG, "unknown partition %d", d->partition);
  if (d->local_len < 0 || d->local_len > kMaxRows) return fail(RA_ERR_INVALID_ARG, "local_len out of range");
  if (d->partition == RA_PART_ZIGZAG && (d->local_len % 2) != 0)
    return fail(RA_ERR_INVALID_ARG, "zigzag needs an even local_len");
  if (d->reverse_order != 0 && d->reverse_order != 1) return fail(RA_ERR_INVALID_ARG, "reverse_order must be 0/1");
  if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (d->receive < RA_RECV_AUTO || d->receive > RA_RECV_FUSED)
    return fail(RA_ERR_INVALID_ARG, "unknown receive %d", d->receive);
  if (d->key_split < 0 || d->key_split > kMaxKeySplit)
    return fail(RA_ERR_INVALID_ARG, "key_split %d out of range (0..%d)", d->key_split, kMaxKeySplit);
  ra_step_desc s{};
  s.batch = d->batch;
  s.heads_q = d->heads_q;
  s.heads_kv = d->heads_kv;
  s.head_dim = d->head_dim;
  s.q_len = d->local_len;
  s.kv_len = d->local_len;
  s.dtype = d->dtype;
  s.scale = d->scale;
  return check_shape(&s, true);
}

// The receive of one block (K and V, `bytes` each) into a slot on stream xs.
hipError_t receive_block(void* dst_k, const void* src_k, void* dst_v, const void* src_v, size_t bytes,
                         hipStream_t xs) {
  hipError_t e = hipMemcpyAsync(dst_k, src_k, bytes, hipMemcpyDeviceToDevice, xs);
  if (e != hipSuccess) return e;
  return hipMemcpyAsync(dst_v, src_v, bytes, hipMemcpyDeviceToDevice, xs);
}

int32_t owner_of(const ra_ring_desc* d, int32_t step) {
  const int32_t n = d->world;
  return d->reverse_order ? (d->rank + step) % n : ((d->rank - step) % n + n) % n;
}

}  // namespace

// Launcher of the matrix-core probe (probe.hip).
namespace ra {
hipError_t launch_mfma_probe(int32_t blocks, int32_t iters, float* sink, uint64_t* stamps, hipStream_t s);
}  // namespace ra

extern "C" {

const char* ring_attn_last_error(void) { return g_last_error; }

int32_t ring_attn_abi_version(void) { return 104; }

int ring_attn_partition_segments(int32_t partition, int32_t world, int32_t rank, int64_t local_len,
                                 ra_segment* segs, int32_t* n_segs) {
  if (segs == nullptr || n_segs == nullptr) return fail(RA_ERR_INVALID_ARG, "segs/n_segs is NULL");
  if (world < 1 || rank < 0 || rank >= world) return fail(RA_ERR_INVALID_ARG, "bad world/rank");
  if (local_len < 0 || local_len > kMaxRows) return fail(RA_ERR_INVALID_ARG, "local_len out of range");
  switch (partition) {
    case RA_PART_CONTIGUOUS:
      segs[0] = {(int64_t)rank * local_len, local_len, 1};
      *n_segs = 1;
      return RA_OK;
    case RA_PART_ZIGZAG: {
      if (local_len % 2) return fail(RA_ERR_INVALID_ARG, "zigzag needs an even local_len");
      const int64_t g = local_len / 2;
      segs[0] = {(int64_t)rank * g, g, 1};
      segs[1] = {(int64_t)(2 * world - 1 - rank) * g, g, 1};
      *n_segs = 2;
      return RA_OK;
    }
    case RA_PART_STRIPED:
      segs[0] = {(int64_t)rank, local_len, (int64_t)world};
      *n_segs = 1;
      return RA_OK;
    default:
      return fail(RA_ERR_INVALID_ARG, "unknown partition %d", partition);
  }
}

int ring_attn_ring_step_desc(const ra_ring_desc* d, int32_t step, ra_step_desc* out, int32_t* owner) {
  int rc = check_ring_desc(d);
  if (rc) return rc;
  if (out == nullptr) return fail(RA_ERR_INVALID_ARG, "out is NULL");
  if (step < 0 || step >= d->world) return fail(RA_ERR_INVALID_ARG, "step out of range");
  ra_step_desc s{};
  s.batch = d->batch;
  s.heads_q = d->heads_q;
  s.heads_kv = d->heads_kv;
  s.head_dim = d->head_dim;
  s.q_len = d->local_len;
  s.kv_len = d->local_len;
  s.dtype = d->dtype;
  s.causal = d->causal;
  s.scale = d->scale;
  const int32_t j = owner_of(d, step);
  rc = ring_attn_partition_segments(d->partition, d->world, d->rank, d->local_len, s.q_seg, &s.n_q_seg);
  if (rc) return rc;
  rc = ring_attn_partition_segments(d->partition, d->world, j, d->local_len, s.kv_seg, &s.n_kv_seg);
  if (rc) return rc;
  *out = s;
  if (owner) *owner = j;
  return RA_OK;
}

int64_t ring_attn_visible_pairs(const ra_step_desc* d) {
  if (check_step_desc(d) != RA_OK) return -1;
  return pairs_of(d);
}

int ring_attn_step(const ra_step_desc* d, const void* q, const void* k, const void* v, float* o_acc, float* m,
                   float* l, int32_t flags, void* stream) {
  int rc = check_step_desc(d);
  if (rc) return rc;
  if (flags & ~RA_STEP_INIT) return fail(RA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool has_rows = d->q_len > 0 && d->batch > 0;
  if (has_rows) {
    if (!q || !o_acc || !m || !l) return fail(RA_ERR_INVALID_ARG, "q/o_acc/m/l must not be NULL");
    if (d->kv_len > 0 && (!k || !v)) return fail(RA_ERR_INVALID_ARG, "k/v must not be NULL");
    if (!aligned16(q) || !aligned16(o_acc) || (k && !aligned16(k)) || (v && !aligned16(v)))
      return fail(RA_ERR_INVALID_ARG, "q/k/v/o_acc must be 16-byte aligned");
  }
  if (!has_rows) return RA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool init = flags & RA_STEP_INIT;
  hipError_t e;
  if (pairs_of(d) == 0) {
    // no key of this block is visible to any row
    if (!init) return RA_OK;
    e = ra::launch_init_state(o_acc, m, l, (int64_t)d->batch * d->heads_q * d->q_len, d->head_dim, s);
    return e == hipSuccess ? RA_OK : hip_fail(e, "init_state launch");
  }
  ra::StepArgs a = make_args(d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o_acc;
  a.m = m;
  a.l = l;
  a.init = init;
  e = launch_step(a, d->head_dim, d->dtype, s);
  return e == hipSuccess ? RA_OK : hip_fail(e, "step launch");
}

int ring_attn_merge(const ra_step_desc* d, float* o_a, float* m_a, float* l_a, const float* o_b, const float* m_b,
                    const float* l_b, void* stream) {
  int rc = check_shape(d, false);
  if (rc) return rc;
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->q_len;
  if (rows == 0) return RA_OK;
  if (!o_a || !m_a || !l_a || !o_b || !m_b || !l_b) return fail(RA_ERR_INVALID_ARG, "state pointers must not be NULL");
  if (!aligned16(o_a) || !aligned16(o_b)) return fail(RA_ERR_INVALID_ARG, "o_a/o_b must be 16-byte aligned");
  hipError_t e = ra::launch_merge(o_a, m_a, l_a, o_b, m_b, l_b, rows, d->head_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RA_OK : hip_fail(e, "merge launch");
}

int ring_attn_finalize(const ra_step_desc* d, const float* o_acc, const float* m, const float* l, void* out,
                       float* lse, void* stream) {
  int rc = check_shape(d, false);
  if (rc) return rc;
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->q_len;
  if (rows == 0) return RA_OK;
  if (!o_acc || !m || !l || !out) return fail(RA_ERR_INVALID_ARG, "o_acc/m/l/out must not be NULL");
  if (!aligned16(o_acc) || !aligned16(out)) return fail(RA_ERR_INVALID_ARG, "o_acc/out must be 16-byte aligned");
  hipError_t e =
      ra::launch_finalize(o_acc, m, l, out, lse, rows, d->head_dim, d->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RA_OK : hip_fail(e, "finalize launch");
}

size_t ring_attn_forward_workspace_size(const ra_ring_desc* d) {
  if (check_ring_desc(d) != RA_OK) return 0;
  RingLayout L;
  ring_layout(d, &L);
  return L.total;
}

namespace {

// Per-thread cache of the drivers' ordering events (never timed): one set per
// calling thread and device, created on first use and reused until
// ring_attn_release_thread_events() destroys them. A thread enqueues one
// driver call completely before the next, and a stream wait binds to the
// record made just before it, so reusing the set is safe.
struct DriverEvents {
  bool created = false;
  hipEvent_t ready[2] = {nullptr, nullptr};  // slot filled (copy stream)
  hipEvent_t freed[2] = {nullptr, nullptr};  // slot no longer read (compute stream)
};
constexpr int kMaxDevices = 64;
thread_local DriverEvents g_events[kMaxDevices];

hipError_t driver_events(DriverEvents** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DriverEvents& ev = g_events[dev];
  if (!ev.created) {
    for (int i = 0; i < 2; ++i) {
      if ((e = hipEventCreateWithFlags(&ev.ready[i], hipEventDisableTiming)) != hipSuccess) return e;
      if ((e = hipEventCreateWithFlags(&ev.freed[i], hipEventDisableTiming)) != hipSuccess) return e;
    }
    ev.created = true;
  }
  *out = &ev;
  return hipSuccess;
}

}  // namespace

namespace {

// Arguments every forward entry point checks before anything is enqueued.
int check_forward_args(const ra_ring_desc* d, const void* q_local, const void* const* k_blocks,
                       const void* const* v_blocks, const void* out, void* const* step_events) {
  int rc = check_ring_desc(d);
  if (rc) return rc;
  const int n = d->world;
  const bool has_rows = d->local_len > 0 && d->batch > 0;
  if (!k_blocks || !v_blocks) return fail(RA_ERR_INVALID_ARG, "k_blocks/v_blocks must not be NULL");
  if (has_rows) {
    if (!q_local || !out) return fail(RA_ERR_INVALID_ARG, "q_local/out must not be NULL");
    if (!aligned16(q_local) || !aligned16(out)) return fail(RA_ERR_INVALID_ARG, "q_local/out must be 16-byte aligned");
    for (int j = 0; j < n; ++j) {
      if (!k_blocks[j] || !v_blocks[j]) return fail(RA_ERR_INVALID_ARG, "block %d pointer is NULL", j);
      if (!aligned16(k_blocks[j]) || !aligned16(v_blocks[j]))
        return fail(RA_ERR_INVALID_ARG, "block %d is not 16-byte aligned", j);
    }
  }
  if (step_events)
    for (int i = 0; i < 2 * n; ++i)
      if (!step_events[i]) return fail(RA_ERR_INVALID_ARG, "step_events[%d] is NULL", i);
  return RA_OK;
}

// The ring of one device, after validation: `base` is the 256-byte aligned
// start of a workspace laid out by ring_layout. With xs == cs every receive
// copy runs on the compute stream and no event is created or recorded.
int forward_run(const ra_ring_desc* d, const RingLayout& L, const void* q_local, const void* const* k_blocks,
                const void* const* v_blocks, void* out, float* lse, char* base, hipStream_t cs, hipStream_t xs,
                void* const* step_events) {
  const int n = d->world;
  int rc;
  // Plan the steps on the host: descriptors and which launch.
  std::vector<ra_step_desc> steps(n);
  std::vector<int32_t> owner(n);
  std::vector<int64_t> pairs(n);
  int first = -1, last = -1;
  for (int s = 0; s < n; ++s) {
    rc = ring_attn_ring_step_desc(d, s, &steps[s], &owner[s]);
    if (rc) return rc;
    pairs[s] = pairs_of(&steps[s]);
    if (pairs[s] > 0) {
      if (first < 0) first = s;
      last = s;
    }
  }

  void* slot_k[2] = {base + L.off_slot[0][0], base + L.off_slot[1][0]};
  void* slot_v[2] = {base + L.off_slot[0][1], base + L.off_slot[1][1]};
  float* o = reinterpret_cast<float*>(base + L.off_o);
  float* m = reinterpret_cast<float*>(base + L.off_m);
  float* l = reinterpret_cast<float*>(base + L.off_l);

  // Fused receive: the block of step s+1 is copied by step s's kernel when
  // step s launches one; the other receives go on the compute stream.
  const bool fused = d->dtype == RA_BF16 && (d->receive == RA_RECV_AUTO || d->receive == RA_RECV_FUSED);
  if (fused) xs = cs;
  const bool two_streams = xs != cs;
  DriverEvents* ev = nullptr;
  hipError_t e;
  if (two_streams)
    if ((e = driver_events(&ev)) != hipSuccess) return hip_fail(e, "event creation");
  bool freed_recorded[2] = {false, false};

  // The copy stream must not start before work already queued on the compute
  // stream that produced the inputs: order it after the compute stream once
  // (only when something will be copied, so that a captured call leaves no
  // branch of the copy stream unjoined).
  if (two_streams && n > 1) {
    if ((e = hipEventRecord(ev->freed[0], cs)) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(xs, ev->freed[0], 0)) != hipSuccess) return hip_fail(e, "stream wait");
  }

  auto enqueue_receive = [&](int s) -> hipError_t {
    // step s reads slot s%2; it was last read by step s-2
    const int slot = s & 1;
    hipError_t err;
    if (freed_recorded[slot] && two_streams)
      if ((err = hipStreamWaitEvent(xs, ev->freed[slot], 0)) != hipSuccess) return err;
    if ((err = receive_block(slot_k[slot], k_blocks[owner[s]], slot_v[slot], v_blocks[owner[s]], L.block_bytes,
                             xs)) != hipSuccess)
      return err;
    return two_streams ? hipEventRecord(ev->ready[slot], xs) : hipSuccess;
  };

  for (int s = 0; s < n; ++s) {
    // receive the block of step s+1 while step s computes
    const bool rx_in_step = fused && pairs[s] > 0 && s + 1 < n;
    if (s + 1 < n && !rx_in_step)
      if ((e = enqueue_receive(s + 1)) != hipSuccess) return hip_fail(e, "receive copy");
    const void* kb = k_blocks[owner[s]];
    const void* vb = v_blocks[owner[s]];
    if (s > 0) {
      kb = slot_k[s & 1];
      vb = slot_v[s & 1];
      if (two_streams)
        if ((e = hipStreamWaitEvent(cs, ev->ready[s & 1], 0)) != hipSuccess) return hip_fail(e, "stream wait");
    }
    if (step_events)
      if ((e = hipEventRecord(static_cast<hipEvent_t>(step_events[2 * s]), cs)) != hipSuccess)
        return hip_fail(e, "step event");
    if (pairs[s] > 0) {
      ra::StepArgs a = make_args(&steps[s]);
      a.q = q_local;
      a.k = kb;
      a.v = vb;
      a.o = o;
      a.m = m;
      a.l = l;
      a.init = (s == first);
      a.final_ = (s == last);
      a.out = out;
      a.lse = lse;
      if (rx_in_step) {
        // slot (s+1)%2 was last read by step s-1, which is complete
        const int slot = (s + 1) & 1;
        a.rx_src[0] = k_blocks[owner[s + 1]];
        a.rx_src[1] = v_blocks[owner[s + 1]];
        a.rx_dst[0] = slot_k[slot];
        a.rx_dst[1] = slot_v[slot];
        a.rx_bytes = (int64_t)L.block_bytes;
      }
      if (L.split > 1) {
        a.split = L.split;
        a.po = reinterpret_cast<float*>(base + L.off_po);
        a.pm = reinterpret_cast<float*>(base + L.off_pm);
        a.pl = reinterpret_cast<float*>(base + L.off_pl);
      }
      if ((e = launch_step(a, d->head_dim, d->dtype, cs)) != hipSuccess) return hip_fail(e, "step launch");
    }
    if (step_events)
      if ((e = hipEventRecord(static_cast<hipEvent_t>(step_events[2 * s + 1]), cs)) != hipSuccess)
        return hip_fail(e, "step event");
    if (s > 0 && two_streams) {
      if ((e = hipEventRecord(ev->freed[s & 1], cs)) != hipSuccess) return hip_fail(e, "event record");
      freed_recorded[s & 1] = true;
    }
  }

  if (last < 0) {
    // no step saw any key: every row is empty
    const int64_t rows = (int64_t)L.state_rows;
    if ((e = ra::launch_init_state(o, m, l, rows, d->head_dim, cs)) != hipSuccess) return hip_fail(e, "init");
    if ((e = ra::launch_finalize(o, m, l, out, lse, rows, d->head_dim, d->dtype, cs)) != hipSuccess)
      return hip_fail(e, "finalize");
  }
  // The copy stream's last work is ordered before the compute stream's last
  // step (which waited on it), so the caller only needs to sync compute_stream.
  return RA_OK;
}

// Scratch of ring_attn_forward_noalloc: receive slots and state live in this
// file-scope device array instead of a caller's workspace. Each device holds
// its own copy (at its own address) from the time the library's code is
// loaded there until the process ends. In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current and kept in g_scratch_addr.
constexpr size_t kScratchBytes = (size_t)RA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

int ring_attn_forward(const ra_ring_desc* d, const void* q_local, const void* const* k_blocks,
                      const void* const* v_blocks, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* compute_stream, void* copy_stream, void* const* step_events) {
  int rc = check_forward_args(d, q_local, k_blocks, v_blocks, out, step_events);
  if (rc) return rc;
  RingLayout L;
  ring_layout(d, &L);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace_bytes);
  if (copy_stream != nullptr && copy_stream == compute_stream)
    return fail(RA_ERR_INVALID_ARG, "copy_stream must differ from compute_stream (or be NULL)");
  if (!(d->local_len > 0 && d->batch > 0)) return RA_OK;
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  hipStream_t cs = static_cast<hipStream_t>(compute_stream);
  hipStream_t xs = copy_stream ? static_cast<hipStream_t>(copy_stream) : cs;
  return forward_run(d, L, q_local, k_blocks, v_blocks, out, lse, base, cs, xs, step_events);
}

int ring_attn_forward_noalloc(const ra_ring_desc* d, const void* q_local, const void* const* k_blocks,
                              const void* const* v_blocks, void* out, float* lse, void* stream) {
  int rc = check_forward_args(d, q_local, k_blocks, v_blocks, out, nullptr);
  if (rc) return rc;
  RingLayout L;
  ring_layout(d, &L);
  const size_t need = L.total - 256;  // the scratch is already 256-byte aligned
  if (need > kScratchBytes)
    return fail(RA_ERR_WORKSPACE, "share needs %zu bytes of scratch, the no-allocation forward has %zu", need,
                kScratchBytes);
  if (!(d->local_len > 0 && d->batch > 0)) return RA_OK;
  void* base = nullptr;
  const hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  hipStream_t cs = static_cast<hipStream_t>(stream);
  return forward_run(d, L, q_local, k_blocks, v_blocks, out, lse, static_cast<char*>(base), cs, cs, nullptr);
}

namespace {

struct UlyssesLayout {
  int64_t hq, hkv, ls;  // heads of this device, rows per shard
  size_t es;            // element size
  size_t off_q, off_k, off_v, off_out, off_lse, total;
};

int check_ulysses_desc(const ra_ulysses_desc* d) {
  if (d == nullptr) return fail(RA_ERR_INVALID_ARG, "ulysses desc is NULL");
  if (d->world < 1) return fail(RA_ERR_INVALID_ARG, "world must be >= 1");
  if (d->rank < 0 || d->rank >= d->world) return fail(RA_ERR_INVALID_ARG, "rank out of range");
  if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (d->seq_len < 0 || d->seq_len > kMaxRows) return fail(RA_ERR_INVALID_ARG, "seq_len out of range");
  if (d->heads_q < 1 || d->heads_kv < 1 || d->heads_q % d->world != 0 || d->heads_kv % d->world != 0)
    return fail(RA_ERR_INVALID_ARG, "heads_q (%d) and heads_kv (%d) must be divisible by world (%d)", d->heads_q,
                d->heads_kv, d->world);
  if (d->seq_len % d->world != 0)
    return fail(RA_ERR_INVALID_ARG, "seq_len (%lld) must be divisible by world (%d)", (long long)d->seq_len,
                d->world);
  // the attention this device runs: its heads over the whole sequence
  ra_step_desc s{};
  s.batch = d->batch;
  s.heads_q = d->heads_q / d->world;
  s.heads_kv = d->heads_kv / d->world;
  s.head_dim = d->head_dim;
  s.q_len = d->seq_len;
  s.kv_len = d->seq_len;
  s.dtype = d->dtype;
  s.scale = d->scale;
  return check_shape(&s, true);
}

void ulysses_layout(const ra_ulysses_desc* d, UlyssesLayout* L) {
  L->hq = d->heads_q / d->world;
  L->hkv = d->heads_kv / d->world;
  L->ls = d->seq_len / d->world;
  L->es = d->dtype == RA_BF16 ? 2 : 4;
  const size_t rows_q = (size_t)d->batch * L->hq * (size_t)d->seq_len;
  const size_t rows_kv = (size_t)d->batch * L->hkv * (size_t)d->seq_len;
  size_t off = 0;
  L->off_q = off;
  off += align256(rows_q * d->head_dim * L->es);
  L->off_k = off;
  off += align256(rows_kv * d->head_dim * L->es);
  L->off_v = off;
  off += align256(rows_kv * d->head_dim * L->es);
  L->off_out = off;
  off += align256(rows_q * d->head_dim * L->es);
  L->off_lse = off;
  off += align256(rows_q * 4);
  L->total = off + 256;  // room to align the caller's base pointer
}

// One all-to-all leg for this device: for every shard j and batch b, `rows`
// consecutive heads of `width` bytes each move between the shard (head pitch
// `width`, first head `shard_head`, heads per batch `shard_heads`) and the
// head-sharded buffer (head pitch `full_pitch`, segment j at byte j * width).
// shards_out picks the direction. One copy kernel per 64 shards.
hipError_t all_to_all_leg(const ra_ulysses_desc* d, char* full, const char* const* shards_in,
                          char* const* shards_out, int64_t rows, int64_t shard_heads, int64_t shard_head,
                          size_t width, size_t full_pitch, hipStream_t s) {
  for (int j0 = 0; j0 < d->world; j0 += ra::kA2AShards) {
    ra::A2ALeg a{};
    a.full = full;
    a.j0 = j0;
    a.nshards = d->world - j0 < ra::kA2AShards ? d->world - j0 : ra::kA2AShards;
    a.to_shards = shards_out != nullptr;
    for (int k = 0; k < a.nshards; ++k)
      a.shard[k] = shards_out ? shards_out[j0 + k] : const_cast<char*>(shards_in[j0 + k]);
    a.batch = d->batch;
    a.rows = rows;
    a.shard_heads = shard_heads;
    a.shard_head = shard_head;
    a.width = (int64_t)width;
    a.full_pitch = (int64_t)full_pitch;
    const hipError_t e = ra::launch_a2a_leg(a, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t ring_attn_ulysses_workspace_size(const ra_ulysses_desc* d) {
  if (check_ulysses_desc(d) != RA_OK) return 0;
  UlyssesLayout L;
  ulysses_layout(d, &L);
  return L.total;
}

int ring_attn_ulysses_forward(const ra_ulysses_desc* d, const void* const* q_shards, const void* const* k_shards,
                              const void* const* v_shards, void* const* out_shards, float* const* lse_shards,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_ulysses_desc(d);
  if (rc) return rc;
  if (!q_shards || !k_shards || !v_shards || !out_shards)
    return fail(RA_ERR_INVALID_ARG, "q/k/v/out shard arrays must not be NULL");
  const bool has_rows = d->seq_len > 0 && d->batch > 0;
  if (has_rows)
    for (int j = 0; j < d->world; ++j) {
      if (!q_shards[j] || !k_shards[j] || !v_shards[j] || !out_shards[j])
        return fail(RA_ERR_INVALID_ARG, "shard %d pointer is NULL", j);
      if (!aligned16(q_shards[j]) || !aligned16(k_shards[j]) || !aligned16(v_shards[j]) || !aligned16(out_shards[j]))
        return fail(RA_ERR_INVALID_ARG, "shard %d is not 16-byte aligned", j);
      if (lse_shards && !lse_shards[j]) return fail(RA_ERR_INVALID_ARG, "lse shard %d pointer is NULL", j);
      if (lse_shards && (reinterpret_cast<uintptr_t>(lse_shards[j]) & 3u) != 0)
        return fail(RA_ERR_INVALID_ARG, "lse shard %d is not 4-byte aligned", j);
    }
  UlyssesLayout L;
  ulysses_layout(d, &L);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace_bytes);
  if (!has_rows) return RA_OK;

  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t row_bytes = (size_t)d->head_dim * L.es;
  const size_t seg = (size_t)L.ls * row_bytes;         // one head of one shard
  const size_t full = (size_t)d->seq_len * row_bytes;  // one head of the whole sequence
  const char* const* qs = reinterpret_cast<const char* const*>(q_shards);
  const char* const* ks = reinterpret_cast<const char* const*>(k_shards);
  const char* const* vs = reinterpret_cast<const char* const*>(v_shards);
  hipError_t e;
  // first all-to-all: this device's heads of every sequence shard
  if ((e = all_to_all_leg(d, base + L.off_q, qs, nullptr, L.hq, d->heads_q, (int64_t)d->rank * L.hq, seg, full,
                          s)) != hipSuccess ||
      (e = all_to_all_leg(d, base + L.off_k, ks, nullptr, L.hkv, d->heads_kv, (int64_t)d->rank * L.hkv, seg, full,
                          s)) != hipSuccess ||
      (e = all_to_all_leg(d, base + L.off_v, vs, nullptr, L.hkv, d->heads_kv, (int64_t)d->rank * L.hkv, seg, full,
                          s)) != hipSuccess)
    return hip_fail(e, "ulysses gather");

  // local attention: every query of the sequence against every key, for this
  // device's heads, in one launch with the state kept in registers
  ra::StepArgs a{};
  a.q_len = d->seq_len;
  a.kv_len = d->seq_len;
  a.batch = d->batch;
  a.heads_q = (int32_t)L.hq;
  a.heads_kv = (int32_t)L.hkv;
  a.group = (int32_t)(L.hq / L.hkv);
  const double scale = d->scale > 0.0f ? (double)d->scale : 1.0 / std::sqrt((double)d->head_dim);
  a.scale_log2 = (float)(scale * 1.4426950408889634074);
  a.causal = d->causal;
  a.n_q_seg = 1;
  a.n_kv_seg = 1;
  a.qs[0] = {0, d->seq_len, 1};
  a.ks[0] = {0, d->seq_len, 1};
  a.q = base + L.off_q;
  a.k = base + L.off_k;
  a.v = base + L.off_v;
  a.init = 1;
  a.final_ = 1;
  a.out = base + L.off_out;
  a.lse = reinterpret_cast<float*>(base + L.off_lse);
  if ((e = launch_step(a, d->head_dim, d->dtype, s)) != hipSuccess) return hip_fail(e, "ulysses attention launch");

  // second all-to-all: this device's heads back into every sequence shard
  char* const* os = reinterpret_cast<char* const*>(out_shards);
  if ((e = all_to_all_leg(d, base + L.off_out, nullptr, os, L.hq, d->heads_q, (int64_t)d->rank * L.hq, seg, full,
                          s)) != hipSuccess)
    return hip_fail(e, "ulysses scatter");
  if (lse_shards) {
    char* const* ls = reinterpret_cast<char* const*>(lse_shards);
    if ((e = all_to_all_leg(d, base + L.off_lse, nullptr, ls, L.hq, d->heads_q, (int64_t)d->rank * L.hq,
                            (size_t)L.ls * 4, (size_t)d->seq_len * 4, s)) != hipSuccess)
      return hip_fail(e, "ulysses scatter (lse)");
  }
  return RA_OK;
}

/* ---- backward ------------------------------------------------------------ */

namespace {

float scale_of(const ra_step_desc* d) {
  return d->scale > 0.0f ? d->scale : (float)(1.0 / std::sqrt((double)d->head_dim));
}

int check_backward_shape(const ra_step_desc* d) { return check_shape(d, true); }

hipError_t launch_bwd(const ra::BwdArgs& a, int head_dim, int dtype, hipStream_t s) {
  return dtype == RA_BF16 ? ra::launch_bwd_bf16(a, head_dim, s) : ra::launch_bwd_f32(a, head_dim, s);
}

struct BwdLayout {
  size_t block_bytes, rows;
  size_t off_slot[2][2];
  size_t off_dq, off_terms, total;
};

void bwd_layout(const ra_ring_desc* d, BwdLayout* L) {
  const size_t es = d->dtype == RA_BF16 ? 2 : 4;
  L->block_bytes = (size_t)d->batch * d->heads_kv * (size_t)d->local_len * d->head_dim * es;
  L->rows = (size_t)d->batch * d->heads_q * (size_t)d->local_len;
  size_t off = 0;
  for (int s = 0; s < 2; ++s)
    for (int t = 0; t < 2; ++t) {
      L->off_slot[s][t] = off;
      off += align256(L->block_bytes);
    }
  L->off_dq = off;
  off += align256(L->rows * d->head_dim * 4);
  L->off_terms = off;
  off += align256(L->rows * 2 * 4);
  L->total = off + 256;
}

}  // namespace

int ring_attn_backward_prep(const ra_step_desc* d, const void* out, const void* d_out, const float* lse,
                            float* terms, void* stream) {
  int rc = check_shape(d, false);
  if (rc) return rc;
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->q_len;
  if (rows == 0) return RA_OK;
  if (!out || !d_out || !lse || !terms) return fail(RA_ERR_INVALID_ARG, "out/d_out/lse/terms must not be NULL");
  hipError_t e = ra::launch_bwd_prep(out, d_out, lse, terms, rows, d->head_dim, d->dtype, scale_of(d),
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RA_OK : hip_fail(e, "backward prep launch");
}

int ring_attn_backward_step(const ra_step_desc* d, const void* q, const void* k, const void* v, const void* d_out,
                            const float* terms, float* dq_acc, float* dk_acc, float* dv_acc, int32_t flags,
                            void* stream) {
  int rc = check_backward_shape(d);
  if (rc) return rc;
  if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  rc = check_segments(d->q_seg, d->n_q_seg, d->q_len, d->causal, "q");
  if (rc) return rc;
  rc = check_segments(d->kv_seg, d->n_kv_seg, d->kv_len, d->causal, "kv");
  if (rc) return rc;
  if (flags & ~RA_BWD_INIT_DQ) return fail(RA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool has_rows = d->q_len > 0 && d->batch > 0;
  if (!has_rows) return RA_OK;
  if (!q || !d_out || !terms || !dq_acc) return fail(RA_ERR_INVALID_ARG, "q/d_out/terms/dq_acc must not be NULL");
  if (d->kv_len > 0 && (!k || !v || !dk_acc || !dv_acc))
    return fail(RA_ERR_INVALID_ARG, "k/v/dk_acc/dv_acc must not be NULL");
  if (!aligned16(q) || !aligned16(d_out) || !aligned16(dq_acc) || (k && !aligned16(k)) || (v && !aligned16(v)) ||
      (dk_acc && !aligned16(dk_acc)) || (dv_acc && !aligned16(dv_acc)) || !aligned16(terms))
    return fail(RA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool init = flags & RA_BWD_INIT_DQ;
  hipError_t e;
  if (pairs_of(d) == 0) {
    if (!init) return RA_OK;
    e = ra::launch_zero(dq_acc, (size_t)d->batch * d->heads_q * d->q_len * d->head_dim * 4, s);
    return e == hipSuccess ? RA_OK : hip_fail(e, "dq clear");
  }
  ra::BwdArgs a{};
  a.s = make_args(d);
  a.s.q = q;
  a.s.k = k;
  a.s.v = v;
  a.dout = d_out;
  a.terms = terms;
  a.dq = dq_acc;
  a.dk = dk_acc;
  a.dv = dv_acc;
  a.scale = scale_of(d);
  a.init_dq = init;
  e = launch_bwd(a, d->head_dim, d->dtype, s);
  return e == hipSuccess ? RA_OK : hip_fail(e, "backward step launch");
}

size_t ring_attn_backward_workspace_size(const ra_ring_desc* d) {
  if (check_ring_desc(d) != RA_OK) return 0;
  BwdLayout L;
  bwd_layout(d, &L);
  return L.total;
}

int ring_attn_backward(const ra_ring_desc* d, const void* q_local, const void* const* k_blocks,
                       const void* const* v_blocks, const void* out, const void* d_out, const float* lse, void* dq,
                       float* const* dk_acc, float* const* dv_acc, void* workspace, size_t workspace_bytes,
                       void* compute_stream, void* copy_stream, void* const* step_events) {
  int rc = check_ring_desc(d);
  if (rc) return rc;
  const int n = d->world;
  const bool has_rows = d->local_len > 0 && d->batch > 0;
  if (!k_blocks || !v_blocks || !dk_acc || !dv_acc)
    return fail(RA_ERR_INVALID_ARG, "k_blocks/v_blocks/dk_acc/dv_acc must not be NULL");
  if (has_rows) {
    if (!q_local || !out || !d_out || !lse || !dq) return fail(RA_ERR_INVALID_ARG, "q/out/d_out/lse/dq must not be NULL");
    if (!aligned16(q_local) || !aligned16(out) || !aligned16(d_out) || !aligned16(dq))
      return fail(RA_ERR_INVALID_ARG, "q/out/d_out/dq must be 16-byte aligned");
    for (int j = 0; j < n; ++j) {
      if (!k_blocks[j] || !v_blocks[j] || !dk_acc[j] || !dv_acc[j])
        return fail(RA_ERR_INVALID_ARG, "block %d pointer is NULL", j);
      if (!aligned16(k_blocks[j]) || !aligned16(v_blocks[j]) || !aligned16(dk_acc[j]) || !aligned16(dv_acc[j]))
        return fail(RA_ERR_INVALID_ARG, "block %d is not 16-byte aligned", j);
    }
  }
  if (step_events)
    for (int i = 0; i < 2 * n; ++i)
      if (!step_events[i]) return fail(RA_ERR_INVALID_ARG, "step_events[%d] is NULL", i);
  BwdLayout L;
  bwd_layout(d, &L);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace_bytes);
  if (copy_stream != nullptr && copy_stream == compute_stream)
    return fail(RA_ERR_INVALID_ARG, "copy_stream must differ from compute_stream (or be NULL)");
  if (!has_rows) return RA_OK;

  std::vector<ra_step_desc> steps(n);
  std::vector<int32_t> owner(n);
  std::vector<int64_t> pairs(n);
  int first = -1;
  for (int s = 0; s < n; ++s) {
    rc = ring_attn_ring_step_desc(d, s, &steps[s], &owner[s]);
    if (rc) return rc;
    pairs[s] = pairs_of(&steps[s]);
    if (pairs[s] > 0 && first < 0) first = s;
  }

  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  void* slot_k[2] = {base + L.off_slot[0][0], base + L.off_slot[1][0]};
  void* slot_v[2] = {base + L.off_slot[0][1], base + L.off_slot[1][1]};
  float* dq_acc = reinterpret_cast<float*>(base + L.off_dq);
  float* terms = reinterpret_cast<float*>(base + L.off_terms);

  hipStream_t cs = static_cast<hipStream_t>(compute_stream);
  hipStream_t xs = copy_stream ? static_cast<hipStream_t>(copy_stream) : cs;
  DriverEvents* ev = nullptr;
  hipError_t e = driver_events(&ev);
  if (e != hipSuccess) return hip_fail(e, "event creation");
  bool freed_recorded[2] = {false, false};
  if (xs != cs && n > 1) {
    if ((e = hipEventRecord(ev->freed[0], cs)) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(xs, ev->freed[0], 0)) != hipSuccess) return hip_fail(e, "stream wait");
  }
  auto enqueue_receive = [&](int s) -> hipError_t {
    const int slot = s & 1;
    hipError_t err;
    if (freed_recorded[slot] && xs != cs)
      if ((err = hipStreamWaitEvent(xs, ev->freed[slot], 0)) != hipSuccess) return err;
    if ((err = receive_block(slot_k[slot], k_blocks[owner[s]], slot_v[slot], v_blocks[owner[s]], L.block_bytes,
                             xs)) != hipSuccess)
      return err;
    return hipEventRecord(ev->ready[slot], xs);
  };

  const float scale = d->scale > 0.0f ? d->scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  if ((e = ra::launch_bwd_prep(out, d_out, lse, terms, (int64_t)L.rows, d->head_dim, d->dtype, scale, cs)) !=
      hipSuccess)
    return hip_fail(e, "backward prep launch");
  for (int s = 0; s < n; ++s) {
    if (s + 1 < n)
      if ((e = enqueue_receive(s + 1)) != hipSuccess) return hip_fail(e, "receive copy");
    const void* kb = k_blocks[owner[s]];
    const void* vb = v_blocks[owner[s]];
    if (s > 0) {
      kb = slot_k[s & 1];
      vb = slot_v[s & 1];
      if (xs != cs)
        if ((e = hipStreamWaitEvent(cs, ev->ready[s & 1], 0)) != hipSuccess) return hip_fail(e, "stream wait");
    }
    if (step_events)
      if ((e = hipEventRecord(static_cast<hipEvent_t>(step_events[2 * s]), cs)) != hipSuccess)
        return hip_fail(e, "step event");
    if (pairs[s] > 0) {
      ra::BwdArgs a{};
      a.s = make_args(&steps[s]);
      a.s.q = q_local;
      a.s.k = kb;
      a.s.v = vb;
      a.dout = d_out;
      a.terms = terms;
      a.dq = dq_acc;
      a.dk = dk_acc[owner[s]];
      a.dv = dv_acc[owner[s]];
      a.scale = scale;
      a.init_dq = (s == first);
      if ((e = launch_bwd(a, d->head_dim, d->dtype, cs)) != hipSuccess) return hip_fail(e, "backward step launch");
    }
    if (step_events)
      if ((e = hipEventRecord(static_cast<hipEvent_t>(step_events[2 * s + 1]), cs)) != hipSuccess)
        return hip_fail(e, "step event");
    if (s > 0 && xs != cs) {
      if ((e = hipEventRecord(ev->freed[s & 1], cs)) != hipSuccess) return hip_fail(e, "event record");
      freed_recorded[s & 1] = true;
    }
  }
  const int64_t n_dq = (int64_t)L.rows * d->head_dim;
  if (first < 0) {
    if ((e = ra::launch_zero(dq, (size_t)n_dq * (d->dtype == RA_BF16 ? 2 : 4), cs)) != hipSuccess)
      return hip_fail(e, "dq clear");
    return RA_OK;
  }
  if ((e = ra::launch_convert(dq_acc, dq, n_dq, d->dtype, cs)) != hipSuccess) return hip_fail(e, "dq convert");
  return RA_OK;
}

int ring_attn_events_create(int32_t n, void** events) {
  if (n < 0 || (n > 0 && events == nullptr)) return fail(RA_ERR_INVALID_ARG, "bad event array");
  for (int i = 0; i < n; ++i) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(static_cast<hipEvent_t>(events[j]));
      return hip_fail(err, "hipEventCreate");
    }
    events[i] = e;
  }
  return RA_OK;
}

int ring_attn_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return fail(RA_ERR_INVALID_ARG, "NULL argument");
  hipError_t e = hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
  return e == hipSuccess ? RA_OK : hip_fail(e, "hipEventElapsedTime");
}

int ring_attn_mfma_probe(int32_t blocks, int32_t iters, float* sink, uint64_t* stamps, void* stream) {
  if (blocks <= 0 || iters <= 0) return fail(RA_ERR_INVALID_ARG, "blocks and iters must be positive");
  if (!sink || !stamps) return fail(RA_ERR_INVALID_ARG, "NULL buffer");
  const hipError_t e = ra::launch_mfma_probe(blocks, iters, sink, stamps, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RA_OK : hip_fail(e, "mfma probe launch");
}

int ring_attn_events_destroy(int32_t n, void* const* events) {
  if (n < 0 || (n > 0 && events == nullptr)) return fail(RA_ERR_INVALID_ARG, "bad event array");
  for (int i = 0; i < n; ++i)
    if (events[i]) (void)hipEventDestroy(static_cast<hipEvent_t>(events[i]));
  return RA_OK;
}

int ring_attn_release_thread_events(void) {
  hipError_t first = hipSuccess;
  for (DriverEvents& ev : g_events) {
    if (!ev.created) continue;
    for (int i = 0; i < 2; ++i) {
      const hipError_t a = hipEventDestroy(ev.ready[i]);
      const hipError_t b = hipEventDestroy(ev.freed[i]);
      if (first == hipSuccess) first = a != hipSuccess ? a : b;
      ev.ready[i] = ev.freed[i] = nullptr;
    }
    ev.created = false;
  }
  return first == hipSuccess ? RA_OK : hip_fail(first, "hipEventDestroy");
}

int ring_attn_synchronize(void* stream) {
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RA_OK : hip_fail(e, "hipStreamSynchronize");
}

}  // extern "C"
