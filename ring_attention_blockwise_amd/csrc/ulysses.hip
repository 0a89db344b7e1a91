// One all-to-all leg of the Ulysses sequence <-> head exchange ("lecture 30",
// sections 3.3-3.4), this device's share, as a single copy kernel: for every
// shard j, batch b and head r of the leg, `width` contiguous bytes move
// between shard j (head pitch `width`, first head `shard_head` of
// `shard_heads` per batch) and the head-sharded buffer (head pitch
// `full_pitch`, shard j's segment at byte j * width of the head). One launch
// per leg (per 64 shards) instead of one strided copy per (shard, batch);
// each element is moved once, with non-temporal loads and stores.
#include "common.h"
#include "ulysses_leg.h"

namespace ra {
namespace {

typedef int i32x4v __attribute__((ext_vector_type(4)));

constexpr int kThreadsA2A = 256;
constexpr int kUnrollA2A = 4;  // accesses per thread and block
constexpr int kPerBlock = kThreadsA2A * kUnrollA2A;

template <typename T>
__global__ void __launch_bounds__(kThreadsA2A) a2a_leg_kernel(A2ALeg a, int64_t chunks_per_seg) {
  const int64_t blk = blockIdx.x;
  const int64_t seg = blk / chunks_per_seg;
  const int64_t chunk = blk % chunks_per_seg;
  const int64_t r = seg % a.rows;
  const int64_t b = (seg / a.rows) % a.batch;
  const int jj = (int)(seg / (a.rows * a.batch));
  char* fptr = a.full + (b * a.rows + r) * a.full_pitch + (int64_t)(a.j0 + jj) * a.width;
  char* sptr = a.shard[jj] + (b * a.shard_heads + a.shard_head + r) * a.width;
  const T* src = reinterpret_cast<const T*>(a.to_shards ? fptr : sptr);
  T* dst = reinterpret_cast<T*>(a.to_shards ? sptr : fptr);
  const int64_t n = a.width / (int64_t)sizeof(T);
  const int64_t i0 = chunk * kPerBlock + threadIdx.x;
  T v[kUnrollA2A];
#pragma unroll
  for (int k = 0; k < kUnrollA2A; ++k) {
    const int64_t i = i0 + (int64_t)k * kThreadsA2A;
    if (i < n) v[k] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int k = 0; k < kUnrollA2A; ++k) {
    const int64_t i = i0 + (int64_t)k * kThreadsA2A;
    if (i < n) __builtin_nontemporal_store(v[k], dst + i);
  }
}

}  // namespace

hipError_t launch_a2a_leg(const A2ALeg& a, hipStream_t s) {
  const int64_t segs = (int64_t)a.nshards * a.batch * a.rows;
  if (segs == 0 || a.width == 0) return hipSuccess;
  // 16-byte accesses when every segment start is 16-byte aligned, else 4
  // (every pointer and pitch here is a multiple of 4 bytes)
  bool wide = (a.width % 16 == 0) && (a.full_pitch % 16 == 0) && ((reinterpret_cast<uintptr_t>(a.full)) % 16 == 0);
  for (int k = 0; k < a.nshards; ++k) wide = wide && (reinterpret_cast<uintptr_t>(a.shard[k]) % 16 == 0);
  const int64_t unit = wide ? 16 : 4;
  const int64_t chunks = (a.width / unit + kPerBlock - 1) / kPerBlock;
  const dim3 grid((unsigned)(segs * chunks));
  if (wide)
    a2a_leg_kernel<i32x4v><<<grid, kThreadsA2A, 0, s>>>(a, chunks);
  else
    a2a_leg_kernel<int><<<grid, kThreadsA2A, 0, s>>>(a, chunks);
  return hipGetLastError();
}

}  // namespace ra
