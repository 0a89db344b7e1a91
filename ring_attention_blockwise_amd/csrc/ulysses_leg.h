// Internal: arguments of one all-to-all leg copy kernel (ulysses.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

constexpr int kA2AShards = 64;  // shard pointers per launch

struct A2ALeg {
  char* full;                   // head-sharded buffer
  char* shard[kA2AShards];      // shards j0 .. j0 + nshards - 1
  int32_t j0;
  int32_t nshards;
  int32_t to_shards;            // 1: full -> shards, 0: shards -> full
  int64_t batch;
  int64_t rows;                 // heads of this device per batch
  int64_t shard_heads;          // heads per batch in a shard
  int64_t shard_head;           // first head of this device in a shard
  int64_t width;                // bytes of one head of one shard
  int64_t full_pitch;           // bytes of one head in the full buffer
};

hipError_t launch_a2a_leg(const A2ALeg& a, hipStream_t s);

}  // namespace ra
