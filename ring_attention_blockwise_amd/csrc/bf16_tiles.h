// Building blocks of the bf16 step kernels on the CDNA4 matrix cores
// (gfx950): vector types, the LDS layout of the K/V tile ring, buffer-to-LDS
// copies, and the register layouts of v_mfma_f32_32x32x16_bf16 operands.
// Internal to libring_attn.
#pragma once

#include "common.h"

namespace ra {
namespace bf16k {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 64;                   // keys per tile
constexpr int kStages = 4;                // LDS ring of K/V tiles
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, dword access
constexpr int kWaitVmcnt0 = 0x0F70;       // s_waitcnt vmcnt(0), other counters unchecked
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// LDS ring: kStages K tiles, then kStages V tiles, rows of D bf16. The
// 16-byte units of a row are XOR-swizzled (applied through the global offset
// of the copy), so the K reads (16 lanes x 16 B over 16 rows) and the V
// transposed reads (4 rows x 4 units per half-wave) are free of bank
// conflicts.
template <int D>
struct Layout {
  static constexpr int kRowBytes = D * 2;                        // one K or V row
  static constexpr int kUnits = D / 8;                           // 16-byte units per row
  static constexpr int kTileBytes = kBN * kRowBytes;             // one K (or V) tile
  static constexpr int kVBase = kStages * kTileBytes;           // K stages, then V stages
  static constexpr int kSmemBytes = 2 * kStages * kTileBytes;
  static constexpr int kDChunks = D / 16;                        // K=16 steps of S^T
  static constexpr int kDBlocks = D / 32;                        // 32-row blocks of O^T

  // Stored position of logical 16-byte unit c of row `row` is c ^ swz(row).
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

template <class T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_ptr(uint32_t addr) {
  return (const __attribute__((address_space(3))) T*)(uintptr_t)addr;
}

// A wave-uniform 64-bit address held in SGPRs.
__device__ __forceinline__ uint64_t uniform_address(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Raw buffer resource over `nbytes` bytes at the uniform address base + off.
__device__ __forceinline__ i32x4 resource_at(uint64_t base, uint64_t off, int nbytes) {
  const uint64_t a = base + off;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = kBufferWord3;
  return r;
}

// A wave's NB consecutive 1 KB blocks of a tile copied into LDS with one M0
// write: lane i of block j lands at lds_dst + 1024 j + 16 i. The per-lane
// byte offsets are computed once (block j's minus 1024 j: the instruction
// offset 1024 j moves the global and the LDS address alike). M0 is declared
// clobbered; nothing else in these kernels keeps a value in it.
template <int NB>
__device__ __forceinline__ void dma16_blocks(const i32x4& rsrc, uint32_t lds_dst, const int (&voff)[NB]) {
  static_assert(NB == 1 || NB == 2 || NB == 4, "one, two or four blocks");
  if constexpr (NB == 4)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "buffer_load_dwordx4 %3, %2, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %4, %2, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %5, %2, 0 offen offset:3072 lds"
        :
        : "s"(lds_dst), "v"(voff[0]), "s"(rsrc), "v"(voff[1 % NB]), "v"(voff[2 % NB]), "v"(voff[3 % NB])
        : "memory", "m0");
  else if constexpr (NB == 2)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "buffer_load_dwordx4 %3, %2, 0 offen offset:1024 lds"
        :
        : "s"(lds_dst), "v"(voff[0]), "s"(rsrc), "v"(voff[1 % NB])
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_dst), "v"(voff[0]), "s"(rsrc)
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// K (A operand of S^T = K Q^T) read address of lane (qcol, hh) for head_dim
// chunk c of a tile in stage 0 and key block 0: row qcol, logical unit
// 2c + hh. Stage and key block add compile-time offsets.
template <int D>
__device__ __forceinline__ uint32_t k_read_address(uint32_t smem_base, int qcol, int hh, int c) {
  using Ly = Layout<D>;
  return smem_base + qcol * Ly::kRowBytes + (((2 * c + hh) ^ Ly::k_swz(qcol)) << 4);
}

// V^T read address for ds_read_b64_tr_b16 and head_dim block db of a tile in
// stage 0: within each 16-lane group, source lane s = 4t + q points at row
// (4*hh + t) of the 8-row slice and at head_dim offset 32*db +
// 16*(group16 & 1) + 4q; the instruction hands output lane j element j%4 of
// source lane 4t + j/4, i.e. V[row t][d = ... + j].
template <int D>
__device__ __forceinline__ uint32_t v_read_address(uint32_t smem_base, int lane, int db) {
  using Ly = Layout<D>;
  const int hh = lane >> 5;
  const int grp16 = lane >> 4;
  const int t4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  const int v_row = 4 * hh + t4;
  const int unit = 4 * db + 2 * (grp16 & 1) + (q4 >> 1);
  return smem_base + Ly::kVBase + v_row * Ly::kRowBytes + ((unit ^ Ly::v_swz(v_row)) << 4) + ((q4 & 1) << 3);
}

// Operand of MFMA i of O^T += V^T P^T for the tile in stage ST: key block
// kb, 16-key chunk c and head_dim block db; V^T is fetched by two
// transposing reads.
template <int D, int ST>
__device__ __forceinline__ bf16x8 read_vt(int i, const uint32_t* v_addr) {
  using Ly = Layout<D>;
  const int db = i % Ly::kDBlocks;
  const int kc = i / Ly::kDBlocks;  // (kb, c) = (kc / 2, kc % 2)
  const int slice = ST * Ly::kTileBytes + (kc * 16) * Ly::kRowBytes;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_ptr<s16x4>(v_addr[db] + slice));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_ptr<s16x4>(v_addr[db] + slice + 8 * Ly::kRowBytes));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace bf16k
}  // namespace ra
