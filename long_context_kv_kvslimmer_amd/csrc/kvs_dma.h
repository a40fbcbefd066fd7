// Tile streaming helpers for gfx950 kernels: 16-byte buffer loads written straight into
// LDS (no register staging), 32-slot tiles in a ring, XOR-swizzled rows.
#pragma once

#include "kvs_common.h"

namespace kvs {

constexpr int kT2 = 32;              // slots per tile
constexpr int kRing2 = 4;            // tile buffers
constexpr int kW2 = 4;               // waves that share one tile's loads

template <int D>
struct Dma {
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int ROWB = 2 * D;               // bytes per row
  static constexpr int TILEB = kT2 * ROWB;         // bytes per K (or V) tile
  static constexpr int RPI = 1024 / ROWB;          // rows filled by one wave-wide 16-byte load
  static constexpr int IPW = TILEB / 1024 / kW2;   // such loads per wave per K (or V) tile
};

// Position of row r's 16-byte chunks: chunk c sits at c ^ swz(r).  The XOR masks are linear
// in the row bits and were chosen by measuring LDS bank conflicts (SQ_LDS_BANK_CONFLICT) of
// every read pattern these kernels use: 16 rows x 4 chunks per 16x16x32 MFMA operand (pass 2,
// decode), 32 rows x 2 chunks per 32x32x16 operand (pass 1), the transposed V reads of pass 1
// and of the decode, and whole-row reads (merge, cosine).  At D = 128 all of them are
// conflict-free; at D = 64 all but the whole-row reads.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    // row bits 0..3 -> masks 0xE, 0x8, 0xB, 0x4
    return ((r & 1) ? 0xE : 0) ^ ((r & 2) ? 0x8 : 0) ^ ((r & 4) ? 0xB : 0) ^ ((r & 8) ? 0x4 : 0);
  } else {
    return (r ^ ((r & 2) << 1)) & 7;
  }
}

// byte offset of 16-byte chunk c of row r inside a tile
template <int D>
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * (2 * D) + ((c ^ swz<D>(r)) << 4);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0): loads beyond the range
// return zeros.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4_t r;
  r.x = (uint32_t)a;
  r.y = (uint32_t)(a >> 32) & 0xffffu;
  r.z = bytes;
  r.w = 0x00020000u;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uint64_t>((const lds_u8*)p);
}

// Buffer loads written straight to LDS: lane i's 16 (or 4) bytes land at lds + 16 i (4 i).
// They are issued as inline assembly with no register results, so the compiler does not
// order them against unrelated LDS reads; the caller tracks completion with wait_vm.
__device__ __forceinline__ void dma16(const u32x4_t& rs, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(off), "s"(rs)
               : "memory", "m0");
}

__device__ __forceinline__ void dma4(const u32x4_t& rs, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(off), "s"(rs)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding (loads
// return in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until every LDS operation of this wave has completed (lgkmcnt 0; vmcnt and expcnt
// left at their maxima).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// x[l] + x[l ^ 16] and x[l] + x[l ^ 32] by lane swaps (no LDS round trip); both lanes of a
// pair add the same two values in the same order, so they hold identical bits.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace kvs
