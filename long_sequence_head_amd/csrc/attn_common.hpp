// Device helpers shared by the kernels (gfx950): vector types,
// LDS swizzles, the XCD-aware workgroup order, cross-half lane reductions,
// wait/barrier helpers and the LDS-DMA load. Header-only; every helper is
// inline and internal to the including translation unit.
#pragma once

#include "lsh_internal.hpp"

#include <cstdint>

namespace lsh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();

// 16-byte chunk swizzles inside a 256-byte (128 x bf16) LDS row.
__device__ __forceinline__ int swz_k(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int swz_v(int row, int c) {
  return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
}

// Workgroups are handed to the 8 XCDs round-robin; remap so that each XCD
// walks a contiguous range of work items (for attention, (b, h, query-block)
// items, so the K/V stream of a head is shared inside one XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int X = 8;
  const int per = n / X, rem = n % X;
  const int x = bid % X, k = bid / X;
  return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// Value of lane l^32 (the other half of the wavefront) for both halves:
// r[0] + r[1] / max(r[0], r[1]) combine the two halves.
__device__ __forceinline__ float pair_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// Item -> (b, h, query block) and the per-item key-tile list.
struct Item {
  int b, h, qblk;
};

__device__ __forceinline__ Item decode_item(int item, int n_qblk, int H) {
  Item it;
  it.qblk = item % n_qblk;
  const int bh = item / n_qblk;
  it.h = bh % H;
  it.b = bh / H;
  return it;
}

constexpr int kTileBytes = kBN * kD * 2;   // one 64 x 128 bf16 tile

// s_waitcnt with vmcnt = N (6 bits: [3:0] and [15:14]); expcnt and lgkmcnt
// left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer descriptor over [base, base + rec) bytes, stride 0: loads past rec
// return zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int rec) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = rec;
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(LDS_AS const unsigned char*)p;
}

// One 1-KiB load of a wavefront into LDS: lane l's 16 bytes at voffset land
// at LDS address lds + 16 l. Issued from inline asm so that the compiler does
// not track it: tracked, every control-flow join makes the compiler wait for
// all such loads in flight before the next LDS read. The kernels order their
// LDS reads after the data with an explicit s_waitcnt and a barrier.
__device__ __forceinline__ void lds_dma16(uint32_t lds, uint32_t voffset, const i32x4& rsrc) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0v), "v"(voffset), "s"(rsrc) : "memory");
}

// Transposing reads of a 64-row x 128-column bf16 tile whose rows are
// stored with swz_v. Fragment i = (kb * 2 + jj) * 4 + db is the A operand
// (32 columns x 16 rows) of a 32x32x16 MFMA: columns 32 db .. 32 db + 31,
// rows kb * 32 + jj * 16 + 0..15. Lane (16 g + 4 e + a) points at row
// 8 part + 4 (g / 2) + e of that 16-row group, columns 32 db + 16 (g % 2)
// + 4 a, and receives 4 rows of column 32 db + lane % 32 per read. Row
// 16 jj + 8 (i >> 2) + 4 hh + (i & 3) of the group lands in slot i of lane
// half hh: the order in which a 32x32 MFMA result holds its rows, so a
// result packed register by register is the matching B operand.
__device__ __forceinline__ void tr_offsets(int lane, uint32_t (&ofs)[2][4]) {
  const int tg = lane >> 4, te = (lane >> 2) & 3, ta = lane & 3;
#pragma unroll
  for (int part = 0; part < 2; ++part)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int row = 8 * part + 4 * (tg >> 1) + te;
      const int col = db * 32 + 16 * (tg & 1) + 4 * ta;
      ofs[part][db] = (uint32_t)(row * 256 + (swz_v(row, col >> 3) << 4) + (col & 7) * 2);
    }
}

__device__ __forceinline__ bf16x8 tr_read(const unsigned char* tile, const uint32_t (&ofs)[2][4],
                                          int i) {
  const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
  const LDS_AS unsigned char* b = (LDS_AS const unsigned char*)tile + (kb * 32 + jj * 16) * 256;
  const s16x4 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b + ofs[0][db]));
  const s16x4 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b + ofs[1][db]));
  const s16x8 w8 = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w8);
}

}  // namespace
}  // namespace lsh
