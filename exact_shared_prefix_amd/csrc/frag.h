// MFMA operand fragments in LDS, direct global -> LDS copies and exact
// MFMA transposes, shared by the forward and backward kernels (gfx950).
//
// MFMA operands staged in LDS are kept "fragment-native": one operand of a
// wave (64 lanes x 8 bf16) is 1 KB with lane l's 16 bytes at byte 16 l, so
// every fragment read or write is one lane-linear 16-byte access. Operands
// needed transposed (Q^T, dO^T for dV, dK; K^T for dQ) are produced by an
// MFMA against a unit fragment, which moves a 32 x 32 block into accumulator
// layout exactly (one nonzero product per element).
#pragma once

#include "common.h"

namespace dkv {

constexpr int kFrag = 512;  // u16 elements per fragment

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_void;

// Direct global -> LDS copy of 16 (4) bytes per lane: lane l's bytes land at
// lds_base + 16 l (4 l); lds_base is the same for the whole wave. Written as
// inline assembly so that the compiler does not treat every later LDS read
// as possibly overwritten by the copy (it would wait for all outstanding
// memory operations before each one); the kernel waits for the copies itself.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  // the low 32 bits of a generic pointer into LDS are its LDS address (the
  // shared aperture's base has zero low bits); no null-pointer check needed
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}
// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m)
               : "memory", "m0");
}
// Same as dma16s with the LDS destination given as an LDS byte address.
__device__ __forceinline__ void dma16sl(const void* base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t voff, void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(m)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

__device__ __forceinline__ bf16x8 frag_ld(const u16* f, int lane) { return lds_b128(f + 8 * lane); }
__device__ __forceinline__ void frag_st(u16* f, int lane, bf16x8 v) {
  Frag x{v};
  *reinterpret_cast<uint4*>(f + 8 * lane) = x.u;
}

// B operand holding a single 1.0 at k-slot e_on (0..7) for lanes with on set.
// Used as the right factor of an MFMA that copies its left operand into the
// accumulator layout, i.e. transposes a fragment exactly.
__device__ __forceinline__ bf16x8 unit_frag(bool on, int e_on) {
  const uint32_t one = 0x3f80u << (16 * (e_on & 1));
  const int wsel = e_on >> 1;
  Frag f;
  f.u.x = (on && wsel == 0) ? one : 0u;
  f.u.y = (on && wsel == 1) ? one : 0u;
  f.u.z = (on && wsel == 2) ? one : 0u;
  f.u.w = (on && wsel == 3) ? one : 0u;
  return f.v;
}

// k-slot e of lane half hl in a P / dS fragment (and in every operand that is
// paired with one) stands for query row 8 (e / 4) + 4 hl + e % 4 of its
// 16-row step: the row order of the 32x32 accumulator.
//
// Transpose of a 32 x 32 block X held as two A-operand fragments (k = columns
// 0..15 and 16..31 in natural order): returns X in accumulator layout (lane ->
// column, register r -> row 8 (r/4) + 4 hl + r%4).
__device__ __forceinline__ f32x16 xpose_nat(bf16x8 a0, bf16x8 a1, int lane) {
  asm volatile("" : "+v"(lane));
  const int n = lane & 31, hl = lane >> 5;
  const bool mine = hl == ((n >> 3) & 1);
  f32x16 d = mfma32(a0, unit_frag(mine && (n >> 4) == 0, n & 7), f32x16{});
  return mfma32(a1, unit_frag(mine && (n >> 4) == 1, n & 7), d);
}
__device__ __forceinline__ void pack2(const f32x16& x, bf16x8& f0, bf16x8& f1) {
  f0 = pack_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
  f1 = pack_bf16x8(x[8], x[9], x[10], x[11], x[12], x[13], x[14], x[15]);
}

// Row-major 32 x 128 bf16 tiles with an XOR swizzle ("row tiles"). Row r is
// 256 bytes; its 16-byte chunk c sits at chunk position c ^ row_swz(r). The
// swizzle makes both ways a tile is read free of LDS bank conflicts: A
// fragments (lane -> row l % 32, 8 consecutive columns) by 16-byte reads, and
// B fragments with k running over rows (lane -> column, 8 rows) by the
// transposing 8-byte read, which gives lane i of each 16-lane group, in slot j,
// element i % 4 of the 4 elements addressed by lane i / 4 + 4 j of its group.
// A tile is copied by 8 direct copies of 1 KB (4 rows each), lane l of copy m
// fetching row 4 m + l / 16, chunk (l % 16) ^ row_swz(4 m + l / 16).
__device__ __forceinline__ int row_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Byte offsets of this lane's reads: A fragment kk of a tile is at
// row_a_base(lane) ^ (32 kk); the B fragment (d tile dt, 16-row step ks) is
// the pair of transposing reads at 4096 ks + 2048 h + (row_b_base(lane) ^
// (64 dt + 32 h)), h = 0, 1, holding rows 16 ks + 8 h + 4 (lane / 32) + 0..3.
__device__ __forceinline__ uint32_t row_a_base(int lane) {
  const int r = lane & 31, hl = lane >> 5;
  return 256 * r + 16 * (row_swz(r) ^ hl);
}
__device__ __forceinline__ uint32_t row_b_base(int lane) {
  const int g = lane >> 4, L = lane & 15, a = L & 3, j = L >> 2, hl = g >> 1, x = g & 1;
  return 1024 * hl + 320 * j + 8 * (a & 1) + 16 * ((2 * x + (a >> 1)) ^ hl);
}
__device__ __forceinline__ bf16x8 row_ld_a(const u16* tile, uint32_t off) {
  return lds_b128(reinterpret_cast<const u16*>(reinterpret_cast<const char*>(tile) + off));
}
typedef short tr4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 row_ld_b(const u16* tile, uint32_t off0, uint32_t off1) {
  typedef __attribute__((address_space(3))) tr4_t lds_tr4;
  char* t = const_cast<char*>(reinterpret_cast<const char*>(tile));
  const tr4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4*)(t + off0));
  const tr4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4*)(t + off1));
  Frag f;
  f.h[0] = __builtin_bit_cast(uint2, x0);
  f.h[1] = __builtin_bit_cast(uint2, x1);
  return f.v;
}

// Wait until at most N vector-memory operations of this wave (the direct
// copies above included) are outstanding, then an LDS barrier.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace dkv
