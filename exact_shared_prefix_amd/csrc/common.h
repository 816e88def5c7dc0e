// Internal definitions shared by the forward/backward kernels and the C ABI.
// gfx950 (CDNA4) only: wave64, bf16 MFMA 32x32x16, LDS tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <vector>

namespace dkv {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- problem --
// Host-side description of one packed micro-batch as a forest of segments in
// depth-first order: segment v is rows [start, start + len), and a row of v
// attends every key of v's proper ancestors plus the keys of v up to itself.
// One shared-prompt group is a root (the prompt) with one leaf per response;
// several groups are several such trees; deeper trees are multi-level shared
// prefixes. subtree_end = end of the last row of v's subtree.
struct Segment { int start = 0, len = 0, parent = -1, subtree_end = 0; };
struct Problem {
  int T = 0;          // packed tokens
  int Hq = 0, Hkv = 0, G = 0, d = 0;
  float scale = 0.f;  // softmax scale
  std::vector<Segment> segs;
};
constexpr int kMaxRegions = 4;   // key regions of a row: at most 3 ancestors + its own segment

// Forward work item: query rows [r0, r1) of one segment; its key regions are
// regions[reg_off .. reg_off + n_reg): the ancestors' whole segments, root
// first, then its own segment up to r1 (causal there).
struct FwdItem { int r0, r1, reg_off, n_reg; };
// Key region [k0, k1); blk = index of its first 32-key block in the
// transposed fragment layout (blocks are cut per segment, so every 64-key tile
// of a region starts on a block).
struct Region { int k0, k1, blk; };

// 32-key block of the transposed fragment layout: keys [key0, key0 + 32)
// clamped to [key0, kend) (kend = end of the block's region).
struct KeyBlock { int key0, kend; };

// Backward work item: keys [kb, ke) of one KV tile, query rows [r0, r1).
// Every row in [r0, r1) with row >= key attends the key (prompt keys are seen
// by all later rows, response keys only by their own response's later rows,
// and the scheduler never pairs a response tile with foreign rows).
struct BwdItem { int kb, ke, r0, r1; };

// Forward workgroup: kFwdWaves waves of 32 query rows.
constexpr int kFwdWaves = 8;
constexpr int kFwdRows = 32 * kFwdWaves;
// dK/dV workgroup: kBwdWaves waves of 32 keys each.
constexpr int kBwdWaves = 8;
constexpr int kBwdKeys = 32 * kBwdWaves;
// dQ workgroup: kDqWaves waves of 32 query rows; K / V tiles of kDqBlocks
// 32-key blocks.
constexpr int kDqWaves = 8;
constexpr int kDqBlocks = 2;
constexpr int kDqRows = 32 * kDqWaves;

// Launch-time block -> (item, head) decomposition that keeps each head group
// on one XCD (workgroups are dealt to the 8 XCDs round-robin by block id).
struct HeadMap { int n_items, H, mode; };

__host__ __device__ inline int headmap_grid(const HeadMap& m) {
  if (m.mode == 1) return m.n_items * m.H;
  if (m.mode == 2) { int rep = 8 / m.H; return ((m.n_items + rep - 1) / rep) * 8; }
  return m.n_items * m.H;
}

__host__ __device__ inline HeadMap make_headmap(int n_items, int H) {
  HeadMap m{n_items, H, 0};
  if (H % 8 == 0) m.mode = 1;
  else if (8 % H == 0) m.mode = 2;
  return m;
}

// returns false for padding blocks
__device__ inline bool headmap_decode(const HeadMap& m, int b, int& item, int& head) {
  if (m.mode == 1) {
    int hp = m.H >> 3, x = b & 7, s = b >> 3;
    head = x * hp + s % hp;
    item = s / hp;
  } else if (m.mode == 2) {
    int rep = 8 / m.H, x = b & 7, s = b >> 3;
    head = x % m.H;
    item = s * rep + x / m.H;
  } else {
    item = b / m.H;
    head = b % m.H;
  }
  return item < m.n_items;
}

// ----------------------------------------------------------------- device --
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32: A lane -> row l%16, k = 8 (l/16) + e; B lane -> column l%16, same
// k; D lane -> column l%16, rows 4 (l/16) + r.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

union Frag {
  bf16x8 v;
  uint4 u;
  uint2 h[2];
};

__device__ __forceinline__ bf16x8 lds_b128(const u16* p) {
  Frag f;
  f.u = *reinterpret_cast<const uint4*>(p);
  return f.v;
}

__device__ __forceinline__ bf16x8 lds_2xb64(const u16* p0, const u16* p1) {
  Frag f;
  f.h[0] = *reinterpret_cast<const uint2*>(p0);
  f.h[1] = *reinterpret_cast<const uint2*>(p1);
  return f.v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 x = {a, b};
  bf16x2 r = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  Frag f;
  f.u.x = pack_bf16x2(a0, a1);
  f.u.y = pack_bf16x2(a2, a3);
  f.u.z = pack_bf16x2(a4, a5);
  f.u.w = pack_bf16x2(a6, a7);
  return f.v;
}

__device__ __forceinline__ uint32_t u16_of(const uint4& v, int e) {
  uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Compiler-only fence: no instruction is scheduled across it. Used to issue a
// block of LDS operand reads before the MFMA chain that consumes them, so the
// reads' latency overlaps instead of each MFMA waiting on its own read.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Scheduling hint for the region that ends here: issue NR LDS reads first,
// then NM MFMAs (so the reads' latency overlaps and each MFMA waits only for
// its own operand).
template <int NR, int NM>
__device__ __forceinline__ void reads_then_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS reads
  __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // MFMA
}

// Scheduling hint for the region that ends here: a chain of NM MFMAs whose
// operands come from NR = RPM * NM LDS reads is issued with the reads DEPTH
// MFMAs ahead of their use (DEPTH * RPM reads first, then RPM reads after each
// MFMA), so each MFMA waits only for reads issued long before it.
template <int NM, int RPM, int DEPTH>
__device__ __forceinline__ void pipelined_mfma() {
  static_assert(DEPTH >= 1 && DEPTH <= NM, "depth");
  __builtin_amdgcn_sched_group_barrier(0x100, DEPTH * RPM, 0);
#pragma unroll
  for (int i = 0; i < NM - DEPTH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, DEPTH, 0);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then s_barrier; the memory clobber keeps the compiler from
// moving memory accesses across it. Unlike __syncthreads() it does not wait
// for outstanding global loads, direct-to-LDS loads or atomics; code that
// needs those complete waits for them explicitly first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max / sum of x over lanes l and l ^ 32. v_permlane32_swap exchanges the
// two 32-lane halves between its two operands; with x in both, the pair
// holds x(l) and x(l ^ 32) in some order on every lane.
__device__ __forceinline__ float wave_swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dkv
