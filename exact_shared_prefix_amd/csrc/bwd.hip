// Backward kernels for shared-prompt attention.
//
// "DualKV: Shared-Prompt Flash Attention for Efficient RL Training with Large
// Rollouts and Long Contexts" (research-map summary, section Approach): the
// backward walks the same two disjoint KV regions as the forward, and the
// shared prompt's key/value gradients are accumulated over all N sequences
// with fp32 atomics. Here:
//  1. pre_kernel:  D_t = sum_d dO_t * O_t (fp32), stored negated beside -LSE_t log2 e;
//                  zero_kernel clears the fp32 dK, dV accumulators.
//  2. dkv_kernel:  key-stationary dK, dV. A workgroup owns 256 keys of one KV
//                  head (8 waves x 32 keys) and walks the query rows that
//                  attend them in 32-row steps, for each of the G query heads
//                  of the group. A prompt tile's rows are every later row of
//                  the packed batch, cut into row chunks that spread over the
//                  chip; each chunk adds its partial dK, dV with fp32 atomics,
//                  which is where the N sequences' prompt gradients meet.
//     dq_kernel:   query-stationary dQ: a workgroup owns 256 query rows of one
//                  head and walks their two KV regions like the forward,
//                  recomputing S and dP; dQ is written once, without atomics
//                  (fp32 atomics run at a fixed rate per lane on this GPU, and
//                  a key-stationary dQ would need one per row, d and key tile).
//  3. convert_kernel: fp32 dK, dV -> bf16 (dK scaled by the softmax scale).
// Deterministic mode replaces the dK/dV atomics by per-item partials that
// reduce_kernel sums in a fixed order (the dQ kernel has no atomics at all),
// so the whole backward is bitwise reproducible.
#include "common.h"
#include "frag.h"

namespace dkv {

// ------------------------------------------------------------------ pre --
// One 16-lane group per (row, head): 16 lanes x 8 elements = 128 (d=64: 8 lanes).
// Writes rs[h][t] = {-LSE_t log2 e, -D_t}: the two per-row values both passes
// read, the LSE already in the base-2 form the exponentials use and D negated,
// the value the dP products' accumulators start from (they end as dP - D).
template <int D>
__global__ __launch_bounds__(256) void pre_kernel(const u16* __restrict__ o,
                                                  const u16* __restrict__ dO,
                                                  const float* __restrict__ lse,
                                                  float2* __restrict__ rs, int T, int Hq) {
  constexpr int LPR = D / 8;  // lanes per (row, head)
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rh = gid / LPR;   // row * Hq + head
  const int sub = (int)(gid % LPR);
  float acc = 0.f;
  const bool valid = rh < (long long)T * Hq;
  if (valid) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + rh * D + sub * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(dO + rh * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = __uint_as_float(u16_of(a, e) << 16);
      float y = __uint_as_float(u16_of(b, e) << 16);
      acc = fmaf(x, y, acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (valid && sub == 0) {
    const int t = (int)(rh / Hq), h = (int)(rh % Hq);
    const size_t i = (size_t)h * T + t;
    rs[i] = make_float2(-lse[i] * kLog2e, -acc);
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// -------------------------------------------------------------------- dKV --
// End of a dK/dV work item: wave w's 32 keys of dK, dV (accumulator layout:
// lane -> d column 32 dt + l % 32, register r -> key 8 (r/4) + 4 (l/32) + r%4).
// Atomic mode adds them to the fp32 accumulators (where the N sequences'
// prompt gradients meet; keys past the tile end add exact zeros to the tile's
// last key). Deterministic mode stores the item's partials
// ([item][g][key][d], dK then dV), summed in item order by reduce_kernel.
template <int D>
__device__ __forceinline__ void store_dkv(const f32x16* dkacc, const f32x16* dvacc,
                                          float* __restrict__ dk_acc, float* __restrict__ dv_acc,
                                          float* __restrict__ part, const BwdItem& it, int item_id,
                                          int g, int w, int lane, int Hkv) {
  constexpr int NDT = D / 32;
  const int hl = lane >> 5, l32 = lane & 31;
  if (part) {
    float* pk = part + ((size_t)item_id * Hkv + g) * (size_t)(2 * kBwdKeys * D) + 32 * w * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 8 * (r >> 2) + 4 * hl + (r & 3);
        pk[kl * D + 32 * dt + l32] = dkacc[dt][r];
        pk[(size_t)kBwdKeys * D + kl * D + 32 * dt + l32] = dvacc[dt][r];
      }
    return;
  }
  const int kw = it.kb + 32 * w;
  const size_t krow = (size_t)Hkv * D;
  if (kw < it.ke) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float* dkp = dk_acc + (size_t)g * D + 32 * dt + l32;
      float* dvp = dv_acc + (size_t)g * D + 32 * dt + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kw + 8 * (r >> 2) + 4 * hl + (r & 3);
        const size_t off = (size_t)min(kk, it.ke - 1) * krow;
        const bool ok = kk < it.ke;
        unsafeAtomicAdd(dkp + off, ok ? dkacc[dt][r] : 0.f);
        unsafeAtomicAdd(dvp + off, ok ? dvacc[dt][r] : 0.f);
      }
    }
  }
}

// Wave w owns keys kb + 32 w .. + 31: V fragments, half of the K fragments
// (d = 128) and the dK, dV accumulators in registers, the other K fragments in
// its own LDS slots. Per 32-row step (query rows
// qb.., head h):
//   S = Q K^T, P = exp2(S c - LSE log2 e), dP = dO V^T, dS = P (dP - D),
//   dV += P^T dO, dK += dS^T Q.
// The dP accumulator starts at -D rather than zero, so dS is one product.
// S and dP are computed with queries as rows, so a lane owns one key and the
// P / dS accumulators are directly the A operands of the dV / dK products.
// Q and dO arrive by direct copies one step ahead. For d = 128 they are
// swizzled row tiles, read as A fragments by 16-byte reads and as the B
// fragments of the dV, dK products by transposing reads; for d = 64 they are
// A-operand fragments and the Q^T, dO^T B fragments are made per step by MFMA
// transposes, one d tile per wave.
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves, 1) void dkv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dO, const float2* __restrict__ rs,
    float* __restrict__ dk_acc, float* __restrict__ dv_acc, float* __restrict__ part,
    const BwdItem* __restrict__ items, HeadMap hm, int T, int Hq, int Hkv, float c) {
  constexpr int NW = kBwdWaves;
  constexpr int BQ = 32;
  constexpr int NKK = D / 16;     // A fragments per 32-row block
  constexpr int NDT = D / 32;     // 32-wide d tiles
  static_assert(kBwdKeys == 32 * NW, "one 32-key block per wave");
  static_assert((2 * NKK) % NW == 0 && 2 * NDT <= NW, "copies and transposes per wave");
  constexpr bool kRow = D == 128;   // row tiles and transposing reads
  // One LDS block with the step buffers first: every read of a Q / dO tile is
  // then a per-lane base register plus an immediate offset below 64 KB.
  constexpr int TS = NKK * kFrag;             // u16 per Q or dO tile
  constexpr int XS = kRow ? 8 : NDT * 2 * kFrag;
  __shared__ __attribute__((aligned(16))) u16 smem[4 * TS + 2 * NW * 64 * 2 + NW * TS + 2 * XS];
  u16* const QA0 = smem;
  u16* const QA1 = smem + TS;
  u16* const OA0 = smem + 2 * TS;
  u16* const OA1 = smem + 3 * TS;
  float* const LD0 = reinterpret_cast<float*>(smem + 4 * TS);   // per wave: -LSE log2 e (32) | -D (32)
  float* const LD1 = LD0 + NW * 64;
  u16* const KF = reinterpret_cast<u16*>(LD1 + NW * 64);          // K B fragments per wave
  // Q^T, dO^T B fragments [dt][ks] (d = 64 only)
  u16* const QT = KF + NW * TS;
  u16* const OT = QT + XS;

  int item_id, g;
  if (!headmap_decode(hm, blockIdx.x, item_id, g)) return;
  const BwdItem it = items[item_id];
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
  const int hl = lane >> 5, l32 = lane & 31;
  const size_t qrow = (size_t)Hq * D, krow = (size_t)Hkv * D;
  const int kw = it.kb + 32 * w;   // first key of this wave
  const int key = kw + l32;        // this lane's key (S / dP column)
  const int nsteps = ((it.r1 - it.r0 + BQ - 1) / BQ) * G;

  // K, V fragments (lane -> key, 8 consecutive d); keys past the tile end
  // read the tile's last key and are masked out of P. V and the first NKR K
  // fragments stay in registers, the other K fragments in the wave's LDS slots
  // (for d = 128 all of K would not fit in the 256 VGPRs of a wave beside the
  // accumulators; for d = 64 it does).
  constexpr int NKR = kRow ? NKK / 2 : NKK;
  u16* kfl = KF + w * NKK * kFrag;
  bf16x8 vf[NKK];
  bf16x8 kf[NKR > 0 ? NKR : 1];
  {
    const int kc = min(key, it.ke - 1);
    const u16* kp = k + (size_t)kc * krow + (size_t)g * D + 8 * hl;
    const u16* vp = v + (size_t)kc * krow + (size_t)g * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Frag b;
      b.u = *reinterpret_cast<const uint4*>(vp + 16 * kk);
      vf[kk] = b.v;
      if (kk < NKR) {
        Frag a;
        a.u = *reinterpret_cast<const uint4*>(kp + 16 * kk);
        kf[kk < NKR ? kk : 0] = a.v;
      } else {
        dma16(kp + 16 * kk, kfl + kk * kFrag);
      }
    }
  }
  // complete the V, K loads here, so that no wait for them lands inside the
  // step loop (where it would also wait for the copies in flight)
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(vf[kk]));
#pragma unroll
  for (int kk = 0; kk < NKR; ++kk) asm volatile("" ::"v"(kf[kk]));

  f32x16 dkacc[NDT], dvacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) { dkacc[dt] = f32x16{}; dvacc[dt] = f32x16{}; }

  // Copies for step st: fragments f = w, w + NW, ... of [Q | dO], and this
  // wave's own copy of the 32 LSE and D values. Rows past the chunk end read
  // its last row; their P is masked to zero.
  auto stage = [&](int qb, int h, u16* qa, u16* oa, float* ld) {
    const int row = min(qb + l32, it.r1 - 1);
    const int lim = it.r1 - 1 - qb;   // last valid row of the step, relative to qb
    if constexpr (kRow) {
      // 1 KB copy f of [Q | dO]: rows 4 m .. 4 m + 3 of the row tile, m = f % NKK;
      // wave-uniform base (row qb, head h) plus a 32-bit per-lane byte offset
      const size_t base = (size_t)qb * qrow + (size_t)h * D;
#pragma unroll
      for (int j = 0; j < 2 * NKK / NW; ++j) {
        const int f = w + NW * j, m = f % NKK;
        const int r = 4 * m + (lane >> 4);
        const uint32_t chunk = (uint32_t)((lane & 15) ^ row_swz(r));
        const uint32_t voff = 2u * ((uint32_t)min(r, lim) * (uint32_t)qrow + 8u * chunk);
        if (f < NKK) dma16s(q + base, voff, qa + m * kFrag);
        else dma16s(dO + base, voff, oa + m * kFrag);
      }
    } else {
      const u16* qp = q + (size_t)row * qrow + (size_t)h * D + 8 * hl;
      const u16* op = dO + (size_t)row * qrow + (size_t)h * D + 8 * hl;
#pragma unroll
      for (int j = 0; j < 2 * NKK / NW; ++j) {
        const int f = w + NW * j;
        if (f < NKK) dma16(qp + 16 * f, qa + f * kFrag);
        else dma16(op + 16 * (f - NKK), oa + (f - NKK) * kFrag);
      }
    }
    // lane l < 32: -LSE log2 e of row qb + l; lane 32 + l: -D of that row
    dma4s(rs + (size_t)h * T + qb, 4u * (2u * (uint32_t)min(l32, lim) + (uint32_t)hl), ld + 64 * w);
  };
  const uint32_t abase = row_a_base(lane), bbase = row_b_base(lane);

  // step st covers rows qb .. qb + 31 of query head g G + st % G; (nq, nh) is
  // the row block and head of step st + 1, whose copies it issues
  auto step = [&](int st, int qb, int nq, int nh, const u16* qa, const u16* oa, const float* ld,
                  u16* qan, u16* oan, float* ldn) {
    vm_barrier<0>();   // this step's copies landed; every wave is done with the last step

    // Q^T (job < NDT) and dO^T B fragments of d tile job % NDT
    if (!kRow && w < 2 * NDT) {
      const int dt = w % NDT;
      const u16* src = w < NDT ? qa : oa;
      u16* dst = w < NDT ? QT : OT;
      bf16x8 f0, f1;
      pack2(xpose_nat(frag_ld(src + 2 * dt * kFrag, lane), frag_ld(src + (2 * dt + 1) * kFrag, lane), lane),
            f0, f1);
      frag_st(dst + (2 * dt) * kFrag, lane, f0);
      frag_st(dst + (2 * dt + 1) * kFrag, lane, f1);
    }

    // accumulator register r <-> query row qb + 8 (r/4) + 4 hl + r%4
    bf16x8 pf[2], sf[2];
    const bool active = kw < it.ke && kw <= qb + BQ - 1;
    if (active) {
      // -D of the step's rows (read before the S products, which hide its latency)
      f32x16 ndacc;
      {
        const float* lw = ld + 64 * w;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 d4 = *reinterpret_cast<const float4*>(lw + 32 + 8 * g4 + 4 * hl);
          ndacc[4 * g4 + 0] = d4.x;
          ndacc[4 * g4 + 1] = d4.y;
          ndacc[4 * g4 + 2] = d4.z;
          ndacc[4 * g4 + 3] = d4.w;
        }
      }
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sacc = mfma32(kRow ? row_ld_a(qa, abase ^ (32 * kk)) : frag_ld(qa + kk * kFrag, lane),
                      kk < NKR ? kf[kk < NKR ? kk : 0] : frag_ld(kfl + kk * kFrag, lane), sacc);
      pipelined_mfma<NKK, 2, 2>();
      const float* lw = ld + 64 * w;
      if ((kw + 31 > qb) || (kw + 32 > it.ke) || (qb + BQ > it.r1)) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(lw + 8 * g4 + 4 * hl);
          const float la[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = qb + 8 * g4 + 4 * hl + e;
            const float p = fast_exp2(fmaf(sacc[4 * g4 + e], c, la[e]));
            sacc[4 * g4 + e] = (key > row || key >= it.ke || row >= it.r1) ? 0.f : p;
          }
        }
      } else {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(lw + 8 * g4 + 4 * hl);
          const float la[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[4 * g4 + e] = fast_exp2(fmaf(sacc[4 * g4 + e], c, la[e]));
        }
      }
      pack2(sacc, pf[0], pf[1]);

      f32x16 dpacc = ndacc;   // starts at -D, ends as dP - D
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        dpacc = mfma32(kRow ? row_ld_a(oa, abase ^ (32 * kk)) : frag_ld(oa + kk * kFrag, lane), vf[kk], dpacc);
      pipelined_mfma<NKK, 1, 4>();
      if (st + 1 < nsteps) stage(nq, g * G + nh, qan, oan, ldn);
#pragma unroll
      for (int r = 0; r < 16; ++r) dpacc[r] = sacc[r] * dpacc[r];   // dS from the fp32 P
      pack2(dpacc, sf[0], sf[1]);
      // dS complete before the dV, dK products: with its registers free the
      // B-fragment reads of those products are issued an MFMA ahead (mixed
      // in with the dS arithmetic, each product waited for its own reads)
      sched_fence();
    }
    if (!active && st + 1 < nsteps) stage(nq, g * G + nh, qan, oan, ldn);

    if constexpr (kRow) {
      if (active) {
        // dV[key][d] += P^T dO, dK[key][d] += dS^T Q, B fragments by transposing reads
        auto bfrag = [&](const u16* tile, int dt, int ks) __attribute__((always_inline)) {
          return row_ld_b(tile, 4096 * ks + (bbase ^ (64 * dt)), 4096 * ks + 2048 + (bbase ^ (64 * dt + 32)));
        };
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) dvacc[dt] = mfma32(pf[ks], bfrag(oa, dt, ks), dvacc[dt]);
        pipelined_mfma<2 * NDT, 2, 2>();
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) dkacc[dt] = mfma32(sf[ks], bfrag(qa, dt, ks), dkacc[dt]);
        pipelined_mfma<2 * NDT, 2, 2>();
      }
      return;
    }
    lds_barrier();   // Q^T, dO^T fragments complete

    if (active) {
      // dV[key][d] += P^T dO, dK[key][d] += dS^T Q
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) dvacc[dt] = mfma32(pf[ks], frag_ld(OT + (2 * dt + ks) * kFrag, lane), dvacc[dt]);
      pipelined_mfma<2 * NDT, 1, 4>();
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) dkacc[dt] = mfma32(sf[ks], frag_ld(QT + (2 * dt + ks) * kFrag, lane), dkacc[dt]);
      pipelined_mfma<2 * NDT, 1, 4>();
    }
  };

  // The step loop alternates between two statically distinct buffer sets.
  // (cq, ch): row block and head offset of the current step, kept in scalar
  // registers and advanced head first
  int cq = it.r0, ch = 0;
  auto advance = [&](int& q_, int& h_) __attribute__((always_inline)) {
    if (++h_ == G) { h_ = 0; q_ += BQ; }
  };
  if (nsteps > 0) stage(cq, g * G, QA0, OA0, LD0);
  for (int st = 0; st < nsteps; st += 2) {
    int nq = cq, nh = ch;
    advance(nq, nh);
    step(st, cq, nq, nh, QA0, OA0, LD0, QA1, OA1, LD1);
    cq = nq; ch = nh;
    if (st + 1 < nsteps) {
      advance(nq, nh);
      step(st + 1, cq, nq, nh, QA1, OA1, LD1, QA0, OA0, LD0);
      cq = nq; ch = nh;
    }
  }

  store_dkv<D>(dkacc, dvacc, dk_acc, dv_acc, part, it, item_id, g, w, lane, Hkv);
}

// ------------------------------------------------------------- reduce --
// Deterministic mode: for key tile `tile` and KV head g, sum the partials of
// the tile's items in item order (fixed, so the result is bitwise
// reproducible) and write dK = bf16(scale * sum), dV = bf16(sum).
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(
    const float* __restrict__ part, const BwdItem* __restrict__ items,
    const int* __restrict__ tile_off, const int* __restrict__ tile_items, u16* __restrict__ dK,
    u16* __restrict__ dV, int Hkv, float scale) {
  const int tile = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int i0 = tile_off[tile], i1 = tile_off[tile + 1];
  if (i0 >= i1) return;
  const BwdItem first = items[tile_items[i0]];
  const int nkeys = first.ke - first.kb;
  const size_t krow = (size_t)Hkv * D;
  for (int idx = threadIdx.x; idx < nkeys * D / 4; idx += 256) {
    const int kl = (4 * idx) / D, dc = (4 * idx) % D;
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int i = i0; i < i1; ++i) {
      const float* pk = part + ((size_t)tile_items[i] * Hkv + g) * (size_t)(2 * kBwdKeys * D) + kl * D + dc;
      const float4 a = *reinterpret_cast<const float4*>(pk);
      const float4 b = *reinterpret_cast<const float4*>(pk + (size_t)kBwdKeys * D);
      sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
      sv.x += b.x; sv.y += b.y; sv.z += b.z; sv.w += b.w;
    }
    const size_t o = (size_t)(first.kb + kl) * krow + (size_t)g * D + dc;
    uint2 wk, wv;
    wk.x = pack_bf16x2(sk.x * scale, sk.y * scale);
    wk.y = pack_bf16x2(sk.z * scale, sk.w * scale);
    wv.x = pack_bf16x2(sv.x, sv.y);
    wv.y = pack_bf16x2(sv.z, sv.w);
    *reinterpret_cast<uint2*>(dK + o) = wk;
    *reinterpret_cast<uint2*>(dV + o) = wv;
  }
}

// --------------------------------------------------------------------- dQ --
// Query-stationary dQ. A workgroup (8 waves x 32 rows) owns 256 query rows of
// one head inside one segment and walks the same two KV regions as the
// forward: for each 64-key tile, S^T = K Q^T, P^T = exp2(S^T c - LSE log2 e),
// dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T. dQ stays in
// registers and is written once, so no atomics are needed. K and V tiles
// arrive by direct global -> LDS copies one tile ahead, V as A-operand
// fragments. For d = 128 each 32-key block of K is a swizzled row tile, read as
// the A fragments of S^T and, by transposing reads, as the K^T A fragments of
// the dQ product; for d = 64, K arrives as A fragments and K^T is made from
// them by MFMA transposes.

// NR: the most key regions any item has (2 for one prompt level, up to
// kMaxRegions).
template <int D, int NR>
__global__ __launch_bounds__(64 * kDqWaves, 1) void dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dO, const float2* __restrict__ rs,
    u16* __restrict__ dQ, const FwdItem* __restrict__ items, const Region* __restrict__ regions,
    HeadMap hm, int T, int Hq, int Hkv, float c, float scale) {
  constexpr int NW = kDqWaves;
  constexpr int NB = kDqBlocks;   // 32-key blocks per tile
  constexpr int BK = 32 * NB;     // keys per tile
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NTF = NB * NKK;   // K (or V) fragments per tile: NB key blocks x NKK
  constexpr int NJOB = 2 * NTF;   // copies per tile (K and V)
  static_assert(NJOB % NW == 0, "copies per wave");
  constexpr bool kRow = D == 128;   // K as row tiles, K^T by transposing reads
  __shared__ __attribute__((aligned(16))) u16 KA0[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 KA1[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 VA0[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 VA1[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 KT[kRow ? 8 : NB * NDT * 2 * kFrag];   // [kb2][dt][ks], d = 64

  int item_id, h;
  if (!headmap_decode(hm, blockIdx.x, item_id, h)) return;
  const FwdItem it = items[item_id];
  const int G = Hq / Hkv;
  const int g = h / G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
  const int hl = lane >> 5, l32 = lane & 31;
  const uint32_t abase = row_a_base(lane), bbase = row_b_base(lane);
  const int t0 = it.r0 + 32 * w;   // first query row of this wave
  const int t = t0 + l32;          // this lane's query row
  const int tc = min(t, it.r1 - 1);
  const bool wave_rows = t0 < it.r1;
  const size_t qrow = (size_t)Hq * D, krow = (size_t)Hkv * D;

  // Q, dO fragments: B operands (lane -> query column, 8 consecutive d)
  bf16x8 qf[NKK], of[NKK];
  {
    const u16* qp = q + (size_t)tc * qrow + (size_t)h * D + 8 * hl;
    const u16* op = dO + (size_t)tc * qrow + (size_t)h * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Frag a, b;
      a.u = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      b.u = *reinterpret_cast<const uint4*>(op + 16 * kk);
      qf[kk] = a.v;
      of[kk] = b.v;
    }
  }
  const float2 rst = rs[(size_t)h * T + tc];
  const float nlse2 = rst.x, ndv = rst.y;   // -LSE log2 e, -D
  // complete these loads before the tile loop (see the forward-copy waits)
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qf[kk]), "v"(of[kk]));
  asm volatile("" ::"v"(nlse2), "v"(ndv));
  f32x16 ndl;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl[r] = ndv;

  f32x16 dqacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dqacc[dt] = f32x16{};

  // key regions of the item (ancestor segments, then its own up to r1), kept in
  // scalar registers; tile i of the item is tile i - tbeg[x] of region x
  static_assert(NR >= 1 && NR <= kMaxRegions, "region count");
  int rk0[NR], rk1[NR], rblk[NR], tbeg[NR + 1];
  tbeg[0] = 0;
#pragma unroll
  for (int x = 0; x < NR; ++x) {
    const Region rg = x < it.n_reg ? regions[it.reg_off + x] : Region{0, 0, 0};
    rk0[x] = rg.k0;
    rk1[x] = rg.k1;
    rblk[x] = rg.blk;
    tbeg[x + 1] = tbeg[x] + (rg.k1 - rg.k0 + BK - 1) / BK;
  }
  const int ntiles = tbeg[NR];
  // tile i: keys [kb, ke) of its region (ke = region end), b0 = its first block
  auto tile_region = [&](int i, int& kb, int& ke, int& b0) __attribute__((always_inline)) {
    kb = 0; ke = 0; b0 = 0;
#pragma unroll
    for (int x = 0; x < NR; ++x)
      if (i >= tbeg[x] && i < tbeg[x + 1]) {
        kb = rk0[x] + (i - tbeg[x]) * BK;
        ke = rk1[x];
        b0 = rblk[x] + (i - tbeg[x]) * (BK / 32);
      }
  };
  auto tile_bounds = [&](int i, int& kb, int& ke) __attribute__((always_inline)) {
    int b0;
    tile_region(i, kb, ke, b0);
  };

  // copies of tile i: job f = w, w + NW, ...: tensor f / NTF, key block
  // (f / NKK) % NB, d chunk f % NKK; keys past the region end read its last key
  // (wave-uniform base at key kb, KV head g, plus a 32-bit per-lane byte offset)
  auto stage = [&](int i, u16* ka, u16* va) {
    int kb, ke;
    tile_bounds(i, kb, ke);
    const int lim = ke - 1 - kb;   // last key of the region, relative to kb
    const size_t base = (size_t)kb * krow + (size_t)g * D;
#pragma unroll
    for (int j = 0; j < NJOB / NW; ++j) {
      const int f = w + NW * j;
      const int kb2 = (f / NKK) % NB, kk = f % NKK;
      if (kRow && f < NTF) {
        // rows 4 kk .. 4 kk + 3 of K row tile kb2
        const int r = 4 * kk + (lane >> 4);
        const uint32_t chunk = (uint32_t)((lane & 15) ^ row_swz(r));
        const uint32_t voff = 2u * ((uint32_t)min(32 * kb2 + r, lim) * (uint32_t)krow + 8u * chunk);
        dma16s(k + base, voff, ka + f * kFrag);
      } else {
        const uint32_t voff =
            2u * ((uint32_t)min(32 * kb2 + l32, lim) * (uint32_t)krow + 16u * kk + 8u * hl);
        dma16s((f < NTF ? k : v) + base, voff, (f < NTF ? ka : va) + (f % NTF) * kFrag);
      }
    }
  };

  auto tile = [&](int i, const u16* ka, const u16* va, u16* kan, u16* van) {
    int kb, ke;
    tile_bounds(i, kb, ke);
    vm_barrier<0>();   // tile i's copies landed; every wave is done with tile i - 1
    if (i + 1 < ntiles) stage(i + 1, kan, van);
    // K^T A fragments (lane -> d, k-slots in accumulator key order)
#pragma unroll
    for (int p = w; !kRow && p < NB * NDT; p += NW) {
      const int kb2 = p / NDT, dt = p % NDT;
      bf16x8 f0, f1;
      pack2(xpose_nat(frag_ld(ka + (kb2 * NKK + 2 * dt) * kFrag, lane),
                      frag_ld(ka + (kb2 * NKK + 2 * dt + 1) * kFrag, lane), lane),
            f0, f1);
      frag_st(KT + ((kb2 * NDT + dt) * 2) * kFrag, lane, f0);
      frag_st(KT + ((kb2 * NDT + dt) * 2 + 1) * kFrag, lane, f1);
    }
    if (!kRow) lds_barrier();
    if (!wave_rows) return;
#pragma unroll
    for (int kb2 = 0; kb2 < NB; ++kb2) {
      const int k0 = kb + 32 * kb2;   // first key of this 32-key block
      if (k0 > t0 + 31 || k0 >= ke) continue;
      // S^T[key][query]: register r <-> key k0 + 8 (r/4) + 4 hl + r%4
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sacc = mfma32(kRow ? row_ld_a(ka + kb2 * NKK * kFrag, abase ^ (32 * kk))
                           : frag_ld(ka + (kb2 * NKK + kk) * kFrag, lane),
                      qf[kk], sacc);
      pipelined_mfma<NKK, 1, 4>();
      // dP^T does not depend on P: its products go first, so the exponentials
      // below overlap the end of the chain
      f32x16 dpacc = ndl;   // starts at -D, ends as dP^T - D
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) dpacc = mfma32(frag_ld(va + (kb2 * NKK + kk) * kFrag, lane), of[kk], dpacc);
      pipelined_mfma<NKK, 1, 4>();
      const bool need_mask = (k0 + 31 > t0) || (k0 + 32 > ke);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const float p = fast_exp2(fmaf(sacc[r], c, nlse2));
          sacc[r] = (key > t || key >= ke) ? 0.f : p;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], c, nlse2));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dpacc[r] = sacc[r] * dpacc[r];   // dS from the fp32 P
      bf16x8 sf[2];
      pack2(dpacc, sf[0], sf[1]);
      if constexpr (kRow) {
        const u16* kt = ka + kb2 * NKK * kFrag;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            dqacc[dt] = mfma32(row_ld_b(kt, 4096 * ks + (bbase ^ (64 * dt)), 4096 * ks + 2048 + (bbase ^ (64 * dt + 32))),
                               sf[ks], dqacc[dt]);
        pipelined_mfma<2 * NDT, 2, 2>();
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            dqacc[dt] = mfma32(frag_ld(KT + ((kb2 * NDT + dt) * 2 + ks) * kFrag, lane), sf[ks], dqacc[dt]);
        pipelined_mfma<2 * NDT, 1, 4>();
      }
    }
  };

  if (ntiles > 0) stage(0, KA0, VA0);
  for (int i = 0; i < ntiles; i += 2) {
    tile(i, KA0, VA0, KA1, VA1);
    if (i + 1 < ntiles) tile(i + 1, KA1, VA1, KA0, VA0);
  }

  // dQ = scale * dQ^T^T: lane -> query row t, register r -> d 32 dt + 8 (r/4) + 4 hl + r%4
  if (t < it.r1) {
    u16* dqp = dQ + (size_t)t * qrow + (size_t)h * D + 4 * hl;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 w2;
        w2.x = pack_bf16x2(dqacc[dt][4 * g4 + 0] * scale, dqacc[dt][4 * g4 + 1] * scale);
        w2.y = pack_bf16x2(dqacc[dt][4 * g4 + 2] * scale, dqacc[dt][4 * g4 + 3] * scale);
        *reinterpret_cast<uint2*>(dqp + 32 * dt + 8 * g4) = w2;
      }
  }
}

// --------------------------------------------------------------- convert --
// dQ = bf16(scale * dQacc), dK = bf16(scale * dKacc), dV = bf16(dVacc).
__global__ __launch_bounds__(256) void convert_kernel(const float4* __restrict__ src,
                                                      uint2* __restrict__ dst, size_t n4,
                                                      float mul) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const float4 x = src[i];
    uint2 r;
    r.x = pack_bf16x2(x.x * mul, x.y * mul);
    r.y = pack_bf16x2(x.z * mul, x.w * mul);
    dst[i] = r;
  }
}

static int stream_grid(size_t n4) {
  size_t b = (n4 + 255) / 256;
  return (int)(b < 8192 ? (b ? b : 1) : 8192);
}

hipError_t launch_bwd(const Problem& pb, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dQ, void* dK,
                      void* dV, const BwdItem* items_dev, int n_items, const FwdItem* qitems_dev,
                      const Region* qregions_dev, int n_qitems, int max_qregions, float2* rs, float* dk_acc, float* dv_acc, float* part,
                      const int* tile_off, const int* tile_items, int n_tiles, hipStream_t stream,
                      int phase_mask) {
  const size_t nk = (size_t)pb.T * pb.Hkv * pb.d;
  const float c = pb.scale * kLog2e;
  // 1. D and (atomic mode) zeroed dK / dV accumulators
  if (phase_mask & 1) {
    const long long lanes = (long long)pb.T * pb.Hq * (pb.d / 8);
    dim3 grid((unsigned)((lanes + 255) / 256));
    if (pb.d == 128)
      hipLaunchKernelGGL(pre_kernel<128>, grid, dim3(256), 0, stream, (const u16*)o,
                         (const u16*)dO, lse, rs, pb.T, pb.Hq);
    else
      hipLaunchKernelGGL(pre_kernel<64>, grid, dim3(256), 0, stream, (const u16*)o,
                         (const u16*)dO, lse, rs, pb.T, pb.Hq);
    if (!part) {
      hipLaunchKernelGGL(zero_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                         (float4*)dk_acc, nk / 4);
      hipLaunchKernelGGL(zero_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                         (float4*)dv_acc, nk / 4);
    }
  }
  // 2. dK / dV (key-stationary): atomics into the accumulators, or (part != null)
  //    per-item partials
  if ((phase_mask & 2) && n_items > 0) {
    HeadMap hm = make_headmap(n_items, pb.Hkv);
    dim3 grid(headmap_grid(hm)), block(64 * kBwdWaves);
    if (pb.d == 128)
      hipLaunchKernelGGL((dkv_kernel<128>), grid, block, 0, stream, (const u16*)q,
                         (const u16*)k, (const u16*)v, (const u16*)dO, rs, dk_acc, dv_acc,
                         part, items_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
    else
      hipLaunchKernelGGL((dkv_kernel<64>), grid, block, 0, stream, (const u16*)q,
                         (const u16*)k, (const u16*)v, (const u16*)dO, rs, dk_acc, dv_acc,
                         part, items_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
  }
  // 8. dQ (query-stationary), written directly as bf16
  if ((phase_mask & 8) && n_qitems > 0) {
    HeadMap hm = make_headmap(n_qitems, pb.Hq);
    dim3 grid(headmap_grid(hm)), block(64 * kDqWaves);
    const bool deep = max_qregions > 2;
    auto kern = pb.d == 128 ? (deep ? dq_kernel<128, kMaxRegions> : dq_kernel<128, 2>)
                            : (deep ? dq_kernel<64, kMaxRegions> : dq_kernel<64, 2>);
    hipLaunchKernelGGL(kern, grid, block, 0, stream, (const u16*)q, (const u16*)k, (const u16*)v,
                       (const u16*)dO, rs, (u16*)dQ, qitems_dev, qregions_dev, hm, pb.T, pb.Hq,
                       pb.Hkv, c, pb.scale);
  }
  // 4. dK, dV to bf16: convert the accumulators, or reduce the partials in order
  if (phase_mask & 4) {
    if (part) {
      if (n_tiles > 0) {
        dim3 grid((unsigned)(n_tiles * pb.Hkv));
        if (pb.d == 128)
          hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(256), 0, stream, part, items_dev,
                             tile_off, tile_items, (u16*)dK, (u16*)dV, pb.Hkv, pb.scale);
        else
          hipLaunchKernelGGL(reduce_kernel<64>, grid, dim3(256), 0, stream, part, items_dev,
                             tile_off, tile_items, (u16*)dK, (u16*)dV, pb.Hkv, pb.scale);
      }
    } else {
      hipLaunchKernelGGL(convert_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                         (const float4*)dk_acc, (uint2*)dK, nk / 4, pb.scale);
      hipLaunchKernelGGL(convert_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                         (const float4*)dv_acc, (uint2*)dV, nk / 4, 1.0f);
    }
  }
  return hipGetLastError();
}

}  // namespace dkv
