// Backward kernels for shared-prompt attention.
//
// DualKV pages (p1 "Approach"): the backward walks the same two disjoint KV
// regions as the forward and accumulates the shared prompt's key/value
// gradients over all N sequences with fp32 atomics. Here:
//  1. pre_kernel:  D_t = sum_d dO_t * O_t (fp32), and zero-fill of the fp32
//                  accumulators for dQ, dK, dV.
//  2. main_kernel: KV-stationary. A workgroup owns 128 keys of one KV head
//                  (4 waves x 32 keys, K and V fragments in registers) and
//                  walks a chunk of query rows in blocks of 32 rows, for each
//                  of the G query heads of the group:
//                    S = Q K^T, P = exp2(S c - LSE_2), dP = dO V^T,
//                    dS = P (dP - D), dV += P^T dO, dK += dS^T Q,
//                    dQ += dS K (fp32 atomics into the dQ accumulator).
//                  A prompt tile's rows are every later row of the packed
//                  batch, split into row chunks so the work spreads over the
//                  chip; partial dK/dV of every chunk are added with fp32
//                  atomics, which is where the N sequences' prompt gradients
//                  meet.
//  3. convert_kernel: fp32 accumulators -> bf16 (dQ, dK scaled by the softmax
//                  scale here once).
// MFMA orientation: S is computed with queries as rows, so a lane owns one key
// column and the S/dS accumulators serve directly as the A operand of
// dV = P^T dO and dK = dS^T Q. dS takes one trip through LDS for dQ = dS K.
#include "common.h"

namespace dkv {

// ------------------------------------------------------------------ pre --
// One 16-lane group per (row, head): 16 lanes x 8 elements = 128 (d=64: 8 lanes).
template <int D>
__global__ __launch_bounds__(256) void pre_kernel(const u16* __restrict__ o,
                                                  const u16* __restrict__ dO,
                                                  float* __restrict__ delta, int T, int Hq) {
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
    delta[(size_t)h * T + t] = acc;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ main --
// Column position of query q (0..31) inside a transposed Q/dO row: bits 2 and 3
// of q are swapped, so the eight queries one MFMA k-step takes from a lane
// half -- 16ks + 4hl + {0..3} and 16ks + 8 + 4hl + {0..3}, the order in which
// the S/dP accumulator holds them -- sit in eight consecutive columns and load
// as one 16-byte read.
__device__ __forceinline__ int qperm(int q) { return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1); }

// Transposed Q/dO block in LDS: row = d, 64 column positions in 8 blocks of 8
// (the 32 permuted queries occupy 4 of them) plus padding; the block index is
// XOR-ed with (row >> 4) & 7. Both the transposing 4-byte stores and the
// 16-byte MFMA operand reads then hit distinct banks.
constexpr int kTS = 72;

// MFMA operands read from LDS in blocks of this many 16-byte reads ahead of
// the products that use them.
#ifndef DKV_READ_AHEAD
#define DKV_READ_AHEAD 2
#endif
constexpr int kReadAhead = DKV_READ_AHEAD;
__device__ __forceinline__ int tpos(int row, int pos) {
  return row * kTS + ((((pos >> 3) ^ (row >> 4)) & 7) << 3) + (pos & 7);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void main_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq_acc, float* __restrict__ dk_acc, float* __restrict__ dv_acc,
    const BwdItem* __restrict__ items, HeadMap hm, int T, int Hq, int Hkv, float c) {
  constexpr int NT = 64 * NW;     // threads
  constexpr int BKW = 32 * NW;    // keys per workgroup, 32 per wave
  constexpr int BQ = 32;          // query rows per step
  constexpr int NDC = D / 8;      // 8-element chunks per row
  constexpr int RS = D + 8;       // Qs / dOs row stride
  constexpr int KTS = BKW + 8;    // Kt row stride (row = d, keys)
  constexpr int SS = BKW + 8;     // dSs row stride (row = query, keys)
  constexpr int NDQ = 2 * (D / 16) / NW;       // dQ 16x16 tiles per wave
  constexpr int UNITS = 2 * (BQ / 2) * NDC;    // (tensor, row pair, d chunk) staging units
  constexpr int UPT = (UNITS + NT - 1) / NT;   // units per thread
  static_assert((2 * (D / 16)) % NW == 0 && NDQ >= 1, "dQ tiles must divide evenly over the waves");
  static_assert(NW % 2 == 0, "dQ tiles of a wave share their query rows");
  static_assert((D / 16) % kReadAhead == 0 && kReadAhead % 2 == 0, "read-ahead depth");
  __shared__ __attribute__((aligned(16))) u16 Qs[BQ * RS];
  __shared__ __attribute__((aligned(16))) u16 dOs[BQ * RS];
  __shared__ __attribute__((aligned(16))) u16 QdOt[2][D * kTS];   // transposed [Q, dO]
  __shared__ __attribute__((aligned(16))) u16 Kt[D * KTS];
  __shared__ __attribute__((aligned(16))) u16 dSs[BQ * SS];
  __shared__ __attribute__((aligned(16))) f32x4 dq_stash[NDQ][NT];   // dQ of the previous step
  __shared__ __attribute__((aligned(16))) float lse2s[BQ];
  __shared__ __attribute__((aligned(16))) float dels[BQ];

  int item_id, g;
  if (!headmap_decode(hm, blockIdx.x, item_id, g)) return;
  const BwdItem it = items[item_id];
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int l16 = lane & 15, g16 = lane >> 4;
  const size_t qrow = (size_t)Hq * D, krow = (size_t)Hkv * D;
  const int kw = it.kb + 32 * w;          // first key of this wave
  const int key = kw + l32;               // this lane's key (S/dP column)
  const bool wave_keys = kw < it.ke;
  const int nqb = (it.r1 - it.r0 + BQ - 1) / BQ;
  const int nsteps = nqb * G;

  // K and V fragments: B operands of S = Q K^T and dP = dO V^T (lane -> key
  // column, 8 consecutive d). Keys past the tile end read the tile's last key:
  // they are masked out of P and dS, and their dK/dV are never written.
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int kc = min(key, it.ke - 1);
    const u16* kp = k + (size_t)kc * krow + (size_t)g * D + 8 * hl;
    const u16* vp = v + (size_t)kc * krow + (size_t)g * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      Frag a, b;
      a.u = *reinterpret_cast<const uint4*>(kp + 16 * kk);
      b.u = *reinterpret_cast<const uint4*>(vp + 16 * kk);
      kf[kk] = a.v;
      vf[kk] = b.v;
    }
  }
  // K^T of the workgroup's keys in LDS: B operand of dQ = dS K (row = d).
  for (int blk = tid; blk < (BKW / 4) * NDC; blk += NT) {
    const int kq = blk % (BKW / 4), dc = blk / (BKW / 4);
    uint4 r4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = min(it.kb + 4 * kq + j, it.ke - 1);
      r4[j] = *reinterpret_cast<const uint4*>(k + (size_t)kk * krow + (size_t)g * D + dc * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w2;
      w2.x = u16_of(r4[0], e) | (u16_of(r4[1], e) << 16);
      w2.y = u16_of(r4[2], e) | (u16_of(r4[3], e) << 16);
      *reinterpret_cast<uint2*>(Kt + (dc * 8 + e) * KTS + 4 * kq) = w2;
    }
  }
#pragma unroll
  for (int i = 0; i < NDQ; ++i) dq_stash[i][tid] = f32x4{};

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) { dkacc[i] = f32x16{}; dvacc[i] = f32x16{}; }

  // Staging of one step's Q and dO blocks through registers: unit u =
  // (tensor, row pair rp, d chunk dc), chunk fastest. Every memory operation
  // of the step loop is unconditional, so the compiler counts them statically
  // and never waits for a prefetch or an atomic early: rows past the chunk
  // end read the chunk's last row (their LSE becomes +inf when staged, which
  // zeroes their P and dS), the last step prefetches itself, and dQ atomics of
  // a row past the end add 0.
  uint4 sreg[UPT][2];
  float lreg, dreg;
  auto load_step = [&](int st) {
    const int qb = it.r0 + (st / G) * BQ, h = g * G + (st % G);
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = (tid + NT * j) % UNITS;
      const int tsr = u / ((BQ / 2) * NDC), rem = u % ((BQ / 2) * NDC), dc = rem % NDC, rp = rem / NDC;
      const u16* base = (tsr == 0 ? q : dO) + (size_t)h * D + dc * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = min(qb + 2 * rp + i, it.r1 - 1);
        sreg[j][i] = *reinterpret_cast<const uint4*>(base + (size_t)row * qrow);
      }
    }
    const int row = min(qb + (lane & (BQ - 1)), it.r1 - 1);
    lreg = lse[(size_t)h * T + row];
    dreg = delta[(size_t)h * T + row];
  };
  auto store_step = [&](int qb) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + NT * j;
      if (UNITS % NT == 0 || u < UNITS) {
        const int tsr = u / ((BQ / 2) * NDC), rem = u % ((BQ / 2) * NDC), dc = rem % NDC, rp = rem / NDC;
        u16* rowl = tsr == 0 ? Qs : dOs;
        *reinterpret_cast<uint4*>(rowl + (2 * rp) * RS + dc * 8) = sreg[j][0];
        *reinterpret_cast<uint4*>(rowl + (2 * rp + 1) * RS + dc * 8) = sreg[j][1];
        u16* trl = QdOt[tsr];
        const int col = qperm(2 * rp);  // 2rp and 2rp + 1 stay adjacent
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint32_t*>(trl + tpos(dc * 8 + e, col)) =
              u16_of(sreg[j][0], e) | (u16_of(sreg[j][1], e) << 16);
      }
    }
    if (tid < BQ) {
      lse2s[tid] = qb + tid < it.r1 ? lreg * kLog2e : INFINITY;
      dels[tid] = dreg;
    }
  };
  // dQ atomics of the previous step, from the LDS stash (each lane its own)
  int pend_qb = it.r0, pend_h = g * G;
  auto issue_dq = [&]() {
#pragma unroll
    for (int i = 0; i < NDQ; ++i) {
      const int t = w + NW * i;
      const int mt = t & 1, d0 = 16 * (t >> 1);
      const int row0 = pend_qb + 16 * mt + 4 * g16;
      const f32x4 a4 = dq_stash[i][tid];
      float* dqp = dq_acc + (size_t)pend_h * D + d0 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = row0 + r < it.r1;
        unsafeAtomicAdd(dqp + (size_t)min(row0 + r, it.r1 - 1) * qrow, ok ? a4[r] : 0.f);
      }
    }
  };

  load_step(0);
  for (int st = 0; st < nsteps; ++st) {
    const int qb = it.r0 + (st / G) * BQ, h = g * G + (st % G);
    lds_barrier();   // previous step finished with the staged blocks and dSs
    store_step(qb);
    lds_barrier();
    issue_dq();

    u16* sp = dSs + 32 * w + l32;
    if (wave_keys && kw <= qb + BQ - 1) {
      // element r: query row qb + 8 (r/4) + 4 hl + r%4, key column `key`
      const bool need_mask = (kw + 31 > qb) || (kw + 32 > it.ke);
      bf16x8 pf0, pf1, sf0, sf1;
      {
        const u16* qp = Qs + l32 * RS + 8 * hl;
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int k0 = 0; k0 < D / 16; k0 += kReadAhead) {
          bf16x8 xa[kReadAhead];
#pragma unroll
          for (int kk = 0; kk < kReadAhead; ++kk) xa[kk] = lds_b128(qp + 16 * (k0 + kk));
#pragma unroll
          for (int kk = 0; kk < kReadAhead; ++kk) sacc = mfma32(xa[kk], kf[k0 + kk], sacc);
          reads_then_mfma<kReadAhead, kReadAhead>();
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(lse2s + 8 * g4 + 4 * hl);
          const float la[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float x = fast_exp2(fmaf(sacc[r], c, -la[e]));
            if (need_mask) {
              const int row = qb + 8 * g4 + 4 * hl + e;
              if (key > row || key >= it.ke) x = 0.f;
            }
            sacc[r] = x;
          }
        }
        pf0 = pack_bf16x8(sacc[0], sacc[1], sacc[2], sacc[3], sacc[4], sacc[5], sacc[6], sacc[7]);
        pf1 = pack_bf16x8(sacc[8], sacc[9], sacc[10], sacc[11], sacc[12], sacc[13], sacc[14], sacc[15]);
      }
      {
        // dS = P (dP - D), with P as the bf16 value the dV product consumes
        const u16* op = dOs + l32 * RS + 8 * hl;
        f32x16 dpacc = f32x16{};
#pragma unroll
        for (int k0 = 0; k0 < D / 16; k0 += kReadAhead) {
          bf16x8 xa[kReadAhead];
#pragma unroll
          for (int kk = 0; kk < kReadAhead; ++kk) xa[kk] = lds_b128(op + 16 * (k0 + kk));
#pragma unroll
          for (int kk = 0; kk < kReadAhead; ++kk) dpacc = mfma32(xa[kk], vf[k0 + kk], dpacc);
          reads_then_mfma<kReadAhead, kReadAhead>();
        }
        const Frag fp0{pf0}, fp1{pf1};
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 d4 = *reinterpret_cast<const float4*>(dels + 8 * g4 + 4 * hl);
          const float da[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            const uint32_t word = r < 8 ? (r < 2 ? fp0.u.x : r < 4 ? fp0.u.y : r < 6 ? fp0.u.z : fp0.u.w)
                                        : (r < 10 ? fp1.u.x : r < 12 ? fp1.u.y : r < 14 ? fp1.u.z : fp1.u.w);
            const float pr = __uint_as_float((r & 1) ? (word & 0xffff0000u) : (word << 16));
            dpacc[r] = pr * (dpacc[r] - da[e]);
          }
        }
        sf0 = pack_bf16x8(dpacc[0], dpacc[1], dpacc[2], dpacc[3], dpacc[4], dpacc[5], dpacc[6], dpacc[7]);
        sf1 = pack_bf16x8(dpacc[8], dpacc[9], dpacc[10], dpacc[11], dpacc[12], dpacc[13], dpacc[14], dpacc[15]);
      }
      // dV[key][d] += P^T dO and dK[key][d] += dS^T Q: B operands are one
      // 16-byte read of the column-permuted transposed blocks.
#pragma unroll
      for (int d0 = 0; d0 < D / 32; d0 += kReadAhead / 2) {
        bf16x8 tb[kReadAhead];
#pragma unroll
        for (int j = 0; j < kReadAhead / 2; ++j) {
          tb[2 * j] = lds_b128(QdOt[1] + tpos(32 * (d0 + j) + l32, 8 * hl));
          tb[2 * j + 1] = lds_b128(QdOt[1] + tpos(32 * (d0 + j) + l32, 16 + 8 * hl));
        }
#pragma unroll
        for (int j = 0; j < kReadAhead / 2; ++j) {
          dvacc[d0 + j] = mfma32(pf0, tb[2 * j], dvacc[d0 + j]);
          dvacc[d0 + j] = mfma32(pf1, tb[2 * j + 1], dvacc[d0 + j]);
        }
        reads_then_mfma<kReadAhead, kReadAhead>();
      }
#pragma unroll
      for (int d0 = 0; d0 < D / 32; d0 += kReadAhead / 2) {
        bf16x8 tb[kReadAhead];
#pragma unroll
        for (int j = 0; j < kReadAhead / 2; ++j) {
          tb[2 * j] = lds_b128(QdOt[0] + tpos(32 * (d0 + j) + l32, 8 * hl));
          tb[2 * j + 1] = lds_b128(QdOt[0] + tpos(32 * (d0 + j) + l32, 16 + 8 * hl));
        }
#pragma unroll
        for (int j = 0; j < kReadAhead / 2; ++j) {
          dkacc[d0 + j] = mfma32(sf0, tb[2 * j], dkacc[d0 + j]);
          dkacc[d0 + j] = mfma32(sf1, tb[2 * j + 1], dkacc[d0 + j]);
        }
        reads_then_mfma<kReadAhead, kReadAhead>();
      }
      // prefetch the next step's blocks (their registers stay live only
      // through the dQ phase), then dS (bf16) into LDS as [query][key]
      load_step(min(st + 1, nsteps - 1));
      const Frag f0{sf0}, f1{sf1};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t word = r < 8 ? (r < 2 ? f0.u.x : r < 4 ? f0.u.y : r < 6 ? f0.u.z : f0.u.w)
                                    : (r < 10 ? f1.u.x : r < 12 ? f1.u.y : r < 14 ? f1.u.z : f1.u.w);
        sp[(8 * (r >> 2) + 4 * hl + (r & 3)) * SS] = (r & 1) ? (u16)(word >> 16) : (u16)(word & 0xffffu);
      }
    } else {
      // this wave's keys all come after the block's rows (or past the tile): dS = 0
      load_step(min(st + 1, nsteps - 1));
#pragma unroll
      for (int r = 0; r < 16; ++r) sp[(8 * (r >> 2) + 4 * hl + (r & 3)) * SS] = 0;
    }
    lds_barrier();   // dSs complete
    // dQ[q][d] += dS[q][key] K[key][d] over all BKW keys of the workgroup, on
    // 16x16x32 tiles: the 2 x D/16 (query, d) tiles are dealt to the waves, and
    // all tiles of a wave share their query rows (t = w + NW i keeps t & 1).
    {
      const u16* ap = dSs + (16 * (w & 1) + l16) * SS + 8 * g16;
      bf16x8 da[BKW / 32];
#pragma unroll
      for (int ks = 0; ks < BKW / 32; ++ks) da[ks] = lds_b128(ap + 32 * ks);
#pragma unroll
      for (int i = 0; i < NDQ; ++i) {
        const u16* bp = Kt + (16 * ((w + NW * i) >> 1) + l16) * KTS + 8 * g16;
        bf16x8 db[BKW / 32];
#pragma unroll
        for (int ks = 0; ks < BKW / 32; ++ks) db[ks] = lds_b128(bp + 32 * ks);
        f32x4 a4 = f32x4{};
#pragma unroll
        for (int ks = 0; ks < BKW / 32; ++ks) a4 = mfma16(da[ks], db[ks], a4);
        dq_stash[i][tid] = a4;
      }
    }
    pend_qb = qb;
    pend_h = h;
  }
  issue_dq();

  // partial dK / dV of this chunk: fp32 atomics (the cross-sequence prompt
  // sum); keys past the tile end hold exact zeros and add them to the last key
  if (wave_keys) {
    float* dkp = dk_acc + (size_t)g * D + l32;
    float* dvp = dv_acc + (size_t)g * D + l32;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kw + 8 * (r >> 2) + 4 * hl + (r & 3);
        const size_t off = (size_t)min(kk, it.ke - 1) * krow + 32 * dt;
        const bool ok = kk < it.ke;
        unsafeAtomicAdd(dkp + off, ok ? dkacc[dt][r] : 0.f);
        unsafeAtomicAdd(dvp + off, ok ? dvacc[dt][r] : 0.f);
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
                      void* dV, const BwdItem* items_dev, int n_items, float* delta,
                      float* dq_acc, float* dk_acc, float* dv_acc, hipStream_t stream,
                      int phase_mask) {
  const size_t nq = (size_t)pb.T * pb.Hq * pb.d, nk = (size_t)pb.T * pb.Hkv * pb.d;
  // 1. D and zeroed accumulators
  if (phase_mask & 1) {
    const long long lanes = (long long)pb.T * pb.Hq * (pb.d / 8);
    dim3 grid((unsigned)((lanes + 255) / 256));
    if (pb.d == 128)
      hipLaunchKernelGGL(pre_kernel<128>, grid, dim3(256), 0, stream, (const u16*)o,
                         (const u16*)dO, delta, pb.T, pb.Hq);
    else
      hipLaunchKernelGGL(pre_kernel<64>, grid, dim3(256), 0, stream, (const u16*)o,
                         (const u16*)dO, delta, pb.T, pb.Hq);
    hipLaunchKernelGGL(zero_kernel, dim3(stream_grid(nq / 4)), dim3(256), 0, stream,
                       (float4*)dq_acc, nq / 4);
    hipLaunchKernelGGL(zero_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                       (float4*)dk_acc, nk / 4);
    hipLaunchKernelGGL(zero_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                       (float4*)dv_acc, nk / 4);
  }
  // 2. main
  if ((phase_mask & 2) && n_items > 0) {
    HeadMap hm = make_headmap(n_items, pb.Hkv);
    dim3 grid(headmap_grid(hm)), block(64 * kBwdWaves);
    const float c = pb.scale * kLog2e;
    if (pb.d == 128)
      hipLaunchKernelGGL((main_kernel<128, kBwdWaves>), grid, block, 0, stream, (const u16*)q,
                         (const u16*)k, (const u16*)v, (const u16*)dO, lse, delta, dq_acc,
                         dk_acc, dv_acc, items_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
    else
      hipLaunchKernelGGL((main_kernel<64, kBwdWaves>), grid, block, 0, stream, (const u16*)q,
                         (const u16*)k, (const u16*)v, (const u16*)dO, lse, delta, dq_acc,
                         dk_acc, dv_acc, items_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
  }
  // 3. convert
  if (phase_mask & 4) {
    hipLaunchKernelGGL(convert_kernel, dim3(stream_grid(nq / 4)), dim3(256), 0, stream,
                       (const float4*)dq_acc, (uint2*)dQ, nq / 4, pb.scale);
    hipLaunchKernelGGL(convert_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                       (const float4*)dk_acc, (uint2*)dK, nk / 4, pb.scale);
    hipLaunchKernelGGL(convert_kernel, dim3(stream_grid(nk / 4)), dim3(256), 0, stream,
                       (const float4*)dv_acc, (uint2*)dV, nk / 4, 1.0f);
  }
  return hipGetLastError();
}

}  // namespace dkv
