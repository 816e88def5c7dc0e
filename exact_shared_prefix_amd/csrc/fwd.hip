// Forward kernel: shared-prompt attention over two KV regions in one launch.
//
// DualKV research-map summary (section Approach) and arXiv abstract: a tiled flash-attention forward
// whose query tile walks the shared prompt's KV region and then its own
// response's KV region, keeping one online-softmax state across both.
//
// gfx950 design:
//  * one workgroup = 8 waves x 32 query rows = 256 rows of one query head, all
//    in one segment (the prompt or one response);
//  * S^T = K Q^T on bf16 MFMA 32x32x16 with Q in registers: a lane owns one
//    query column, so the row max / row sum are lane-local plus one swap
//    between the wave halves;
//  * O^T += V^T P^T takes P^T straight from the S^T accumulator as its B
//    operand; the V^T A fragments are made once per call by a transpose pass
//    over V (xpose_kv_kernel) and copied like K;
//  * 64-key K and V^T tiles arrive by direct global -> LDS copies two steps
//    ahead, as fragment-native A operands (lane-linear 16-byte LDS reads);
//  * the two waves of a SIMD run one phase apart, so one issues its matrix
//    products while the other computes its softmax;
//  * scores are kept in the log2 domain (scale * log2 e folded in), exp2 on the
//    transcendental unit, against a reference that is only moved (with an O
//    rescale) when the exponentials outgrow 2^20: no per-tile row max in the
//    common case; LSE is written in natural log.
#include "common.h"
#include "frag.h"

namespace dkv {

// Transposed fragments of K or V: for every 32-key block b of the per-region
// block list and KV head g, the A operands X^T[d][key] of the 2 * D / 32
// (d tile, 16-key step) pairs, in the k-slot order of a P^T (dS^T) B operand:
// lane l = 32 hl + i holds d = 32 dt + i and, in slot e, key
// key0 + 16 ks + 8 (e / 4) + 4 hl + e % 4 (keys past the region end repeat
// its last key). Layout [block][g][dt][ks][64 lanes][8].
template <int D>
__global__ __launch_bounds__(256) void xpose_kv_kernel(const u16* __restrict__ src,
                                                       u16* __restrict__ dst,
                                                       const KeyBlock* __restrict__ blocks, int Hkv) {
  constexpr int NF = 2 * (D / 32);
  constexpr int LD = D + 8;   // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) u16 tile[32 * LD];
  const int b = blockIdx.x, g = blockIdx.y;
  const KeyBlock kb = blocks[b];
  const size_t krow = (size_t)Hkv * D;
  for (int x = threadIdx.x; x < 32 * (D / 8); x += 256) {
    const int r = x / (D / 8), c = x % (D / 8);
    const int key = min(kb.key0 + r, kb.kend - 1);
    *reinterpret_cast<uint4*>(tile + r * LD + 8 * c) =
        *reinterpret_cast<const uint4*>(src + (size_t)key * krow + (size_t)g * D + 8 * c);
  }
  __syncthreads();
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, hl = lane >> 5, i = lane & 31;
  for (int f = wv; f < NF; f += 4) {
    const int dt = f >> 1, ks = f & 1;
    u16 e8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e8[e] = tile[(16 * ks + 8 * (e >> 2) + 4 * hl + (e & 3)) * LD + 32 * dt + i];
    uint4 w4;
    w4.x = e8[0] | ((uint32_t)e8[1] << 16);
    w4.y = e8[2] | ((uint32_t)e8[3] << 16);
    w4.z = e8[4] | ((uint32_t)e8[5] << 16);
    w4.w = e8[6] | ((uint32_t)e8[7] << 16);
    *reinterpret_cast<uint4*>(dst + (((size_t)b * Hkv + g) * NF + f) * kFrag + 8 * lane) = w4;
  }
}

// ZERO_SCALE: the softmax scale is 0, so a masked score (-inf) times the scale
// is not -inf and masked probabilities are zeroed explicitly. NR: the most key
// regions any item has (2 for one prompt level, up to kMaxRegions).
template <int D, bool ZERO_SCALE, int NR>
__global__ __launch_bounds__(64 * kFwdWaves, 1) void fwd_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ vt,
    u16* __restrict__ o, float* __restrict__ lse, const FwdItem* __restrict__ items,
    const Region* __restrict__ regions, HeadMap hm, int T, int Hq, int Hkv,
    float c /* softmax scale * log2(e) */) {
  constexpr int NW = kFwdWaves;
  constexpr int BK = 64;          // keys per tile
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NTF = 2 * NKK;    // K (or V^T) fragments per tile
  constexpr int NL = NW / 2;      // leading waves; the other NL waves issue the copies
  constexpr int NC = NTF / NL;    // copies of each tensor per trailing wave and tile
  static_assert(NW == 8 && NTF % NL == 0, "copies per wave");
  __shared__ __attribute__((aligned(16))) u16 KA0[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 KA1[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 VT0[NTF * kFrag];   // V^T A fragments [kb2][dt][ks]
  __shared__ __attribute__((aligned(16))) u16 VT1[NTF * kFrag];

  int item_id, h;
  if (!headmap_decode(hm, blockIdx.x, item_id, h)) return;
  const FwdItem it = items[item_id];
  const int G = Hq / Hkv;
  const int g = h / G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
  // Waves w and w + 4 share a SIMD and run the same step sequence one phase
  // apart (the trailing wave passes one extra barrier first): while one runs
  // its matrix products the other runs its softmax.
  const bool lead = w < NL;
  const int hl = lane >> 5, l32 = lane & 31;
  const int t0 = it.r0 + 32 * w;   // first query row of this wave
  const int t = t0 + l32;          // this lane's query row
  const size_t qrow = (size_t)Hq * D, krow = (size_t)Hkv * D;

  // Q fragments: B operand of S^T = K Q^T (lane -> query column, 8 consecutive d)
  bf16x8 qf[NKK];
  {
    const u16* qp = q + (size_t)min(t, it.r1 - 1) * qrow + (size_t)h * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Frag a;
      a.u = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      qf[kk] = a.v;
    }
  }
  // complete the Q loads here, so that no wait for them lands inside the tile
  // loop (where it would also wait for the copies in flight)
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qf[kk]));

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  float m2 = -1e30f;  // running max of the log2-domain scores (reference point)
  float lsum = 0.f;   // this lane's partial row sum (its half of the keys)
  f32x16 s[2];        // S^T of the current tile: block kb2, register r <-> key kb + 32 kb2 + 8 (r/4) + 4 hl + r%4
  bf16x8 pf[2][2];    // P^T of the previous tile, B operands of O^T += V^T P^T

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
  const int n = tbeg[NR];
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

  // copies of tile i by the trailing waves (copy f = (w - NL) + NL j):
  // K: key block f / NKK, d chunk f % NKK, keys past the region end read its
  // last key; V^T: block f / (2 NDT) of the tile (clamped to the last block
  // the tile needs), fragment f % (2 NDT)
  auto copy_k = [&](int i, u16* dst) __attribute__((always_inline)) {
    int kb, ke;
    tile_bounds(i, kb, ke);
    const u16* base = k + (size_t)kb * krow + (size_t)g * D;
    // the buffer's LDS address, materialised here rather than kept live (as
    // one register per copy) across the loop
    uint32_t l0 = lds_addr(dst);
    asm volatile("" : "+s"(l0));
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int f = (w - NL) + NL * j;
      const int kb2 = f / NKK, kk = f % NKK;
      const uint32_t row = (uint32_t)min(32 * kb2 + l32, ke - 1 - kb);
      dma16sl(base, 2u * (row * (uint32_t)krow + 16 * kk + 8 * hl), l0 + 2u * f * kFrag);
    }
  };
  auto copy_vt = [&](int i, u16* dst) __attribute__((always_inline)) {
    int kb, ke, b0;
    tile_region(i, kb, ke, b0);
    const int blast = b0 + (ke - 1 - kb) / 32;
    uint32_t l0 = lds_addr(dst);
    asm volatile("" : "+s"(l0));
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int f = (w - NL) + NL * j;
      const int blk = min(b0 + f / (2 * NDT), blast);
      const u16* base = vt + ((size_t)blk * Hkv + g) * (2 * NDT * kFrag);
      dma16sl(base, 2u * ((f % (2 * NDT)) * kFrag + 8 * lane), l0 + 2u * f * kFrag);
    }
  };
  // products of step j: S^T of tile j, then O^T += V^T P^T of tile j - 1
  auto mfma_part = [&](int j, const u16* ka, const u16* vt_prev) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (j < n) {
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = mfma32(frag_ld(ka + (kb2 * NKK + kk) * kFrag, lane), qf[kk], s[kb2]);
      pipelined_mfma<2 * NKK, 1, 2>();
    }
    if (j > 0) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            oacc[dt] = mfma32(frag_ld(vt_prev + ((kb2 * NDT + dt) * 2 + ks) * kFrag, lane), pf[kb2][ks], oacc[dt]);
      pipelined_mfma<4 * NDT, 1, 2>();
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // softmax of step j: mask, running max, P^T = exp2(S^T c - m) (bf16)
  auto valu_part = [&](int j) __attribute__((always_inline)) {
    int kb, ke;
    tile_bounds(j, kb, ke);
    // masked scores become -inf and their exp2 exact zeros (also every score of
    // a tile that lies wholly after this wave's rows)
    const bool need_mask = (kb + BK > ke) || (kb + BK - 1 > t0);
    if (need_mask) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = kb + 32 * kb2 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (jj >= ke || jj > t) s[kb2][r] = -INFINITY;
        }
    }
    // P^T against the current reference m2 first; the reference only moves
    // (and O, l are rescaled) when some lane's sum leaves (0, 2^20] bounds, i.e.
    // a score exceeds m2 by about 20 (log2 units): the first tile, and rarely
    // later. O / l and the LSE do not depend on the reference.
    auto expo = [&]() __attribute__((always_inline)) {
      float ps = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[r] = fast_exp2(fmaf(s[kb2][r], c, -m2));
          if (ZERO_SCALE && need_mask && s[kb2][r] == -INFINITY) x[r] = 0.f;
          ps += x[r];
        }
        pack2(x, pf[kb2][0], pf[kb2][1]);
      }
      return ps;
    };
    float ps = expo();
    if (!__all(ps <= 1048576.f)) {   // > 2^20, inf or NaN in some lane
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
      mx = wave_swap32_max(mx);
      const float mnew = fmaxf(m2, mx * c);
      const float alpha = fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      ps = expo();
    }
    lsum += ps;
  };

  // Step j of a wave: phase M (products of step j) then phase S (softmax of
  // tile j). Phase M of a leading wave coincides with phase S of step j - 1 of
  // its trailing partner, and the other way round. The trailing waves copy
  // K(j + 2) and V^T(j + 1) during their phase S(j) and wait for them at the
  // barrier that ends their phase S(j + 1), which is where the leading waves
  // start phase M(j + 2) (K(j + 2) lands in the buffer K(j) used, V^T(j + 1)
  // in the one V^T(j - 1) used).
  auto step = [&](int j, u16* ka, u16* vt_prev) __attribute__((always_inline)) {
    lds_barrier();     // leading: K(j), V^T(j - 1) landed (the trailing waves waited for them)
    mfma_part(j, ka, vt_prev);
    vm_barrier<0>();   // trailing: copies issued in phase S(j - 1) landed
    if (!lead) {
      if (j + 2 < n) copy_k(j + 2, ka);
      if (j + 1 < n) copy_vt(j + 1, vt_prev);
    }
    if (j < n) valu_part(j);
  };

  if (!lead) {
    if (n > 0) copy_k(0, KA0);
    vm_barrier<0>();
    if (n > 1) copy_k(1, KA1);
    if (n > 0) copy_vt(0, VT0);
  }
  // steps 0 .. n (step n only finishes tile n - 1), two per iteration so that
  // every buffer is a static LDS address
  for (int j = 0; j <= n; j += 2) {
    step(j, KA0, VT1);
    if (j + 1 <= n) step(j + 1, KA1, VT0);
  }
  if (lead) lds_barrier();

  // O = O^T^T / l: lane -> query row t, register r -> d 32 dt + 8 (r/4) + 4 hl + r%4
  const float ltot = wave_swap32_sum(lsum);
  if (t < it.r1) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    u16* op = o + (size_t)t * qrow + (size_t)h * D + 4 * hl;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 w2;
        w2.x = pack_bf16x2(oacc[dt][4 * g4 + 0] * inv, oacc[dt][4 * g4 + 1] * inv);
        w2.y = pack_bf16x2(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * g4) = w2;
      }
    if (hl == 0)
      lse[(size_t)h * T + t] = ltot > 0.f ? (m2 + fast_log2(ltot)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_xpose_kv(const Problem& pb, const void* src, void* dst, const KeyBlock* blocks_dev,
                           int n_blocks, hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  dim3 grid(n_blocks, pb.Hkv), block(256);
  if (pb.d == 128)
    hipLaunchKernelGGL(xpose_kv_kernel<128>, grid, block, 0, stream, (const u16*)src, (u16*)dst,
                       blocks_dev, pb.Hkv);
  else
    hipLaunchKernelGGL(xpose_kv_kernel<64>, grid, block, 0, stream, (const u16*)src, (u16*)dst,
                       blocks_dev, pb.Hkv);
  return hipGetLastError();
}

hipError_t launch_fwd(const Problem& pb, const void* q, const void* k, const void* vt, void* o,
                      float* lse, const FwdItem* items_dev, const Region* regions_dev, int n_items,
                      int max_regions, hipStream_t stream) {
  if (n_items == 0) return hipSuccess;
  HeadMap hm = make_headmap(n_items, pb.Hq);
  dim3 grid(headmap_grid(hm)), block(64 * kFwdWaves);
  const float c = pb.scale * kLog2e;
  const bool z = c == 0.f, deep = max_regions > 2;
  auto kern = pb.d == 128 ? (deep ? (z ? fwd_kernel<128, true, kMaxRegions> : fwd_kernel<128, false, kMaxRegions>)
                                  : (z ? fwd_kernel<128, true, 2> : fwd_kernel<128, false, 2>))
                          : (deep ? (z ? fwd_kernel<64, true, kMaxRegions> : fwd_kernel<64, false, kMaxRegions>)
                                  : (z ? fwd_kernel<64, true, 2> : fwd_kernel<64, false, 2>));
  hipLaunchKernelGGL(kern, grid, block, 0, stream, (const u16*)q, (const u16*)k, (const u16*)vt,
                     (u16*)o, lse, items_dev, regions_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
  return hipGetLastError();
}

}  // namespace dkv
