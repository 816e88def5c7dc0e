// Forward kernel: shared-prompt attention over two KV regions in one launch.
//
// DualKV pages (p1 "Approach", p2 abstract): a tiled flash-attention forward
// whose query tile walks the shared prompt's KV region and then its own
// response's KV region, keeping one online-softmax state across both.
//
// gfx950 design:
//  * one workgroup = 8 waves x 32 query rows = 256 rows of one query head, all
//    in one segment (the prompt or one response); two waves per SIMD;
//  * S^T = K Q^T on bf16 MFMA 32x32x16 with Q in registers: a lane owns one
//    query column, so the row max / row sum are lane-local plus one swap
//    between the wave halves;
//  * O^T += V^T P^T takes P^T straight from the S^T accumulator as its B
//    operand; the V^T A fragments are made once per tile by MFMA transposes
//    (one 32 x 32 block per wave);
//  * 64-key K and V tiles arrive by direct global -> LDS copies one tile ahead,
//    as fragment-native A operands (lane-linear 16-byte LDS accesses only);
//  * scores are kept in the log2 domain (scale * log2 e folded in), exp2 on the
//    transcendental unit; the running max moves only when a row's max grows
//    by more than 2^8, so the O rescale is skipped in almost every tile; LSE
//    is written in natural log.
#include "common.h"
#include "frag.h"

namespace dkv {

template <int D>
__global__ __launch_bounds__(64 * kFwdWaves, 1) void fwd_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    u16* __restrict__ o, float* __restrict__ lse, const FwdItem* __restrict__ items,
    HeadMap hm, int T, int Hq, int Hkv, float c /* softmax scale * log2(e) */) {
  constexpr int NW = kFwdWaves;
  constexpr int BK = 64;          // keys per tile
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NTF = 2 * NKK;    // K (or V) fragments per tile: 2 key blocks x NKK
  constexpr int NJOB = 2 * NTF;   // copies per tile (K and V)
  static_assert(NJOB % NW == 0 && 2 * NDT <= NW, "copies and transposes per wave");
  __shared__ __attribute__((aligned(16))) u16 KA0[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 KA1[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 VA0[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 VA1[NTF * kFrag];
  __shared__ __attribute__((aligned(16))) u16 VT[2 * NDT * 2 * kFrag];   // V^T A fragments [kb2][dt][ks]

  int item_id, h;
  if (!headmap_decode(hm, blockIdx.x, item_id, h)) return;
  const FwdItem it = items[item_id];
  const int G = Hq / Hkv;
  const int g = h / G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
  const int hl = lane >> 5, l32 = lane & 31;
  const int t0 = it.r0 + 32 * w;   // first query row of this wave
  const int t = t0 + l32;          // this lane's query row
  const bool wave_rows = t0 < it.r1;
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

  const int nA = (it.a_end + BK - 1) / BK;
  const int nB = it.r1 > it.b_start ? (it.r1 - it.b_start + BK - 1) / BK : 0;
  const int ntiles = nA + nB;
  auto tile_bounds = [&](int i, int& kb, int& ke) {
    if (i < nA) { kb = i * BK; ke = it.a_end; }
    else { kb = it.b_start + (i - nA) * BK; ke = it.r1; }
  };
  // copies of tile i: job f = w, w + NW, ...: tensor f / NTF, key block
  // (f / NKK) % 2, d chunk f % NKK; keys past the region end read its last key
  auto stage = [&](int i, u16* ka, u16* va) {
    int kb, ke;
    tile_bounds(i, kb, ke);
#pragma unroll
    for (int j = 0; j < NJOB / NW; ++j) {
      const int f = w + NW * j;
      const int kb2 = (f / NKK) % 2, kk = f % NKK;
      const int key = min(kb + 32 * kb2 + l32, ke - 1);
      const u16* src = (f < NTF ? k : v) + (size_t)key * krow + (size_t)g * D + 16 * kk + 8 * hl;
      dma16(src, (f < NTF ? ka : va) + (f % NTF) * kFrag);
    }
  };

  auto tile = [&](int i, const u16* ka, const u16* va, u16* kan, u16* van) {
    int kb, ke;
    tile_bounds(i, kb, ke);
    vm_barrier<0>();   // tile i's copies landed; every wave is done with tile i - 1
    if (i + 1 < ntiles) stage(i + 1, kan, van);
    // V^T A fragments of (key block, d tile) pair w: lane -> d, k-slots in
    // accumulator key order
    if (w < 2 * NDT) {
      const int kb2 = w / NDT, dt = w % NDT;
      bf16x8 f0, f1;
      pack2(xpose_nat(frag_ld(va + (kb2 * NKK + 2 * dt) * kFrag, lane),
                      frag_ld(va + (kb2 * NKK + 2 * dt + 1) * kFrag, lane), lane),
            f0, f1);
      frag_st(VT + ((kb2 * NDT + dt) * 2) * kFrag, lane, f0);
      frag_st(VT + ((kb2 * NDT + dt) * 2 + 1) * kFrag, lane, f1);
    }
    lds_barrier();
    if (!wave_rows || kb > t0 + 31) return;   // every key of the tile lies after this wave's rows

    // S^T[key][query]: block kb2, register r <-> key kb + 32 kb2 + 8 (r/4) + 4 hl + r%4
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = mfma32(frag_ld(ka + (kb2 * NKK + kk) * kFrag, lane), qf[kk], s[kb2]);
    pipelined_mfma<2 * NKK, 1, 4>();

    // masked scores become -inf and their exp2 exact zeros
    const bool need_mask = (kb + BK > ke) || (kb + BK - 1 > t0);
    if (need_mask) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb + 32 * kb2 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (j >= ke || j > t) s[kb2][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
    mx = wave_swap32_max(mx);
    // lazy rescaling: the reference max only moves when some row's max exceeds
    // it by more than 8 (log2 units); O / l and the LSE do not depend on it
    if (__any(mx * c > m2 + 8.f)) {
      const float mnew = fmaxf(m2, mx * c);
      const float alpha = fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    }
    bf16x8 pf[2][2];
    float ps = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fast_exp2(fmaf(s[kb2][r], c, -m2));
        // explicit zero: with a softmax scale of 0, -inf * c is not -inf
        if (need_mask && s[kb2][r] == -INFINITY) x = 0.f;
        s[kb2][r] = x;
        ps += x;
      }
      pack2(s[kb2], pf[kb2][0], pf[kb2][1]);
    }
    lsum += ps;

    // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          oacc[dt] = mfma32(frag_ld(VT + ((kb2 * NDT + dt) * 2 + ks) * kFrag, lane), pf[kb2][ks], oacc[dt]);
    pipelined_mfma<4 * NDT, 1, 4>();
  };

  // The tile loop alternates between two statically distinct buffer sets.
  if (ntiles > 0) stage(0, KA0, VA0);
  for (int i = 0; i < ntiles; i += 2) {
    tile(i, KA0, VA0, KA1, VA1);
    if (i + 1 < ntiles) tile(i + 1, KA1, VA1, KA0, VA0);
  }

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

hipError_t launch_fwd(const Problem& pb, const void* q, const void* k, const void* v, void* o,
                      float* lse, const FwdItem* items_dev, int n_items, hipStream_t stream) {
  if (n_items == 0) return hipSuccess;
  HeadMap hm = make_headmap(n_items, pb.Hq);
  dim3 grid(headmap_grid(hm)), block(64 * kFwdWaves);
  const float c = pb.scale * kLog2e;
  if (pb.d == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, grid, block, 0, stream, (const u16*)q, (const u16*)k,
                       (const u16*)v, (u16*)o, lse, items_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, grid, block, 0, stream, (const u16*)q, (const u16*)k,
                       (const u16*)v, (u16*)o, lse, items_dev, hm, pb.T, pb.Hq, pb.Hkv, c);
  return hipGetLastError();
}

}  // namespace dkv
