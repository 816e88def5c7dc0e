// Forward kernel: shared-prompt attention over two KV regions in one launch.
//
// DualKV pages (p1 "Approach", p2 abstract): a tiled flash-attention forward
// whose query tile walks the shared prompt's KV region and then its own
// response's KV region, keeping one online-softmax state across both.
//
// gfx950 design:
//  * one workgroup = 4 waves = 128 query rows of one query head, all rows of a
//    tile in one segment (prompt or one response);
//  * S^T = K Q^T on bf16 MFMA 32x32x16: a lane owns one query column, so the
//    row max / row sum are lane-local plus one swap between wave halves;
//  * O^T += V^T P^T reuses the S^T accumulator layout directly as the B
//    operand (no LDS round trip for P); V is staged transposed in LDS;
//  * K/V tiles of 64 keys go global -> registers -> LDS with the next tile's
//    global loads in flight during the current tile's math;
//  * scores are kept in the log2 domain (scale * log2 e folded in), exp2 on
//    the hardware transcendental unit; LSE is written in natural log.
#include "common.h"

namespace dkv {

// Column position of key j (0..63) in a V^T tile row: bits 2 and 3 of j are
// swapped, so the eight keys one MFMA k-step takes from a lane half (16 ks +
// 4 hl + {0..3} and 16 ks + 8 + 4 hl + {0..3}) are eight consecutive columns.
__device__ __forceinline__ int kperm(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    u16* __restrict__ o, float* __restrict__ lse, const FwdItem* __restrict__ items,
    HeadMap hm, int T, int Hq, int Hkv, float c /* softmax scale * log2(e) */) {
  constexpr int BK = 64;        // keys per LDS tile
  constexpr int KS = D + 8;     // K tile row stride (elements), padded against bank conflicts
  constexpr int VS = BK + 8;    // V^T tile row stride (16-byte aligned rows)
  constexpr int KLD = BK * D / 8 / 256;  // 16-byte K loads per thread per tile
  constexpr int NDC = D / 8;    // 8-element chunks per row
  __shared__ __attribute__((aligned(16))) u16 Ks[BK * KS];
  __shared__ __attribute__((aligned(16))) u16 Vt[D * VS];

  int item_id, h;
  if (!headmap_decode(hm, blockIdx.x, item_id, h)) return;
  const FwdItem it = items[item_id];
  const int G = Hq / Hkv;
  const int g = h / G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int t0 = it.r0 + 32 * w;      // first query row of this wave
  const int t = t0 + l32;             // this lane's query row
  const bool wave_active = t0 < it.r1;
  const bool row_valid = t < it.r1;
  const size_t qrow = (size_t)Hq * D, krow = (size_t)Hkv * D;

  // Q fragments, B operand of S^T = K Q^T: lane -> query column, 8 consecutive d.
  bf16x8 qf[D / 16];
  {
    const u16* qp = q + (size_t)t * qrow + (size_t)h * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      Frag f;
      f.u = row_valid ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qf[kk] = f.v;
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m2 = -1e30f;  // running max of the log2-domain scores
  float lsum = 0.f;   // this lane's partial row sum (its half of the keys)

  const int nA = (it.a_end + BK - 1) / BK;
  const int nB = it.r1 > it.b_start ? (it.r1 - it.b_start + BK - 1) / BK : 0;
  const int ntiles = nA + nB;

  uint4 kreg[KLD];
  uint4 vreg[4];
  const int vkg = tid & 15, vdc = tid >> 4;   // V: 4-key group, 8-wide d chunk
  const bool vthread = tid < 16 * NDC;

  auto tile_bounds = [&](int i, int& kb, int& ke) {
    if (i < nA) { kb = i * BK; ke = it.a_end; }
    else { kb = it.b_start + (i - nA) * BK; ke = it.r1; }
  };
  auto load_tile = [&](int i) {
    int kb, ke;
    tile_bounds(i, kb, ke);
    const u16* kbase = k + (size_t)g * D;
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      int idx = tid + 256 * j, row = idx / NDC, ch = idx % NDC;
      int key = kb + row;
      kreg[j] = key < ke ? *reinterpret_cast<const uint4*>(kbase + (size_t)key * krow + ch * 8)
                         : make_uint4(0, 0, 0, 0);
    }
    if (vthread) {
      const u16* vbase = v + (size_t)g * D + vdc * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int key = kb + 4 * vkg + j;
        vreg[j] = key < ke ? *reinterpret_cast<const uint4*>(vbase + (size_t)key * krow)
                           : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      int idx = tid + 256 * j, row = idx / NDC, ch = idx % NDC;
      *reinterpret_cast<uint4*>(Ks + row * KS + ch * 8) = kreg[j];
    }
    if (vthread) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w2;
        w2.x = u16_of(vreg[0], e) | (u16_of(vreg[1], e) << 16);
        w2.y = u16_of(vreg[2], e) | (u16_of(vreg[3], e) << 16);
        *reinterpret_cast<uint2*>(Vt + (vdc * 8 + e) * VS + kperm(4 * vkg)) = w2;
      }
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int i = 0; i < ntiles; ++i) {
    int kb, ke;
    tile_bounds(i, kb, ke);
    __syncthreads();
    store_tile();
    __syncthreads();
    if (i + 1 < ntiles) load_tile(i + 1);

    if (!wave_active || kb > t0 + 31) continue;  // every key of the tile lies after this wave's rows

    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
      const u16* kp = Ks + (32 * sb + l32) * KS + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s[sb] = mfma32(lds_b128(kp + 16 * kk), qf[kk], s[sb]);
    }
    // S^T element (sb, r) is key kb + 32 sb + 8 (r/4) + 4 hl + r%4 for query t.
    const bool need_mask = (kb + BK > ke) || (kb + BK - 1 > t0);
    float mx = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int j = kb + 32 * sb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (j >= ke || j > t) s[sb][r] = -INFINITY;
          mx = fmaxf(mx, s[sb][r]);
        }
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
    }
    mx = wave_swap32_max(mx);
    // Lazy rescaling: the reference max m2 only moves when a row's max exceeds
    // it by more than 8 (log2 units), so P stays below 2^8 and the O/l
    // rescale is skipped unless some row of the wave needs it. O / l and the
    // LSE do not depend on the reference.
    if (__any(mx * c > m2 + 8.f)) {
      const float mnew = fmaxf(m2, mx * c);
      const float alpha = fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i2 = 0; i2 < D / 32; ++i2) oacc[i2] *= alpha;
    }

    bf16x8 pf[2][2];
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fast_exp2(fmaf(s[sb][r], c, -m2));
        if (need_mask && s[sb][r] == -INFINITY) x = 0.f;
        p[r] = x;
        ps += x;
      }
      pf[sb][0] = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      pf[sb][1] = pack_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
    }
    lsum += ps;

    // O^T[d][q] += V^T[d][key] P^T[key][q]; k-slot (hl, e) of both operands is
    // key 4 hl + e (e < 4) or 8 + 4 hl + (e - 4) inside each 16-key step, which
    // the permuted V^T columns hold as 8 consecutive elements at 8 hl.
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const u16* vp = Vt + (32 * dt + l32) * VS + 8 * hl;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) oacc[dt] = mfma32(lds_b128(vp + 32 * sb + 16 * kh), pf[sb][kh], oacc[dt]);
    }
  }

  const float ltot = wave_swap32_sum(lsum);
  if (row_valid) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    u16* op = o + (size_t)t * qrow + (size_t)h * D + 4 * hl;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
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
  dim3 grid(headmap_grid(hm)), block(256);
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
