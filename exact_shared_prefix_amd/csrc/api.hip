// C ABI: argument checks, packed-layout descriptors, work lists, launches.
//
// The packed layout is the DualKV one (arXiv abstract: P + NR tokens per
// micro-batch; research-map summary, section Approach: a shared-context KV
// region and per-sequence response KV regions). Work lists are built on the
// host and copied into the caller's workspace on the caller's stream through
// pinned staging buffers; no device memory is allocated here.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dualkv.h"
#include "common.h"

namespace dkv {
hipError_t launch_fwd(const Problem& pb, const void* q, const void* k, const void* vt, void* o,
                      float* lse, const FwdItem* items_dev, const Region* regions_dev, int n_items,
                      int max_regions, hipStream_t stream);
hipError_t launch_xpose_kv(const Problem& pb, const void* src, void* dst, const KeyBlock* blocks_dev,
                           int n_blocks, hipStream_t stream);
hipError_t launch_bwd(const Problem& pb, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dQ, void* dK,
                      void* dV, const BwdItem* items_dev, int n_items, const FwdItem* qitems_dev,
                      const Region* qregions_dev, int n_qitems, int max_qregions, float2* rs,
                      float* dk_acc, float* dv_acc, float* part,
                      const int* tile_off, const int* tile_items, int n_tiles, hipStream_t stream,
                      int phase_mask);
}  // namespace dkv

using namespace dkv;

namespace {

// Query rows per dK/dV work item (the grid of row chunks): the largest of
// 2048, 1024, 512, 256 that gives the dK/dV pass at least kBwdMinGroups
// workgroups (one per CU), else the one that gives it the most. Shorter
// chunks mean more partial dK/dV flushes, so they are taken only where the
// pass would otherwise leave CUs idle.
constexpr int kBwdChunk = 2048;
constexpr int kMinBwdChunk = 256;
constexpr long long kBwdMinGroups = 256;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Head / size checks shared by every entry point (T already known).
dualkv_status check_heads(long long T, int Hq, int Hkv, int d, Problem& pb) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return DUALKV_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DUALKV_ERR_UNSUPPORTED;
  if (T >= (1LL << 31)) return DUALKV_ERR_INVALID_ARG;
  // element offsets are 64-bit everywhere; this bound keeps every launch grid
  // (one lane per 8 elements in the preprocess) well inside 32 bits
  if (T * (long long)std::max(Hq, Hkv) * d >= (1LL << 40)) return DUALKV_ERR_INVALID_ARG;
  // per-lane copy offsets within a 64-key tile are 32-bit
  if ((long long)Hkv * d >= (1LL << 20)) return DUALKV_ERR_INVALID_ARG;
  pb.T = (int)T;
  pb.Hq = Hq;
  pb.Hkv = Hkv;
  pb.G = Hq / Hkv;
  pb.d = d;
  return DUALKV_OK;
}

// One group given by P, N and uniform R or host offsets[N + 1] (offsets[0] == P,
// non-decreasing), starting at row `start`: a root segment (the prompt) with
// one leaf per response. Appends them to pb.segs.
dualkv_status add_group(int start, int P, int R, int N, const int32_t* offsets, Problem& pb,
                        long long& end) {
  if (P < 0 || N < 1) return DUALKV_ERR_INVALID_ARG;
  if (offsets) {
    if (offsets[0] != P) return DUALKV_ERR_INVALID_ARG;
    for (int n = 0; n < N; ++n)
      if (offsets[n + 1] < offsets[n]) return DUALKV_ERR_INVALID_ARG;
  } else if (R < 0) {
    return DUALKV_ERR_INVALID_ARG;
  }
  std::vector<int> off(N + 1);
  for (int n = 0; n <= N; ++n) {
    const long long on = offsets ? (long long)start + offsets[n] : (long long)start + P + (long long)n * R;
    if (on >= (1LL << 31)) return DUALKV_ERR_INVALID_ARG;
    off[n] = (int)on;
  }
  const int root = (int)pb.segs.size();
  pb.segs.push_back({start, P, -1, 0});
  for (int n = 0; n < N; ++n) pb.segs.push_back({off[n], off[n + 1] - off[n], root, 0});
  end = off[N];
  return DUALKV_OK;
}

// subtree_end of every segment (segments are in depth-first order, so a
// subtree is the segment and the run of later segments that descend from it)
void finish_segments(Problem& pb) {
  for (Segment& sg : pb.segs) sg.subtree_end = sg.start + sg.len;
  for (int v = (int)pb.segs.size() - 1; v >= 0; --v) {
    const int p = pb.segs[v].parent;
    if (p >= 0) pb.segs[p].subtree_end = std::max(pb.segs[p].subtree_end, pb.segs[v].subtree_end);
  }
}

// Single-group problem (the dualkv_fwd / dualkv_bwd arguments).
dualkv_status check_shape(int P, int R, int N, const int32_t* offsets, int Hq, int Hkv, int d,
                          Problem& pb) {
  pb.segs.clear();
  long long T = 0;
  const dualkv_status st = add_group(0, P, R, N, offsets, pb, T);
  if (st != DUALKV_OK) return st;
  finish_segments(pb);
  return check_heads(T, Hq, Hkv, d, pb);
}

// B groups back to back (the *_groups entry points): group b has prompt length
// group_P[b] and group_N[b] responses whose lengths are group_R[...] taken in
// order (sum of group_N entries in all).
dualkv_status check_groups(int B, const int32_t* group_P, const int32_t* group_N,
                           const int32_t* resp_len, int Hq, int Hkv, int d, Problem& pb) {
  pb.segs.clear();
  if (B < 1 || !group_P || !group_N || !resp_len) return DUALKV_ERR_INVALID_ARG;
  long long start = 0;
  size_t r = 0;
  std::vector<int32_t> offs;
  for (int b = 0; b < B; ++b) {
    const int N = group_N[b];
    if (N < 1 || group_P[b] < 0 || start >= (1LL << 31)) return DUALKV_ERR_INVALID_ARG;
    offs.assign(1, group_P[b]);
    for (int n = 0; n < N; ++n, ++r) {
      if (resp_len[r] < 0) return DUALKV_ERR_INVALID_ARG;
      const long long o = (long long)offs.back() + resp_len[r];
      if (o >= (1LL << 31)) return DUALKV_ERR_INVALID_ARG;
      offs.push_back((int32_t)o);
    }
    long long end = 0;
    const dualkv_status st = add_group((int)start, group_P[b], 0, N, offs.data(), pb, end);
    if (st != DUALKV_OK) return st;
    start = end;
  }
  finish_segments(pb);
  return check_heads(start, Hq, Hkv, d, pb);
}

// A forest of segments in depth-first order (the *_tree entry points): segment
// i has node_len[i] rows (stored right after segment i - 1) and parent
// node_parent[i], -1 for a root, else a segment on the path from a root to
// segment i - 1 (depth-first order); at most kMaxRegions - 1 = 3 ancestors.
dualkv_status check_tree(int n_nodes, const int32_t* node_len, const int32_t* node_parent, int Hq,
                         int Hkv, int d, Problem& pb) {
  pb.segs.clear();
  if (n_nodes < 1 || !node_len || !node_parent) return DUALKV_ERR_INVALID_ARG;
  std::vector<int> path;   // segments from the current root down to segment i - 1
  long long start = 0;
  for (int i = 0; i < n_nodes; ++i) {
    const int par = node_parent[i];
    if (node_len[i] < 0 || par < -1 || par >= i) return DUALKV_ERR_INVALID_ARG;
    while (!path.empty() && path.back() != par) path.pop_back();
    if (par >= 0 && path.empty()) return DUALKV_ERR_INVALID_ARG;   // parent not on the path
    if ((int)path.size() >= kMaxRegions) return DUALKV_ERR_INVALID_ARG;
    path.push_back(i);
    pb.segs.push_back({(int)start, node_len[i], par, 0});
    start += node_len[i];
    if (start >= (1LL << 31)) return DUALKV_ERR_INVALID_ARG;
  }
  finish_segments(pb);
  return check_heads(start, Hq, Hkv, d, pb);
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work-list upload. A copy from pageable host memory may wait for the stream
// to drain, which would leave the GPU idle between launches, so lists are
// staged through a small ring of pinned host buffers per device. A slot is
// reused only after the event recorded behind its previous copy completed.
class Staging {
 public:
  hipError_t upload(void* dst, const void* src, size_t n, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu_);
    Slot& sl = ring_[dev][next_[dev]];
    next_[dev] = (next_[dev] + 1) % kSlots;
    if (sl.pending) {
      if ((e = hipEventSynchronize(sl.ev)) != hipSuccess) return e;
      sl.pending = false;
    }
    if (!sl.ev && (e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming)) != hipSuccess)
      return e;
    if (sl.cap < n) {
      if (sl.host && (e = hipHostFree(sl.host)) != hipSuccess) return e;
      sl.host = nullptr;
      sl.cap = 0;
      const size_t cap = std::max<size_t>(n, 64 << 10);
      if ((e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault)) != hipSuccess) return e;
      sl.cap = cap;
    }
    std::memcpy(sl.host, src, n);
    if ((e = hipMemcpyAsync(dst, sl.host, n, hipMemcpyHostToDevice, stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(sl.ev, stream)) != hipSuccess) return e;
    sl.pending = true;
    return hipSuccess;
  }

 private:
  static constexpr int kDevices = 16, kSlots = 8;
  struct Slot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
  };
  std::mutex mu_;
  Slot ring_[kDevices][kSlots];
  int next_[kDevices] = {};
};

hipError_t upload(void* dst, const void* src, size_t n, hipStream_t stream) {
  static Staging* staging = new Staging();  // process lifetime, never torn down
  return staging->upload(dst, src, n, stream);
}

// 32-key blocks of the transposed K / V fragments, cut per segment;
// base[v] = first block of segment v.
std::vector<KeyBlock> key_blocks(const Problem& pb, std::vector<int>* base = nullptr) {
  std::vector<KeyBlock> blocks;
  if (base) base->clear();
  for (const Segment& sg : pb.segs) {
    if (base) base->push_back((int)blocks.size());
    for (int kb = sg.start; kb < sg.start + sg.len; kb += 32) blocks.push_back({kb, sg.start + sg.len});
  }
  return blocks;
}

// Forward (and dQ) work list: query tiles of `rows` rows of one segment, with
// their key regions (ancestor segments root first, then the own segment up to
// the tile's last row), longest (most keys) first so the tail of the grid is
// short.
std::vector<FwdItem> fwd_items(const Problem& pb, std::vector<Region>* regions, int rows = kFwdRows) {
  std::vector<int> base;
  key_blocks(pb, &base);
  struct Tmp { FwdItem it; int keys; };
  std::vector<Tmp> tmp;
  std::vector<Region> regs;
  std::vector<int> anc;
  for (int v = 0; v < (int)pb.segs.size(); ++v) {
    const Segment& sg = pb.segs[v];
    anc.clear();
    for (int a = sg.parent; a >= 0; a = pb.segs[a].parent) anc.push_back(a);
    for (int r = sg.start; r < sg.start + sg.len; r += rows) {
      const int r1 = std::min(sg.start + sg.len, r + rows);
      const int off = (int)regs.size();
      int keys = 0;
      for (int x = (int)anc.size() - 1; x >= 0; --x) {
        const Segment& as = pb.segs[anc[x]];
        regs.push_back({as.start, as.start + as.len, base[anc[x]]});
        keys += as.len;
      }
      regs.push_back({sg.start, r1, base[v]});
      keys += r1 - sg.start;
      tmp.push_back({{r, r1, off, (int)anc.size() + 1}, keys});
    }
  }
  std::stable_sort(tmp.begin(), tmp.end(), [](const Tmp& x, const Tmp& y) { return x.keys > y.keys; });
  std::vector<FwdItem> items;
  for (const Tmp& t : tmp) items.push_back(t.it);
  if (regions) *regions = std::move(regs);
  return items;
}

// dK/dV items of a chunk size C: every key tile paired with each C-row chunk
// its attending rows (from the tile's first key to the end of its segment's
// subtree) touch.
long long bwd_item_count(const Problem& pb, int C) {
  long long n = 0;
  for (const Segment& sg : pb.segs)
    for (int kb = sg.start; kb < sg.start + sg.len; kb += kBwdKeys)
      if (kb < sg.subtree_end) n += (sg.subtree_end - 1) / C - kb / C + 1;
  return n;
}

int chunk_rows(const Problem& pb) {
  int best = kBwdChunk;
  long long most = 0;
  for (int C = kBwdChunk; C >= kMinBwdChunk; C /= 2) {
    const long long n = bwd_item_count(pb, C);
    if (n * pb.Hkv >= kBwdMinGroups) return C;
    if (n > most) { most = n; best = C; }
  }
  return best;
}

// dK/dV work list: kBwdKeys-key tiles of each segment, each paired with the
// rows that attend it: the later rows of the segment's subtree (every later row
// of its group for a prompt tile, the later rows of its own response for a
// response tile), cut on a fixed grid of chunk_rows(pb)-row chunks.
// Items are ordered chunk-major so workgroups running together share query
// rows. With tl_out != null, also returns each tile's items (ascending) as a
// CSR list.
struct TileLists { std::vector<int> off, items; };
std::vector<BwdItem> bwd_items(const Problem& pb, TileLists* tl_out = nullptr) {
  struct Tile { int kb, ke, rend; };
  std::vector<Tile> tiles;
  for (const Segment& sg : pb.segs) {
    const int e = sg.start + sg.len;
    for (int kb = sg.start; kb < e; kb += kBwdKeys) tiles.push_back({kb, std::min(e, kb + kBwdKeys), sg.subtree_end});
  }
  std::vector<BwdItem> items;
  std::vector<std::vector<int>> per_tile(tiles.size());
  const int chunk = chunk_rows(pb);
  const int nchunks = (pb.T + chunk - 1) / chunk;
  for (int cidx = 0; cidx < nchunks; ++cidx) {
    const int c0 = cidx * chunk, c1 = std::min(pb.T, c0 + chunk);
    for (size_t ti = 0; ti < tiles.size(); ++ti) {
      const Tile& tl = tiles[ti];
      const int r0 = std::max(c0, tl.kb), r1 = std::min(c1, tl.rend);
      if (r0 < r1) {
        per_tile[ti].push_back((int)items.size());
        items.push_back({tl.kb, tl.ke, r0, r1});
      }
    }
  }
  if (tl_out) {
    tl_out->off.assign(1, 0);
    tl_out->items.clear();
    for (const auto& v : per_tile) {
      tl_out->items.insert(tl_out->items.end(), v.begin(), v.end());
      tl_out->off.push_back((int)tl_out->items.size());
    }
  }
  return items;
}

// Forward workspace: work list, key blocks, V^T fragments
// [block][Hkv][d/32][2][64][8] bf16.
struct FwdLayout {
  size_t items, regions, blocks, vt, total;
};
FwdLayout fwd_layout(const Problem& pb, size_t n_items, size_t n_regions, size_t n_blocks) {
  FwdLayout L{};
  size_t off = 0;
  L.items = off;   off = align_up(off + std::max<size_t>(1, n_items) * sizeof(FwdItem));
  L.regions = off; off = align_up(off + std::max<size_t>(1, n_regions) * sizeof(Region));
  L.blocks = off; off = align_up(off + std::max<size_t>(1, n_blocks) * sizeof(KeyBlock));
  L.vt = off;     off = align_up(off + n_blocks * pb.Hkv * (size_t)pb.d * 32 * sizeof(uint16_t));
  L.total = off;
  return L;
}

struct BwdLayout {
  size_t items, qitems, qregions, rowstat, dk, dv, part, tile_off, tile_items, total;
};

// Atomic mode: fp32 dK, dV accumulators [T][Hkv][d]. Deterministic mode:
// per-item partials [n_items][Hkv][2][kBwdKeys][d] and the tile CSR lists.
BwdLayout bwd_layout(const Problem& pb, size_t n_items, size_t n_qitems, size_t n_qregions,
                     bool det, size_t n_tiles) {
  BwdLayout L{};
  size_t off = 0;
  L.items = off;    off = align_up(off + n_items * sizeof(BwdItem));
  L.qitems = off;   off = align_up(off + n_qitems * sizeof(FwdItem));
  L.qregions = off; off = align_up(off + std::max<size_t>(1, n_qregions) * sizeof(Region));
  L.rowstat = off; off = align_up(off + (size_t)pb.Hq * pb.T * 2 * sizeof(float));   // {-LSE log2 e, D}
  if (det) {
    L.part = off;       off = align_up(off + n_items * pb.Hkv * 2 * (size_t)kBwdKeys * pb.d * sizeof(float));
    L.tile_off = off;   off = align_up(off + (n_tiles + 1) * sizeof(int));
    L.tile_items = off; off = align_up(off + n_items * sizeof(int));
  } else {
    L.dk = off; off = align_up(off + (size_t)pb.T * pb.Hkv * pb.d * sizeof(float));
    L.dv = off; off = align_up(off + (size_t)pb.T * pb.Hkv * pb.d * sizeof(float));
  }
  L.total = off;
  return L;
}

size_t fwd_ws_bytes(const Problem& pb) {
  std::vector<Region> regs;
  const size_t ni = fwd_items(pb, &regs).size();
  return fwd_layout(pb, ni, regs.size(), key_blocks(pb).size()).total;
}

// Sizes of the backward's lists, counted without building them: dK/dV items
// (key tiles x the row chunks their attending rows touch), key tiles, dQ
// items (query tiles) and their key regions (ancestors + own segment each).
struct BwdCounts { size_t items = 0, tiles = 0, qitems = 0, qregions = 0; };
BwdCounts bwd_counts(const Problem& pb) {
  BwdCounts n;
  std::vector<int> depth(pb.segs.size(), 0);
  for (size_t v = 0; v < pb.segs.size(); ++v) {
    const Segment& sg = pb.segs[v];
    if (sg.parent >= 0) depth[v] = depth[sg.parent] + 1;
    const int e = sg.start + sg.len;
    for (int kb = sg.start; kb < e; kb += kBwdKeys) ++n.tiles;
    const size_t q = (size_t)(sg.len + kDqRows - 1) / kDqRows;
    n.qitems += q;
    n.qregions += q * (depth[v] + 1);
  }
  n.items = (size_t)bwd_item_count(pb, chunk_rows(pb));
  return n;
}

BwdLayout bwd_layout_of(const Problem& pb, const BwdCounts& n, bool det) {
  return bwd_layout(pb, std::max<size_t>(1, n.items), std::max<size_t>(1, n.qitems), n.qregions, det,
                    n.tiles);
}

size_t bwd_ws_bytes(const Problem& pb, bool det) { return bwd_layout_of(pb, bwd_counts(pb), det).total; }

dualkv_status fwd_impl(Problem& pb, const void* q, const void* k, const void* v, void* o,
                       float* lse, float softmax_scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return DUALKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return DUALKV_ERR_INVALID_ARG;
  pb.scale = softmax_scale;
  std::vector<Region> regs;
  const std::vector<FwdItem> items = fwd_items(pb, &regs);
  const std::vector<KeyBlock> blocks = key_blocks(pb);
  const FwdLayout L = fwd_layout(pb, items.size(), regs.size(), blocks.size());
  int max_regions = 1;
  for (const FwdItem& it : items) max_regions = std::max(max_regions, it.n_reg);
  if (!workspace || workspace_bytes < L.total) return DUALKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DUALKV_ERR_INVALID_ARG;
  if (items.empty()) return DUALKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (upload(ws + L.items, items.data(), items.size() * sizeof(FwdItem), s) != hipSuccess ||
      upload(ws + L.regions, regs.data(), regs.size() * sizeof(Region), s) != hipSuccess ||
      (!blocks.empty() &&
       upload(ws + L.blocks, blocks.data(), blocks.size() * sizeof(KeyBlock), s) != hipSuccess))
    return DUALKV_ERR_HIP;
  if (launch_xpose_kv(pb, v, ws + L.vt, reinterpret_cast<const KeyBlock*>(ws + L.blocks),
                      (int)blocks.size(), s) != hipSuccess ||
      launch_fwd(pb, q, k, ws + L.vt, o, lse, reinterpret_cast<const FwdItem*>(ws + L.items),
                 reinterpret_cast<const Region*>(ws + L.regions), (int)items.size(), max_regions,
                 s) != hipSuccess)
    return DUALKV_ERR_HIP;
  return DUALKV_OK;
}

dualkv_status bwd_impl(Problem& pb, const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                       float softmax_scale, int deterministic, void* workspace,
                       size_t workspace_bytes, void* stream, int phase_mask) {
  if (phase_mask < 1 || phase_mask > 15) return DUALKV_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return DUALKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return DUALKV_ERR_INVALID_ARG;
  pb.scale = softmax_scale;
  const bool det = deterministic != 0;
  const BwdCounts cnt = bwd_counts(pb);
  const BwdLayout L = bwd_layout_of(pb, cnt, det);
  if (!workspace || workspace_bytes < L.total) return DUALKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DUALKV_ERR_INVALID_ARG;
  if (pb.T == 0) return DUALKV_OK;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // build and upload only what the requested phases read: the dK/dV pass and
  // the ordered reduction read the item list, the reduction also the tile
  // lists, the dQ pass its query-tile list and key regions
  const bool need_items = (phase_mask & 2) || (det && (phase_mask & 4));
  const bool need_tiles = det && (phase_mask & 4);
  const bool need_q = (phase_mask & 8) != 0;
  TileLists tl;
  std::vector<BwdItem> items;
  if (need_items) items = bwd_items(pb, need_tiles ? &tl : nullptr);
  std::vector<Region> qregs;
  std::vector<FwdItem> qitems;
  if (need_q) qitems = fwd_items(pb, &qregs, kDqRows);
  if (items.size() > cnt.items || qitems.size() > cnt.qitems || qregs.size() > cnt.qregions)
    return DUALKV_ERR_HIP;   // the counts size the workspace; they cannot fall short
  if (need_items && !items.empty() &&
      upload(ws + L.items, items.data(), items.size() * sizeof(BwdItem), s) != hipSuccess)
    return DUALKV_ERR_HIP;
  if (need_tiles && !items.empty() &&
      (upload(ws + L.tile_off, tl.off.data(), tl.off.size() * sizeof(int), s) != hipSuccess ||
       upload(ws + L.tile_items, tl.items.data(), tl.items.size() * sizeof(int), s) != hipSuccess))
    return DUALKV_ERR_HIP;
  if (need_q && !qitems.empty() &&
      (upload(ws + L.qitems, qitems.data(), qitems.size() * sizeof(FwdItem), s) != hipSuccess ||
       upload(ws + L.qregions, qregs.data(), qregs.size() * sizeof(Region), s) != hipSuccess))
    return DUALKV_ERR_HIP;
  int max_qregions = 1;
  for (const FwdItem& it : qitems) max_qregions = std::max(max_qregions, it.n_reg);
  const int n_tiles = (int)cnt.tiles;
  if (launch_bwd(pb, q, k, v, o, lse, dO, dQ, dK, dV, reinterpret_cast<const BwdItem*>(ws + L.items),
                 (int)items.size(), reinterpret_cast<const FwdItem*>(ws + L.qitems),
                 reinterpret_cast<const Region*>(ws + L.qregions), (int)qitems.size(), max_qregions,
                 reinterpret_cast<float2*>(ws + L.rowstat),
                 det ? nullptr : reinterpret_cast<float*>(ws + L.dk),
                 det ? nullptr : reinterpret_cast<float*>(ws + L.dv),
                 det ? reinterpret_cast<float*>(ws + L.part) : nullptr,
                 reinterpret_cast<const int*>(ws + L.tile_off),
                 reinterpret_cast<const int*>(ws + L.tile_items), det ? n_tiles : 0, s,
                 phase_mask) != hipSuccess)
    return DUALKV_ERR_HIP;
  return DUALKV_OK;
}

// ------------------------------------------------ allocation-free forward --
// dualkv_fwd_noalloc: the forward with its workspace in a fixed device array
// of this library (one per GPU, held until the process ends) instead of a
// caller buffer, and its work lists built on the device by describe_kernel
// from the shape passed by value, so the call allocates nothing and copies
// nothing from the host. Everything in the array is written before it is
// read, so nothing needs clearing between calls; calls that overlap on one
// GPU share the array and race.
constexpr size_t kScratchBytes = DUALKV_NOALLOC_SCRATCH_BYTES;
constexpr int kNoallocMaxResp = 256;     // responses per call (offsets travel by value)
constexpr int kNoallocMaxItems = 4096;   // forward work items (256-row query tiles)
constexpr int kNoallocMaxDevices = 16;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DescribeArgs {
  int P, N;
  int items_prompt, n_items;
  int off[kNoallocMaxResp + 1];   // o_0 = P .. o_N = T
};

// Segment s of the single-group layout: s = 0 is the prompt [0, P), s = n + 1
// is response n [o_n, o_{n+1}).
__device__ inline int seg_begin(const DescribeArgs& a, int s) { return s == 0 ? 0 : a.off[s - 1]; }
__device__ inline int seg_end(const DescribeArgs& a, int s) { return s == 0 ? a.P : a.off[s]; }

// One workgroup writes the three lists fwd_items / key_blocks build on the
// host, in the same order: the query tiles (kFwdRows rows of one segment) in
// generation order get their key regions (the prompt tile [0, r1); a
// response tile the whole prompt, then its own rows up to r1), and are then
// placed by a stable rank on their key count, longest first.
__global__ __launch_bounds__(1024) void describe_kernel(DescribeArgs a, FwdItem* __restrict__ items,
                                                        Region* __restrict__ regions,
                                                        KeyBlock* __restrict__ blocks) {
  __shared__ int item_base[kNoallocMaxResp + 2];    // first item of segment s
  __shared__ int block_base[kNoallocMaxResp + 2];   // first 32-key block of segment s
  __shared__ int keys[kNoallocMaxItems];
  const int nseg = a.N + 1;
  if (threadIdx.x == 0) {
    int it = 0, bl = 0;
    for (int s = 0; s < nseg; ++s) {
      item_base[s] = it;
      block_base[s] = bl;
      const int len = seg_end(a, s) - seg_begin(a, s);
      it += (len + kFwdRows - 1) / kFwdRows;
      bl += (len + 31) / 32;
    }
    item_base[nseg] = it;
    block_base[nseg] = bl;
  }
  __syncthreads();
  // items in generation order: key counts, regions
  for (int i = threadIdx.x; i < a.n_items; i += blockDim.x) {
    int s = 0;
    while (item_base[s + 1] <= i) ++s;
    const int b0 = seg_begin(a, s), b1 = seg_end(a, s);
    const int r0 = b0 + (i - item_base[s]) * kFwdRows, r1 = min(b1, r0 + kFwdRows);
    if (s == 0) {
      keys[i] = r1;
      regions[i] = Region{0, r1, block_base[0]};
    } else {
      keys[i] = a.P + (r1 - b0);
      const int ro = a.items_prompt + 2 * (i - a.items_prompt);
      regions[ro] = Region{0, a.P, block_base[0]};
      regions[ro + 1] = Region{b0, r1, block_base[s]};
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.n_items; i += blockDim.x) {
    int s = 0;
    while (item_base[s + 1] <= i) ++s;
    const int b0 = seg_begin(a, s), b1 = seg_end(a, s);
    const int r0 = b0 + (i - item_base[s]) * kFwdRows, r1 = min(b1, r0 + kFwdRows);
    const int ki = keys[i];
    int rank = 0;
    for (int j = 0; j < a.n_items; ++j) rank += (keys[j] > ki) || (keys[j] == ki && j < i);
    items[rank] = s == 0 ? FwdItem{r0, r1, i, 1}
                         : FwdItem{r0, r1, a.items_prompt + 2 * (i - a.items_prompt), 2};
  }
  for (int b = threadIdx.x; b < block_base[nseg]; b += blockDim.x) {
    int s = 0;
    while (block_base[s + 1] <= b) ++s;
    blocks[b] = KeyBlock{seg_begin(a, s) + 32 * (b - block_base[s]), seg_end(a, s)};
  }
}

// Device address of this GPU's scratch array, looked up once per device
// with that device current (the array's name is only a host-side handle).
hipError_t scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptr[kNoallocMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoallocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

dualkv_status fwd_noalloc_impl(const Problem& pb, int P, const void* q, const void* k, const void* v,
                               void* o, float* lse, float softmax_scale, void* stream) {
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return DUALKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return DUALKV_ERR_INVALID_ARG;
  const int N = (int)pb.segs.size() - 1;
  if (N > kNoallocMaxResp) return DUALKV_ERR_UNSUPPORTED;
  DescribeArgs a{};
  a.P = P;
  a.N = N;
  long long n_blocks = 0;
  for (int s = 0; s <= N; ++s) {
    const Segment& sg = pb.segs[s];
    if (s > 0) a.off[s - 1] = sg.start;
    const int ni = (sg.len + kFwdRows - 1) / kFwdRows;
    if (s == 0) a.items_prompt = ni;
    a.n_items += ni;
    n_blocks += (sg.len + 31) / 32;
  }
  a.off[N] = pb.T;
  if (a.n_items > kNoallocMaxItems) return DUALKV_ERR_WORKSPACE;
  const int n_regions = a.items_prompt + 2 * (a.n_items - a.items_prompt);
  Problem sized = pb;
  sized.scale = softmax_scale;
  const FwdLayout L = fwd_layout(sized, a.n_items, n_regions, (size_t)n_blocks);
  if (L.total > kScratchBytes) return DUALKV_ERR_WORKSPACE;
  if (a.n_items == 0) return DUALKV_OK;
  void* base = nullptr;
  if (scratch_ptr(&base) != hipSuccess) return DUALKV_ERR_HIP;
  char* ws = static_cast<char*>(base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  FwdItem* items = reinterpret_cast<FwdItem*>(ws + L.items);
  Region* regions = reinterpret_cast<Region*>(ws + L.regions);
  KeyBlock* blocks = reinterpret_cast<KeyBlock*>(ws + L.blocks);
  hipLaunchKernelGGL(describe_kernel, dim3(1), dim3(1024), 0, s, a, items, regions, blocks);
  if (hipGetLastError() != hipSuccess) return DUALKV_ERR_HIP;
  const int max_regions = a.n_items > a.items_prompt ? 2 : 1;
  if (launch_xpose_kv(sized, v, ws + L.vt, blocks, (int)n_blocks, s) != hipSuccess ||
      launch_fwd(sized, q, k, ws + L.vt, o, lse, items, regions, a.n_items, max_regions, s) != hipSuccess)
    return DUALKV_ERR_HIP;
  return DUALKV_OK;
}

}  // namespace

extern "C" {

size_t dualkv_fwd_workspace_bytes(int P, int R, int N, const int32_t* offsets, int Hq, int Hkv,
                                  int d) {
  Problem pb;
  if (check_shape(P, R, N, offsets, Hq, Hkv, d, pb) != DUALKV_OK) return 0;
  return fwd_ws_bytes(pb);
}

size_t dualkv_bwd_workspace_bytes(int P, int R, int N, const int32_t* offsets, int Hq, int Hkv,
                                  int d, int deterministic) {
  Problem pb;
  if (check_shape(P, R, N, offsets, Hq, Hkv, d, pb) != DUALKV_OK) return 0;
  return bwd_ws_bytes(pb, deterministic != 0);
}

dualkv_status dualkv_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int P,
                         int R, int N, const int32_t* offsets, int Hq, int Hkv, int d,
                         float softmax_scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Problem pb;
  const dualkv_status st = check_shape(P, R, N, offsets, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return fwd_impl(pb, q, k, v, o, lse, softmax_scale, workspace, workspace_bytes, stream);
}

dualkv_status dualkv_bwd_phases(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                                int P, int R, int N, const int32_t* offsets, int Hq, int Hkv,
                                int d, float softmax_scale, int deterministic, void* workspace,
                                size_t workspace_bytes, void* stream, int phase_mask) {
  Problem pb;
  const dualkv_status st = check_shape(P, R, N, offsets, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return bwd_impl(pb, q, k, v, o, lse, dO, dQ, dK, dV, softmax_scale, deterministic, workspace,
                  workspace_bytes, stream, phase_mask);
}

dualkv_status dualkv_bwd(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dQ, void* dK, void* dV, int P,
                         int R, int N, const int32_t* offsets, int Hq, int Hkv, int d,
                         float softmax_scale, int deterministic, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return dualkv_bwd_phases(q, k, v, o, lse, dO, dQ, dK, dV, P, R, N, offsets, Hq, Hkv, d,
                           softmax_scale, deterministic, workspace, workspace_bytes, stream, 15);
}

size_t dualkv_fwd_workspace_bytes_groups(int B, const int32_t* group_P, const int32_t* group_N,
                                         const int32_t* resp_len, int Hq, int Hkv, int d) {
  Problem pb;
  if (check_groups(B, group_P, group_N, resp_len, Hq, Hkv, d, pb) != DUALKV_OK) return 0;
  return fwd_ws_bytes(pb);
}

size_t dualkv_bwd_workspace_bytes_groups(int B, const int32_t* group_P, const int32_t* group_N,
                                         const int32_t* resp_len, int Hq, int Hkv, int d,
                                         int deterministic) {
  Problem pb;
  if (check_groups(B, group_P, group_N, resp_len, Hq, Hkv, d, pb) != DUALKV_OK) return 0;
  return bwd_ws_bytes(pb, deterministic != 0);
}

dualkv_status dualkv_fwd_groups(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, const int32_t* group_P, const int32_t* group_N,
                                const int32_t* resp_len, int Hq, int Hkv, int d,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* stream) {
  Problem pb;
  const dualkv_status st = check_groups(B, group_P, group_N, resp_len, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return fwd_impl(pb, q, k, v, o, lse, softmax_scale, workspace, workspace_bytes, stream);
}

dualkv_status dualkv_bwd_groups(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                                int B, const int32_t* group_P, const int32_t* group_N,
                                const int32_t* resp_len, int Hq, int Hkv, int d,
                                float softmax_scale, int deterministic, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Problem pb;
  const dualkv_status st = check_groups(B, group_P, group_N, resp_len, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return bwd_impl(pb, q, k, v, o, lse, dO, dQ, dK, dV, softmax_scale, deterministic, workspace,
                  workspace_bytes, stream, 15);
}

const char* dualkv_status_string(dualkv_status s) {
  switch (s) {
    case DUALKV_OK: return "ok";
    case DUALKV_ERR_INVALID_ARG: return "invalid argument";
    case DUALKV_ERR_UNSUPPORTED: return "unsupported head_dim or mode";
    case DUALKV_ERR_WORKSPACE: return "workspace missing or too small";
    case DUALKV_ERR_HIP: return "HIP runtime or kernel launch error";
  }
  return "unknown status";
}

size_t dualkv_fwd_workspace_bytes_tree(int n_nodes, const int32_t* node_len,
                                       const int32_t* node_parent, int Hq, int Hkv, int d) {
  Problem pb;
  if (check_tree(n_nodes, node_len, node_parent, Hq, Hkv, d, pb) != DUALKV_OK) return 0;
  return fwd_ws_bytes(pb);
}

size_t dualkv_bwd_workspace_bytes_tree(int n_nodes, const int32_t* node_len,
                                       const int32_t* node_parent, int Hq, int Hkv, int d,
                                       int deterministic) {
  Problem pb;
  if (check_tree(n_nodes, node_len, node_parent, Hq, Hkv, d, pb) != DUALKV_OK) return 0;
  return bwd_ws_bytes(pb, deterministic != 0);
}

dualkv_status dualkv_fwd_tree(const void* q, const void* k, const void* v, void* o, float* lse,
                              int n_nodes, const int32_t* node_len, const int32_t* node_parent,
                              int Hq, int Hkv, int d, float softmax_scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Problem pb;
  const dualkv_status st = check_tree(n_nodes, node_len, node_parent, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return fwd_impl(pb, q, k, v, o, lse, softmax_scale, workspace, workspace_bytes, stream);
}

dualkv_status dualkv_bwd_tree(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                              int n_nodes, const int32_t* node_len, const int32_t* node_parent,
                              int Hq, int Hkv, int d, float softmax_scale, int deterministic,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Problem pb;
  const dualkv_status st = check_tree(n_nodes, node_len, node_parent, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return bwd_impl(pb, q, k, v, o, lse, dO, dQ, dK, dV, softmax_scale, deterministic, workspace,
                  workspace_bytes, stream, 15);
}

dualkv_status dualkv_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int P, int R, int N, const int32_t* offsets, int Hq, int Hkv,
                                 int d, float softmax_scale, void* stream) {
  Problem pb;
  const dualkv_status st = check_shape(P, R, N, offsets, Hq, Hkv, d, pb);
  if (st != DUALKV_OK) return st;
  return fwd_noalloc_impl(pb, P, q, k, v, o, lse, softmax_scale, stream);
}

}  // extern "C"
