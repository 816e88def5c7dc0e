/*
 * dualkv.h -- C ABI of the MI355X (gfx950) shared-prompt attention library.
 *
 * The operation (DualKV pages: the research-map summary "DualKV: Shared-Prompt
 * Flash Attention for Efficient RL Training with Large Rollouts and Long
 * Contexts", section Approach; the arXiv abstract of that paper; the forum
 * topic "DualKV: Eliminating N-fold Prompt Recomputation in RL Training of
 * LLMs", its body): one
 * micro-batch is packed as a shared prompt of P tokens followed by N
 * responses, [prompt][resp_0]...[resp_{N-1}], T = P + sum_n R_n tokens instead
 * of N(P + R). With o_0 = P and o_{n+1} = o_n + R_n, packed row t attends
 *   A(t) = {0 .. t}                      if t < P        (prompt, causal)
 *   A(t) = {0 .. P-1} u {o_n .. t}       if o_n <= t < o_{n+1}
 * i.e. the whole prompt KV region plus its own response region causally. This
 * is exactly standard attention on the N sequences [prompt; resp_n] with the
 * prompt computed once; the prompt's dK/dV are summed over all N sequences.
 *
 * Conventions for every entry point below:
 *  - Tensors are device pointers to contiguous row-major arrays, 16-byte
 *    aligned. bf16 means IEEE bfloat16 (raw 16-bit storage).
 *      q, o, dO, dQ : [T][Hq][d]  bf16
 *      k, v, dK, dV : [T][Hkv][d] bf16
 *      lse          : [Hq][T]     fp32, natural-log log-sum-exp of the scaled
 *                                 scores of each row (used by the backward)
 *  - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention);
 *    Hq must be a multiple of Hkv. Hq == Hkv is plain multi-head attention.
 *  - Score of (t, j) is softmax_scale * <q_t, k_j>, softmax_scale finite and
 *    >= 0 (0 gives uniform attention over A(t)).
 *  - Response lengths: offsets == NULL means N responses of R tokens each.
 *    Otherwise offsets is a HOST array of N+1 int32 with offsets[0] == P,
 *    offsets non-decreasing and offsets[N] == T (R is ignored). Empty
 *    responses (R_n = 0) and P == 0 (the replicated, unshared layout) are
 *    allowed.
 *  - Supported head_dim d: 64, 128. T < 2^31, T * max(Hq, Hkv) * d < 2^40
 *    and Hkv * d < 2^20.
 *  - Ownership: the caller owns every device buffer, including the
 *    workspace; the library allocates no device memory. Its only state is a
 *    small ring of pinned host staging buffers (grown on demand, kept for the
 *    life of the process) used to upload work lists. Outputs are overwritten,
 *    never accumulated into.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and the call returns without waiting for the device. The small
 *    work list is uploaded into the workspace with an asynchronous
 *    host-to-device copy on the same stream. Two calls that share a workspace
 *    must be ordered. Calls are thread-safe.
 *  - Errors: arguments are checked before any HIP call. DUALKV_ERR_INVALID_ARG
 *    for bad shapes, offsets, pointers, alignment or scale;
 *    DUALKV_ERR_UNSUPPORTED for a head_dim or mode not built;
 *    DUALKV_ERR_WORKSPACE if workspace_bytes is below the *_workspace_bytes
 *    figure; DUALKV_ERR_HIP if a HIP call or kernel launch fails. Nothing is
 *    printed and no exception crosses the ABI. On error no output is written
 *    unless the error is DUALKV_ERR_HIP.
 */
#ifndef DUALKV_H
#define DUALKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DUALKV_OK = 0,
  DUALKV_ERR_INVALID_ARG = 1,
  DUALKV_ERR_UNSUPPORTED = 2,
  DUALKV_ERR_WORKSPACE = 3,
  DUALKV_ERR_HIP = 4
} dualkv_status;

/* Workspace (device bytes) dualkv_fwd needs for this problem: the work
 * list, the 32-key block list and V^T fragments written by a transpose pass
 * over v (about the size of v). 0 if the arguments are invalid. Pure host
 * computation. */
size_t dualkv_fwd_workspace_bytes(int P, int R, int N, const int32_t* offsets,
                                  int Hq, int Hkv, int d);

/* Workspace dualkv_bwd needs: the two work lists, the per-row pairs
 * {-LSE * log2(e), -D}, D = rowsum(dO*O), [Hq][T] fp32, and either fp32
 * accumulators for dK and dV [T][Hkv][d] (atomic mode) or, with
 * deterministic != 0, per-work-item dK/dV partials plus the lists of
 * each key tile's items (dQ is written directly in both modes). 0 if the
 * arguments are invalid. */
size_t dualkv_bwd_workspace_bytes(int P, int R, int N, const int32_t* offsets,
                                  int Hq, int Hkv, int d, int deterministic);

/* Forward pass (research-map summary, section Approach, and the arXiv
 * abstract: one launch that
 * walks the prompt KV region and then the row's own response KV region).
 * Reads q, k, v; writes o (bf16) and lse (fp32, natural log), and the V^T
 * fragments into the workspace (two launches on `stream`). */
dualkv_status dualkv_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int P, int R, int N, const int32_t* offsets,
                         int Hq, int Hkv, int d, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass of L = sum_t <dO_t, O_t> (research-map summary, section
 * Approach: gradients of the
 * shared prompt accumulated across all N sequences with fp32 atomics).
 * Reads q, k, v, o, lse (from dualkv_fwd on the same inputs) and dO; writes
 * dQ, dK, dV (bf16). deterministic = 0 adds the row-chunk partials of dK and
 * dV with fp32 atomics (last bits depend on their order); deterministic != 0
 * stores the partials and sums them in a fixed order, so repeated calls on the
 * same inputs are bitwise identical (larger workspace, see above). */
dualkv_status dualkv_bwd(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                         int P, int R, int N, const int32_t* offsets,
                         int Hq, int Hkv, int d, float softmax_scale, int deterministic,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The backward of dualkv_bwd split into its stream-ordered phases, so a
 * caller can time or interleave them: bit 1 = preprocess (D = rowsum(dO*O),
 * paired with the base-2 LSE; in atomic mode also zeroed fp32 dK, dV
 * accumulators), bit 2 = key-stationary
 * dK, dV pass (two KV regions; atomics into the accumulators, or partials in
 * deterministic mode), bit 8 = query-stationary dQ pass (writes dQ), bit 4 =
 * finish (accumulators -> bf16 dK, dV, or the ordered reduction of the
 * partials). Same arguments and checks as dualkv_bwd, which is phase_mask 15.
 * Bit 1 must run before bits 2, 4 and 8, and bit 2 before bit 4, on the same
 * workspace with the same arguments; a mask of 0 or above 15 is
 * DUALKV_ERR_INVALID_ARG. */
dualkv_status dualkv_bwd_phases(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                                int P, int R, int N, const int32_t* offsets,
                                int Hq, int Hkv, int d, float softmax_scale, int deterministic,
                                void* workspace, size_t workspace_bytes, void* stream,
                                int phase_mask);

/* Several shared-prompt groups in one call. The DualKV summary page quotes its
 * GRPO speed-ups at a micro-batch size of 8 ("Key results") and states that
 * one shared prefix is assumed per micro-batch group ("Limitations"); the
 * reading taken here is that a micro-batch holds several such groups. The B groups are packed back to back in the same
 * [T][H][d] tensors: group b occupies rows [s_b, s_{b+1}) with s_0 = 0; its
 * first group_P[b] rows are its prompt, followed by its group_N[b] responses,
 * whose lengths are the next group_N[b] entries of resp_len (HOST int32 arrays:
 * group_P and group_N of B entries, resp_len of sum(group_N) entries). A row
 * attends only keys of its own group, by the single-group rule (prompt rows:
 * causal within the group's prompt; response rows: the group's whole prompt and
 * their own response causally). Groups are independent: the result equals one
 * single-group call per group on its rows. Every other convention (layouts,
 * LSE, scale, workspace, asynchrony, errors; group_N[b] >= 1, group_P[b] >= 0,
 * resp_len >= 0, B >= 1, NULL arrays are DUALKV_ERR_INVALID_ARG) is that of
 * the single-group entry points, which are the B = 1 case. */
size_t dualkv_fwd_workspace_bytes_groups(int B, const int32_t* group_P, const int32_t* group_N,
                                         const int32_t* resp_len, int Hq, int Hkv, int d);
size_t dualkv_bwd_workspace_bytes_groups(int B, const int32_t* group_P, const int32_t* group_N,
                                         const int32_t* resp_len, int Hq, int Hkv, int d,
                                         int deterministic);
dualkv_status dualkv_fwd_groups(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, const int32_t* group_P, const int32_t* group_N,
                                const int32_t* resp_len, int Hq, int Hkv, int d,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* stream);
dualkv_status dualkv_bwd_groups(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                                int B, const int32_t* group_P, const int32_t* group_N,
                                const int32_t* resp_len, int Hq, int Hkv, int d,
                                float softmax_scale, int deterministic, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Multi-level shared prefixes. The DualKV summary page names, as a limitation,
 * that only one shared prefix per group is handled and tree-structured
 * prefixes are not ("Limitations"). Here the packed rows form a forest of
 * segments stored in depth-first order: segment i holds node_len[i] rows,
 * right after segment i - 1 (segment 0 starts at row 0), and its parent is
 * node_parent[i] (-1 for a root; otherwise a segment on the path from the
 * current root to segment i - 1, so every subtree is a contiguous run of
 * rows). A row of segment v attends every key of v's proper ancestors and the
 * keys of v up to itself (causal). One shared-prompt group is a root prompt
 * with one leaf per response, so the single- and multi-group entry points are
 * special cases. At most 3 ancestors per segment (4 levels); node_len >= 0;
 * HOST int32 arrays of n_nodes >= 1 entries; anything else, or a parent that
 * breaks the depth-first order, is DUALKV_ERR_INVALID_ARG. Every other
 * convention is that of the single-group entry points. */
size_t dualkv_fwd_workspace_bytes_tree(int n_nodes, const int32_t* node_len,
                                       const int32_t* node_parent, int Hq, int Hkv, int d);
size_t dualkv_bwd_workspace_bytes_tree(int n_nodes, const int32_t* node_len,
                                       const int32_t* node_parent, int Hq, int Hkv, int d,
                                       int deterministic);
dualkv_status dualkv_fwd_tree(const void* q, const void* k, const void* v, void* o, float* lse,
                              int n_nodes, const int32_t* node_len, const int32_t* node_parent,
                              int Hq, int Hkv, int d, float softmax_scale, void* workspace,
                              size_t workspace_bytes, void* stream);
dualkv_status dualkv_bwd_tree(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                              int n_nodes, const int32_t* node_len, const int32_t* node_parent,
                              int Hq, int Hkv, int d, float softmax_scale, int deterministic,
                              void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory or stage host copies (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): dualkv_fwd with no workspace argument. Same arguments, layouts,
 * checks and results as dualkv_fwd (bitwise: the kernels are the same); the
 * work lists and the V^T fragments live in a fixed device array inside the
 * library, DUALKV_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library's
 * code is loaded on that GPU and held until the process ends. The work lists
 * are built on the device from the shape passed by value, so the call makes no
 * allocation of any kind, no host-to-device copy and no synchronisation: it
 * enqueues three kernels on `stream`. Limits: at most 256 responses
 * (DUALKV_ERR_UNSUPPORTED beyond), at most 4096 query tiles of 256 rows, and
 * work lists plus V^T (about 2 * T * Hkv * d bytes) within the array
 * (DUALKV_ERR_WORKSPACE beyond); these checks come before any HIP call.
 * Every call on one GPU uses that GPU's array, and everything a call reads
 * there it has written first, so nothing carries over from the previous
 * call; but calls that overlap in time on one GPU (other streams, other
 * threads) race on it and must be ordered by the caller. */
#define DUALKV_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dualkv_status dualkv_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int P, int R, int N, const int32_t* offsets,
                                 int Hq, int Hkv, int d, float softmax_scale, void* stream);

/* Static English description of a status code (never NULL). */
const char* dualkv_status_string(dualkv_status s);

#ifdef __cplusplus
}
#endif

#endif /* DUALKV_H */
