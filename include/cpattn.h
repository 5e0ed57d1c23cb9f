/*
 * cpattn.h -- blockwise (ring / context-parallel) attention for AMD gfx950.
 *
 * A query block computes a partial attention result against one visiting
 * key/value block and returns it as the pair (O, LSE): the softmax-weighted
 * sum of the visible values and the natural log of the softmax denominator
 * over those keys ("Context Parallelism in ART", section 02, the attention
 * definition and the LSE summary (o_A, L_A)).  Partials over disjoint key
 * sets combine exactly with the log-sum-exp merge (same page, section 03),
 * done here in fp32.  A ring of N ranks is emulated on one GPU by visiting,
 * in round k, the key/value block of rank (r - k) mod N (ML-systems lesson on
 * sequence/context parallelism, the ring-attention section).
 *
 * Conventions shared by every entry point:
 *  - Status: every function returns CPATTN_OK (0) or a negative cpattn_status.
 *    No exception crosses this interface.  cpattn_last_error() gives a message
 *    for the calling thread's last failure.
 *  - Memory: tensors, outputs and position data passed to compute calls are
 *    device pointers owned by the caller, who keeps them alive until the
 *    stream has finished with them.  The library allocates device memory only
 *    inside mask descriptors (released by cpattn_mask_free), and holds one
 *    static buffer per GPU for cpattn_mask_tree_static.
 *  - Streams: `stream` is a hipStream_t (NULL = the legacy default stream).
 *    Compute calls validate their arguments synchronously, then enqueue work
 *    on the stream and return without waiting.  A launch failure returns
 *    CPATTN_EDEVICE with the HIP error text.  Compute calls enqueue kernels
 *    only (no allocation, copy, memset or synchronisation), so they may be
 *    captured in a HIP graph, and calls on different streams share no state;
 *    the kernels are deterministic, so equal inputs give equal bits.  Mask
 *    constructors copy and synchronise on their stream and are not for
 *    capture.
 *  - Fail fast: unsupported combinations return CPATTN_EUNSUPPORTED; nothing
 *    falls back to another code path.
 *  - Extents (token counts, head counts, block counts, tree shapes) are
 *    runtime arguments; nothing recompiles when they change.
 *  - Numerics: scores are accumulated in fp32 from bf16 or fp32 inputs, the
 *    softmax runs in fp32, O and LSE are fp32, LSE is a natural log.  A row
 *    that sees no key of the visiting block gets O = 0 and LSE = -inf (with
 *    accumulate set, such a row keeps its running value).  NaN inputs
 *    propagate.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_VERSION_MAJOR 0
#define CPATTN_VERSION_MINOR 9

typedef enum {
    CPATTN_OK = 0,
    CPATTN_EINVAL = -1,        /* malformed argument: sizes, ranks, tree links */
    CPATTN_EUNSUPPORTED = -2,  /* well-formed but not implemented: dtype, head dim, layout */
    CPATTN_EDEVICE = -3,       /* HIP runtime or launch failure */
    CPATTN_ENOMEM = -4         /* device allocation failed (mask descriptors only) */
} cpattn_status;

typedef enum { CPATTN_BF16 = 0, CPATTN_F32 = 1 } cpattn_dtype;

/* A [n_heads][n_tok][d] tensor in device memory.  Element (h, i, c) lives at
 * data + h*stride_head + i*stride_tok + c (strides in elements; the last
 * dimension is contiguous).  `data` must be 16-byte aligned and both strides
 * multiples of 8 elements (bf16) or 4 elements (f32). */
typedef struct {
    const void* data;
    int32_t dtype;          /* cpattn_dtype */
    int32_t reserved;
    int64_t n_heads;
    int64_t n_tok;
    int64_t d;              /* head dimension: 64 or 128 */
    int64_t stride_head;
    int64_t stride_tok;
} cpattn_tensor;

/* Global position of row i of a block: base + stride * i (stride >= 1).
 * Contiguous blocks use stride 1; the striped layout, where rank r holds the
 * positions x with x % P == r (mstar PR 1141, the ring exchange), uses
 * base = r, stride = P. */
typedef struct {
    int64_t base;
    int64_t stride;
} cpattn_posmap;

/* Opaque visibility descriptor.  Immutable after creation; safe to share
 * between calls and streams.  Visibility of key position x to query position
 * y is "x <= y < end[x]", where end[x] is one past the last position of the
 * subtree of x's segment (or +infinity for a causal mask). */
typedef struct cpattn_mask cpattn_mask;

/* Causal visibility over positions [0, n_pos): key x is visible to query y
 * iff x <= y ("Context Parallelism in ART", section 02: a causal query reads
 * positions up through its own).  Allocates no device memory.
 * EINVAL if n_pos < 0 or out is NULL. */
int cpattn_mask_causal(int64_t n_pos, cpattn_mask** out);

/* Prefix-tree visibility ("Context Parallelism in ART", section 02 and the
 * tiny tree of section 03): a query sees the earlier-or-equal tokens of its
 * own segment and every token of every strict ancestor segment.
 *   seg_id[n_tok]: host array, segment of each physical position (0..n_seg-1);
 *                  each segment must occupy one contiguous run.
 *   parent[n_seg]: host array, parent segment (-1 for a root).
 * The row must be stored in depth-first preorder: every segment's subtree
 * occupies one contiguous range that starts with the segment itself (a
 * parent precedes its children and no subtree is interleaved with another).
 * Returns EUNSUPPORTED for a tree that is not stored that way, EINVAL for
 * out-of-range ids, split segments or parent cycles, ENOMEM/EDEVICE on
 * allocation or upload failure.  The upload is enqueued on `stream` and is
 * complete when the function returns (the host arrays may be freed). */
int cpattn_mask_tree(const int32_t* seg_id, int64_t n_tok, const int32_t* parent, int32_t n_seg,
                     void* stream, cpattn_mask** out);

/* cpattn_mask_tree for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops that build a descriptor per input,
 * harnesses that forbid hipMalloc): the same descriptor, same arguments,
 * checks and errors, built without any device allocation.  Its device arrays
 * live in a static buffer of the library, one per GPU, held until the process
 * ends: at most CPATTN_STATIC_MAX_TOK tokens and CPATTN_STATIC_MAX_SEG
 * segments (9 MiB), larger trees return EUNSUPPORTED.  The descriptor returned
 * belongs to the library and is the same object on every call on the current
 * device: each call replaces that device's previous descriptor (its device
 * arrays are rewritten in order on `stream`; work still using the previous
 * one must be on `stream` or finished), and calls that overlap on one GPU
 * (other threads or streams) race.  cpattn_mask_free accepts it and does
 * nothing.  It is used like any descriptor, cpattn_mask_with_window included
 * (whose result is an ordinary, allocated descriptor).  The first call on a
 * device looks up the buffer's device address and reserves host bookkeeping
 * for the largest tree; later calls allocate nothing. */
#define CPATTN_STATIC_MAX_TOK (1 << 20)
#define CPATTN_STATIC_MAX_SEG (1 << 16)
int cpattn_mask_tree_static(const int32_t* seg_id, int64_t n_tok, const int32_t* parent, int32_t n_seg,
                            void* stream, cpattn_mask** out);

/* Sliding-window attention on logical positions ("Context Parallelism in
 * ART", section 06): a new descriptor with the visibility of `m` restricted
 * to the keys whose logical position is within `window` tokens of the
 * query's, the query included (logical position = position along the
 * root-to-leaf path: the tokens of the strict ancestor segments plus the
 * earlier tokens of the own segment; for a causal mask, the position itself).
 * With window 3, query B8 of the section's tiny tree sees physical positions
 * 3, 7, 8, not the last three physical addresses.  The new descriptor owns
 * copies of m's device arrays (m may be freed first) and is used like any
 * other; partial, ring, plan and merge calls honour its window, and the
 * kernels skip tiles outside it.  1 <= window <= 2^30, else EINVAL; ENOMEM /
 * EDEVICE on allocation or upload failure (enqueued on `stream`, complete on
 * return). */
int cpattn_mask_with_window(const cpattn_mask* m, int64_t window, void* stream, cpattn_mask** out);

/* Releases a descriptor and its device arrays.  The caller guarantees that no
 * enqueued work still uses it.  NULL is accepted. */
int cpattn_mask_free(cpattn_mask* m);

/* Number of positions a descriptor covers (its n_pos / n_tok), or -1. */
int64_t cpattn_mask_npos(const cpattn_mask* m);

/* Partial attention of one query block against one key/value block: the
 * (O, LSE) pair of one ring round ("Context Parallelism in ART", sections 02
 * and 03; the masks are those of section 02).
 *   q: [H][n_q][d], k and v: [H_kv][n_k][d]; one dtype, one d.  H_kv must
 *      divide H: grouped-query attention ("Context Parallelism in ART",
 *      section 02, the measured model has 32 query and 4 KV heads), query
 *      head h reads K/V head h / (H / H_kv); H_kv = H is plain multi-head.
 *   q_pos, k_pos: global positions of the rows (checked against the mask's
 *                 n_pos: every row's position must lie in [0, n_pos)).
 *   scale: multiplies q.k before the softmax (usually 1/sqrt(d)).
 *   o_out / lse_out: fp32 device arrays [H][n_q][d] and [H][n_q], contiguous.
 *   accumulate = 0: write the partial (O, LSE).
 *   accumulate = 1: read the running (O, LSE) already in o_out/lse_out and
 *                   replace it by its merge with this partial, in fp32.
 * Zero-sized blocks (n_q == 0 or n_k == 0) are a successful no-op when
 * accumulate is set and write (0, -inf) rows otherwise. */
int cpattn_partial(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                   const cpattn_mask* mask, cpattn_posmap q_pos, cpattn_posmap k_pos, float scale,
                   float* o_out, float* lse_out, int accumulate, void* stream);

/* Merge of n_parts partial results ("Context Parallelism in ART", section 03,
 * the stable form with m = max of the LSEs), all fp32 in device memory:
 *   o_parts[p]: [n_rows][d], lse_parts[p]: [n_rows]   (n_rows = heads*rows)
 *   o_out: [n_rows][d], lse_out: [n_rows]; may alias o_parts[0]/lse_parts[0].
 * o_parts and lse_parts are HOST arrays of device pointers.  Rows whose
 * every part has LSE = -inf give (0, -inf).  1 <= n_parts <= 64, d >= 1. */
int cpattn_merge(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                 int64_t n_rows, int64_t d, float* o_out, float* lse_out, void* stream);

/* Ring emulation on one GPU (K/V blocks may have fewer heads than the
 * queries, as in cpattn_partial).  N ranks each hold one query block q_blocks[r]
 * and one key/value block (k_blocks[r], v_blocks[r]) with positions pos[r].
 * For each rank r in ranks[0..n_ranks_run), every round k = 0..N-1 computes
 * the partial of q_blocks[r] against the K/V block of rank (r - k) mod N and
 * merges it into o_out[r]/lse_out[r] (round 0 writes, later rounds merge).
 * Rounds in which no query of r sees any key of the visiting block are
 * skipped (their merge would be the identity).  The ranks are independent, so
 * one launch runs the next non-empty round of every rank (as the ranks of a
 * real ring run their rounds concurrently); each rank's rounds are still
 * merged in ring order.
 *   q_blocks, k_blocks, v_blocks, pos: host arrays of N entries.
 *   o_out, lse_out: host arrays of N device pointers ([H][n_q_r][d] and
 *                   [H][n_q_r] fp32); entries of ranks not run may be NULL.
 *   ranks: host array of rank ids to run (NULL with n_ranks_run = N: all).
 * 1 <= N <= 64. */
int cpattn_ring_emulate(int N, const cpattn_tensor* q_blocks, const cpattn_tensor* k_blocks,
                        const cpattn_tensor* v_blocks, const cpattn_posmap* pos,
                        const int* ranks, int n_ranks_run, const cpattn_mask* mask, float scale,
                        float* const* o_out, float* const* lse_out, void* stream);

/* Ring emulation where each rank holds C chunks of the sequence, for
 * layouts that are not one affine run per rank.  The zig-zag (folded) layout
 * of the causal load-balancing section of the ML-systems lesson splits the
 * sequence into 2N chunks and gives rank r chunks r and 2N-1-r (C = 2), so
 * that every rank does the same causal work (the lesson's worked example (c):
 * 9 pairs per rank instead of 3, 7, 11, 15).
 *   Arrays of N*C entries, chunk c of rank r at index r*C + c: q_chunks,
 *   k_chunks, v_chunks (tensors as in cpattn_ring_emulate; a chunk's queries
 *   and keys sit at the same positions pos[r*C + c]) and o_out, lse_out
 *   (device pointers, [H][n_tok][d] and [H][n_tok] fp32 per chunk; entries of
 *   ranks not run may be NULL).
 * In round k every chunk of rank r meets every key chunk of rank (r - k) mod N
 * (in chunk order); pairs with no visible key are skipped; the partials of a
 * query chunk merge in that order.  C = 1 is cpattn_ring_emulate.
 * 1 <= N <= 64, 1 <= C <= 8.  Errors as for cpattn_ring_emulate. */
int cpattn_ring_emulate_chunks(int N, int C, const cpattn_tensor* q_chunks, const cpattn_tensor* k_chunks,
                               const cpattn_tensor* v_chunks, const cpattn_posmap* pos,
                               const int* ranks, int n_ranks_run, const cpattn_mask* mask, float scale,
                               float* const* o_out, float* const* lse_out, void* stream);

/* Per-rank work report of a ring (host only; no device work).  For N ranks
 * with C chunks each (chunk r*C + c has n_tok[r*C + c] tokens at positions
 * pos[r*C + c]), work[r*N + k] receives the number of visible (query, key)
 * pairs, per head, of rank r's queries against the keys held by rank
 * (r - k) mod N, i.e. rank r's work in round k (ML-systems lesson, causal
 * load balancing: a ring round lasts as long as its busiest rank).  Counted
 * exactly from the mask with integer arithmetic.  n_tok, pos and work are
 * host arrays (N*C, N*C and N*N entries).  EINVAL on bad sizes or positions
 * outside the mask. */
int cpattn_ring_plan(int N, int C, const int64_t* n_tok, const cpattn_posmap* pos, const cpattn_mask* mask,
                     int64_t* work);

/* Learned attention sink, applied once to a complete (fully merged) result
 * ("Context Parallelism in ART", section 06: a per-head sink logit adds
 * probability mass with zero value to the softmax denominator, and belongs to
 * the whole query, not to every ring stage):
 *   L' = logaddexp(L, a_h),  O' = O * exp(L - L'),  in place.
 *   o: [n_heads][n_rows][d] fp32 (16-byte aligned), lse: [n_heads][n_rows]
 *   fp32, sink_logits: [n_heads] fp32 in natural-log units; all device memory.
 * A row with no visible key (L = -inf) becomes (0, a_h).  Applying it to each
 * partial before merging would count the sink once per partial; call it after
 * the last merge.  EUNSUPPORTED if d % 4 != 0 or misaligned; EINVAL on bad
 * sizes or NULL pointers. */
int cpattn_apply_sink(float* o, float* lse, const float* sink_logits, int64_t n_heads, int64_t n_rows,
                      int64_t d, void* stream);

/* ---- backward ("Context Parallelism in ART", section 04) ----------------
 * Gradients use the global softmax derivative: for a query with complete
 * output o and log-sum-exp L (over ALL of its visible keys, i.e. the merged
 * forward result) and output gradient g, D = dot(g, o) and for every visible
 * key j of any stage: p_j = exp(s_j - L), dS_j = p_j (dot(g, v_j) - D),
 * dV_j += p_j g, dQ += scale dS_j k_j, dK_j += scale dS_j q.  A stage needs
 * only its own key block plus the query's L and D, and the stages'
 * contributions add.  Sliding-window descriptors apply their window here as in
 * the forward (a key outside a query's window gets no gradient from it). */

/* delta[h][i] = dot(dout[h][i][:], o[h][i][:]) for a complete output o
 * (fp32 [H][n][d], contiguous, 16-byte aligned) and output gradient dout
 * (bf16 or fp32, same shape); delta: fp32 [H][n] device memory, 4-byte
 * aligned.  EUNSUPPORTED for a misaligned o or delta. */
int cpattn_backward_delta(const float* o, const cpattn_tensor* dout, float* delta, void* stream);

/* Gradient contributions of one (query block, key/value block) pair, ADDED to
 * dq (fp32 [H][n_q][d]), dk and dv (fp32 [H_kv][n_k][d]); all contiguous
 * device memory that the caller zero-fills before the first contribution.
 * q, k, v, mask, positions and scale as in cpattn_partial; lse and delta:
 * fp32 [H][n_q], the queries' complete LSE and D; dout: the output gradient
 * of the queries (dtype, heads, tokens and d of q).  Grouped-query K/V are
 * supported (every query head's contribution is added to its K/V head). */
int cpattn_partial_backward(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                            const cpattn_mask* mask, cpattn_posmap q_pos, cpattn_posmap k_pos, float scale,
                            const float* lse, const float* delta, const cpattn_tensor* dout,
                            float* dq, float* dk, float* dv, void* stream);

/* Backward of the ring emulated by cpattn_ring_emulate (all N ranks): in
 * round k rank r's queries meet the keys of rank (r - k) mod N; rank r's dQ
 * stays in dq[r], and the dK/dV contributions for rank b's keys, which a real
 * ring returns to their owner, are added to dk[b], dv[b].  Each round is one
 * dQ launch and one dK/dV launch (a round pairs every key block with one
 * query block, so no two jobs of a launch write the same rows).  Host arrays
 * of N entries: q_blocks, k_blocks, v_blocks, pos, lse, delta, dout_blocks,
 * dq, dk, dv (device pointers, zero-filled by the caller). */
int cpattn_ring_backward(int N, const cpattn_tensor* q_blocks, const cpattn_tensor* k_blocks,
                         const cpattn_tensor* v_blocks, const cpattn_posmap* pos, const cpattn_mask* mask,
                         float scale, const float* const* lse, const float* const* delta,
                         const cpattn_tensor* dout_blocks, float* const* dq, float* const* dk, float* const* dv,
                         void* stream);

/* Backward of cpattn_ring_emulate_chunks (all N ranks, C chunks each, chunk
 * c of rank r at index r*C + c; zig-zag: C = 2): in round k every query chunk
 * of rank r meets every key chunk of rank (r - k) mod N; dQ stays with the
 * query chunk, dK/dV are added to the key chunk's buffers.  Per round, C dQ
 * launches (one per key chunk index, so no two jobs write the same dQ rows)
 * and C dK/dV launches (one per query chunk index).  Host arrays of N*C
 * entries as in cpattn_ring_backward.  1 <= N <= 64, 1 <= C <= 8; C = 1 is
 * cpattn_ring_backward. */
int cpattn_ring_backward_chunks(int N, int C, const cpattn_tensor* q_chunks, const cpattn_tensor* k_chunks,
                                const cpattn_tensor* v_chunks, const cpattn_posmap* pos, const cpattn_mask* mask,
                                float scale, const float* const* lse, const float* const* delta,
                                const cpattn_tensor* dout_chunks, float* const* dq, float* const* dk,
                                float* const* dv, void* stream);

/* Adjoints of cpattn_merge ("Context Parallelism in ART", section 04): for
 * the merged result (o, lse) of parts (o_p, lse_p), w_p = exp(lse_p - lse),
 * an output gradient g_o and an optional LSE gradient g_lse (NULL: zero),
 *   g_o_parts[p]   = w_p g_o,
 *   g_lse_parts[p] = w_p (dot(g_o, o_p - o) + g_lse).
 * A part with lse_p = -inf (or a row with lse = -inf) gets w_p = 0.  Rows of
 * d fp32 values, as in cpattn_merge: o_parts, lse_parts, g_o_parts and
 * g_lse_parts are HOST arrays of n_parts device pointers; o, g_o and every O
 * array 16-byte aligned, d % 4 == 0 (else EUNSUPPORTED).  Outputs are written
 * (not added).  1 <= n_parts <= 64. */
int cpattn_merge_backward(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                          int64_t n_rows, int64_t d, const float* o, const float* lse, const float* g_o,
                          const float* g_lse, float* const* g_o_parts, float* const* g_lse_parts, void* stream);

/* Adjoints of cpattn_apply_sink (same page, section 06), from the buffers it
 * leaves: o = y = w O and lse = L' = logaddexp(L, a_h), where O, L are the
 * result before the sink.  With u = exp(a_h - L') (the sink's share of the
 * softmax mass) and w = 1 - u, for an output gradient g_o:
 *   g_o_in  = w g_o                              (gradient of O)
 *   g_lse_in = u dot(g_o, y)   = w (1 - w) dot(g_o, O)   (gradient of L)
 *   g_sink[h] = -sum over the head's rows of g_lse_in
 * (L' itself is taken as unused downstream).  o, g_o, g_o_in: [n_heads]
 * [n_rows][d] fp32, 16-byte aligned, d % 4 == 0; lse, g_lse_in: [n_heads]
 * [n_rows]; sink_logits, g_sink: [n_heads]; all device memory, outputs
 * written.  The per-head sum runs in a fixed order (deterministic). */
int cpattn_sink_backward(const float* o, const float* lse, const float* sink_logits, int64_t n_heads,
                         int64_t n_rows, int64_t d, const float* g_o, float* g_o_in, float* g_lse_in,
                         float* g_sink, void* stream);

/* Measurement helper, not a step of the attention path: streams `bytes` of
 * device memory once, 16 bytes per lane and step, with `grid` workgroups of
 * 256 lanes looping grid-stride (grid <= 0: one lane per 16 bytes, no loop).
 * It gives the HBM-bound kernels above a bandwidth ceiling measured on the
 * same device (the HBM3E figure of the MI355X data sheet is not reached by a
 * plain stream).  kind 0 reads src; dst must hold 16 bytes, which are left
 * as they are for zero-filled or random data.  kind 1 copies src to dst
 * (the two must not overlap).  src and dst are 16-byte aligned device
 * pointers owned by the caller; bytes is a multiple of 16, grid <= 2^20.
 * Asynchronous on `stream`; errors as for the other calls. */
int cpattn_stream_probe(int kind, const void* src, void* dst, int64_t bytes, int grid, void* stream);

/* Message for the calling thread's last failed call ("" if none). */
const char* cpattn_last_error(void);

/* (major << 16) | minor */
int cpattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
