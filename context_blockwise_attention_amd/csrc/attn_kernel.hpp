// attn_kernel.hpp -- partial blockwise attention on gfx950 (CDNA4) MFMA.
//
// One workgroup = 4 waves = kBM = 128 query rows of one head of one job; each
// wave owns 32 query rows.  The workgroup walks the key tiles (BN keys each)
// that its queries can see, stages K and V^T in LDS (double buffered), and
// keeps an online softmax per query row in registers ("Context Parallelism in
// ART", section 02: the FlashAttention-style tile loop that never writes the
// probability matrix, returning O and the log-sum-exp).  The epilogue either
// writes (O, LSE) or merges it into a running (O, LSE) with the stable
// log-sum-exp merge (same page, section 03), all in fp32.
//
// Layout choices for 64-wide wavefronts and the 32x32 MFMA:
//  * Scores are computed transposed, S^T = K Q^T, so that MFMA output lane l
//    holds ONE query (column l % 32) and 16 keys: the row max and row sum
//    need one cross-lane exchange (lane l with lane l ^ 32) per tile.
//  * K rows are fed to the MFMA in a permuted order (kperm) chosen so that the
//    16 score values a lane holds are exactly the 8-key groups that the next
//    MFMA (O^T += V^T P^T) wants as its B operand: P never leaves registers.
//  * V is transposed while it is staged into LDS (V^T rows = head dims), so
//    the A operand of O^T += V^T P^T is one 16-byte LDS read per lane.
//  * O^T accumulators: lane l holds its query's D/2 output values.
//  * The running max is only raised when a tile's max exceeds it by more than
//    kTau (in the base-2 exponent), so the accumulator rescale -- a pass
//    over every accumulator register -- is rare; probabilities stay below
//    2^kTau, far inside fp32 and bf16 range, and the final normalisation uses
//    the same stale max for numerator and denominator, so the result is the
//    same softmax.  (The bf16 kernel goes one step further and skips the
//    tile's max while the probabilities against the stale reference stay
//    small: see softmax_phase in attn_bf16_kernel.hpp.)
//  * Global loads go through buffer resources: 32-bit offsets, and rows past
//    the end of a block read as zero (those keys are masked out).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxJobs = 16;
constexpr int kThreads = 256;  // 4 waves
constexpr int kBM = 128;       // query rows per workgroup
constexpr float kTau = 8.0f;   // lazy-rescale threshold (base-2 exponent)
constexpr float kSumCap = 65536.0f;   // bf16 kernel: largest per-lane tile sum kept without the tile max (2^16)
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit dwords (gfx9 family)

enum MaskKind : int32_t { kCausal = 0, kTree = 1 };

// One (query block, key/value block, output) triple of a launch.
struct JobArgs {
    const void* q;
    const void* k;
    const void* v;
    float* o;
    float* lse;
    int64_t q_sh, k_sh, v_sh;      // head strides (elements)
    int32_t q_st, k_st, v_st;      // token strides (elements)
    int32_t qbase, qstride;        // global position of query row i: qbase + qstride * i
    int32_t kbase, kstride;        // same for key rows
    int32_t n_q, n_k;
    int32_t accumulate;
    int32_t q_tiles;   // ceil(n_q / rows per workgroup)
    int32_t kv_group;  // query heads per key/value head (grouped-query attention; 1 = one K/V head per query head)
};

struct MaskArgs {
    const int32_t* seg;     // [n_pos] segment of each position (tree only)
    const int4* segtab;     // [n_seg] {run_start, run_end, parent, subtree_end}
    const int32_t* end;     // [n_pos] subtree end of each position (tree only)
    const int32_t* lpos;    // [n_pos] logical (root-to-leaf) position (tree with a window only)
    int32_t n_pos;
    int32_t kind;
    int32_t window;         // sliding window in logical positions (0 = none)
};

struct LaunchArgs {
    JobArgs jobs[kMaxJobs];
    MaskArgs mask;
    int32_t n_jobs;
    int32_t heads;
    int32_t total_wg;        // work slots = grid size (some slots may be empty)
    int32_t sum_q_tiles;     // sum of q_tiles over the jobs
    int32_t heads_per_xcd;   // ceil(heads / 8) with at least 8 heads, else 0
    float scale_log2;        // scale * log2(e)
};

// ---------------------------------------------------------------------------
// Work slot of workgroup `bid` -> (job, head, q-tile), or false for an empty
// slot.  Workgroups are dispatched round-robin over the 8 XCDs (bid % 8).
// With at least 8 heads, XCD x runs one eighth of the heads of every job
// (contiguous ranges when the head count divides by 8, else h = x mod 8):
// every XCD gets the same share of every job, so no XCD is left with only the
// light job of a launch.  Within an XCD the items run one (job, head) group
// after another, the group's q-tiles heaviest (last) first, so the ~32
// workgroups in flight on the XCD read the same head's K/V and share its L2.
// With fewer heads the same group order is dealt round-robin over the XCDs.
// An XCD starts its workgroups strictly in order and deals them round-robin
// over its four shader engines (measured with per-workgroup hardware ids), so
// slot p and slot p + 4 land on the same engine.  With q-tiles in plain
// descending order one engine would always get the heaviest of every four
// and fall behind, and the in-order dealer would hold the other engines' free
// CUs waiting for it (on the diagonal launch of the 64K row 5% of the CU time
// went to such gaps).  So the second half of every block of eight is
// reversed: slots p and p + 4 then hold tiles whose weights (linear in the
// q-tile on a causal diagonal) sum to the same value in every block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool work_item(const LaunchArgs& a, int bid, int* job, int* head, int* qtile) {
    const bool by_xcd = a.heads_per_xcd > 0;
    const int x = bid & 7;
    int p = by_xcd ? (bid >> 3) : bid;
    const int hg = by_xcd ? a.heads_per_xcd : a.heads;   // head groups per job seen by this slot stream
    // heads divisible by 8: XCD x runs the contiguous heads [x*hg, (x+1)*hg),
    // so the query heads of one K/V head (grouped-query attention) share as
    // few L2s as possible; otherwise heads h = x (mod 8), which balances the
    // XCDs when the count is uneven
    const bool ranges = by_xcd && (a.heads & 7) == 0;
    for (int j = 0; j < a.n_jobs; ++j) {
        const int qt = a.jobs[j].q_tiles;
        const int n = hg * qt;
        if (p < n) {
            const int hi = p / qt;
            const int r = p - hi * qt;
            const int h = !by_xcd ? hi : ranges ? x * hg + hi : x + 8 * hi;
            if (h >= a.heads) return false;
            *job = j;
            *head = h;
            const int rb = ((r & 4) && (r | 7) < qt) ? (r ^ 3) : r;   // complete blocks of 8 only
            *qtile = qt - 1 - rb;
            return true;
        }
        p -= n;
    }
    return false;
}

// ---------------------------------------------------------------------------
// element traits
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
    using op8 = bf16x8;                      // 8 consecutive k values for one MFMA lane
    static constexpr int kEPC = 8;           // elements per 16-byte chunk
    static constexpr int kPad = 8;           // LDS row padding (elements)
    static __device__ __forceinline__ f32x16 mfma_k16(const op8& a, const op8& b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Elem<float> {
    using op8 = f32x8;
    static constexpr int kEPC = 4;
    static constexpr int kPad = 4;
    // 16 values of k split into 8 fp32 MFMAs of k = 2; lane group g supplies
    // element 8g + e in the e-th one, identically for A and B.
    static __device__ __forceinline__ f32x16 mfma_k16(const op8& a, const op8& b, f32x16 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
};

template <typename T, int D, int BN>
struct Tile {
    static constexpr int EPC = Elem<T>::kEPC;
    static constexpr int KS = D + Elem<T>::kPad;   // K row stride (elements) in LDS
    static constexpr int VS = BN + Elem<T>::kPad;  // V^T row stride (elements) in LDS
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE_BYTES = (K_ELEMS + V_ELEMS) * (int)sizeof(T) + 2 * BN * 4;   // + horizons, logical positions
    static constexpr int K_CHUNKS = BN * D / EPC;            // 16-byte chunks of a K tile
    static constexpr int K_PER_THREAD = (K_CHUNKS + kThreads - 1) / kThreads;
    static constexpr int KG = BN / 4;                          // 4-key groups of a V tile
    static constexpr int V_GROUPS = KG * (D / EPC);            // 4 keys x EPC dims each
    static constexpr int V_PER_THREAD = (V_GROUPS + kThreads - 1) / kThreads;
    static constexpr int KB = BN / 32;                         // 32-key MFMA blocks per tile
    static constexpr int DSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    static constexpr int KSTEPS = BN / 16;
};

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 8 consecutive elements as one MFMA operand (16-byte aligned LDS source).
__device__ __forceinline__ bf16x8 load_op8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load_op8(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::op8 as_op8(u32x4 lo, u32x4 hi);
template <>
__device__ __forceinline__ bf16x8 as_op8<__bf16>(u32x4 lo, u32x4) { return __builtin_bit_cast(bf16x8, lo); }
template <>
__device__ __forceinline__ f32x8 as_op8<float>(u32x4 lo, u32x4 hi) {
    f32x4 a = __builtin_bit_cast(f32x4, lo), b = __builtin_bit_cast(f32x4, hi);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// max / sum of a value with the same value of lane l ^ 32
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Candidate key tiles of one query tile.
//
// With the row stored in depth-first preorder, key x is visible to query y
// iff x <= y < end[x].  For a query tile covering positions [y0, y1] every
// visible key lies in the union of: the positions [run_start(s), y1] with
// s = seg(y0) (its own segment, plus anything after y0 inside the tile), and
// the runs of the strict ancestors of s.  A key of a segment starting inside
// (y0, y1] is covered by the first range; any ancestor of such a segment whose
// run starts at or before y0 is an ancestor-or-self of s.  The ranges are
// walked from s up to the root, tiles in descending order, and a tile already
// visited through a later range is not visited again.  All state is
// wave-uniform (scalar registers).
// ---------------------------------------------------------------------------
// The key block's position map and size: what the tile walk needs of a job
// (kept apart so that the walk's state fits in a few scalar registers).
struct KeyBlock {
    int32_t kbase, kstride, n_k;
};

// Segment-table entry, read through the scalar cache (the index is
// wave-uniform and the table is constant for the launch).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 seg_entry(const MaskArgs& M, int s) {
    return ((const __attribute__((address_space(4))) i32x4*)M.segtab)[s];
}

// Each range of key positions becomes a range of tiles [t_lo, t] (clipped
// below the tiles already emitted), and the tiles [fa, fb] of it are full
// (every key visible to every query row of the tile).  Both are decided once
// per range, so producing a tile is a compare and a decrement; moving to the
// next range is the rare path.
//
// With a sliding window (WIN; "Context Parallelism in ART", section 06: a
// query sees the keys within `window` tokens of its logical, root-to-leaf,
// position), each range is first clipped to the keys some query of the tile
// can reach (logical position >= the tile's lowest query position - window
// + 1), and a tile is full only if its first key lies within the window of
// the tile's highest query position.  Inside one segment's run the logical
// position is the physical one minus the run's offset `lbase` (run start
// minus its logical position; 0 for a causal mask).
template <int BN, bool WIN = false>
struct TileCursor {
    int t;        // next tile to emit; the range is exhausted when t < t_lo
    int t_lo;     // lowest tile of the current range
    int fa, fb;   // full tiles of the current range (none when fa > fb)
    int seg;      // segment whose run is the current range (tree); -1 = no further range
    int lq_min, lq_max;   // WIN: bounds of the query tile's logical positions

    __device__ __forceinline__ static int ceil_div(int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }
    __device__ __forceinline__ static int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
    __device__ __forceinline__ static int64_t ceil_div64(int64_t a, int64_t b) {
        return a >= 0 ? (a + b - 1) / b : -((-a) / b);
    }

    // Enters the key positions [pa, pb] inside the block.  A tile is full if
    // it lies inside the range, full_ok holds (every key's subtree contains
    // the whole query tile) and its last key index is at most j_last (and,
    // with a window, its first key is within reach of every query).  False
    // (state unchanged) if no tile below the ones emitted is left.
    __device__ __forceinline__ bool set_range(int pa, int pb, bool full_ok, int j_last, const KeyBlock& J,
                                              const MaskArgs& M, int lbase) {
        if (WIN) {
            pa = (int)max((int64_t)pa, (int64_t)lq_min - M.window + 1 + lbase);
            if (pa > pb) return false;
        }
        int lo, hi;
        if (J.kstride == 1) {
            lo = pa - J.kbase;
            hi = pb - J.kbase;
        } else {
            lo = ceil_div(pa - J.kbase, J.kstride);
            hi = floor_div(pb - J.kbase, J.kstride);
        }
        lo = max(lo, 0);
        hi = min(hi, J.n_k - 1);
        if (lo > hi) return false;
        const int th = min(hi / BN, t);
        const int tl = lo / BN;
        if (th < tl) return false;
        t = th;
        t_lo = tl;
        // tile u is full iff u*BN >= lo, u*BN + BN - 1 <= min(hi, j_last)
        // (j_last + 1 <= 0 leaves fb < 0: no tile full)
        fa = full_ok ? (lo + BN - 1) / BN : 1;
        fb = full_ok ? min(hi + 1, j_last + 1) / BN - 1 : 0;
        if (WIN && full_ok) {
            // first key index within the window of every query of the tile
            const int64_t thr = (int64_t)lq_max - M.window + 1 + lbase;
            const int64_t jthr = max((int64_t)0, ceil_div64(thr - J.kbase, J.kstride));
            fa = (int)min((int64_t)0x3fffffff, max((int64_t)fa, (jthr + BN - 1) / BN));
        }
        return true;
    }

    // run offset of segment s's run: run start minus its logical position
    __device__ __forceinline__ static int run_lbase(const MaskArgs& M, int run_start) {
        return run_start - ((const __attribute__((address_space(4))) int32_t*)M.lpos)[run_start];
    }

    // The first range: the query tile's own run up to y1 (its keys after y0
    // are not visible to the first query row: j_last is y0's key index).
    __device__ void init(const KeyBlock& J, const MaskArgs& M, int y0, int y1) {
        t = 0x7ffffffe;   // nothing emitted yet
        t_lo = 0x7fffffff;
        seg = -1;
        const int j_own = J.kstride == 1 ? y0 - J.kbase : floor_div(y0 - J.kbase, J.kstride);
        if (M.kind == kCausal) {
            if (WIN) {
                lq_min = y0;
                lq_max = y1;
            }
            set_range(0, y1, true, j_own, J, M, 0);
            return;
        }
        seg = ((const __attribute__((address_space(4))) int32_t*)M.seg)[y0];
        const i32x4 st = seg_entry(M, seg);
        int lbase = 0;
        if (WIN) {
            const auto* lp = (const __attribute__((address_space(4))) int32_t*)M.lpos;
            const bool one_seg = ((const __attribute__((address_space(4))) int32_t*)M.seg)[y1] == seg;
            // a tile that crosses a segment boundary keeps every key in reach
            // and has no full tile (its positions are not one logical run)
            lq_min = one_seg ? lp[y0] : -(1 << 30);
            lq_max = one_seg ? lp[y1] : (1 << 30);
            lbase = run_lbase(M, st.x);
        }
        set_range(st.x, y1, st.w > y1, j_own, J, M, lbase);
    }

    // Moves to the runs of the ancestor segments until one has a tile left.
    __device__ bool advance(const KeyBlock& J, const MaskArgs& M, int y1) {
        while (seg >= 0) {
            seg = seg_entry(M, seg).z;
            if (seg < 0) break;
            const i32x4 sp = seg_entry(M, seg);
            if (set_range(sp.x, sp.y - 1, sp.w > y1, 0x7ffffffe, J, M, WIN ? run_lbase(M, sp.x) : 0)) return true;
        }
        return false;
    }

    // Produces the next tile; returns false when the walk is over.
    __device__ __forceinline__ bool next(const KeyBlock& J, const MaskArgs& M, int y1, int* tile, int* full) {
        if (t < t_lo && !advance(J, M, y1)) return false;
        *tile = t;
        *full = (t >= fa) & (t <= fb);
        --t;
        return true;
    }
};

// ---------------------------------------------------------------------------
// Epilogue shared by the kernels: lane (query qi, half g) holds the O^T
// accumulators of its query (dims b*32 + (i/4)*8 + g*4 + i%4), the running
// max m_run (base 2, scaled) and its half of the denominator.  Writes the
// partial (O, LSE), or merges it into the running (O, LSE) already stored:
// M = max(L_old, L_new), w = exp(L - M), O = (w_old O_old + w_new O_new) /
// (w_old + w_new), L = M + log(w_old + w_new).  LSE is a natural log.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void write_result(const JobArgs& J, int head, int qi, int g, const f32x16* acc,
                                             float m_run, float l_run) {
    constexpr int DBLK = D / 32;
    const float l_tot = xhalf_sum(l_run);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_new = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    if (qi >= J.n_q) return;
    float* orow = J.o + (int64_t)head * J.n_q * D + (int64_t)qi * D;
    float* lrow = J.lse + (int64_t)head * J.n_q + qi;
    if (!J.accumulate) {
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 v = {acc[b][q4 * 4 + 0] * inv, acc[b][q4 * 4 + 1] * inv, acc[b][q4 * 4 + 2] * inv,
                                 acc[b][q4 * 4 + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + b * 32 + q4 * 8 + g * 4) = v;
            }
        if (g == 0) *lrow = lse_new;
    } else {
        // the running LSE and O are read together (one memory round trip)
        f32x4 old[DBLK * 4];
        const float lse_old = *lrow;
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                old[b * 4 + q4] = *reinterpret_cast<const f32x4*>(orow + b * 32 + q4 * 8 + g * 4);
        // Branch-free, so that the loads above are not sunk behind a test of
        // the LSE: when both sides are empty (M = -inf) the weights are 0 and
        // the row is rewritten as (0, -inf).
        const float M = fmaxf(lse_old, lse_new);
        const bool none = M == -INFINITY;
        const float wa = none ? 0.f : expf(lse_old - M), wb = none ? 0.f : expf(lse_new - M);
        const float z = wa + wb;
        const float rz = none ? 0.f : 1.f / z;
        const float wbn = wb * inv;
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (wa * old[b * 4 + q4][e] + wbn * acc[b][q4 * 4 + e]) * rz;
                *reinterpret_cast<f32x4*>(orow + b * 32 + q4 * 8 + g * 4) = v;
            }
        if (g == 0) *lrow = none ? -INFINITY : M + logf(z);
    }
}

// ---------------------------------------------------------------------------
// the register-staged kernel (fp32 inputs; the bf16 path is attn_bf16_kernel.hpp)
// ---------------------------------------------------------------------------
template <typename T, int D, int BN, bool WIN>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
partial_attention_kernel(const LaunchArgs args) {
    using E = Elem<T>;
    using TL = Tile<T, D, BN>;
    using op8 = typename E::op8;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // ---- work item ------------------------------------------------------
    int ji, head, qtile;
    if (!work_item(args, blockIdx.x, &ji, &head, &qtile)) return;
    // integer division runs on the vector ALU; keep the results scalar
    ji = wave_uniform(ji);
    head = wave_uniform(head);
    qtile = wave_uniform(qtile);
    const JobArgs& J = args.jobs[ji];
    const KeyBlock kblk{J.kbase, J.kstride, J.n_k};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_uniform(tid >> 6);   // scalar: the wave index is uniform per wave
    const int r32 = lane & 31;
    const int g = lane >> 5;

    const int q_first = qtile * kBM;
    const int q_last = min(q_first + kBM, J.n_q) - 1;
    const int y0 = J.qbase + J.qstride * q_first;
    const int y1 = J.qbase + J.qstride * q_last;

    // this lane's query row
    const int qi = q_first + wave * 32 + r32;
    const int ypos = J.qbase + J.qstride * qi;
    // sliding window (see the bf16 kernel): causal -> lowest visible key
    // index; tree -> the query's logical position
    const bool tree_q = args.mask.kind == kTree;
    int jlo = 0, ly = 0;
    if (WIN) {
        if (tree_q) {
            ly = qi < J.n_q ? args.mask.lpos[ypos] : 0;
        } else {
            const int lowest = ypos - args.mask.window + 1 - J.kbase;
            jlo = lowest <= 0 ? 0 : (lowest + J.kstride - 1) / J.kstride;
        }
    }

    const T* qh = reinterpret_cast<const T*>(J.q) + head * J.q_sh;
    const int kv_head = head / J.kv_group;
    const T* kh = reinterpret_cast<const T*>(J.k) + kv_head * J.k_sh;
    const T* vh = reinterpret_cast<const T*>(J.v) + kv_head * J.v_sh;
    const auto qr = make_rsrc(qh, ((J.n_q - 1) * J.q_st + D) * (int)sizeof(T));
    const auto kr = make_rsrc(kh, ((J.n_k - 1) * J.k_st + D) * (int)sizeof(T));
    const auto vr = make_rsrc(vh, ((J.n_k - 1) * J.v_st + D) * (int)sizeof(T));

    // Q^T operand: 8 consecutive dims per lane per 16-dim step (rows past the
    // block read as zero; they are never stored)
    op8 qreg[TL::DSTEPS];
    {
        const int qoff = qi * J.q_st * (int)sizeof(T);
#pragma unroll
        for (int s = 0; s < TL::DSTEPS; ++s) {
            const int off = qoff + (s * 16 + 8 * g) * (int)sizeof(T);
            u32x4 lo = buf_load16(qr, off);
            u32x4 hi = sizeof(T) == 4 ? buf_load16(qr, off + 16) : lo;
            qreg[s] = as_op8<T>(lo, hi);
        }
    }

    // permuted K row fed by this lane (see the header comment)
    const int kperm_i = (r32 >> 3) * 4 + (r32 & 3);
    const int kperm = (kperm_i >> 3) * 16 + ((r32 & 7) >> 2) * 8 + (kperm_i & 7);

    f32x16 acc[TL::DBLK];
#pragma unroll
    for (int b = 0; b < TL::DBLK; ++b) acc[b] = f32x16{};
    float m_run = -INFINITY;   // running (lazily raised) max of scaled scores, base 2
    float l_run = 0.f;         // this lane's half of the running denominator

    // ---- staging registers -------------------------------------------------
    // K: thread chunk c -> row c / (D/EPC), column chunk c % (D/EPC).
    // V: thread group gi -> keys 4*(gi % KG) .. +3, dims EPC*(gi / KG) .. ;
    //    consecutive lanes take consecutive key groups so that the transposed
    //    LDS writes of one instruction fill consecutive 8-byte slots of a row.
    u32x4 kreg[TL::K_PER_THREAD];
    u32x4 vreg[TL::V_PER_THREAD][4];
    int endreg = 0, lreg = 0;

    const bool tree = args.mask.kind == kTree;
    auto stage_load = [&](int tile) {
        const int j0 = tile * BN;
#pragma unroll
        for (int i = 0; i < TL::K_PER_THREAD; ++i) {
            const int c = tid + i * kThreads;
            if (c < TL::K_CHUNKS) {
                const int row = c / (D / TL::EPC), col = c % (D / TL::EPC);
                kreg[i] = buf_load16(kr, ((j0 + row) * J.k_st + col * TL::EPC) * (int)sizeof(T));
            }
        }
#pragma unroll
        for (int i = 0; i < TL::V_PER_THREAD; ++i) {
            const int gi = tid + i * kThreads;
            if (gi < TL::V_GROUPS) {
                const int kg = gi % TL::KG, dc = gi / TL::KG;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vreg[i][r] = buf_load16(vr, ((j0 + 4 * kg + r) * J.v_st + dc * TL::EPC) * (int)sizeof(T));
            }
        }
        if (tree && tid < BN) {
            const int j = j0 + tid;
            endreg = j < J.n_k ? args.mask.end[J.kbase + J.kstride * j] : (int)0x80000000;
        }
        if (WIN && tree && tid >= BN && tid < 2 * BN) {
            const int j = j0 + tid - BN;
            lreg = j < J.n_k ? args.mask.lpos[J.kbase + J.kstride * j] : 0;
        }
    };

    auto stage_store = [&](int buf) {
        T* Ks = reinterpret_cast<T*>(smem + buf * TL::STAGE_BYTES);
        T* Vt = Ks + TL::K_ELEMS;
        int* Es = reinterpret_cast<int*>(Vt + TL::V_ELEMS);
#pragma unroll
        for (int i = 0; i < TL::K_PER_THREAD; ++i) {
            const int c = tid + i * kThreads;
            if (c < TL::K_CHUNKS) {
                const int row = c / (D / TL::EPC), col = c % (D / TL::EPC);
                *reinterpret_cast<u32x4*>(Ks + row * TL::KS + col * TL::EPC) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < TL::V_PER_THREAD; ++i) {
            const int gi = tid + i * kThreads;
            if (gi < TL::V_GROUPS) {
                const int kg = gi % TL::KG, dc = gi / TL::KG;
                if constexpr (sizeof(T) == 2) {
                    // 4 keys x 8 dims -> 8 dims x 4 keys: each output is the 16-bit
                    // half of one dim from each key (v_perm_b32 byte selects:
                    // low half -> bytes 1:0, high half -> bytes 3:2)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int w32 = e >> 1;
                        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                        const uint32_t lo = __builtin_amdgcn_perm(vreg[i][1][w32], vreg[i][0][w32], sel);
                        const uint32_t hi = __builtin_amdgcn_perm(vreg[i][3][w32], vreg[i][2][w32], sel);
                        *reinterpret_cast<u32x2*>(Vt + (dc * 8 + e) * TL::VS + 4 * kg) = u32x2{lo, hi};
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const u32x4 col = {vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
                        *reinterpret_cast<u32x4*>(Vt + (dc * 4 + e) * TL::VS + 4 * kg) = col;
                    }
                }
            }
        }
        if (tree && tid < BN) Es[tid] = endreg;
        if (WIN && tree && tid >= BN && tid < 2 * BN) Es[tid] = lreg;   // Ls = Es + BN
    };

    // ---- tile walk ------------------------------------------------------------
    TileCursor<BN, WIN> cur;
    cur.init(kblk, args.mask, y0, y1);
    int tile, full;
    bool have = cur.next(kblk, args.mask, y1, &tile, &full);
    if (have) stage_load(tile);
    int buf = 0;
    const float c2 = args.scale_log2;

    while (have) {
        stage_store(buf);
        __syncthreads();
        int ntile, nfull;
        const bool nhave = cur.next(kblk, args.mask, y1, &ntile, &nfull);
        if (nhave) stage_load(ntile);

        const T* Ks = reinterpret_cast<const T*>(smem + buf * TL::STAGE_BYTES);
        const T* Vt = Ks + TL::K_ELEMS;
        const int* Es = reinterpret_cast<const int*>(Vt + TL::V_ELEMS);

        // S^T = K Q^T for this wave's 32 queries
        f32x16 s[TL::KB];
#pragma unroll
        for (int kb = 0; kb < TL::KB; ++kb) {
            s[kb] = f32x16{};
            const T* krow = Ks + (kb * 32 + kperm) * TL::KS + 8 * g;
#pragma unroll
            for (int ds = 0; ds < TL::DSTEPS; ++ds) s[kb] = E::mfma_k16(load_op8(krow + ds * 16), qreg[ds], s[kb]);
        }

        // elementwise visibility on partial tiles: key in the block and
        // kpos <= ypos < end[kpos]
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < TL::KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int jl = kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
                    const int j = tile * BN + jl;
                    bool vis = j < J.n_k && J.kbase + J.kstride * j <= ypos;
                    if (tree) vis = vis && ypos < Es[jl];
                    if (WIN) vis = vis && (tree ? ly - Es[BN + jl] < args.mask.window : j >= jlo);
                    if (!vis) s[kb][i] = -INFINITY;
                }
            }
        }

        // online softmax for this lane's query, with a lazily raised max
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < TL::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = xhalf_max(mx) * c2;
        const bool raise = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            // lanes that keep their max multiply by exactly 1 (their max may
            // still be -inf, and -inf - -inf would be NaN)
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;   // 0 when m_run = -inf
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < TL::DBLK; ++b) acc[b] *= alpha;
            m_run = raise ? mx : m_run;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float psum = 0.f;
        op8 pb[TL::KSTEPS];
#pragma unroll
        for (int kb = 0; kb < TL::KB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m_use));
                psum += p;
                pb[kb * 2 + (i >> 3)][i & 7] = (T)p;
            }
        }
        l_run += psum;

        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < TL::KSTEPS; ++ks) {
#pragma unroll
            for (int b = 0; b < TL::DBLK; ++b)
                acc[b] = E::mfma_k16(load_op8(Vt + (b * 32 + r32) * TL::VS + ks * 16 + 8 * g), pb[ks], acc[b]);
        }

        have = nhave;
        tile = ntile;
        full = nfull;
        buf ^= 1;
    }

    // ---- epilogue: normalise, then write or merge ------------------------------
    write_result<D>(J, head, qi, g, acc, m_run, l_run);
}

}  // namespace cpattn
