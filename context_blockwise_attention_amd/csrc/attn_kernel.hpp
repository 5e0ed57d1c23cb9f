// attn_kernel.hpp -- partial blockwise attention on gfx950 (CDNA4) MFMA.
//
// One workgroup = 4 waves = BM = 128 query rows of one head of one job; each
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
//  * O^T accumulators: lane l holds its query's 64 (D=128) output values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxJobs = 16;
constexpr int kThreads = 256;  // 4 waves
constexpr int kBM = 128;       // query rows per workgroup
constexpr int kMaxTreeDepth = 1 << 20;

enum MaskKind : int32_t { kCausal = 0, kTree = 1 };

// One (query block, key/value block, output) triple of a launch.
struct JobArgs {
    const void* q;
    const void* k;
    const void* v;
    float* o;
    float* lse;
    int64_t q_sh, q_st, k_sh, k_st, v_sh, v_st;  // element strides (head, token)
    int64_t qbase, qstride, kbase, kstride;       // global positions of rows
    int32_t n_q, n_k;
    int32_t accumulate;
    int32_t q_tiles;   // ceil(n_q / kBM)
    int32_t wg_begin;  // first work item of this job
    int32_t pad_;
};

struct MaskArgs {
    const int32_t* seg;     // [n_pos] segment of each position (tree only)
    const int4* segtab;     // [n_seg] {run_start, run_end, parent, subtree_end}
    const int32_t* end;     // [n_pos] subtree end of each position (tree only)
    int64_t n_pos;
    int32_t kind;
    int32_t n_seg;
};

struct LaunchArgs {
    JobArgs jobs[kMaxJobs];
    MaskArgs mask;
    int32_t n_jobs;
    int32_t heads;
    int32_t total_wg;   // work items (the grid is rounded up to a multiple of 8)
    float scale_log2;   // scale * log2(e)
};

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
    static constexpr int STAGE_BYTES = (K_ELEMS + V_ELEMS) * (int)sizeof(T) + BN * 4;
    static constexpr int K_CHUNKS = BN * D / EPC;            // 16-byte chunks of a K tile
    static constexpr int K_PER_THREAD = (K_CHUNKS + kThreads - 1) / kThreads;
    static constexpr int V_GROUPS = (BN / 4) * (D / EPC);     // 4 keys x EPC dims each
    static constexpr int V_PER_THREAD = (V_GROUPS + kThreads - 1) / kThreads;
    static constexpr int KB = BN / 32;                         // 32-key MFMA blocks per tile
    static constexpr int DSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    static constexpr int KSTEPS = BN / 16;
};

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 8 consecutive elements as one MFMA operand (16-byte aligned source).
__device__ __forceinline__ bf16x8 load_op8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load_op8(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
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
// visited through a later range is not visited again.
// ---------------------------------------------------------------------------
template <int BN>
struct TileCursor {
    int t;           // next tile to emit (descending)
    int t_lo;        // lowest tile of the current range
    int j_lo, j_hi;  // current range in key indices, inclusive
    int visited_lo;  // lowest tile emitted so far
    int seg;         // segment whose run is the current range (tree); -1 = done
    int own;         // current range is the query tile's own range
    int full_ok;     // every key of the current range is visible to every query row
    int end_s;       // subtree end of the current segment (tree)

    __device__ __forceinline__ static int64_t ceil_div(int64_t a, int64_t b) {
        return a >= 0 ? (a + b - 1) / b : -((-a) / b);
    }
    __device__ __forceinline__ static int64_t floor_div(int64_t a, int64_t b) {
        return a >= 0 ? a / b : -((-a + b - 1) / b);
    }

    // Key index range of the positions [pa, pb] inside the block; returns
    // false if empty.
    __device__ __forceinline__ bool set_range(int64_t pa, int64_t pb, const JobArgs& J) {
        int64_t lo = ceil_div(pa - J.kbase, J.kstride);
        int64_t hi = floor_div(pb - J.kbase, J.kstride);
        if (lo < 0) lo = 0;
        if (hi > J.n_k - 1) hi = J.n_k - 1;
        if (lo > hi) return false;
        j_lo = (int)lo;
        j_hi = (int)hi;
        int tl = j_lo / BN, th = j_hi / BN;
        if (th >= visited_lo) th = visited_lo - 1;
        t_lo = tl;
        t = th;
        return true;
    }

    __device__ void init(const JobArgs& J, const MaskArgs& M, int64_t y0, int64_t y1) {
        visited_lo = 0x7fffffff;
        own = 1;
        t = -1;
        t_lo = 0;
        if (M.kind == kCausal) {
            seg = -1;
            end_s = 0x7fffffff;
            full_ok = 1;
            set_range(0, y1, J);
            return;
        }
        seg = wave_uniform(M.seg[y0]);
        int4 st = M.segtab[seg];
        end_s = wave_uniform(st.w);
        full_ok = (int64_t)end_s > y1;
        if (!set_range(wave_uniform(st.x), y1, J)) t = t_lo - 1;
    }

    // Produces the next tile; returns false when the walk is over.
    __device__ bool next(const JobArgs& J, const MaskArgs& M, int64_t y0, int64_t y1,
                         int* tile, int* full) {
        while (t < t_lo || t < 0) {
            // current range exhausted: move to the parent segment's run
            if (seg < 0) return false;
            int4 st = M.segtab[seg];
            int p = wave_uniform(st.z);
            if (p < 0) { seg = -1; return false; }
            seg = p;
            int4 sp = M.segtab[p];
            own = 0;
            end_s = wave_uniform(sp.w);
            full_ok = (int64_t)end_s > y1;
            if (!set_range(wave_uniform(sp.x), (int64_t)wave_uniform(sp.y) - 1, J)) t = -1;
        }
        int tt = t;
        --t;
        if (tt < visited_lo) visited_lo = tt;
        // classification: full iff the whole tile lies in the range, the tile is
        // not ragged, every key precedes every query and all horizons pass y1.
        int k0 = tt * BN, k1 = tt * BN + BN - 1;
        int f = full_ok && k0 >= j_lo && k1 <= j_hi && k1 < J.n_k;
        if (f && own) {
            int64_t kmax = J.kbase + J.kstride * (int64_t)k1;
            f = kmax <= y0;
        }
        *tile = tt;
        *full = f;
        return true;
    }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename T, int D, int BN>
__global__ void __launch_bounds__(kThreads)
partial_attention_kernel(const LaunchArgs args) {
    using E = Elem<T>;
    using TL = Tile<T, D, BN>;
    using op8 = typename E::op8;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // ---- work item: XCD-aware mapping -----------------------------------
    // Workgroups are dispatched round-robin over the 8 XCDs; give every XCD a
    // contiguous range of work items so that the workgroups sharing one head's
    // K/V run on the same XCD and share its L2.
    const int nwg = gridDim.x;
    const int per_xcd = nwg / 8;
    const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (w >= args.total_wg) return;
    int ji = 0;
    while (ji + 1 < args.n_jobs && w >= args.jobs[ji + 1].wg_begin) ++ji;
    const JobArgs& J = args.jobs[ji];
    const int local = w - J.wg_begin;
    const int head = local / J.q_tiles;
    const int qtile = J.q_tiles - 1 - (local % J.q_tiles);   // heavy (late) tiles first

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r32 = lane & 31;
    const int g = lane >> 5;

    const int q_first = qtile * kBM;
    const int q_last = min(q_first + kBM, J.n_q) - 1;
    const int64_t y0 = J.qbase + J.qstride * (int64_t)q_first;
    const int64_t y1 = J.qbase + J.qstride * (int64_t)q_last;

    // this lane's query row
    const int qi = q_first + wave * 32 + r32;
    const bool q_valid = qi < J.n_q;
    const int qi_ld = q_valid ? qi : J.n_q - 1;
    const int64_t ypos = J.qbase + J.qstride * (int64_t)qi;

    const T* qp = reinterpret_cast<const T*>(J.q) + head * J.q_sh + (int64_t)qi_ld * J.q_st;
    const T* kp = reinterpret_cast<const T*>(J.k) + head * J.k_sh;
    const T* vp = reinterpret_cast<const T*>(J.v) + head * J.v_sh;

    // Q^T operand: 8 consecutive dims per lane per 16-dim step
    op8 qreg[TL::DSTEPS];
#pragma unroll
    for (int s = 0; s < TL::DSTEPS; ++s)
        qreg[s] = load_op8(qp + s * 16 + 8 * g);

    // permuted K row fed by this lane (see the header comment)
    const int kperm_i = (r32 >> 3) * 4 + (r32 & 3);
    const int kperm = (kperm_i >> 3) * 16 + ((r32 & 7) >> 2) * 8 + (kperm_i & 7);

    f32x16 acc[TL::DBLK];
#pragma unroll
    for (int b = 0; b < TL::DBLK; ++b) acc[b] = f32x16{};
    float m_run = -INFINITY;   // running max of scaled scores (log2 domain)
    float l_run = 0.f;         // this lane's half of the running denominator

    // ---- staging registers -------------------------------------------------
    u32x4 kreg[TL::K_PER_THREAD];
    u32x4 vreg[TL::V_PER_THREAD][4];
    int endreg = 0;

    const bool tree = args.mask.kind == kTree;
    auto stage_load = [&](int tile) {
        const int j0 = tile * BN;
#pragma unroll
        for (int i = 0; i < TL::K_PER_THREAD; ++i) {
            int c = threadIdx.x + i * kThreads;
            if (c < TL::K_CHUNKS) {
                int row = c / (D / TL::EPC), col = c % (D / TL::EPC);
                int j = min(j0 + row, J.n_k - 1);
                kreg[i] = *reinterpret_cast<const u32x4*>(kp + (int64_t)j * J.k_st + col * TL::EPC);
            }
        }
#pragma unroll
        for (int i = 0; i < TL::V_PER_THREAD; ++i) {
            int gi = threadIdx.x + i * kThreads;
            if (gi < TL::V_GROUPS) {
                int kg = gi / (D / TL::EPC), dc = gi % (D / TL::EPC);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int j = min(j0 + 4 * kg + r, J.n_k - 1);
                    vreg[i][r] = *reinterpret_cast<const u32x4*>(vp + (int64_t)j * J.v_st + dc * TL::EPC);
                }
            }
        }
        if (tree && threadIdx.x < BN) {
            int j = j0 + threadIdx.x;
            endreg = j < J.n_k ? args.mask.end[J.kbase + J.kstride * (int64_t)j] : (int)0x80000000;
        }
    };

    auto stage_store = [&](int buf) {
        T* Ks = reinterpret_cast<T*>(smem + buf * TL::STAGE_BYTES);
        T* Vt = Ks + TL::K_ELEMS;
        int* Es = reinterpret_cast<int*>(Vt + TL::V_ELEMS);
#pragma unroll
        for (int i = 0; i < TL::K_PER_THREAD; ++i) {
            int c = threadIdx.x + i * kThreads;
            if (c < TL::K_CHUNKS) {
                int row = c / (D / TL::EPC), col = c % (D / TL::EPC);
                *reinterpret_cast<u32x4*>(Ks + row * TL::KS + col * TL::EPC) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < TL::V_PER_THREAD; ++i) {
            int gi = threadIdx.x + i * kThreads;
            if (gi < TL::V_GROUPS) {
                int kg = gi / (D / TL::EPC), dc = gi % (D / TL::EPC);
                if constexpr (sizeof(T) == 2) {
                    // 4 keys x 8 dims -> 8 dims x 4 keys; each output is 4 bf16
                    // of one dim: pick 16-bit halves with v_perm_b32.
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int w32 = e >> 1;
                        // byte selectors: low half -> bytes 1:0, high half -> bytes 3:2
                        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                        uint32_t lo = __builtin_amdgcn_perm(vreg[i][1][w32], vreg[i][0][w32], sel);
                        uint32_t hi = __builtin_amdgcn_perm(vreg[i][3][w32], vreg[i][2][w32], sel);
                        *reinterpret_cast<u32x2*>(Vt + (dc * 8 + e) * TL::VS + 4 * kg) = u32x2{lo, hi};
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        u32x4 col = {vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
                        *reinterpret_cast<u32x4*>(Vt + (dc * 4 + e) * TL::VS + 4 * kg) = col;
                    }
                }
            }
        }
        if (tree && threadIdx.x < BN) Es[threadIdx.x] = endreg;
    };

    // ---- tile walk ------------------------------------------------------------
    TileCursor<BN> cur;
    cur.init(J, args.mask, y0, y1);
    int tile, full;
    bool have = cur.next(J, args.mask, y0, y1, &tile, &full);
    if (have) stage_load(tile);
    int buf = 0;
    const float c2 = args.scale_log2;

    while (have) {
        stage_store(buf);
        __syncthreads();
        int ntile, nfull;
        const bool nhave = cur.next(J, args.mask, y0, y1, &ntile, &nfull);
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
            for (int ds = 0; ds < TL::DSTEPS; ++ds) {
                op8 a = load_op8(krow + ds * 16);
                s[kb] = E::mfma_k16(a, qreg[ds], s[kb]);
            }
        }

        // elementwise visibility on partial tiles: x <= y < end[x], key in range
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < TL::KB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int jl = kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
                    const int j = tile * BN + jl;
                    const int64_t x = J.kbase + J.kstride * (int64_t)j;
                    bool vis = j < J.n_k && x <= ypos;
                    if (tree) vis = vis && ypos < (int64_t)Es[jl];
                    if (!vis) s[kb][i] = -INFINITY;
                }
            }
        }

        // online softmax for this lane's query
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < TL::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * c2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        op8 pb[TL::KSTEPS];
#pragma unroll
        for (int kb = 0; kb < TL::KB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m_use));
                psum += p;
                pb[kb * 2 + (i >> 3)][i & 7] = (T)p;
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int b = 0; b < TL::DBLK; ++b) acc[b] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < TL::KSTEPS; ++ks) {
#pragma unroll
            for (int b = 0; b < TL::DBLK; ++b) {
                op8 a = load_op8(Vt + (b * 32 + r32) * TL::VS + ks * 16 + 8 * g);
                acc[b] = E::mfma_k16(a, pb[ks], acc[b]);
            }
        }

        have = nhave;
        tile = ntile;
        full = nfull;
        buf ^= 1;
    }

    // ---- epilogue: normalise, then write or merge ------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_new = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    if (!q_valid) return;
    float* orow = J.o + (int64_t)head * J.n_q * D + (int64_t)qi * D;
    float* lrow = J.lse + (int64_t)head * J.n_q + qi;
    if (!J.accumulate) {
#pragma unroll
        for (int b = 0; b < TL::DBLK; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 v = {acc[b][q4 * 4 + 0] * inv, acc[b][q4 * 4 + 1] * inv,
                           acc[b][q4 * 4 + 2] * inv, acc[b][q4 * 4 + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + b * 32 + q4 * 8 + g * 4) = v;
            }
        if (g == 0) *lrow = lse_new;
    } else {
        const float lse_old = *lrow;
        const float M = fmaxf(lse_old, lse_new);
        if (M == -INFINITY) return;   // both sides empty: keep (0, -inf)
        const float wa = expf(lse_old - M), wb = expf(lse_new - M);
        const float z = wa + wb;
        const float rz = 1.f / z;
        const float wbn = wb * inv;
#pragma unroll
        for (int b = 0; b < TL::DBLK; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4* dst = reinterpret_cast<f32x4*>(orow + b * 32 + q4 * 8 + g * 4);
                f32x4 old = *dst;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (wa * old[e] + wbn * acc[b][q4 * 4 + e]) * rz;
                *dst = v;
            }
        if (g == 0) *lrow = M + logf(z);
    }
}

}  // namespace cpattn
