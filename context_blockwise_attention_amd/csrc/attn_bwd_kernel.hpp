// attn_bwd_kernel.hpp -- backward of partial attention on gfx950 MFMA.
//
// "Context Parallelism in ART", section 04 (the global softmax derivative):
// for a query with complete output o, log-sum-exp L and incoming output
// gradient g, and D = dot(g, o), every visible key j of any stage gets
//     p_j = exp(s_j - L),   dS_j = p_j (dot(g, v_j) - D),
//     dV_j += p_j g,   dQ += scale dS_j k_j,   dK_j += scale dS_j q,
// with the complete L and D, so a stage's backward needs no other stage and
// the stages' contributions add.  Two kernels (the fp32 path; bf16 inputs
// use the kernels of attn_bwd_bf16_kernel.hpp):
//
//  * attn_bwd_dq_kernel: a workgroup owns 128 query rows (4 waves x 32) and
//    walks the key tiles they see exactly like the forward kernel
//    (TileCursor); per 32-key tile it recomputes S^T = K Q^T and
//    dP^T = V dO^T (one query per MFMA output lane, keys fed in the permuted
//    order kperm so a lane's 16 values are the next MFMA's B operand), forms
//    dS^T and accumulates dQ^T += K^T dS^T.  dQ is added to the fp32 output.
//  * attn_bwd_dkv_kernel: a workgroup owns 128 keys (4 waves x 32, K and V
//    rows in registers) and walks the query tiles that see them: for a tree
//    stored in depth-first preorder key x is visible exactly to the query
//    positions [x, end[x]), so the tiles are those between the first key's
//    position and the largest horizon.  Per 32-query tile it recomputes
//    S = Q K^T and dP = dO V^T (one key per output lane, query rows fed in the
//    permuted order), and accumulates dV^T += dO^T P and dK^T += Q^T dS.  With
//    grouped-query attention the workgroup also loops over the query heads
//    that share its K/V head, so every dK/dV element has one writer.
//
// Tiles are staged through LDS by the whole workgroup (row-major for the A
// operands read in permuted row order, transposed for the dO^T / Q^T / K^T
// operands), loaded into registers one tile ahead.
#pragma once

#include "attn_kernel.hpp"

namespace cpattn {

constexpr int kBwdThreads = 256;
constexpr int kBwdRows = 128;   // query rows (dQ) or keys (dK/dV) per workgroup
constexpr int kBwdTile = 32;    // keys (dQ) or query rows (dK/dV) per inner tile

// One (query block, key/value block) pair of a backward launch.
struct BwdJob {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;     // [H][n_q] complete log-sum-exp (natural log)
    const float* delta;   // [H][n_q] D = dot(dO, O) per query row
    float* dq;            // [H][n_q][d], added to
    float* dk;            // [H_kv][n_k][d], added to
    float* dv;            // [H_kv][n_k][d], added to
    int64_t q_sh, k_sh, v_sh, do_sh;   // head strides (elements)
    int32_t q_st, k_st, v_st, do_st;   // token strides (elements)
    int32_t qbase, qstride, kbase, kstride;
    int32_t n_q, n_k;
    int32_t kv_group;     // query heads per K/V head
    int32_t tiles;        // 128-row tiles of the side the kernel owns (queries or keys)
};

struct BwdArgs {
    BwdJob jobs[kMaxJobs];
    MaskArgs mask;
    int32_t n_jobs;
    int32_t heads;        // heads the kernel iterates over (query heads for dQ, K/V heads for dK/dV)
    int32_t heads_per_xcd;   // ceil(heads / 8) with at least 8 heads, else 0
    int32_t last_first;   // 1: a head's tiles from the last (dQ: later queries see more keys), 0: from the first (dK/dV)
    int32_t total_wg;
    float scale;
    float scale_log2;     // scale * log2(e)
};

// Workgroup -> (job, head, tile), mapped like the forward's work_item: with at
// least 8 heads, XCD x (= bid mod 8) runs its own heads one after another, so
// the workgroups in flight on an XCD stream the same head's tiles through its
// L2; a head's heaviest tiles go first.
__device__ __forceinline__ bool bwd_item(const BwdArgs& a, int bid, int* job, int* head, int* tile) {
    const bool by_xcd = a.heads_per_xcd > 0;
    const int x = bid & 7;
    int p = by_xcd ? (bid >> 3) : bid;
    const int hg = by_xcd ? a.heads_per_xcd : a.heads;
    const bool ranges = by_xcd && (a.heads & 7) == 0;
    for (int j = 0; j < a.n_jobs; ++j) {
        const int nt = a.jobs[j].tiles;
        const int n = hg * nt;
        if (p < n) {
            const int hi = p / nt;
            const int r = p - hi * nt;
            const int h = !by_xcd ? hi : ranges ? x * hg + hi : x + 8 * hi;
            if (h >= a.heads) return false;
            *job = j;
            *head = h;
            *tile = a.last_first ? nt - 1 - r : r;
            return true;
        }
        p -= n;
    }
    return false;
}

// 32-row staging of a [rows][D] matrix: 4-row groups x 16-byte column chunks.
template <typename T, int D>
struct BwdStage {
    static constexpr int EPC = Elem<T>::kEPC;
    static constexpr int RS = D + Elem<T>::kPad;          // row-major stride (elements)
    static constexpr int TS = kBwdTile + Elem<T>::kPad;   // transposed stride (elements)
    static constexpr int GROUPS = (kBwdTile / 4) * (D / EPC);   // per matrix
    static constexpr int ROW_ELEMS = kBwdTile * RS;
    static constexpr int T_ELEMS = D * TS;
};

// Loads 4 rows x EPC columns (group gi of a 32-row tile starting at row0)
template <typename T, int D>
__device__ __forceinline__ void bwd_load_group(__amdgpu_buffer_rsrc_t r, int st, int row0, int gi, u32x4* v) {
    using S = BwdStage<T, D>;
    const int kg = gi % (kBwdTile / 4), dc = gi / (kBwdTile / 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
        v[rr] = buf_load16(r, ((row0 + 4 * kg + rr) * st + dc * S::EPC) * (int)sizeof(T));
}

// Writes a loaded group row-major (rows != nullptr) and/or transposed.
template <typename T, int D>
__device__ __forceinline__ void bwd_store_group(int gi, const u32x4* v, T* rows, T* trans) {
    using S = BwdStage<T, D>;
    const int kg = gi % (kBwdTile / 4), dc = gi / (kBwdTile / 4);
    if (rows) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<u32x4*>(rows + (4 * kg + rr) * S::RS + dc * S::EPC) = v[rr];
    }
    if (trans) {
        if constexpr (sizeof(T) == 2) {
            // 4 rows x 8 columns -> 8 rows x 4: each output takes one 16-bit
            // half from each input row (v_perm_b32 byte selects)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w32 = e >> 1;
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t lo = __builtin_amdgcn_perm(v[1][w32], v[0][w32], sel);
                const uint32_t hi = __builtin_amdgcn_perm(v[3][w32], v[2][w32], sel);
                *reinterpret_cast<u32x2*>(trans + (dc * 8 + e) * S::TS + 4 * kg) = u32x2{lo, hi};
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u32x4 col = {v[0][e], v[1][e], v[2][e], v[3][e]};
                *reinterpret_cast<u32x4*>(trans + (dc * 4 + e) * S::TS + 4 * kg) = col;
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::op8 load_operand(__amdgpu_buffer_rsrc_t r, int off_bytes) {
    const u32x4 lo = buf_load16(r, off_bytes);
    const u32x4 hi = sizeof(T) == 4 ? buf_load16(r, off_bytes + 16) : lo;
    return as_op8<T>(lo, hi);
}

// permuted row fed by MFMA lane r32 (see attn_kernel.hpp): lane value i of the
// 32x32 output then belongs to row 16 (i / 8) + 8 g + (i % 8)
__device__ __forceinline__ int mfma_row_perm(int r32) {
    const int pi = (r32 >> 3) * 4 + (r32 & 3);
    return (pi >> 3) * 16 + ((r32 & 7) >> 2) * 8 + (pi & 7);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// WIN: sliding window on logical positions, as in the forward (causal: a
// lowest visible key index per query; tree: logical positions compared, the
// keys' staged beside their horizons)
template <typename T, int D, bool WIN>
__global__ void __launch_bounds__(kBwdThreads) attn_bwd_dq_kernel(const BwdArgs args) {
    using E = Elem<T>;
    using S = BwdStage<T, D>;
    using op8 = typename E::op8;
    constexpr int BN = kBwdTile;
    constexpr int DSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int KSTEPS = BN / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int ji, head, qtile;
    if (!bwd_item(args, blockIdx.x, &ji, &head, &qtile)) return;
    ji = wave_uniform(ji);
    head = wave_uniform(head);
    qtile = wave_uniform(qtile);
    const BwdJob& J = args.jobs[ji];
    const KeyBlock kblk{J.kbase, J.kstride, J.n_k};
    const int kvh = head / J.kv_group;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_uniform(tid >> 6);
    const int r32 = lane & 31;
    const int g = lane >> 5;
    const int q_first = qtile * kBwdRows;
    const int q_last = min(q_first + kBwdRows, J.n_q) - 1;
    const int y0 = J.qbase + J.qstride * q_first;
    const int y1 = J.qbase + J.qstride * q_last;
    const int qi = q_first + wave * 32 + r32;
    const int ypos = J.qbase + J.qstride * qi;
    const bool tree = args.mask.kind == kTree;

    const T* qh = reinterpret_cast<const T*>(J.q) + head * J.q_sh;
    const T* doh = reinterpret_cast<const T*>(J.dout) + head * J.do_sh;
    const T* kh = reinterpret_cast<const T*>(J.k) + kvh * J.k_sh;
    const T* vh = reinterpret_cast<const T*>(J.v) + kvh * J.v_sh;
    const auto qr = make_rsrc(qh, ((J.n_q - 1) * J.q_st + D) * (int)sizeof(T));
    const auto dor = make_rsrc(doh, ((J.n_q - 1) * J.do_st + D) * (int)sizeof(T));
    const auto kr = make_rsrc(kh, ((J.n_k - 1) * J.k_st + D) * (int)sizeof(T));
    const auto vr = make_rsrc(vh, ((J.n_k - 1) * J.v_st + D) * (int)sizeof(T));

    op8 qreg[DSTEPS], doreg[DSTEPS];
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) {
        qreg[s] = load_operand<T>(qr, (qi * J.q_st + s * 16 + 8 * g) * (int)sizeof(T));
        doreg[s] = load_operand<T>(dor, (qi * J.do_st + s * 16 + 8 * g) * (int)sizeof(T));
    }
    const bool valid_q = qi < J.n_q;
    const float lse = valid_q ? J.lse[(int64_t)head * J.n_q + qi] : -INFINITY;
    const float lse2 = lse * 1.4426950408889634f;
    const float dlt = valid_q ? J.delta[(int64_t)head * J.n_q + qi] : 0.f;
    const bool live = lse > -INFINITY;   // a row with no visible key has no gradient
    const float c2 = args.scale_log2;
    const int kperm = mfma_row_perm(r32);
    int jlo = 0, ly = 0;
    if (WIN) {
        if (tree) {
            ly = valid_q ? args.mask.lpos[ypos] : 0;
        } else {
            const int lowest = ypos - args.mask.window + 1 - J.kbase;
            jlo = lowest <= 0 ? 0 : (lowest + J.kstride - 1) / J.kstride;
        }
    }

    f32x16 acc[DBLK];
#pragma unroll
    for (int b = 0; b < DBLK; ++b) acc[b] = f32x16{};

    T* Ks = reinterpret_cast<T*>(smem);
    T* Kt = Ks + S::ROW_ELEMS;
    T* Vs = Kt + S::T_ELEMS;
    int* Es = reinterpret_cast<int*>(Vs + S::ROW_ELEMS);   // horizons, then (window) logical positions

    // staging: K (rows and transposed) and V (rows) of a 32-key tile; group
    // gi < GROUPS is K, the next GROUPS are V
    constexpr int GPT = (2 * S::GROUPS + kBwdThreads - 1) / kBwdThreads;
    u32x4 sreg[GPT][4];
    int endreg = 0, lreg = 0;
    auto stage_load = [&](int tile) {
#pragma unroll
        for (int x = 0; x < GPT; ++x) {
            const int gi = tid + x * kBwdThreads;
            if (gi < S::GROUPS) bwd_load_group<T, D>(kr, J.k_st, tile * BN, gi, sreg[x]);
            else if (gi < 2 * S::GROUPS) bwd_load_group<T, D>(vr, J.v_st, tile * BN, gi - S::GROUPS, sreg[x]);
        }
        if (tree && tid < BN) {
            const int j = tile * BN + tid;
            endreg = j < J.n_k ? args.mask.end[J.kbase + J.kstride * j] : (int)0x80000000;
        }
        if (WIN && tree && tid >= BN && tid < 2 * BN) {
            const int j = tile * BN + tid - BN;
            lreg = j < J.n_k ? args.mask.lpos[J.kbase + J.kstride * j] : 0;
        }
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int x = 0; x < GPT; ++x) {
            const int gi = tid + x * kBwdThreads;
            if (gi < S::GROUPS) bwd_store_group<T, D>(gi, sreg[x], Ks, Kt);
            else if (gi < 2 * S::GROUPS) bwd_store_group<T, D>(gi - S::GROUPS, sreg[x], Vs, nullptr);
        }
        if (tree && tid < BN) Es[tid] = endreg;
        if (WIN && tree && tid >= BN && tid < 2 * BN) Es[tid] = lreg;   // Ls = Es + BN
    };

    const int jlim = min(J.n_k - 1, ypos < J.kbase ? -1 : (ypos - J.kbase) / J.kstride);
    TileCursor<BN, WIN> cur;
    cur.init(kblk, args.mask, y0, y1);
    int tile, full;
    bool have = cur.next(kblk, args.mask, y1, &tile, &full);
    if (have) stage_load(tile);
    while (have) {
        __syncthreads();   // the previous tile's operands are no longer read
        stage_store();
        __syncthreads();
        int ntile, nfull;
        const bool nhave = cur.next(kblk, args.mask, y1, &ntile, &nfull);
        if (nhave) stage_load(ntile);

        f32x16 s = {}, dp = {};
        const T* krow = Ks + kperm * S::RS + 8 * g;
        const T* vrow = Vs + kperm * S::RS + 8 * g;
#pragma unroll
        for (int ds = 0; ds < DSTEPS; ++ds) {
            s = E::mfma_k16(load_op8(krow + ds * 16), qreg[ds], s);
            dp = E::mfma_k16(load_op8(vrow + ds * 16), doreg[ds], dp);
        }
        op8 dsb[KSTEPS];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int jl = (i >> 3) * 16 + g * 8 + (i & 7);
            bool vis = live;
            if (!full) {
                vis = vis && tile * BN + jl <= jlim;
                if (tree) vis = vis && ypos < Es[jl];
                if (WIN) vis = vis && (tree ? ly - Es[BN + jl] < args.mask.window : tile * BN + jl >= jlo);
            }
            const float p = vis ? __builtin_amdgcn_exp2f(s[i] * c2 - lse2) : 0.f;
            dsb[i >> 3][i & 7] = (T)(p * (dp[i] - dlt));
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int b = 0; b < DBLK; ++b)
                acc[b] = E::mfma_k16(load_op8(Kt + (b * 32 + r32) * S::TS + ks * 16 + 8 * g), dsb[ks], acc[b]);
        have = nhave;
        tile = ntile;
        full = nfull;
    }

    if (!valid_q) return;
    // lane (query qi, half g) holds dQ^T[d][qi] for d = 32 b + 8 (i / 4) + 4 g + i % 4
    float* row = J.dq + ((int64_t)head * J.n_q + qi) * D;
    const float sc = args.scale;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4* dst = reinterpret_cast<f32x4*>(row + b * 32 + q4 * 8 + g * 4);
            f32x4 v = *dst;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += sc * acc[b][q4 * 4 + e];
            *dst = v;
        }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
// WIN: sliding window on logical positions; the queries' logical positions
// are staged with their LSE and D (tree), and with a causal mask the query
// range ends at the last key's position + window.
template <typename T, int D, bool WIN>
__global__ void __launch_bounds__(kBwdThreads) attn_bwd_dkv_kernel(const BwdArgs args) {
    using E = Elem<T>;
    using S = BwdStage<T, D>;
    using op8 = typename E::op8;
    constexpr int BM = kBwdTile;   // query rows per inner tile
    constexpr int DSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int ji, kvh, ktile;
    if (!bwd_item(args, blockIdx.x, &ji, &kvh, &ktile)) return;
    ji = wave_uniform(ji);
    kvh = wave_uniform(kvh);
    ktile = wave_uniform(ktile);
    const BwdJob& J = args.jobs[ji];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_uniform(tid >> 6);
    const int r32 = lane & 31;
    const int g = lane >> 5;
    const bool tree = args.mask.kind == kTree;
    const int j0 = ktile * kBwdRows;
    const int jk = j0 + wave * 32 + r32;          // this lane's key
    const bool valid_k = jk < J.n_k;
    const int kpos = J.kbase + J.kstride * jk;
    // key jk is visible to the query positions [kpos, horizon)
    const int horizon = !valid_k ? (int)0x80000000 : tree ? args.mask.end[kpos] : 0x7fffffff;

    const T* kh = reinterpret_cast<const T*>(J.k) + kvh * J.k_sh;
    const T* vh = reinterpret_cast<const T*>(J.v) + kvh * J.v_sh;
    const auto kr = make_rsrc(kh, ((J.n_k - 1) * J.k_st + D) * (int)sizeof(T));
    const auto vr = make_rsrc(vh, ((J.n_k - 1) * J.v_st + D) * (int)sizeof(T));
    op8 kreg[DSTEPS], vreg[DSTEPS];
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) {
        kreg[s] = load_operand<T>(kr, (jk * J.k_st + s * 16 + 8 * g) * (int)sizeof(T));
        vreg[s] = load_operand<T>(vr, (jk * J.v_st + s * 16 + 8 * g) * (int)sizeof(T));
    }

    // query rows that can see any key of the workgroup: positions from the
    // first key's to the largest horizon
    __shared__ int s_hmax[4];
    int hmax = horizon;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hmax = max(hmax, __shfl_xor(hmax, off));
    if (lane == 0) s_hmax[wave] = hmax;
    __syncthreads();
    hmax = max(max(s_hmax[0], s_hmax[1]), max(s_hmax[2], s_hmax[3]));
    const int pos_lo = J.kbase + J.kstride * j0;
    auto first_query_at_or_after = [&](int64_t x) -> int {
        if (x <= J.qbase) return 0;
        const int64_t i = (x - J.qbase + J.qstride - 1) / J.qstride;
        return (int)min<int64_t>(i, J.n_q);
    };
    const int i_begin = first_query_at_or_after(pos_lo) / BM * BM;
    int i_end = hmax == (int)0x80000000 ? 0 : first_query_at_or_after((int64_t)hmax);   // exclusive
    if (WIN && !tree) {
        // the workgroup's last key position + window bounds the queries that can see it
        int kl = valid_k ? kpos : (int)0x80000000;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kl = max(kl, __shfl_xor(kl, off));
        if (lane == 0) s_hmax[wave] = kl;
        __syncthreads();
        kl = max(max(s_hmax[0], s_hmax[1]), max(s_hmax[2], s_hmax[3]));
        __syncthreads();
        if (kl != (int)0x80000000) i_end = min(i_end, first_query_at_or_after((int64_t)kl + args.mask.window));
    }
    const int lk = !WIN || !valid_k ? 0 : tree ? args.mask.lpos[kpos] : kpos;

    f32x16 acck[DBLK], accv[DBLK];
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
        acck[b] = f32x16{};
        accv[b] = f32x16{};
    }

    T* Qs = reinterpret_cast<T*>(smem);
    T* Qt = Qs + S::ROW_ELEMS;
    T* Ds_ = Qt + S::T_ELEMS;          // dO rows
    T* Dt = Ds_ + S::ROW_ELEMS;        // dO transposed
    float* L2s = reinterpret_cast<float*>(Dt + S::T_ELEMS);
    float* Dls = L2s + BM;
    int* Lqs = reinterpret_cast<int*>(Dls + BM);   // window on a tree: the queries' logical positions

    const float c2 = args.scale_log2;
    const int qperm = mfma_row_perm(r32);
    constexpr int GPT = (2 * S::GROUPS + kBwdThreads - 1) / kBwdThreads;

    for (int hq = 0; hq < J.kv_group; ++hq) {
        const int head = kvh * J.kv_group + hq;
        const T* qh = reinterpret_cast<const T*>(J.q) + head * J.q_sh;
        const T* doh = reinterpret_cast<const T*>(J.dout) + head * J.do_sh;
        const auto qr = make_rsrc(qh, ((J.n_q - 1) * J.q_st + D) * (int)sizeof(T));
        const auto dor = make_rsrc(doh, ((J.n_q - 1) * J.do_st + D) * (int)sizeof(T));
        const float* lse = J.lse + (int64_t)head * J.n_q;
        const float* delta = J.delta + (int64_t)head * J.n_q;
        u32x4 sreg[GPT][4];
        float lreg = 0.f, dreg = 0.f;
        int lqreg = 0;
        auto stage_load = [&](int q0) {
#pragma unroll
            for (int x = 0; x < GPT; ++x) {
                const int gi = tid + x * kBwdThreads;
                if (gi < S::GROUPS) bwd_load_group<T, D>(qr, J.q_st, q0, gi, sreg[x]);
                else if (gi < 2 * S::GROUPS) bwd_load_group<T, D>(dor, J.do_st, q0, gi - S::GROUPS, sreg[x]);
            }
            if (tid < BM) {
                const int i = q0 + tid;
                lreg = i < J.n_q ? lse[i] : -INFINITY;
                dreg = i < J.n_q ? delta[i] : 0.f;
                if (WIN && tree) lqreg = i < J.n_q ? args.mask.lpos[J.qbase + J.qstride * i] : 0;
            }
        };
        auto stage_store = [&]() {
#pragma unroll
            for (int x = 0; x < GPT; ++x) {
                const int gi = tid + x * kBwdThreads;
                if (gi < S::GROUPS) bwd_store_group<T, D>(gi, sreg[x], Qs, Qt);
                else if (gi < 2 * S::GROUPS) bwd_store_group<T, D>(gi - S::GROUPS, sreg[x], Ds_, Dt);
            }
            if (tid < BM) {
                L2s[tid] = lreg * 1.4426950408889634f;
                Dls[tid] = dreg;
                if (WIN && tree) Lqs[tid] = lqreg;
            }
        };
        if (i_begin < i_end) stage_load(i_begin);
        for (int q0 = i_begin; q0 < i_end; q0 += BM) {
            __syncthreads();
            stage_store();
            __syncthreads();
            if (q0 + BM < i_end) stage_load(q0 + BM);

            f32x16 s = {}, dp = {};
            const T* qrow = Qs + qperm * S::RS + 8 * g;
            const T* drow = Ds_ + qperm * S::RS + 8 * g;
#pragma unroll
            for (int ds = 0; ds < DSTEPS; ++ds) {
                s = E::mfma_k16(load_op8(qrow + ds * 16), kreg[ds], s);
                dp = E::mfma_k16(load_op8(drow + ds * 16), vreg[ds], dp);
            }
            // lane (key jk, half g), value i: query row q0 + 16 (i / 8) + 8 g + i % 8
            op8 pb[2], dsb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int il = (i >> 3) * 16 + 8 * g + (i & 7);
                const int qrow_i = q0 + il;
                const int y = J.qbase + J.qstride * qrow_i;
                const float l2 = L2s[il];
                bool vis = qrow_i < J.n_q && kpos <= y && y < horizon && l2 > -INFINITY;
                if (WIN) vis = vis && (tree ? Lqs[il] : y) - lk < args.mask.window;
                const float p = vis ? __builtin_amdgcn_exp2f(s[i] * c2 - l2) : 0.f;
                pb[i >> 3][i & 7] = (T)p;
                dsb[i >> 3][i & 7] = (T)(p * (dp[i] - Dls[il]));
            }
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int b = 0; b < DBLK; ++b) {
                    accv[b] = E::mfma_k16(load_op8(Dt + (b * 32 + r32) * S::TS + st * 16 + 8 * g), pb[st], accv[b]);
                    acck[b] = E::mfma_k16(load_op8(Qt + (b * 32 + r32) * S::TS + st * 16 + 8 * g), dsb[st], acck[b]);
                }
        }
        __syncthreads();   // the next head's staging overwrites the tiles
    }

    if (!valid_k) return;
    // lane (key jk, half g) holds dK^T / dV^T [d][jk] for d = 32 b + 8 (i / 4) + 4 g + i % 4
    float* krow = J.dk + ((int64_t)kvh * J.n_k + jk) * D;
    float* vrow = J.dv + ((int64_t)kvh * J.n_k + jk) * D;
    const float sc = args.scale;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int c = b * 32 + q4 * 8 + g * 4;
            f32x4 kv = *reinterpret_cast<f32x4*>(krow + c);
            f32x4 vv = *reinterpret_cast<f32x4*>(vrow + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kv[e] += sc * acck[b][q4 * 4 + e];
                vv[e] += accv[b][q4 * 4 + e];
            }
            *reinterpret_cast<f32x4*>(krow + c) = kv;
            *reinterpret_cast<f32x4*>(vrow + c) = vv;
        }
}

// D = dot(dO, O) per query row (fp32), for one [H][n_q] block.  Each lane
// takes 4 consecutive columns (16 bytes of O, 4 elements of dO), d / 4 lanes
// share a row (a power of two dividing 64: 16 or 32) and reduce by shuffles,
// 256 / (d / 4) rows per workgroup.  Both inputs are read once: non-temporal
// loads.  O must be 16-byte aligned; dO's element offsets are multiples of 4
// (its strides are multiples of 8 elements for bf16, 4 for fp32).
template <typename T>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const float* o, const T* dout, int64_t do_sh, int32_t do_st,
                                                        float* delta, int64_t rows, int32_t n_q, int32_t d) {
    using f4v = float __attribute__((ext_vector_type(4)));
    using u2v = unsigned __attribute__((ext_vector_type(2)));
    const int lanes = d >> 2;
    const int64_t row = (int64_t)blockIdx.x * (256 / lanes) + threadIdx.x / lanes;
    const int c = (threadIdx.x % lanes) * 4;
    float acc = 0.f;
    if (row < rows) {
        const int64_t h = row / n_q, i = row - h * n_q;
        const f4v ov = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(o + row * d + c));
        const T* gp = dout + h * do_sh + i * do_st + c;
        f4v gv;
        if constexpr (sizeof(T) == 2) {
            const u2v raw = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(gp));
            gv = f4v{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                     __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        } else {
            gv = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(gp));
        }
        acc = ov.x * gv.x + ov.y * gv.y + ov.z * gv.z + ov.w * gv.w;
    }
    for (int off = lanes >> 1; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && threadIdx.x % lanes == 0) delta[row] = acc;
}

}  // namespace cpattn
