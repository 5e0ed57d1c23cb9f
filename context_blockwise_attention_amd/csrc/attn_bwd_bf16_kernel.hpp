// attn_bwd_bf16_kernel.hpp -- backward of partial attention for bf16 inputs
// on gfx950, built on the same CDNA4 features as the bf16 forward kernel.
//
// Arithmetic and work split as in attn_bwd_kernel.hpp ("Context Parallelism
// in ART", section 04: p = exp(s - L) with the complete L, dS = p (dP - D)).
// What differs is how a tile reaches the matrix cores:
//
//  * Tiles of 32 rows go from HBM straight into LDS with buffer_load ... lds,
//    double buffered: the loads of tile t+1 are issued right after the one
//    workgroup barrier of iteration t and land while tile t is computed.
//  * A tile is stored once, row-major.  Operands that need rows (K and V rows
//    for S^T = K Q^T and dP^T = V dO^T) are 16-byte row reads; operands that
//    need columns (K^T for dQ^T += K^T dS^T) are read from the same rows with
//    ds_read_b64_tr_b16.  The 16-byte chunks of a row are XOR-swizzled by
//    bwd_swizzle so that both access patterns spread over all LDS banks.
#pragma once

#include "attn_bf16_kernel.hpp"
#include "attn_bwd_kernel.hpp"

namespace cpattn {

// 32-row bf16 tile of D columns in LDS (row-major, swizzled 16-byte chunks)
template <int D>
struct BwdTileBf16 {
    static constexpr int ROWS = kBwdTile;
    static constexpr int ROWB = D * 2;                  // bytes per row
    static constexpr int CPR = D / 8;                   // 16-byte chunks per row
    static constexpr int BYTES = ROWS * ROWB;
    static constexpr int RPB = 1024 / ROWB;             // rows per 1 KB direct load (64 lanes x 16 B)
    static constexpr int LOADS = BYTES / 1024;          // direct loads per tile
    static constexpr int LOADS_PER_WAVE = LOADS / 4;    // four waves share a tile
    static constexpr int DSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    static_assert(LOADS % 4 == 0, "tile shape");
};

// Physical chunk of logical chunk c in row r (row within a tile) is
// c ^ bwd_swizzle(r).  A 16-byte row read serves 16 lanes per pass, here 16
// different rows (rows 0-15 or 16-31 in the permuted MFMA order), so the
// swizzle is a permutation of 0-15 over any 16 consecutive rows.  A
// transposed read (ds_read_b64_tr_b16) serves 32 lanes: rows 8g + kq
// (kq = 0-3) at chunks (4b + 2 G2 + t) ^ swizzle with G2, t in {0, 1}, so the
// swizzles of those four rows must differ above bit 1; then the 32 lanes'
// 8-byte words fall in 16 distinct chunks x 2 halves.  With 128-byte rows (d
// 64) two rows share a 256-byte bank line: the same conditions then hold for
// the even and the odd rows separately, over 8 chunks.
template <int D>
__device__ __forceinline__ int bwd_swizzle(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Per-lane offsets of one wave's share of a tile's direct loads: load i of
// wave w fills 1 KB block b = 4 i + w, lane L goes to row b RPB + L / CPR,
// physical chunk L % CPR, so it fetches logical chunk (L % CPR) ^ swizzle.
template <int D>
struct BwdDma {
    using TT = BwdTileBf16<D>;
    int voff[TT::LOADS_PER_WAVE];
    __device__ __forceinline__ void init(int wave, int lane, int st) {
#pragma unroll
        for (int i = 0; i < TT::LOADS_PER_WAVE; ++i) {
            const int row = (4 * i + wave) * TT::RPB + lane / TT::CPR;
            voff[i] = row * st * 2 + (((lane % TT::CPR) ^ bwd_swizzle<D>(row)) * 16);
        }
    }
    // rows row0 .. row0 + 31 of the buffer into the tile at `dst`
    __device__ __forceinline__ void issue(const i32x4& rsrc, int row0, int st, int wave, lds_byte* dst) const {
        const int base = row0 * st * 2;
#pragma unroll
        for (int i = 0; i < TT::LOADS_PER_WAVE; ++i)
            dma_b128(rsrc, voff[i] + base, lds_addr(dst + (4 * i + wave) * 1024));
    }
};

// 16-byte read of logical chunk 2 ds + g of a row: the row's byte offset plus
// the physical chunk, (2 ds + g) ^ swizzle = 2 ds ^ (g ^ swizzle)
struct BwdRowRead {
    int base;   // row * bytes per row
    int x;      // g ^ swizzle(row)
    __device__ __forceinline__ int off(int ds) const { return base + (((2 * ds) ^ x) << 4); }
};

// LDS offsets of the two operand reads a lane makes from a tile:
//  row: 16-byte reads of row `perm` (the MFMA row order), chunk 2 ds + g
//  tr_lo[b], tr_hi[b]: the ds_read_b64_tr_b16 pair that builds the A operand
//  (column block b of the tile's transpose, rows 0-15 of the k-step), as in
//  the forward's V^T reads
template <int D>
struct BwdReadOffsets {
    using TT = BwdTileBf16<D>;
    BwdRowRead row;
    int tr_lo[TT::DBLK], tr_hi[TT::DBLK];
    __device__ __forceinline__ void init(int lane, int perm) {
        const int g = lane >> 5;
        row = BwdRowRead{perm * TT::ROWB, g ^ bwd_swizzle<D>(perm)};
        const int G2 = (lane >> 4) & 1;
        const int kq = (lane & 15) >> 2;
        const int qq = lane & 3;
        const int rlo = 8 * g + kq, rhi = rlo + 4;
#pragma unroll
        for (int b = 0; b < TT::DBLK; ++b) {
            const int c = 4 * b + 2 * G2 + (qq >> 1);
            tr_lo[b] = rlo * TT::ROWB + ((c ^ bwd_swizzle<D>(rlo)) * 16) + (qq & 1) * 8;
            tr_hi[b] = rhi * TT::ROWB + ((c ^ bwd_swizzle<D>(rhi)) * 16) + (qq & 1) * 8;
        }
    }
};

// A operand of a transposed product: column block b, k-step ks of the tile
template <int D>
__device__ __forceinline__ bf16x8 bwd_tr_operand(const lds_byte* tile, const BwdReadOffsets<D>& o, int ks, int b) {
    const lds_byte* p = tile + ks * 16 * BwdTileBf16<D>::ROWB;
    const u32x2 lo = lds_tr4(p + o.tr_lo[b]);
    const u32x2 hi = lds_tr4(p + o.tr_hi[b]);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ void bwd_tile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// dQ (bf16): 128 query rows per workgroup, 64-key tiles stored as two 32-row
// sub-tiles (one barrier per 64 keys; measured ~1% faster than 32-key tiles
// on the 64K tree ring, at 256 registers)
// ---------------------------------------------------------------------------
constexpr int kBwdDqKeyTile = 64;
template <int D, int KT_ = kBwdDqKeyTile / kBwdTile>
struct BwdDqBf16Smem {
    using TT = BwdTileBf16<D>;
    static constexpr int KT = KT_;     // 32-row sub-tiles per key tile
    static constexpr int SLOT = KT * TT::BYTES;
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = 2 * SLOT;
    static constexpr int E_OFF = 4 * SLOT;   // two 256-byte horizon slots (64-lane loads)
    static constexpr int L_OFF = E_OFF + 2 * 256;   // window on a tree: the keys' logical positions
    static constexpr int BYTES = L_OFF + 2 * 256;
};

// WIN: sliding window on logical positions (the forward's rule): causal ->
// a lowest visible key index per query; tree -> the query's logical position
// against each key's, staged beside the horizons.  The tile walk skips and
// classifies tiles with the window (TileCursor<BN, true>).  Windowed runs use
// 32-key tiles (the window's registers do not fit beside two sub-tiles).
template <int D, bool WIN>
__global__ void __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_bf16_kernel(const BwdArgs args) {
    using TT = BwdTileBf16<D>;
    using SM = BwdDqBf16Smem<D, WIN ? 1 : kBwdDqKeyTile / kBwdTile>;
    constexpr int KT = SM::KT;
    constexpr int BN = KT * kBwdTile;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

    int ji, head, qtile;
    if (!bwd_item(args, blockIdx.x, &ji, &head, &qtile)) return;
    ji = wave_uniform(ji);
    head = wave_uniform(head);
    qtile = wave_uniform(qtile);
    const BwdJob& J = args.jobs[ji];
    const KeyBlock kblk{J.kbase, J.kstride, J.n_k};
    const int k_st = J.k_st, v_st = J.v_st;
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

    const __bf16* qh = reinterpret_cast<const __bf16*>(J.q) + head * J.q_sh;
    const __bf16* doh = reinterpret_cast<const __bf16*>(J.dout) + head * J.do_sh;
    const __bf16* kh = reinterpret_cast<const __bf16*>(J.k) + kvh * J.k_sh;
    const __bf16* vh = reinterpret_cast<const __bf16*>(J.v) + kvh * J.v_sh;

    bf16x8 qreg[TT::DSTEPS], doreg[TT::DSTEPS];
    {
        const auto qr = make_rsrc(qh, ((J.n_q - 1) * J.q_st + D) * 2);
        const auto dor = make_rsrc(doh, ((J.n_q - 1) * J.do_st + D) * 2);
#pragma unroll
        for (int s = 0; s < TT::DSTEPS; ++s) {
            qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qr, (qi * J.q_st + s * 16 + 8 * g) * 2));
            doreg[s] = __builtin_bit_cast(bf16x8, buf_load16(dor, (qi * J.do_st + s * 16 + 8 * g) * 2));
        }
    }
    const bool valid_q = qi < J.n_q;
    const float lse = valid_q ? J.lse[(int64_t)head * J.n_q + qi] : -INFINITY;
    // exp2(s c2 - lse2) is 0 for a row without gradient (no visible key, or past the block)
    const float lse2 = lse > -INFINITY ? lse * 1.4426950408889634f : INFINITY;
    const float dlt = valid_q ? J.delta[(int64_t)head * J.n_q + qi] : 0.f;
    const float c2 = args.scale_log2;
    const int jlim = min(J.n_k - 1, ypos < J.kbase ? -1 : (ypos - J.kbase) / J.kstride);
    int jlo = 0, ly = 0;
    if (WIN) {
        if (tree) {
            ly = valid_q ? args.mask.lpos[ypos] : 0;
        } else {
            const int lowest = ypos - args.mask.window + 1 - J.kbase;   // lowest visible key position, block-relative
            jlo = lowest <= 0 ? 0 : (lowest + J.kstride - 1) / J.kstride;
        }
    }

    lds_byte* const lds = to_lds(smem);
    const i32x4 k_rsrc = sgpr_rsrc(kh, (J.n_k - 1) * k_st * 2 + D * 2);
    const i32x4 v_rsrc = sgpr_rsrc(vh, (J.n_k - 1) * v_st * 2 + D * 2);
    const i32x4 e_rsrc = sgpr_rsrc(args.mask.end, args.mask.n_pos * 4);
    const i32x4 l_rsrc = WIN ? sgpr_rsrc(args.mask.lpos, args.mask.n_pos * 4) : i32x4{};
    BwdDma<D> dk, dv;
    dk.init(wave, lane, k_st);
    dv.init(wave, lane, v_st);
    BwdReadOffsets<D> ro;
    ro.init(lane, mfma_row_perm(r32));
    auto issue = [&](int tile, int slot) {
#pragma unroll
        for (int h = 0; h < KT; ++h) {
            dk.issue(k_rsrc, tile * BN + h * 32, k_st, wave, lds + SM::K_OFF + slot * SM::SLOT + h * TT::BYTES);
            dv.issue(v_rsrc, tile * BN + h * 32, v_st, wave, lds + SM::V_OFF + slot * SM::SLOT + h * TT::BYTES);
        }
        if (tree && wave == 0)
            dma_b32(e_rsrc, (kblk.kbase + kblk.kstride * (tile * BN + lane)) * 4, lds_addr(lds + SM::E_OFF + slot * 256));
        if (WIN && tree && wave == 1)
            dma_b32(l_rsrc, (kblk.kbase + kblk.kstride * (tile * BN + lane)) * 4, lds_addr(lds + SM::L_OFF + slot * 256));
    };

    f32x16 acc[TT::DBLK];
#pragma unroll
    for (int b = 0; b < TT::DBLK; ++b) acc[b] = f32x16{};

    TileCursor<BN, WIN> cur;
    cur.init(kblk, args.mask, y0, y1);
    int t_cur, f_cur, t_nxt = 0, f_nxt = 0;
    if (cur.next(kblk, args.mask, y1, &t_cur, &f_cur)) {
        issue(t_cur, 0);
        bool h_nxt = cur.next(kblk, args.mask, y1, &t_nxt, &f_nxt);
        for (int it = 0;; ++it) {
            const int slot = it & 1;
            // this wave's loads of the current tile have landed; after the
            // barrier every wave's have, and every wave is done with the
            // other slot (read in the previous iteration)
            __builtin_amdgcn_s_waitcnt(0xF70);
            bwd_tile_barrier();
            if (h_nxt) issue(t_nxt, slot ^ 1);
            const lds_byte* kt = lds + SM::K_OFF + slot * SM::SLOT;
            const lds_byte* vt = lds + SM::V_OFF + slot * SM::SLOT;

            f32x16 s[KT], dp[KT];
#pragma unroll
            for (int h = 0; h < KT; ++h) {
                s[h] = f32x16{};
                dp[h] = f32x16{};
            }
#pragma unroll
            for (int ds = 0; ds < TT::DSTEPS; ++ds)
#pragma unroll
                for (int h = 0; h < KT; ++h) {
                    s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(kt + h * TT::BYTES + ro.row.off(ds)), qreg[ds],
                                                                   s[h], 0, 0, 0);
                    dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(vt + h * TT::BYTES + ro.row.off(ds)),
                                                                    doreg[ds], dp[h], 0, 0, 0);
                }
            // lane value i of sub-tile h is key 32 h + 16 (i / 8) + 8 g + i % 8 of the tile
            bf16x8 dsb[2 * KT];
            if (f_cur) {
#pragma unroll
                for (int h = 0; h < KT; ++h)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[h][i], c2, -lse2));
                        dsb[2 * h + (i >> 3)][i & 7] = (__bf16)(p * (dp[h][i] - dlt));
                    }
            } else {
                const int lim = jlim - t_cur * BN - 8 * g;
                const int lo = jlo - t_cur * BN - 8 * g;   // window (causal)
                const auto* ep = reinterpret_cast<const __attribute__((address_space(3))) int*>(lds + SM::E_OFF + slot * 256) + 8 * g;
                const auto* lkp = reinterpret_cast<const __attribute__((address_space(3))) int*>(lds + SM::L_OFF + slot * 256) + 8 * g;
#pragma unroll
                for (int h = 0; h < KT; ++h)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int jl = 32 * h + (i >> 3) * 16 + (i & 7);   // + 8 g, folded into lim, lo, ep, lkp
                        bool vis = jl <= lim;
                        if (tree) vis = vis && ypos < ep[jl];
                        if (WIN) vis = vis && (tree ? ly - lkp[jl] < args.mask.window : jl >= lo);
                        const float p = vis ? __builtin_amdgcn_exp2f(fmaf(s[h][i], c2, -lse2)) : 0.f;
                        dsb[2 * h + (i >> 3)][i & 7] = (__bf16)(p * (dp[h][i] - dlt));
                    }
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int ks = 0; ks < 2 * KT; ++ks)
#pragma unroll
                for (int b = 0; b < TT::DBLK; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        bwd_tr_operand<D>(kt + (ks >> 1) * TT::BYTES, ro, ks & 1, b), dsb[ks], acc[b], 0, 0, 0);
            if (!h_nxt) break;
            t_cur = t_nxt;
            f_cur = f_nxt;
            h_nxt = cur.next(kblk, args.mask, y1, &t_nxt, &f_nxt);
        }
    }

    if (!valid_q) return;
    // lane (query qi, half g) holds dQ^T[d][qi] for d = 32 b + 8 (i / 4) + 4 g + i % 4
    float* row = J.dq + ((int64_t)head * J.n_q + qi) * D;
    const float sc = args.scale;
#pragma unroll
    for (int b = 0; b < TT::DBLK; ++b)
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
// dK, dV (bf16): 128 keys per workgroup (32 per wave), 32-query tiles
//
// A wave keeps its keys' K rows in registers (the B operand of S = Q K^T) and
// the workgroup's V rows in LDS (B operand of dP = dO V^T, read per tile), so
// that K, the dK/dV accumulators and one tile's S and dP fit the 256
// registers of two waves per SIMD.  Query tiles (Q, dO and the rows' LSE and
// D) stream through two LDS slots.  For a tree stored in depth-first preorder
// key x is visible exactly to the query positions [x, end[x]): the tiles are
// those from the first key's position to the largest horizon, and a tile is
// full when its first query lies at or after the last key and its last query
// before the smallest horizon.
// ---------------------------------------------------------------------------
template <int D>
struct BwdDkvBf16Smem {
    using TT = BwdTileBf16<D>;
    static constexpr int V_OFF = 0;                       // 128 V rows, 4 tiles of 32
    static constexpr int Q_OFF = 4 * TT::BYTES;           // two slots
    static constexpr int DO_OFF = Q_OFF + 2 * TT::BYTES;  // two slots
    static constexpr int L_OFF = DO_OFF + 2 * TT::BYTES;  // LSE, two 256-byte slots (64-lane loads)
    static constexpr int DL_OFF = L_OFF + 2 * 256;        // D, two slots
    static constexpr int LQ_OFF = DL_OFF + 2 * 256;       // window on a tree: the queries' logical positions
    static constexpr int T_CAP = 1024;                    // window on a tree: query tiles that can see a key
    static constexpr int T_OFF = LQ_OFF + 2 * 256;
    static constexpr int R_OFF = T_OFF + T_CAP * 4;       // per-wave reductions
    static constexpr int BYTES = R_OFF + 128;
};

// WIN: sliding window on logical positions (query and key also within the
// window: ly - lk < window, logical = physical for a causal mask); a tile is
// full only if its largest logical query position is within the window of the
// smallest logical key position.  With a causal mask the query range ends at
// the last key's position + window.  With a tree the subtree's runs are
// walked: inside a run logical positions grow by one per position, so the
// queries within the window of some key of the workgroup are a prefix of each
// run, and only the tiles of those prefixes are visited (a list in LDS; a
// list longer than T_CAP falls back to the whole range).  A list entry is the
// tile's first query, with bit 31 set when the tile lies inside one run and
// its last logical query position is within the window of the smallest
// logical key position (decided from the run's bounds while the list is
// built, so the tile loop reads no positions from memory to decide it).
template <int D, bool WIN>
__global__ void __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkv_bf16_kernel(const BwdArgs args) {
    using TT = BwdTileBf16<D>;
    using SM = BwdDkvBf16Smem<D>;
    constexpr int BM = kBwdTile;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

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

    const __bf16* kh = reinterpret_cast<const __bf16*>(J.k) + kvh * J.k_sh;
    const __bf16* vh = reinterpret_cast<const __bf16*>(J.v) + kvh * J.v_sh;
    bf16x8 kreg[TT::DSTEPS];
    {
        const auto kr = make_rsrc(kh, ((J.n_k - 1) * J.k_st + D) * 2);
#pragma unroll
        for (int s = 0; s < TT::DSTEPS; ++s)
            kreg[s] = __builtin_bit_cast(bf16x8, buf_load16(kr, (jk * J.k_st + s * 16 + 8 * g) * 2));
    }
    lds_byte* const lds = to_lds(smem);
    const int q_st = J.q_st, do_st = J.do_st;
    BwdDma<D> dma_q, dma_do;
    dma_q.init(wave, lane, q_st);
    dma_do.init(wave, lane, do_st);
    {
        // the workgroup's 128 V rows, as four 32-row tiles
        BwdDma<D> dma_v;
        dma_v.init(wave, lane, J.v_st);
        const i32x4 v_rsrc = sgpr_rsrc(vh, (J.n_k - 1) * J.v_st * 2 + D * 2);
#pragma unroll
        for (int t = 0; t < 4; ++t) dma_v.issue(v_rsrc, j0 + t * 32, J.v_st, wave, lds + SM::V_OFF + t * TT::BYTES);
    }

    // query rows that can see a key of the workgroup: positions from the first
    // key's to the largest horizon; the full-tile bounds: last key position and
    // smallest horizon over the valid keys
    int hmax = horizon, hmin = valid_k ? horizon : 0x7fffffff, kmax = valid_k ? kpos : (int)0x80000000;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        hmax = max(hmax, __shfl_xor(hmax, off));
        hmin = min(hmin, __shfl_xor(hmin, off));
        kmax = max(kmax, __shfl_xor(kmax, off));
    }
    int* red = reinterpret_cast<int*>(smem + SM::R_OFF);
    if (lane == 0) {
        red[wave] = hmax;
        red[4 + wave] = hmin;
        red[8 + wave] = kmax;
    }
    __syncthreads();
    hmax = wave_uniform(max(max(red[0], red[1]), max(red[2], red[3])));
    hmin = wave_uniform(min(min(red[4], red[5]), min(red[6], red[7])));
    kmax = wave_uniform(max(max(red[8], red[9]), max(red[10], red[11])));
    const int pos_lo = J.kbase + J.kstride * j0;
    auto first_query_at_or_after = [&](int64_t x) -> int {
        if (x <= J.qbase) return 0;
        const int64_t i = (x - J.qbase + J.qstride - 1) / J.qstride;
        return (int)min<int64_t>(i, J.n_q);
    };
    const int i_begin = first_query_at_or_after(pos_lo) / BM * BM;
    int i_end = hmax == (int)0x80000000 ? 0 : first_query_at_or_after((int64_t)hmax);   // exclusive
    if (WIN && !tree && kmax != (int)0x80000000)
        i_end = min(i_end, first_query_at_or_after((int64_t)kmax + args.mask.window));
    int n_tiles = i_end > i_begin ? (i_end - i_begin + BM - 1) / BM : 0;
    // this lane's key's logical position
    const int lk = !WIN || !valid_k ? 0 : tree ? args.mask.lpos[kpos] : kpos;
    int* tlist = reinterpret_cast<int*>(smem + SM::T_OFF);
    bool use_list = false;
    const auto* segp = (const __attribute__((address_space(4))) int32_t*)args.mask.seg;
    const auto* lposp = (const __attribute__((address_space(4))) int32_t*)args.mask.lpos;
    // smallest logical key position of the workgroup (a tile whose largest
    // logical query position is within the window of it needs no window mask)
    int lkmin = 0;
    if (WIN && tree) {
        int lkm = valid_k ? lk : (int)0x80000000;
        int lkn = valid_k ? lk : 0x7fffffff;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            lkm = max(lkm, __shfl_xor(lkm, off));
            lkn = min(lkn, __shfl_xor(lkn, off));
        }
        if (lane == 0) {
            red[16 + wave] = lkm;
            red[24 + wave] = lkn;
        }
        __syncthreads();
        lkm = wave_uniform(max(max(red[16], red[17]), max(red[18], red[19])));
        lkmin = wave_uniform(min(min(red[24], red[25]), min(red[26], red[27])));
        if (wave == 0) {
            int cnt = 0, last = -1;
            bool over = false;
            int y = pos_lo;
            while (lkm != (int)0x80000000 && y < hmax && !over) {
                const i32x4 run = seg_entry(args.mask, segp[y]);
                const int64_t vis_end = (int64_t)y + max(0, lkm + args.mask.window - lposp[y]);
                const int e = (int)min((int64_t)min(run.y, hmax), vis_end);
                if (e > y) {
                    const int ib = first_query_at_or_after(e);
                    // logical position of a query of this run: lposp[y] + (position - y)
                    const int ly0 = lposp[y];
                    for (int t = first_query_at_or_after(y) / BM * BM; t < ib; t += BM) {
                        if (t <= last) continue;
                        if (cnt == SM::T_CAP) {
                            over = true;
                            break;
                        }
                        const int64_t yt0 = (int64_t)J.qbase + (int64_t)J.qstride * t;
                        const int64_t yt1 = (int64_t)J.qbase + (int64_t)J.qstride * min(t + BM - 1, J.n_q - 1);
                        const bool wfull = yt0 >= run.x && yt1 < run.y &&
                                           (int64_t)ly0 + (yt1 - y) - lkmin < args.mask.window;
                        if (lane == 0) tlist[cnt] = wfull ? (int)((uint32_t)t | 0x80000000u) : t;
                        ++cnt;
                        last = t;
                    }
                }
                y = run.y;   // the next run in storage order
            }
            if (lane == 0) red[20] = over ? -1 : cnt;
        }
        __syncthreads();
        const int c = wave_uniform(red[20]);
        if (c >= 0) {
            use_list = true;
            n_tiles = c;
        }
    }
    const int steps = n_tiles * J.kv_group;   // (query head, tile) pairs, head-major
    // list entry or computed first query of tile t (bit 31: window-full, see above)
    auto tile_entry = [&](int t) { return use_list ? wave_uniform(tlist[t]) : i_begin + t * BM; };
    auto tile_q0 = [&](int t) { return tile_entry(t) & 0x7fffffff; };

    f32x16 acck[TT::DBLK], accv[TT::DBLK];
#pragma unroll
    for (int b = 0; b < TT::DBLK; ++b) {
        acck[b] = f32x16{};
        accv[b] = f32x16{};
    }
    BwdReadOffsets<D> ro;
    ro.init(lane, mfma_row_perm(r32));
    // B operand rows of dP: this wave's 32 V rows (tile `wave` of the V block) in natural order
    const BwdRowRead vread{SM::V_OFF + wave * TT::BYTES + r32 * TT::ROWB, g ^ bwd_swizzle<D>(r32)};

    const int qbase = J.qbase, qstride = J.qstride;
    // (query head, tile) of the next load and of the tile being computed,
    // advanced without divisions; the job's fields are read once
    const int kv_group = J.kv_group, n_q = J.n_q;
    const __bf16* const q_all = reinterpret_cast<const __bf16*>(J.q);
    const __bf16* const do_all = reinterpret_cast<const __bf16*>(J.dout);
    const int64_t q_sh = J.q_sh, do_sh = J.do_sh;
    const float* const lse_all = J.lse;
    const float* const delta_all = J.delta;
    int ld_head = kvh * kv_group, ld_tile = 0;
    auto issue = [&](int slot) {
        const int q0 = tile_q0(ld_tile);
        const __bf16* qh = q_all + ld_head * q_sh;
        const __bf16* doh = do_all + ld_head * do_sh;
        dma_q.issue(sgpr_rsrc(qh, (n_q - 1) * q_st * 2 + D * 2), q0, q_st, wave, lds + SM::Q_OFF + slot * TT::BYTES);
        dma_do.issue(sgpr_rsrc(doh, (n_q - 1) * do_st * 2 + D * 2), q0, do_st, wave,
                     lds + SM::DO_OFF + slot * TT::BYTES);
        if (wave == 0)
            dma_b32(sgpr_rsrc(lse_all + (int64_t)ld_head * n_q, n_q * 4), (q0 + lane) * 4,
                    lds_addr(lds + SM::L_OFF + slot * 256));
        else if (wave == 1)
            dma_b32(sgpr_rsrc(delta_all + (int64_t)ld_head * n_q, n_q * 4), (q0 + lane) * 4,
                    lds_addr(lds + SM::DL_OFF + slot * 256));
        else if (WIN && tree && wave == 2)
            dma_b32(sgpr_rsrc(args.mask.lpos, args.mask.n_pos * 4), (qbase + qstride * (q0 + lane)) * 4,
                    lds_addr(lds + SM::LQ_OFF + slot * 256));
        if (++ld_tile == n_tiles) {
            ld_tile = 0;
            ++ld_head;
        }
    };

    const float c2 = args.scale_log2;
    if (steps > 0) issue(0);
    int cur_tile = 0;
    for (int step = 0; step < steps; ++step) {
        const int slot = step & 1;
        // this wave's loads of the current tile (and, first, the V block)
        // have landed; after the barrier every wave's have, and the other slot
        // is free
        __builtin_amdgcn_s_waitcnt(0xF70);
        if (wave == 0) {
            // The tile's LSEs (this wave's own load) are turned into base-2
            // units once, +inf for rows without gradient, so that each of
            // the 16 probabilities a lane computes per tile takes one fma
            // instead of a multiply, a compare and a select as well (every
            // lane of every wave reads 16 of these rows).
            auto* lw = reinterpret_cast<__attribute__((address_space(3))) float*>(lds + SM::L_OFF + slot * 256);
            const float lse = lw[lane];
            lw[lane] = lse > -INFINITY ? lse * 1.4426950408889634f : INFINITY;
        }
        bwd_tile_barrier();
        if (step + 1 < steps) issue(slot ^ 1);
        const int entry = tile_entry(cur_tile);
        const int q0 = entry & 0x7fffffff;
        if (++cur_tile == n_tiles) cur_tile = 0;
        const lds_byte* qt = lds + SM::Q_OFF + slot * TT::BYTES;
        const lds_byte* dt = lds + SM::DO_OFF + slot * TT::BYTES;
        // The kernel has no room for the 16 row-read offsets the compiler
        // would keep for the whole loop (it spilled up to 76 bytes per lane):
        // the swizzle words are made opaque per tile, so each offset is
        // recomputed next to its read (two vector instructions) and lives
        // only there.
        BwdRowRead rrow = ro.row, rv = vread;
        asm volatile("" : "+v"(rrow.x));
        asm volatile("" : "+v"(rv.x));

        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ds = 0; ds < TT::DSTEPS; ++ds) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(qt + rrow.off(ds)), kreg[ds], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(dt + rrow.off(ds)), lds_op(lds + rv.off(ds)), dp, 0, 0, 0);
        }
        // lane (key jk, half g), value i: query row q0 + il, il = 16 (i / 8) + 8 g + i % 8
        const auto* lp = reinterpret_cast<const __attribute__((address_space(3))) float*>(lds + SM::L_OFF + slot * 256) + 8 * g;
        const auto* dlp = reinterpret_cast<const __attribute__((address_space(3))) float*>(lds + SM::DL_OFF + slot * 256) + 8 * g;
        const int yq0 = qbase + qstride * q0;
        const int yq1 = qbase + qstride * min(q0 + BM - 1, n_q - 1);
        bool full = yq0 >= kmax && (!tree || yq1 < hmin);
        if (WIN)   // and every pair within the window
            full = full && (!tree ? yq1 - pos_lo < args.mask.window
                            : use_list ? entry < 0
                                       : segp[yq0] == segp[yq1] && lposp[yq1] - lkmin < args.mask.window);
        const auto* lqp = reinterpret_cast<const __attribute__((address_space(3))) int*>(lds + SM::LQ_OFF + slot * 256) + 8 * g;
        bf16x8 pb[2], dsb[2];
        // a row without gradient (LSE = -inf) gets p = 0
        auto prob = [&](int i, int il) { return __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lp[il])); };
        if (full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int il = (i >> 3) * 16 + (i & 7);   // + 8 g, folded into lp, dlp
                const float p = prob(i, il);
                pb[i >> 3][i & 7] = (__bf16)p;
                dsb[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dlp[il]));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int il = (i >> 3) * 16 + (i & 7);
                const int qrow = q0 + il + 8 * g;
                const int y = qbase + qstride * qrow;
                bool vis = qrow < n_q && kpos <= y && y < horizon;
                if (WIN) vis = vis && (tree ? lqp[il] : y) - lk < args.mask.window;
                const float p = vis ? prob(i, il) : 0.f;
                pb[i >> 3][i & 7] = (__bf16)p;
                dsb[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dlp[il]));
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int b = 0; b < TT::DBLK; ++b) {
                accv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr_operand<D>(dt, ro, st, b), pb[st], accv[b], 0,
                                                                  0, 0);
                acck[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr_operand<D>(qt, ro, st, b), dsb[st], acck[b],
                                                                  0, 0, 0);
            }
    }

    if (!valid_k) return;
    // lane (key jk, half g) holds dK^T / dV^T [d][jk] for d = 32 b + 8 (i / 4) + 4 g + i % 4
    float* krow = J.dk + ((int64_t)kvh * J.n_k + jk) * D;
    float* vrow = J.dv + ((int64_t)kvh * J.n_k + jk) * D;
    const float sc = args.scale;
#pragma unroll
    for (int b = 0; b < TT::DBLK; ++b)
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

}  // namespace cpattn
