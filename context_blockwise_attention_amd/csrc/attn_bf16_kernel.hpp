// attn_bf16_kernel.hpp -- software-pipelined partial attention for bf16 inputs
// on gfx950 (CDNA4).
//
// Same work decomposition, tile walk, online softmax and epilogue as the
// register-staged kernel in attn_kernel.hpp (one workgroup = 4 waves = 128
// query rows, S^T = K Q^T with one query per lane, lazily raised max), with
// three changes that matter on CDNA4:
//
//  * K, V (and the key horizons of tree masks) go from HBM straight into LDS
//    with buffer_load ... lds (no staging registers, no LDS write
//    instructions).  Rows are XOR-swizzled in 16-byte chunks so that the MFMA
//    operand reads are free of bank conflicts.
//  * V stays row-major in LDS; the A operand of O^T += V^T P^T is read with
//    ds_read_b64_tr_b16, which transposes 16x4 blocks of 16-bit elements
//    across each group of 16 lanes (lane i receives column i % 4 of rows
//    i/4, 4 + i/4, 8 + i/4, 12 + i/4 of the block its group addresses).
//  * Software pipeline: while the matrix cores compute the scores of tile
//    t+1 and accumulate P_t V_t, the vector ALUs turn the scores of tile t
//    into probabilities; the scores of tile t+1 are then masked and their
//    row max taken.  K runs two tiles ahead of its use, V one.
//
// Pipeline invariant at the top of iteration t: S holds the masked scores of
// tile t and m_run already accounts for them; LDS holds K(t+1) in
// kbuf[(t+1)&1], V(t) in vbuf[t&1] and E(t+1) in ebuf[(t+1)&1].  Iteration t
// issues V(t+1) -> vbuf[(t+1)&1] and K(t+2), E(t+2) -> kbuf[t&1], ebuf[t&1];
// every buffer it overwrites was last read in iteration t-1, which all waves
// finished before the barrier that ends iteration t-1.
#pragma once

#include "attn_kernel.hpp"

namespace cpattn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

template <int D>
struct BfTile {
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int ROWB = D * 2;              // bytes per row
    static constexpr int TILE_BYTES = BN * ROWB;    // one K or V tile
    static constexpr int NI = BN * CPR / 256;       // direct loads per thread per tile
    static constexpr int DSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    static constexpr int KSTEPS = BN / 16;
    // LDS map: K[2] | V[2] | E[2]
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = 2 * TILE_BYTES;
    static constexpr int E_OFF = 4 * TILE_BYTES;
    static constexpr int LDS_BYTES = E_OFF + 2 * BN * 4;
};

__device__ __forceinline__ lds_byte* to_lds(void* p) { return (lds_byte*)(p); }

// 16-byte MFMA operand from LDS
__device__ __forceinline__ bf16x8 lds_op(const lds_byte* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}
// transposed 4 x 16-bit read (see the header comment)
__device__ __forceinline__ u32x2 lds_tr4(const lds_byte* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_byte*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

template <int D>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(const LaunchArgs args) {
    using TT = BfTile<D>;
    constexpr int BN = TT::BN;
    constexpr int CPR = TT::CPR;
    constexpr int ROWB = TT::ROWB;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

    // ---- work item (XCD-aware; see the register-staged kernel) -------------
    const int per_xcd = gridDim.x / 8;
    const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (w >= args.total_wg) return;
    int ji = 0;
    while (ji + 1 < args.n_jobs && w >= args.jobs[ji + 1].wg_begin) ++ji;
    const JobArgs& J = args.jobs[ji];
    const int local = w - J.wg_begin;
    // integer division runs on the vector ALU; keep the results scalar
    const int head = wave_uniform(local / J.q_tiles);
    const int qtile = wave_uniform(J.q_tiles - 1 - (local % J.q_tiles));   // heavy (late) tiles first

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_uniform(tid >> 6);   // scalar: the wave index is uniform per wave
    const int r32 = lane & 31;
    const int g = lane >> 5;

    const int q_first = qtile * kBM;
    const int q_last = min(q_first + kBM, J.n_q) - 1;
    const int y0 = J.qbase + J.qstride * q_first;
    const int y1 = J.qbase + J.qstride * q_last;
    const int qi = q_first + wave * 32 + r32;
    const int ypos = J.qbase + J.qstride * qi;
    const bool tree = args.mask.kind == kTree;

    const __bf16* qh = reinterpret_cast<const __bf16*>(J.q) + head * J.q_sh;
    const __bf16* kh = reinterpret_cast<const __bf16*>(J.k) + head * J.k_sh;
    const __bf16* vh = reinterpret_cast<const __bf16*>(J.v) + head * J.v_sh;

    // Q^T operand in registers (rows past the block read as zero)
    bf16x8 qreg[TT::DSTEPS];
    {
        const auto qr = make_rsrc(qh, ((J.n_q - 1) * J.q_st + D) * 2);
        const int qoff = qi * J.q_st * 2;
#pragma unroll
        for (int s = 0; s < TT::DSTEPS; ++s)
            qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qr, qoff + (s * 16 + 8 * g) * 2));
    }

    lds_byte* const lds = to_lds(smem);

    // ---- direct HBM -> LDS loads ----------------------------------------------
    // Load instruction i of wave `wave` fills LDS bytes [1024*b, 1024*b + 1024)
    // of a tile, b = 4i + wave, lane L -> 16-byte slot 64b + L: row r = slot /
    // CPR, slot s = slot % CPR.  K rows store chunk c at slot c ^ (r % CPR),
    // V rows at slot c ^ (4r % CPR); for both the swizzle depends only on the
    // lane and the wave, so the per-lane source offset is the same for every i.
    constexpr int ROWS_PER_BLOCK = 1024 / ROWB;
    const int lrow = lane / CPR;   // row of this lane within its 1 KB block
    const int lslot = lane % CPR;
    // (4i + wave) * ROWS_PER_BLOCK is a multiple of CPR plus wave * ROWS_PER_BLOCK
    const int rmod = (wave * ROWS_PER_BLOCK + lrow) % CPR;
    const int voff_k = lrow * J.k_st * 2 + ((lslot ^ rmod) * 16);
    const int voff_v = lrow * J.v_st * 2 + ((lslot ^ ((4 * rmod) % CPR)) * 16);

    auto issue_kv = [&](const __bf16* base, int st, int voff, int tile, lds_byte* dst) {
        const int j0 = tile * BN;
#pragma unroll
        for (int i = 0; i < TT::NI; ++i) {
            const int b = i * 4 + wave;
            const int row0 = j0 + b * ROWS_PER_BLOCK;   // first key row of this 1 KB block
            // bytes of the block's rows that exist; later rows read as zero
            const int bytes = row0 < J.n_k ? (J.n_k - 1 - row0) * st * 2 + D * 2 : 0;
            const auto r = make_rsrc(base + (int64_t)row0 * st, bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + b * 1024, 16, voff, 0, 0, 0);
        }
    };
    auto issue_e = [&](int tile, lds_byte* dst) {
        if (wave == 0) {
            const int p0 = J.kbase + J.kstride * tile * BN;
            const auto r = make_rsrc(args.mask.end + p0, (args.mask.n_pos - p0) * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, lane * J.kstride * 4, 0, 0, 0);
        }
    };
    auto kbuf = [&](int i) { return lds + TT::K_OFF + (i & 1) * TT::TILE_BYTES; };
    auto vbuf = [&](int i) { return lds + TT::V_OFF + (i & 1) * TT::TILE_BYTES; };
    auto ebuf = [&](int i) { return lds + TT::E_OFF + (i & 1) * BN * 4; };

    // ---- LDS operand offsets (bytes) ------------------------------------------
    // K: lane (r32, g) feeds key row kb*32 + kperm, chunk 2*ds + g.
    const int kperm_i = (r32 >> 3) * 4 + (r32 & 3);
    const int kperm = (kperm_i >> 3) * 16 + ((r32 & 7) >> 2) * 8 + (kperm_i & 7);
    int koff[TT::DSTEPS];
#pragma unroll
    for (int ds = 0; ds < TT::DSTEPS; ++ds) koff[ds] = kperm * ROWB + (((2 * ds + g) ^ (kperm % CPR)) * 16);
    // V (transposed reads): lane l, group G = l / 16, j = l % 16, kq = j / 4,
    // q = j % 4 addresses key row 16*ks + 8*g + 4*h + kq, dims b*32 + 16*(G%2)
    // + 4q .. +3, i.e. chunk 4b + 2(G%2) + q/2, half q%2, at slot chunk ^ (4kq % CPR).
    const int G2 = (lane >> 4) & 1;
    const int kq = (lane & 15) >> 2;
    const int qq = lane & 3;
    int voffb[TT::DBLK];
#pragma unroll
    for (int b = 0; b < TT::DBLK; ++b)
        voffb[b] = (8 * g + kq) * ROWB + (((4 * b + 2 * G2 + (qq >> 1)) ^ ((4 * kq) % CPR)) * 16) + (qq & 1) * 8;

    f32x16 acc[TT::DBLK];
#pragma unroll
    for (int b = 0; b < TT::DBLK; ++b) acc[b] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c2 = args.scale_log2;

    // ---- pipeline stages ------------------------------------------------------
    auto qk = [&](const lds_byte* kb_lds, f32x16* s) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < TT::DSTEPS; ++ds) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(kb_lds + koff[ds]), qreg[ds], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(kb_lds + 32 * ROWB + koff[ds]), qreg[ds], s[1], 0,
                                                           0, 0);
        }
    };
    // visibility of partial tiles: key in the block and kpos <= ypos < end[kpos]
    auto mask = [&](f32x16* s, int tile, const lds_byte* e_lds) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int jl0 = kb * 32 + hf * 16 + g * 8;
                int ends[8];
                if (tree) {
                    const auto* ep = reinterpret_cast<const __attribute__((address_space(3))) int*>(e_lds) + jl0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) ends[e] = ep[e];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = tile * BN + jl0 + e;
                    bool vis = j < J.n_k && J.kbase + J.kstride * j <= ypos;
                    if (tree) vis = vis && ypos < ends[e];
                    s[kb][hf * 8 + e] = vis ? s[kb][hf * 8 + e] : -INFINITY;
                }
            }
        }
    };
    // row max of a tile and the lazy raise of m_run (rescales acc and l_run)
    auto update_max = [&](const f32x16* s) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = xhalf_max(mx) * c2;
        const bool raise = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < TT::DBLK; ++b) acc[b] *= alpha;
            m_run = raise ? mx : m_run;
        }
    };
    // probabilities of a tile, as the B operands of the PV MFMAs
    auto softmax = [&](const f32x16* s, bf16x8* pb) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m_use));
                if (i & 1) ps1 += p; else ps0 += p;
                pb[kb * 2 + (i >> 3)][i & 7] = (__bf16)p;
            }
        }
        l_run += ps0 + ps1;
    };
    auto pv = [&](const lds_byte* v_lds, const bf16x8* pb) {
#pragma unroll
        for (int ks = 0; ks < TT::KSTEPS; ++ks) {
#pragma unroll
            for (int b = 0; b < TT::DBLK; ++b) {
                const lds_byte* p = v_lds + ks * 16 * ROWB + voffb[b];
                const u32x2 lo = lds_tr4(p);
                const u32x2 hi = lds_tr4(p + 4 * ROWB);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], acc[b], 0, 0, 0);
            }
        }
    };

    // ---- prologue ---------------------------------------------------------------
    TileCursor<BN> cur;
    cur.init(J, args.mask, y0, y1);
    int t0, f0, t1 = 0, f1 = 0, t2 = 0, f2 = 0;
    if (cur.next(J, args.mask, y0, y1, &t0, &f0)) {
        bool has1 = cur.next(J, args.mask, y0, y1, &t1, &f1);
        issue_kv(kh, J.k_st, voff_k, t0, kbuf(0));
        issue_kv(vh, J.v_st, voff_v, t0, vbuf(0));
        if (tree) issue_e(t0, ebuf(0));
        if (has1) {
            issue_kv(kh, J.k_st, voff_k, t1, kbuf(1));
            if (tree) issue_e(t1, ebuf(1));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        f32x16 s[2], sn[2];
        bf16x8 pb[TT::KSTEPS];
        qk(kbuf(0), s);
        if (!f0) mask(s, t0, ebuf(0));
        update_max(s);
        // every wave has read kbuf(0) and ebuf(0) before they are refilled
        __syncthreads();
        int it = 0;
        while (has1) {
            const bool has2 = cur.next(J, args.mask, y0, y1, &t2, &f2);
            issue_kv(vh, J.v_st, voff_v, t1, vbuf(it + 1));
            if (has2) {
                issue_kv(kh, J.k_st, voff_k, t2, kbuf(it));
                if (tree) issue_e(t2, ebuf(it));
            }
            // one branch-free block: the probabilities of tile t (vector ALUs)
            // overlap the scores of tile t+1 and O += V(t) P(t) (matrix cores)
            softmax(s, pb);
            qk(kbuf(it + 1), sn);
            pv(vbuf(it), pb);
            // then the visibility mask and row max of tile t+1
            if (!f1) mask(sn, t1, ebuf(it + 1));
            update_max(sn);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            s[0] = sn[0];
            s[1] = sn[1];
            t1 = t2;
            f1 = f2;
            has1 = has2;
            ++it;
        }
        softmax(s, pb);
        pv(vbuf(it), pb);
    }

    write_result<D>(J, head, qi, g, acc, m_run, l_run);
}

}  // namespace cpattn
