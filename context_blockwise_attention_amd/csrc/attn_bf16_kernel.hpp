// attn_bf16_kernel.hpp -- partial attention for bf16 inputs on gfx950 (CDNA4).
//
// Same work decomposition, tile walk, online softmax and epilogue as the
// register-staged kernel in attn_kernel.hpp (S^T = K Q^T with one query per
// lane, lazily raised max), built around three CDNA4 features:
//
//  * K, V (and the key horizons of tree masks) go from HBM straight into LDS
//    with buffer_load ... lds (no staging registers, no LDS write
//    instructions).  Rows are XOR-swizzled in 16-byte chunks so that the MFMA
//    operand reads are free of bank conflicts.
//  * V stays row-major in LDS; the A operand of O^T += V^T P^T is read with
//    ds_read_b64_tr_b16, which transposes 16x4 blocks of 16-bit elements
//    across each group of 16 lanes (lane i receives column i % 4 of rows
//    i/4, 4 + i/4, 8 + i/4, 12 + i/4 of the block its group addresses).
//  * Two waves per SIMD in a ping-pong schedule: one runs its matrix phase
//    while the other runs the vector (softmax) phase, and the roles swap at
//    every workgroup barrier (details at the kernel).
#pragma once

#include "attn_kernel.hpp"

namespace cpattn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

__device__ __forceinline__ lds_byte* to_lds(void* p) { return (lds_byte*)(p); }

// 16-byte MFMA operand from LDS
__device__ __forceinline__ bf16x8 lds_op(const lds_byte* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}
// Raw buffer descriptor (base, stride 0, size in bytes, the flags of
// make_rsrc) as four scalar registers, for the inline-asm loads below.
__device__ __forceinline__ i32x4 sgpr_rsrc(const void* base, int32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = wave_uniform((int32_t)(uint32_t)a);
    r[1] = wave_uniform((int32_t)((a >> 32) & 0xffffu));
    r[2] = wave_uniform(bytes);
    r[3] = kBufferFlags;
    return r;
}
// Direct global -> LDS loads (buffer_load ... lds): lane l's 16 (or 4) bytes
// at buffer offset voff land at LDS byte address lds + 16 l (4 l); offsets
// past the buffer's size read as zero.  They are issued as inline asm so that
// the compiler does not make later LDS reads wait for them: the kernel tracks
// them itself (vmcnt) and synchronises the workgroup before any wave reads
// the destination.  Loads complete in issue order.  The LDS base travels in
// m0, which the asm saves and restores (the compiler treats m0 as reserved);
// GFX9 needs one wait state between an SALU write of m0 and the LDS-DMA
// instruction that reads it, hence the s_nop.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, int voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds)
        : "memory");
}
__device__ __forceinline__ void dma_b32(i32x4 rsrc, int voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds)
        : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const lds_byte* p) {
    return (uint32_t)wave_uniform((int32_t)(uint32_t)reinterpret_cast<uintptr_t>(p));
}

// transposed 4 x 16-bit read (see the header comment)
__device__ __forceinline__ u32x2 lds_tr4(const lds_byte* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_byte*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------------------
// Ping-pong kernel: one workgroup of 8 waves = 256 query rows.  Waves w and
// w + 4 share a SIMD (the dispatcher places them so).  Per key tile each wave
// has a matrix phase and a softmax phase:
//
//   M(t): P(t-1) V(t-1) and S(t) = K(t) Q^T      -> 32 MFMAs per wave
//   V(t): mask, exp, row sum of S(t) (row max     -> vector ALU only
//         only when the reference must move)
//
// After the workgroup barrier that opens iteration t (t = tile sequence
// index), group 0 (waves 0-3) runs M(t) then V(t) and group 1 runs V(t-1)
// then M(t), so each SIMD holds one wave in a matrix phase and one in a
// softmax phase and the matrix cores stay fed while the other wave computes
// exponentials.  There is one barrier per iteration: a second one between the
// phases (forcing the alternation) made the second matrix phase of every
// iteration markedly slower and cost ~15% per tile.
//
// Loads are split between the groups: group 0 issues V(t+1) as its softmax
// phase opens, group 1 issues K(t+2) and E(t+2) after its matrix phase, in
// the time it would otherwise wait at the barrier; each wave loads a quarter
// of a tile.  (A load instruction holds its wave until the CU's load path
// accepts it, about 1 KB per 16 cycles for the whole CU, so the issuing
// wave pays for the tile's transfer; measured per iteration, group 0's
// softmax phase is its longest stretch and group 1 finishes its matrix phase
// early.)  Before the barrier that opens iteration t+1 every wave waits for
// its own older loads, leaving in flight only the ones issued in iteration
// t: V gets about an iteration and a half and K about one iteration to
// arrive before a matrix phase reads it, which hides the HBM/L2 latency (all
// workgroups of a head walk the same tiles at about the same time, so most
// of them wait on the same miss).  K and V rotate over 3 buffers, E over 4:
// every buffer a load overwrites was last read before the barrier that
// precedes the load.  (Wider key tiles would halve the
// barriers per key, but 128-key scores and probabilities do not fit the 256
// registers a wave has at two waves per SIMD.)
// ---------------------------------------------------------------------------
constexpr int kPPThreads = 512;
constexpr int kPPBM = 256;

template <int D, int BN_, int PF_>
struct PPTile {
    static constexpr int BN = BN_;                     // keys per tile
    static constexpr int PF = PF_;                     // prefetch distance (iterations)
    static constexpr int CPR = D / 8;
    static constexpr int ROWB = D * 2;
    static constexpr int TILE_BYTES = BN * ROWB;
    static constexpr int NI = TILE_BYTES / 1024 / 4;   // 1 KB direct loads per wave per tile (4 waves load it)
    static constexpr int RPB = 1024 / ROWB;            // rows per 1 KB block
    static constexpr int DSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    static constexpr int KSTEPS = BN / 16;
    static constexpr int NKB = BN / 32;                // 32-key blocks per tile
    static constexpr int NBUF = PF + 1;                // K and V buffers
    static constexpr int NEB = PF + 2;                 // horizon buffers
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = NBUF * TILE_BYTES;
    static constexpr int E_OFF = 2 * NBUF * TILE_BYTES;
    static constexpr int LDS_BYTES = E_OFF + NEB * BN * 4;
    // sliding window on a tree: the keys' logical positions follow the horizons
    static constexpr int L_OFF = LDS_BYTES;
    static constexpr int LDS_BYTES_WIN = L_OFF + NEB * BN * 4;
    static_assert(NI >= 1 && BN % 64 == 0, "tile shape");
    static_assert(PF == 2, "the tile loop issues loads two iterations ahead");
};

// ---------------------------------------------------------------------------
// Epilogue through LDS.  The same arithmetic as write_result (the partial
// written, or merged into the running result by the stable rule), but the
// accumulators, which a lane holds as 16-byte pieces of its own row (a wave's
// store then touches 32 rows with 32 bytes each), are first written to an
// 8 KB LDS area of the wave and read back row-contiguous, so that every
// global load and store instruction covers whole 256-byte row halves.  Done
// in passes of 64 columns.  The area's 16-byte chunks are XOR-swizzled by
// row (conflict-free writes and reads).  Per-row factors go from the row's
// lanes to the reading lanes by lane shuffles.  `stage` must not be touched
// by any other wave while this runs.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void write_result_staged(const JobArgs& J, int head, int row0, int lane, const f32x16* acc,
                                                    float m_run, float l_run, lds_byte* stage) {
    constexpr int PASSES = D / 64;                // 64 columns per pass
    const int r32 = lane & 31;
    const int g = lane >> 5;
    const int qi = row0 + r32;                    // this lane's accumulator row
    const float l_tot = xhalf_sum(l_run);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_new = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    float* const ohead = J.o + (int64_t)head * J.n_q * D;
    float* const lhead = J.lse + (int64_t)head * J.n_q;
    // per-row factors: out = ca * O_old + cb * acc
    float ca = 0.f, cb = inv, lse_out = lse_new;
    if (J.accumulate) {
        const float lse_old = qi < J.n_q ? lhead[qi] : -INFINITY;
        const float M = fmaxf(lse_old, lse_new);
        const bool none = M == -INFINITY;
        const float wa = none ? 0.f : expf(lse_old - M), wb = none ? 0.f : expf(lse_new - M);
        const float z = wa + wb;
        const float rz = none ? 0.f : 1.f / z;
        ca = wa * rz;
        cb = wb * inv * rz;
        lse_out = none ? -INFINITY : M + logf(z);
    }
    // rows read back by this lane: row 4 it + lane / 16, chunk lane % 16
    const int rsub = lane >> 4, chunk = lane & 15;
    float ra[8], rb[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        ra[it] = __shfl(ca, it * 4 + rsub);
        rb[it] = __shfl(cb, it * 4 + rsub);
    }
    auto lds4 = [&](int row, int c) {
        return reinterpret_cast<__attribute__((address_space(3))) f32x4*>(stage + row * 256 + ((c ^ (row & 15)) << 4));
    };
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        // the running O is read once and the result written once: non-temporal
        // accesses, so the caches keep the K/V tiles other workgroups still
        // read (0.2-0.7% faster on every forward workload, identical results)
        f32x4 old[8];
        if (J.accumulate) {
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int row = it * 4 + rsub;
                old[it] = row0 + row < J.n_q
                              ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ohead + (int64_t)(row0 + row) * D + ps * 64 + chunk * 4))
                              : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        // accumulator blocks 2 ps, 2 ps + 1: lane (r32, g) holds columns
        // 32 b' + 8 q4 + 4 g + e of the pass, i.e. chunk 8 b' + 2 q4 + g
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int b = 2 * ps + bb;
                *lds4(r32, 8 * bb + 2 * q4 + g) =
                    f32x4{acc[b][q4 * 4 + 0], acc[b][q4 * 4 + 1], acc[b][q4 * 4 + 2], acc[b][q4 * 4 + 3]};
            }
        // the wave's own writes are in LDS before its reads (in-order per wave)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int row = it * 4 + rsub;
            const f32x4 a = *lds4(row, chunk);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = J.accumulate ? ra[it] * old[it][e] + rb[it] * a[e] : rb[it] * a[e];
            if (row0 + row < J.n_q) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(ohead + (int64_t)(row0 + row) * D + ps * 64 + chunk * 4));
        }
        // the next pass overwrites the area: every read of this one has returned
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
    }
    if (g == 0 && qi < J.n_q) lhead[qi] = lse_out;
}

template <int D, int BN_, int PF_, bool WIN>
__global__ void __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_pp_kernel(const LaunchArgs args) {
    using TT = PPTile<D, BN_, PF_>;
    constexpr int BN = TT::BN;
    constexpr int PF = TT::PF;
    constexpr int CPR = TT::CPR;
    constexpr int ROWB = TT::ROWB;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

    int ji, head, qtile;
    if (!work_item(args, blockIdx.x, &ji, &head, &qtile)) return;
    ji = wave_uniform(ji);
    head = wave_uniform(head);
    qtile = wave_uniform(qtile);
    // the few job fields the tile loop uses are copied to scalar registers;
    // the rest is read from the kernel arguments where needed (copying the
    // whole descriptor spilled scalar registers into vector lanes)
    const JobArgs& J = args.jobs[ji];
    const KeyBlock kblk{J.kbase, J.kstride, J.n_k};
    const int k_st = J.k_st, v_st = J.v_st;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_uniform(tid >> 6);
    const int group = wave >> 2;
    const int r32 = lane & 31;
    const int g = lane >> 5;

    const int q_first = qtile * kPPBM;
    const int q_last = min(q_first + kPPBM, J.n_q) - 1;
    const int y0 = J.qbase + J.qstride * q_first;
    const int y1 = J.qbase + J.qstride * q_last;
    const int qi = q_first + wave * 32 + r32;
    const int ypos = J.qbase + J.qstride * qi;
    const bool tree = args.mask.kind == kTree;
    // last key index of the block at or before this query's position
    const int jlim = min(J.n_k - 1, ypos < J.kbase ? -1 : (ypos - J.kbase) / J.kstride);
    // Sliding window (WIN): a key is visible only if its logical position is
    // above the query's minus the window.  Causal: logical = physical, so the
    // window is a lower key-index bound jlo per query.  Tree: the query's
    // logical position ly, compared with each key's (staged in LDS).
    int jlo = 0, ly = 0;
    if (WIN) {
        if (tree) {
            const auto lr = make_rsrc(args.mask.lpos, args.mask.n_pos * 4);
            ly = qi < J.n_q ? (int)__builtin_amdgcn_raw_buffer_load_b32(lr, ypos * 4, 0, 0) : 0;
        } else {
            const int lowest = ypos - args.mask.window + 1 - J.kbase;   // lowest visible key position, block-relative
            jlo = lowest <= 0 ? 0 : (lowest + J.kstride - 1) / J.kstride;
        }
    }

    const __bf16* qh = reinterpret_cast<const __bf16*>(J.q) + head * J.q_sh;
    const int kv_head = head / J.kv_group;   // grouped-query attention: query heads share a K/V head
    const __bf16* kh = reinterpret_cast<const __bf16*>(J.k) + kv_head * J.k_sh;
    const __bf16* vh = reinterpret_cast<const __bf16*>(J.v) + kv_head * J.v_sh;

    bf16x8 qreg[TT::DSTEPS];
    {
        const auto qr = make_rsrc(qh, ((J.n_q - 1) * J.q_st + D) * 2);
        const int qoff = qi * J.q_st * 2;
#pragma unroll
        for (int s = 0; s < TT::DSTEPS; ++s)
            qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qr, qoff + (s * 16 + 8 * g) * 2));
    }

    lds_byte* const lds = to_lds(smem);
    // direct loads: wave `wave`, load i fills 1 KB block b = 8i + wave of a
    // tile; lane L -> row b * RPB + L / CPR, slot L % CPR (see the
    // register-budget comment of attn_bf16_kernel for the swizzles)
    const int lrow = lane / CPR;
    const int lslot = lane % CPR;
    const int rmod = (wave * TT::RPB + lrow) % CPR;   // same for wave and wave & 3 (4 * RPB % CPR == 0)
    const int voff_k = lrow * J.k_st * 2 + ((lslot ^ rmod) * 16);
    const int voff_v = lrow * J.v_st * 2 + ((lslot ^ ((4 * rmod) % CPR)) * 16);
    // The head's K and V blocks (and the horizon array) as whole buffers: the
    // ragged tail of the last tile lies past the buffer's size and reads as
    // zero.  Per tile only the row offset (scalar) is added to each lane's
    // constant offset; all offsets stay below 2 GiB (checked on the host).
    const i32x4 k_rsrc = sgpr_rsrc(kh, (J.n_k - 1) * J.k_st * 2 + D * 2);
    const i32x4 v_rsrc = sgpr_rsrc(vh, (J.n_k - 1) * J.v_st * 2 + D * 2);
    const i32x4 e_rsrc = sgpr_rsrc(args.mask.end, args.mask.n_pos * 4);
    const i32x4 l_rsrc = WIN ? sgpr_rsrc(args.mask.lpos, args.mask.n_pos * 4) : i32x4{};
    // a tile is loaded by the four waves of group 0: wave w fills the 1 KB
    // blocks b = 4i + w; the horizons by its first wave
    const int wl = wave & 3;
    int voffk[TT::NI], voffv[TT::NI];
#pragma unroll
    for (int i = 0; i < TT::NI; ++i) {
        const int rows = (i * 4 + wl) * TT::RPB;   // first row of this wave's i-th 1 KB block
        voffk[i] = voff_k + rows * J.k_st * 2;
        voffv[i] = voff_v + rows * J.v_st * 2;
    }
    auto issue_kv = [&](const i32x4& rsrc, const int* voffs, int st, int tile, lds_byte* dst) {
        const int tile_bytes = tile * BN * st * 2;
#pragma unroll
        for (int i = 0; i < TT::NI; ++i) dma_b128(rsrc, voffs[i] + tile_bytes, lds_addr(dst + (i * 4 + wl) * 1024));
    };
    // horizons: the group's first BN/64 waves each load 64 of the tile's entries
    auto issue_e = [&](int tile, int slot) {
        constexpr int W64 = BN / 64;
        static_assert(!WIN || 2 * W64 <= 4, "horizon and logical-position loads fit the loading group");
        if (wl < W64)
            dma_b32(e_rsrc, (kblk.kbase + kblk.kstride * (tile * BN + wl * 64 + lane)) * 4,
                    lds_addr(lds + TT::E_OFF + (slot % TT::NEB) * BN * 4 + wl * 256));
        else if (WIN && wl < 2 * W64)
            dma_b32(l_rsrc, (kblk.kbase + kblk.kstride * (tile * BN + (wl - W64) * 64 + lane)) * 4,
                    lds_addr(lds + TT::L_OFF + (slot % TT::NEB) * BN * 4 + (wl - W64) * 256));
    };
    auto kbuf = [&](int s) { return lds + TT::K_OFF + (s % TT::NBUF) * TT::TILE_BYTES; };
    auto vbuf = [&](int s) { return lds + TT::V_OFF + (s % TT::NBUF) * TT::TILE_BYTES; };
    auto ebuf = [&](int s) { return lds + TT::E_OFF + (s % TT::NEB) * BN * 4; };
    // Wait until at most `pending` of this wave's vector-memory loads are in
    // flight (vmcnt only; the immediate leaves expcnt and lgkmcnt unwaited):
    // the largest immediate not above `pending` among the counts that occur
    // (a quarter tile of V, or of K with or without E; the prologue's K, E and
    // V).  Loads complete in issue order, so this waits for every older load.
    auto wait_older = [&](int pending) {
        constexpr int NI = TT::NI;
        static_assert(2 * NI + 1 < 16, "vmcnt immediate");
        if (pending >= 2 * NI + 1) __builtin_amdgcn_s_waitcnt(0xF70 | (2 * NI + 1));
        else if (pending >= 2 * NI) __builtin_amdgcn_s_waitcnt(0xF70 | (2 * NI));
        else if (pending >= NI + 1) __builtin_amdgcn_s_waitcnt(0xF70 | (NI + 1));
        else if (pending >= NI) __builtin_amdgcn_s_waitcnt(0xF70 | NI);
        else __builtin_amdgcn_s_waitcnt(0xF70);
    };

    const int kperm_i = (r32 >> 3) * 4 + (r32 & 3);
    const int kperm = (kperm_i >> 3) * 16 + ((r32 & 7) >> 2) * 8 + (kperm_i & 7);
    int koff[TT::DSTEPS];
#pragma unroll
    for (int ds = 0; ds < TT::DSTEPS; ++ds) koff[ds] = kperm * ROWB + (((2 * ds + g) ^ (kperm % CPR)) * 16);
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
    f32x16 s[TT::NKB];
    bf16x8 pb[TT::KSTEPS];

    auto qk = [&](const lds_byte* kb_lds) {
#pragma unroll
        for (int kb = 0; kb < TT::NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < TT::DSTEPS; ++ds)
#pragma unroll
            for (int kb = 0; kb < TT::NKB; ++kb)
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(kb_lds + kb * 32 * ROWB + koff[ds]), qreg[ds],
                                                                s[kb], 0, 0, 0);
    };
    auto pv = [&](const lds_byte* v_lds) {
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
    // softmax phase of one tile: mask (partial tiles), lazily raised max,
    // probabilities as the B operands of the next phase's PV MFMAs
    // A masked score becomes -inf in the register that holds it: written as a
    // tied asm operand, so that the masked and the unmasked paths leave the
    // scores in the same registers (with a plain select the compiler gave the
    // two paths different registers and copied all 32 scores on every full
    // tile).  `keep` is the wave's lane mask of visible entries.
    const float neg_inf = -INFINITY;
    auto keep_if = [&](float x, uint64_t keep) {
        asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(x) : "v"(neg_inf), "s"(keep));
        return x;
    };
    auto softmax_phase = [&](int tile, int full, const lds_byte* e_lds) {
        if (!full) {
            // key j (block index) is visible iff j <= jlim and, for trees,
            // ypos < end[kpos(j)]; jl below is the key's index in the tile.
            // Branch-free: one compare (two for trees) and a select per score.
            const int lim = jlim - tile * BN - 8 * g;
            const int lo = jlo - tile * BN - 8 * g;   // window (causal)
            if (tree) {
                const auto* ep = reinterpret_cast<const __attribute__((address_space(3))) int*>(e_lds) + 8 * g;
#pragma unroll
                for (int kb = 0; kb < TT::NKB; ++kb) {
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int jl0 = kb * 32 + hf * 16;   // + 8g, folded into lim and ep
                        int ends[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) ends[e] = ep[jl0 + e];
                        int lks[8];
                        if (WIN) {
                            const auto* lq = ep + (TT::L_OFF - TT::E_OFF) / 4;   // same slot, logical positions
#pragma unroll
                            for (int e = 0; e < 8; ++e) lks[e] = lq[jl0 + e];
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            uint64_t vis = __builtin_amdgcn_ballot_w64(jl0 + e <= lim) &
                                           __builtin_amdgcn_ballot_w64(ypos < ends[e]);
                            if (WIN) vis &= __builtin_amdgcn_ballot_w64(ly - lks[e] < args.mask.window);
                            s[kb][hf * 8 + e] = keep_if(s[kb][hf * 8 + e], vis);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < TT::NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int jl = kb * 32 + (i >> 3) * 16 + (i & 7);
                        uint64_t vis = __builtin_amdgcn_ballot_w64(jl <= lim);
                        if (WIN) vis &= __builtin_amdgcn_ballot_w64(jl >= lo);
                        s[kb][i] = keep_if(s[kb][i], vis);
                    }
            }
        }
        // Probabilities against the reference m (base 2, scaled), packed as
        // the PV operands; returns this lane's sum of them.
        auto probs = [&](float m) {
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < TT::NKB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m));
                    if (kb == 0 && i < 2) (i ? ps1 : ps0) = p;
                    else if (i & 1) ps1 += p;
                    else ps0 += p;
                    pb[kb * 2 + (i >> 3)][i & 7] = (__bf16)p;
                }
            }
            return ps0 + ps1;
        };
        // Fast path: once a row has a reference (m_run finite), its
        // probabilities are taken against it directly, without the tile's
        // max; they are kept only if every lane's sum stays within 2^kSumCap
        // (no probability can then exceed it, and a NaN sum fails the test).
        // Otherwise -- a row still without a reference, or scores that have
        // risen far above it -- the tile is redone on the exact path: row
        // max, reference raised lazily (by more than kTau), probabilities
        // recomputed.  Either way acc, l_run and the probabilities share one
        // reference, so the result is the same softmax.
        // (The windowed instantiation always takes the exact path: keeping
        // the scores live through the fast path's check next to the window's
        // registers spilled.)
        float ps = 0.f;
        bool exact = WIN || __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
        if (!exact) {
            ps = probs(m_run);
            exact = __builtin_amdgcn_ballot_w64(!(ps <= kSumCap)) != 0;
        }
        if (exact) {
            // (rare without a window) keeps the compiler from speculating the
            // exact path's arithmetic into every tile
            if (!WIN) __builtin_amdgcn_sched_barrier(0);
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < TT::NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            mx = xhalf_max(mx) * c2;
            const bool raise = mx > m_run + kTau;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                // rare: keeps the compiler from speculating the 64 accumulator
                // multiplies (by 1) into every tile
                __builtin_amdgcn_sched_barrier(0);
                const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < TT::DBLK; ++b) acc[b] *= alpha;
                m_run = raise ? mx : m_run;
            }
            ps = probs(m_run == -INFINITY ? 0.f : m_run);
            if (!WIN) __builtin_amdgcn_sched_barrier(0);
        }
        l_run += ps;
    };

    // A workgroup barrier orders memory but not arithmetic: keep the compiler
    // from moving vector or matrix instructions across phase boundaries.
    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    // The two waves of a SIMD are in opposite phases.  The one in its matrix
    // phase runs at raised issue priority so that its MFMAs and operand reads
    // go out as soon as they are ready, and the other wave's softmax fills
    // the gaps (without it the older wave wins every conflict).
    auto matrix_priority = [&](bool on) {
        __builtin_amdgcn_sched_barrier(0);
        if (on) __builtin_amdgcn_s_setprio(3);
        else __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // M phase schedule: LDS operand reads run ahead of the MFMAs that use
    // them (8 reads first, then one MFMA followed by its share of reads).
    auto m_schedule = [&](bool with_pv, bool with_qk) {
        if (with_pv) {
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < TT::KSTEPS * TT::DBLK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        if (with_qk) {
            if (!with_pv) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < TT::NKB * TT::DSTEPS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };

    // ---- phase loop ---------------------------------------------------------------
    // Iteration t (tile sequence index t): group 0 runs M(t) = {P(t-1)V(t-1),
    // S(t)} then V(t) = softmax(t); group 1 runs V(t-1) then M(t).  The first
    // (no P V; barriers on both sides of the first matrix phase) and last (no
    // S, no softmax for group 0) iterations are peeled so the steady-state
    // body has no conditional work, and each group runs its own copy of the
    // loop so that its loop-carried registers are allocated once (the G loop is
    // fully unrolled; each copy serves one group).  Every wave passes the same
    // barriers.
    int t_last = 1;   // tiles of the walk + 1 (the epilogue's staging avoids the last V buffer)
#pragma unroll
    for (int G = 0; G < 2; ++G) {
        if (group != G) continue;
        TileCursor<BN, WIN> cur;
        cur.init(kblk, args.mask, y0, y1);
        // tiles t, t+1, t+2 of the walk (h_*: whether they exist)
        int t_cur = 0, f_cur = 0, t_nxt = 0, f_nxt = 0, t_n2 = 0, f_n2 = 0;
        if (!cur.next(kblk, args.mask, y1, &t_cur, &f_cur)) break;   // tile 0
        bool h_nxt = cur.next(kblk, args.mask, y1, &t_nxt, &f_nxt);
        bool h_n2 = false;
        // Loads of K and E after the prologue: by group 1 (see the load
        // schedule above), except with a window, where group 0 issues every
        // load (measured: the window's partial tiles lengthen group 1's
        // softmax phase, and the split made the windowed ring ~1.5% slower)
        constexpr bool kSplitLoads = !WIN;
        // horizon loads per tile of this wave (group 0 in the prologue, then
        // the group that loads K)
        const int e_loads = (tree && wl < (WIN ? 2 : 1) * (BN / 64)) ? 1 : 0;
        // this wave's loads issued in the current iteration (they may stay in
        // flight across the next barrier)
        int pending = 0;
        // K/E of tile s of the walk into buffer slot s
        auto issue_ke = [&](int tile, int s) {
            issue_kv(k_rsrc, voffk, k_st, tile, kbuf(s));
            if (tree) issue_e(tile, s);
        };
        // prologue: group 0 loads K(0), E(0), V(0), K(1), E(1); only K(0) and
        // E(0) must land before barrier 0
        if (G == 0) {
            issue_ke(t_cur, 0);
            issue_kv(v_rsrc, voffv, v_st, t_cur, vbuf(0));
            if (h_nxt) issue_ke(t_nxt, 1);
            wait_older(TT::NI + (h_nxt ? TT::NI + e_loads : 0));
        }
        phase_barrier();                                                // barrier 0
        if (G == 0) {
            qk(kbuf(0));
            m_schedule(false, true);
            phase_barrier();                                            // barrier 1
            if (h_nxt) issue_kv(v_rsrc, voffv, v_st, t_nxt, vbuf(1));
            softmax_phase(t_cur, f_cur, ebuf(0));
            h_n2 = h_nxt && cur.next(kblk, args.mask, y1, &t_n2, &f_n2);
            if (!kSplitLoads && h_n2) issue_ke(t_n2, 2);
            pending = (h_nxt ? TT::NI : 0) + (!kSplitLoads && h_n2 ? TT::NI + e_loads : 0);   // V(1) (K(2), E(2))
        } else {
            h_n2 = h_nxt && cur.next(kblk, args.mask, y1, &t_n2, &f_n2);
            phase_barrier();                                            // barrier 1
            qk(kbuf(0));
            m_schedule(false, true);
            if (kSplitLoads && h_n2) issue_ke(t_n2, 2);   // K(2), E(2)
            pending = kSplitLoads && h_n2 ? TT::NI + e_loads : 0;
        }
        int t = 1;
        while (h_nxt) {
            // iteration t: tile t (= t_nxt) exists; t_n2 / h_n2 describe tile t+1
            const int t_prev = t_cur, f_prev = f_cur;
            t_cur = t_nxt;
            f_cur = f_nxt;
            t_nxt = t_n2;
            f_nxt = f_n2;
            h_nxt = h_n2;
            wait_older(pending);                                        // K(t), E(t), V(t-1) landed
            phase_barrier();                                            // opens iteration t
            if (G == 0) {
                matrix_priority(true);
                pv(vbuf(t - 1));
                qk(kbuf(t));
                m_schedule(true, true);
                matrix_priority(false);                                 // phase boundary
                if (h_nxt) issue_kv(v_rsrc, voffv, v_st, t_nxt, vbuf(t + 1));
                softmax_phase(t_cur, f_cur, ebuf(t));
                h_n2 = h_nxt && cur.next(kblk, args.mask, y1, &t_n2, &f_n2);
                if (!kSplitLoads && h_n2) issue_ke(t_n2, t + 2);
                pending = (h_nxt ? TT::NI : 0) + (!kSplitLoads && h_n2 ? TT::NI + e_loads : 0);
            } else {
                h_n2 = h_nxt && cur.next(kblk, args.mask, y1, &t_n2, &f_n2);
                softmax_phase(t_prev, f_prev, ebuf(t - 1));
                matrix_priority(true);                                  // phase boundary
                pv(vbuf(t - 1));
                qk(kbuf(t));
                m_schedule(true, true);
                matrix_priority(false);
                // K(t+2), E(t+2): issued while this group would wait at the barrier
                if (kSplitLoads && h_n2) issue_ke(t_n2, t + 2);
                pending = kSplitLoads && h_n2 ? TT::NI + e_loads : 0;
            }
            ++t;
        }
        // last iteration t = T: only tile T-1 (= cur) remains; nothing is left in flight
        t_last = t;
        wait_older(0);
        phase_barrier();                                                // barrier 2T
        if (G == 0) {
            pv(vbuf(t - 1));
            m_schedule(true, false);
            phase_barrier();                                            // barrier 2T+1
        } else {
            softmax_phase(t_cur, f_cur, ebuf(t - 1));
            phase_barrier();                                            // barrier 2T+1
            pv(vbuf(t - 1));
            m_schedule(true, false);
        }
    }

    if constexpr (TT::TILE_BYTES >= 2 * 8192) {
        // staging areas: group 0's waves use the K buffers (free since the
        // last S, before barrier 2T), group 1's waves the two V buffers that
        // its last PV does not read (each wave 8 KB)
        lds_byte* stage;
        if (group == 0) {
            stage = lds + TT::K_OFF + wave * 8192;
        } else {
            const int busy = (t_last - 1) % TT::NBUF;
            const int f = (wave - 4) >> 1;                   // 0 or 1: the f-th V buffer other than `busy`
            const int vb = f < busy ? f : f + 1;
            stage = lds + TT::V_OFF + vb * TT::TILE_BYTES + ((wave - 4) & 1) * 8192;
        }
        write_result_staged<D>(J, head, q_first + wave * 32, lane, acc, m_run, l_run, stage);
    } else {
        write_result<D>(J, head, qi, g, acc, m_run, l_run);   // d 64: tiles too small to stage in
    }
}

}  // namespace cpattn
