// merge_kernel.hpp -- merge of n partial (O, LSE) results, and an output fill.
//
// The merge follows the stable log-sum-exp rule ("Context Parallelism in ART",
// section 03): with m the largest LSE of a row, w_p = exp(L_p - m),
// L = m + log(sum w_p) and O = sum w_p O_p / sum w_p, in fp32.  Rows whose
// every LSE is -inf give (0, -inf).  The kernel is bound by HBM bandwidth:
// each row reads n*(d+1) floats and writes d+1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

constexpr int kMaxMergeParts = 64;

// Accesses to data a kernel touches once (streamed parts, outputs): marked
// non-temporal, so the caches do not keep lines nobody reads again (the
// 4-part merge of 524288 rows x 128 ran 5.6 -> 6.2 TB/s, the rate of a plain
// copy; identical results).  Data read again (the merge adjoint's G and
// merged O, once per part) keeps ordinary loads.
using stream_f4 = float __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_once(const float4* p) {
    return __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const stream_f4*>(p)));
}
__device__ __forceinline__ float ld_once(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_once(float4* p, const float4& v) {
    __builtin_nontemporal_store(__builtin_bit_cast(stream_f4, v), reinterpret_cast<stream_f4*>(p));
}
__device__ __forceinline__ void st_once(float* p, float v) { __builtin_nontemporal_store(v, p); }

struct MergeArgs {
    const float* o[kMaxMergeParts];
    const float* l[kMaxMergeParts];
    float* o_out;
    float* l_out;
    int64_t rows;
    int32_t n;
    int32_t d;
    int32_t tpr;   // threads per row (consecutive threads of one workgroup)
};

// One row's d floats move as VEC-float units (VEC = 4 when d % 4 == 0 and
// every row start is 16-byte aligned, else 1).
template <int VEC> struct MergeUnit;
template <> struct MergeUnit<4> { using T = float4; };
template <> struct MergeUnit<1> { using T = float; };

__device__ __forceinline__ void merge_axpy(float4& acc, float w, const float4& v) {
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
}
__device__ __forceinline__ void merge_axpy(float& acc, float w, float v) { acc += w * v; }

// NP = n when 1 <= n <= 8: every LSE and every part's unit of a chunk is
// loaded before any arithmetic, so a thread has all n loads in flight, and the
// weights w_p are computed once per row.  NP = 0 serves any n in groups of 8
// (the last group's surplus slots re-read the final part with weight 0).
template <int NP, int VEC>
__global__ void __launch_bounds__(256) merge_kernel(const MergeArgs a) {
    using U = typename MergeUnit<VEC>::T;
    constexpr int G = NP > 0 ? NP : 8;
    const int rows_per_block = 256 / a.tpr;
    const int sub = threadIdx.x / a.tpr;
    const int t = threadIdx.x % a.tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + sub;
    const bool active = sub < rows_per_block && row < a.rows;
    const int n = NP > 0 ? NP : a.n;

    float m = -INFINITY;
    float z = 0.f;
    float w[G];
    if (active) {
        if (NP > 0) {
#pragma unroll
            for (int j = 0; j < G; ++j) w[j] = a.l[j][row];
#pragma unroll
            for (int j = 0; j < G; ++j) m = fmaxf(m, w[j]);
            const float ms = m == -INFINITY ? 0.f : m;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                w[j] = expf(w[j] - ms);
                z += w[j];
            }
        } else {
            for (int p0 = 0; p0 < n; p0 += G) {
#pragma unroll
                for (int j = 0; j < G; ++j) w[j] = a.l[min(p0 + j, n - 1)][row];
#pragma unroll
                for (int j = 0; j < G; ++j) m = fmaxf(m, w[j]);
            }
            if (m != -INFINITY)
                for (int p0 = 0; p0 < n; p0 += G) {
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const float e = expf(a.l[min(p0 + j, n - 1)][row] - m);
                        z += p0 + j < n ? e : 0.f;
                    }
                }
        }
    }
    const bool empty = m == -INFINITY;
    const float rz = empty ? 0.f : 1.f / z;
    // every thread has read its LSEs before any output LSE is written (the
    // output may alias part 0, and a row may span several waves)
    __syncthreads();
    if (active && !empty) {
        const int units = a.d / VEC;
        for (int c = t; c < units; c += a.tpr) {
            U acc{};
            if (NP > 0) {
                U v[G];
#pragma unroll
                for (int j = 0; j < G; ++j) v[j] = ld_once(reinterpret_cast<const U*>(a.o[j] + row * a.d) + c);
                // the scheduler would otherwise wait for each load before issuing the next
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < G; ++j) merge_axpy(acc, w[j] * rz, v[j]);
            } else {
                for (int p0 = 0; p0 < n; p0 += G) {
                    U v[G];
                    float lp[G];
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const int p = min(p0 + j, n - 1);
                        lp[j] = a.l[p][row];
                        v[j] = ld_once(reinterpret_cast<const U*>(a.o[p] + row * a.d) + c);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < G; ++j) merge_axpy(acc, p0 + j < n ? expf(lp[j] - m) * rz : 0.f, v[j]);
                }
            }
            st_once(reinterpret_cast<U*>(a.o_out + row * a.d) + c, acc);
        }
    } else if (active) {
        for (int c = t; c < a.d / VEC; c += a.tpr) st_once(reinterpret_cast<U*>(a.o_out + row * a.d) + c, U{});
    }
    // the general form re-reads the LSEs above: all of the block's threads are
    // past that before the output LSE (possibly part 0's) is written
    if (NP == 0) __syncthreads();
    if (active && t == 0) a.l_out[row] = empty ? -INFINITY : m + logf(z);
}

// (O, LSE) = (0, -inf) for rows that saw no key at all.
__global__ void __launch_bounds__(256) fill_empty_kernel(float* o, float* lse, int64_t rows, int64_t d) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < rows * d) st_once(o + i, 0.f);
    if (i < rows) lse[i] = -INFINITY;
}

// Learned attention sink applied once to a complete result ("Context
// Parallelism in ART", section 06: the sink is probability mass with zero
// value): L' = logaddexp(L, a_h), O' = O * exp(L - L').  One row of d floats
// per `tpr` consecutive threads, d % 4 == 0, in place.  A row with no visible
// key (L = -inf) becomes (0, a_h).  HBM-bound: reads and writes d + 1 floats.
struct SinkArgs {
    float* o;
    float* lse;
    const float* sink;     // [heads] logits, natural-log units
    int64_t rows;          // heads * rows per head
    int64_t rows_per_head;
    int32_t d;
    int32_t tpr;
};

__global__ void __launch_bounds__(256) sink_kernel(const SinkArgs a) {
    const int rows_per_block = 256 / a.tpr;
    const int sub = threadIdx.x / a.tpr;
    const int t = threadIdx.x % a.tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + sub;
    const bool active = sub < rows_per_block && row < a.rows;
    float l = -INFINITY, lt = -INFINITY, w = 0.f;
    if (active) {
        l = a.lse[row];
        const float s = a.sink[row / a.rows_per_head];
        const float m = fmaxf(l, s);
        lt = m == -INFINITY ? -INFINITY : m + logf(expf(l - m) + expf(s - m));
        w = l == -INFINITY ? 0.f : expf(l - lt);
    }
    // a row may span several waves: all of them read its LSE before it is replaced
    __syncthreads();
    if (!active) return;
    float4* o = reinterpret_cast<float4*>(a.o + row * a.d);
    for (int c = t; c < a.d / 4; c += a.tpr) {
        float4 v = ld_once(o + c);
        v.x *= w;
        v.y *= w;
        v.z *= w;
        v.w *= w;
        st_once(o + c, v);
    }
    if (t == 0) a.lse[row] = lt;
}

// ---------------------------------------------------------------------------
// Adjoints of the merge ("Context Parallelism in ART", section 04): for the
// merged (O, L) of parts (O_p, L_p), w_p = exp(L_p - L), an output gradient G
// and an optional LSE gradient gL,
//     dO_p = w_p G,   dL_p = w_p (dot(G, O_p - O) + gL).
// A part with L_p = -inf (or a row with L = -inf) gets w_p = 0.  One row per
// `tpr` consecutive lanes of one wave (tpr a power of two <= 64, d % 4 == 0),
// the dot products reduced with lane shuffles.  HBM-bound: per row reads
// (n + 2) d + n + 2 floats and writes n (d + 1).
struct MergeBwdArgs {
    const float* o[kMaxMergeParts];
    const float* l[kMaxMergeParts];
    float* go[kMaxMergeParts];
    float* gl[kMaxMergeParts];
    const float* o_m;      // merged O
    const float* l_m;      // merged L
    const float* g;        // gradient of merged O
    const float* g_l;      // gradient of merged L, or null
    int64_t rows;
    int32_t n;
    int32_t d;
    int32_t tpr;
};

__device__ __forceinline__ float row_sum(float v, int tpr) {
    for (int off = tpr >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__global__ void __launch_bounds__(256) merge_backward_kernel(const MergeBwdArgs a) {
    const int rows_per_block = 256 / a.tpr;
    const int sub = threadIdx.x / a.tpr;
    const int t = threadIdx.x % a.tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + sub;
    // rows past the end still take part in the shuffles (with zeros)
    const bool active = row < a.rows;
    const int chunks = a.d / 4;
    const float L = active ? a.l_m[row] : -INFINITY;
    const float gL = active && a.g_l ? a.g_l[row] : 0.f;
    const float4* om = reinterpret_cast<const float4*>(a.o_m + row * a.d);
    const float4* gg = reinterpret_cast<const float4*>(a.g + row * a.d);
    for (int p = 0; p < a.n; ++p) {
        const float lp = active ? a.l[p][row] : -INFINITY;
        const float w = (L == -INFINITY || lp == -INFINITY) ? 0.f : expf(lp - L);
        const float4* op = reinterpret_cast<const float4*>(a.o[p] + row * a.d);
        float4* gop = reinterpret_cast<float4*>(a.go[p] + row * a.d);
        float dot = 0.f;
        if (active) {
            for (int c = t; c < chunks; c += a.tpr) {
                const float4 gv = gg[c], ov = ld_once(op + c), mv = om[c];
                dot += gv.x * (ov.x - mv.x) + gv.y * (ov.y - mv.y) + gv.z * (ov.z - mv.z) + gv.w * (ov.w - mv.w);
                st_once(gop + c, float4{w * gv.x, w * gv.y, w * gv.z, w * gv.w});
            }
        }
        dot = row_sum(dot, a.tpr);
        if (active && t == 0) a.gl[p][row] = w * (dot + gL);
    }
}

// ---------------------------------------------------------------------------
// Adjoints of the sink step (section 06), from the buffers cpattn_apply_sink
// leaves: y = w O and L' = logaddexp(L, a_h), with u = exp(a_h - L') the
// sink's share of the softmax mass and w = 1 - u:
//     dO = w G,   dL = u dot(G, y),   da_h = -sum over the head's rows of u dot(G, y)
// (the same values as w (1 - w) dot(G, O) with O before the sink).  A row with
// no visible key (L = -inf: L' = a_h, y = 0) gets dO = 0, dL = 0.  The row
// terms are written to dL; sink_grad_kernel then sums them per head in a
// fixed order (deterministic).
struct SinkBwdArgs {
    const float* y;
    const float* lse;      // L'
    const float* sink;     // [heads]
    const float* g;
    float* go;
    float* gl;
    int64_t rows;
    int64_t rows_per_head;
    int32_t d;
    int32_t tpr;
};

__global__ void __launch_bounds__(256) sink_backward_kernel(const SinkBwdArgs a) {
    const int rows_per_block = 256 / a.tpr;
    const int sub = threadIdx.x / a.tpr;
    const int t = threadIdx.x % a.tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + sub;
    const bool active = row < a.rows;
    float u = 1.f;
    if (active) {
        const float lt = a.lse[row];
        const float s = a.sink[row / a.rows_per_head];
        u = lt == -INFINITY ? 1.f : fminf(1.f, expf(s - lt));
    }
    const float w = 1.f - u;
    const float4* yv = reinterpret_cast<const float4*>(a.y + row * a.d);
    const float4* gv = reinterpret_cast<const float4*>(a.g + row * a.d);
    float4* gov = reinterpret_cast<float4*>(a.go + row * a.d);
    float dot = 0.f;
    if (active) {
        for (int c = t; c < a.d / 4; c += a.tpr) {
            const float4 gg = ld_once(gv + c), yy = ld_once(yv + c);
            dot += gg.x * yy.x + gg.y * yy.y + gg.z * yy.z + gg.w * yy.w;
            st_once(gov + c, float4{w * gg.x, w * gg.y, w * gg.z, w * gg.w});
        }
    }
    dot = row_sum(dot, a.tpr);
    if (active && t == 0) a.gl[row] = u * dot;
}

// g_sink[h] = -sum_r gl[h][r]; one workgroup per head, fixed reduction order
__global__ void __launch_bounds__(256) sink_grad_kernel(const float* gl, int64_t rows_per_head, float* g_sink) {
    __shared__ float part[256];
    const int h = blockIdx.x;
    float acc = 0.f;
    for (int64_t r = threadIdx.x; r < rows_per_head; r += 256) acc += gl[h * rows_per_head + r];
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) g_sink[h] = -part[0];
}

}  // namespace cpattn
