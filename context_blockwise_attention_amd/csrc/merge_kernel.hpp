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

struct MergeArgs {
    const float* o[kMaxMergeParts];
    const float* l[kMaxMergeParts];
    float* o_out;
    float* l_out;
    int64_t rows;
    int32_t n;
    int32_t d;
    int32_t tpr;   // threads per row (consecutive threads of one workgroup)
    int32_t vec;   // 4 when d % 4 == 0, else 1
};

__global__ void __launch_bounds__(256) merge_kernel(const MergeArgs a) {
    const int rows_per_block = 256 / a.tpr;
    const int sub = threadIdx.x / a.tpr;
    const int t = threadIdx.x % a.tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + sub;
    const bool active = sub < rows_per_block && row < a.rows;

    float m = -INFINITY;
    float z = 0.f;
    if (active) {
        for (int p = 0; p < a.n; ++p) m = fmaxf(m, a.l[p][row]);
        if (m != -INFINITY)
            for (int p = 0; p < a.n; ++p) z += expf(a.l[p][row] - m);
    }
    // every thread has read its LSEs before any output LSE is written (the
    // output may alias part 0)
    __syncthreads();
    if (!active) return;
    const bool empty = m == -INFINITY;
    const float rz = empty ? 0.f : 1.f / z;
    if (a.vec == 4) {
        const int chunks = a.d / 4;
        for (int c = t; c < chunks; c += a.tpr) {
            float4 acc = {0.f, 0.f, 0.f, 0.f};
            if (!empty) {
                for (int p = 0; p < a.n; ++p) {
                    const float w = expf(a.l[p][row] - m);
                    const float4 v = reinterpret_cast<const float4*>(a.o[p] + row * a.d)[c];
                    acc.x += w * v.x;
                    acc.y += w * v.y;
                    acc.z += w * v.z;
                    acc.w += w * v.w;
                }
                acc.x *= rz;
                acc.y *= rz;
                acc.z *= rz;
                acc.w *= rz;
            }
            reinterpret_cast<float4*>(a.o_out + row * a.d)[c] = acc;
        }
    } else {
        for (int c = t; c < a.d; c += a.tpr) {
            float acc = 0.f;
            if (!empty) {
                for (int p = 0; p < a.n; ++p) acc += expf(a.l[p][row] - m) * a.o[p][row * a.d + c];
                acc *= rz;
            }
            a.o_out[row * a.d + c] = acc;
        }
    }
    if (t == 0) a.l_out[row] = empty ? -INFINITY : m + logf(z);
}

// (O, LSE) = (0, -inf) for rows that saw no key at all.
__global__ void __launch_bounds__(256) fill_empty_kernel(float* o, float* lse, int64_t rows, int64_t d) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < rows * d) o[i] = 0.f;
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
        float4 v = o[c];
        v.x *= w;
        v.y *= w;
        v.z *= w;
        v.w *= w;
        o[c] = v;
    }
    if (t == 0) a.lse[row] = lt;
}

}  // namespace cpattn
