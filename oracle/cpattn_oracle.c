/*
 * cpattn_oracle.c -- plain fp64 CPU reference for blockwise attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * path.
 *
 * What it computes (sources are the pages this project is built from):
 *
 *  - Attention of one query against a visible key set
 *    ("Context Parallelism in ART", section 02, the attention definition
 *    s_j = q.k_j/sqrt(d), p_j = softmax, o = sum p_j v_j) together with its
 *    log-sum-exp L_A = log sum_{j in A} exp(s_j) and o_A = sum exp(s_j - L_A) v_j
 *    (same page, section 02, the LSE definition).  The logarithm is natural.
 *
 *  - Visibility, from the same section 02 and the tiny-tree example of
 *    section 03: causal -> key position <= query position; tree -> keys earlier
 *    or equal in the query's own segment plus every token of every strict
 *    ancestor segment.  The predicate is evaluated explicitly per (query, key)
 *    pair by walking the parent links; no precomputed horizon is used, and
 *    nothing assumes the segments are stored in any particular order.
 *
 *  - The two-way merge of partial results in its max-shifted stable form
 *    ("Context Parallelism in ART", section 03: a = exp(L_A - m),
 *    b = exp(L_B - m), L = m + log(a + b), o = (a o_A + b o_B)/(a + b)),
 *    with m read as max(L_A, L_B).  An n-way merge is a left fold of the
 *    two-way merge, which the page states is composable.
 *
 *  - The learned attention sink, applied once to a complete result (same
 *    page, section 06): oracle_apply_sink.
 *
 *  - Backward: attention gradients with the global softmax derivative
 *    (section 04), the merge adjoints (section 04) and the sink adjoints
 *    (section 06).
 *
 *  Readings where the pages are silent:
 *  a query with no visible key gives O = 0 and L = -inf; merging with such a
 *  partial leaves the other side unchanged; merging two empty partials gives
 *  (0, -inf).
 *
 * Inputs may be fp64, fp32 or bf16 (raw 16-bit patterns); every value is
 * widened to fp64 exactly before any arithmetic.  All accumulation is fp64,
 * keys are visited in ascending key index, one query row at a time.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };
enum { OR_CAUSAL = 0, OR_TREE = 1, OR_FULL = 2 };

static double widen(const void* base, int dtype, int64_t idx) {
    if (dtype == OR_F64) return ((const double*)base)[idx];
    if (dtype == OR_F32) return (double)((const float*)base)[idx];
    /* bf16: the 16 stored bits are the top half of an IEEE binary32 */
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Is segment `anc` a strict ancestor of segment `s`?  Walks parent links
 * upward; a walk longer than n_seg steps means a cycle and counts as "no". */
static int is_strict_ancestor(const int32_t* parent, int32_t n_seg, int32_t anc, int32_t s) {
    int32_t cur = parent[s];
    for (int32_t steps = 0; cur >= 0 && steps <= n_seg; ++steps) {
        if (cur == anc) return 1;
        cur = parent[cur];
    }
    return 0;
}

/* Visibility of key at global position xk to query at global position xq. */
static int visible(int kind, const int32_t* seg, const int32_t* parent, int32_t n_seg,
                   int64_t xq, int64_t xk) {
    if (kind == OR_FULL) return 1;
    if (kind == OR_CAUSAL) return xk <= xq;
    int32_t sq = seg[xq], sk = seg[xk];
    if (sq == sk) return xk <= xq;
    return is_strict_ancestor(parent, n_seg, sk, sq);
}

/*
 * Logical positions of a packed tree ("Context Parallelism in ART", section
 * 06: position IDs follow the root-to-leaf path): lp[x] = the number of tokens
 * of the strict ancestor segments of seg(x) plus the number of earlier tokens
 * of seg(x) itself.  Counted plainly over the storage order (no assumption on
 * how segments are laid out).  Returns 0, or -1 on allocation failure.
 */
static int logical_positions(const int32_t* seg, int64_t n_pos, const int32_t* parent, int32_t n_seg,
                             int64_t* lp) {
    int64_t* len = (int64_t*)calloc((size_t)(n_seg > 0 ? n_seg : 1), sizeof(int64_t));
    int64_t* seen = (int64_t*)calloc((size_t)(n_seg > 0 ? n_seg : 1), sizeof(int64_t));
    if (!len || !seen) { free(len); free(seen); return -1; }
    for (int64_t x = 0; x < n_pos; ++x) len[seg[x]] += 1;
    for (int64_t x = 0; x < n_pos; ++x) {
        int64_t anc = 0;
        for (int32_t a = 0; a < n_seg; ++a)
            if (is_strict_ancestor(parent, n_seg, a, seg[x])) anc += len[a];
        lp[x] = anc + seen[seg[x]];
        seen[seg[x]] += 1;
    }
    free(len);
    free(seen);
    return 0;
}

/*
 * oracle_attention: for each head h and each selected query row, attention
 * over the keys the predicate makes visible.
 *
 *   Q element (h, i, c) is at Q[h*q_sh + i*q_st + c]; likewise K and V.
 *   qpos[i], kpos[j]: global positions of query row i and key row j.
 *   kind: OR_CAUSAL, OR_TREE (seg[] indexed by global position, parent[] by
 *         segment, -1 = root) or OR_FULL (every key visible).
 *   rows: the query rows to compute (n_rows of them), or NULL for all nq rows.
 *   O: [H][n_rows][dv] fp64,  L: [H][n_rows] fp64 (natural log).
 * Returns 0, or -1 on a bad argument (negative size, position out of range
 * of seg[] for a tree).
 */
int oracle_attention(int64_t H, int64_t nq, int64_t nk, int64_t d, int64_t dv, int dtype,
                     const void* Q, int64_t q_sh, int64_t q_st,
                     const void* K, int64_t k_sh, int64_t k_st,
                     const void* V, int64_t v_sh, int64_t v_st,
                     const int64_t* qpos, const int64_t* kpos,
                     int kind, const int32_t* seg, int64_t n_pos,
                     const int32_t* parent, int32_t n_seg,
                     int64_t window, double scale, const int64_t* rows, int64_t n_rows,
                     double* O, double* L, int n_threads) {
    if (H < 0 || nq < 0 || nk < 0 || d <= 0 || dv <= 0 || window < 0) return -1;
    if (window > 0 && kind == OR_FULL) return -1;
    if (!rows) n_rows = nq;
    if (kind == OR_TREE) {
        for (int64_t j = 0; j < nk; ++j)
            if (kpos[j] < 0 || kpos[j] >= n_pos) return -1;
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t i = rows ? rows[r] : r;
            if (i < 0 || i >= nq || qpos[i] < 0 || qpos[i] >= n_pos) return -1;
        }
    }
    /* sliding window ("Context Parallelism in ART", section 06): a query sees
     * only the keys whose logical position is within `window` tokens of its
     * own, the current token included; causal logical positions are the
     * global positions themselves */
    int64_t* lp = NULL;
    if (window > 0 && kind == OR_TREE) {
        lp = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_pos > 0 ? n_pos : 1));
        if (!lp || logical_positions(seg, n_pos, parent, n_seg, lp) != 0) { free(lp); return -1; }
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int64_t total = H * n_rows;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nk > 0 ? nk : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < total; ++t) {
            int64_t h = t / n_rows, r = t % n_rows;
            int64_t i = rows ? rows[r] : r;
            double* o = O + (h * n_rows + r) * dv;
            for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
            /* the visible key set A, in ascending key index */
            int64_t n_vis = 0;
            for (int64_t j = 0; j < nk; ++j) {
                if (!visible(kind, seg, parent, n_seg, qpos[i], kpos[j])) continue;
                if (window > 0) {
                    int64_t lq = lp ? lp[qpos[i]] : qpos[i], lk = lp ? lp[kpos[j]] : kpos[j];
                    if (lq - lk >= window) continue;
                }
                idx[n_vis++] = j;
            }
            if (n_vis == 0) {
                L[h * n_rows + r] = -INFINITY;
                continue;
            }
            /* s_j = q . k_j * scale */
            double m = -INFINITY;
            for (int64_t a = 0; a < n_vis; ++a) {
                int64_t j = idx[a];
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc += widen(Q, dtype, h * q_sh + i * q_st + c) *
                           widen(K, dtype, h * k_sh + j * k_st + c);
                s[a] = acc * scale;
                if (s[a] > m) m = s[a];
            }
            /* L_A = log sum exp(s_j), evaluated with the max shift */
            double z = 0.0;
            for (int64_t a = 0; a < n_vis; ++a) z += exp(s[a] - m);
            double lse = m + log(z);
            L[h * n_rows + r] = lse;
            /* o_A = sum exp(s_j - L_A) v_j */
            for (int64_t a = 0; a < n_vis; ++a) {
                int64_t j = idx[a];
                double p = exp(s[a] - lse);
                for (int64_t c = 0; c < dv; ++c) o[c] += p * widen(V, dtype, h * v_sh + j * v_st + c);
            }
        }
        free(s);
        free(idx);
    }
    free(lp);
    return 0;
}

/*
 * oracle_attention_backward: gradients of attention of the selected query
 * rows, given each row's complete output O and log-sum-exp L (over all of its
 * visible keys, not only this call's) and the incoming output gradient G
 * ("Context Parallelism in ART", section 04, the global softmax derivative):
 * with p_j = exp(s_j - L) over the keys of this call that the row sees and
 * D = dot(G, O),
 *     dS_j = p_j (dot(G, v_j) - D),   dV_j += p_j G,
 *     dQ   += scale dS_j k_j,          dK_j += scale dS_j q.
 * Because p_j and D are global, summing the calls over any partition of the
 * keys gives the gradients of the unpartitioned attention.
 *   O, G, dQ: [H][n_rows][d or dv] for the selected rows; L: [H][n_rows];
 *   dK: [H][nk][d], dV: [H][nk][dv].  All fp64, accumulated into (the caller
 *   zeroes them).  Rows are processed one after another (dK and dV are
 *   shared).  Returns 0, or -1 on a bad argument.
 */
int oracle_attention_backward(int64_t H, int64_t nq, int64_t nk, int64_t d, int64_t dv, int dtype,
                              const void* Q, int64_t q_sh, int64_t q_st,
                              const void* K, int64_t k_sh, int64_t k_st,
                              const void* V, int64_t v_sh, int64_t v_st,
                              const int64_t* qpos, const int64_t* kpos,
                              int kind, const int32_t* seg, int64_t n_pos,
                              const int32_t* parent, int32_t n_seg,
                              int64_t window, double scale, const int64_t* rows, int64_t n_rows,
                              const double* O, const double* L, const double* G,
                              double* dQ, double* dK, double* dV) {
    if (H < 0 || nq < 0 || nk < 0 || d <= 0 || dv <= 0 || window < 0) return -1;
    if (window > 0 && kind == OR_FULL) return -1;
    if (!rows) n_rows = nq;
    if (kind == OR_TREE) {
        for (int64_t j = 0; j < nk; ++j)
            if (kpos[j] < 0 || kpos[j] >= n_pos) return -1;
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t i = rows ? rows[r] : r;
            if (i < 0 || i >= nq || qpos[i] < 0 || qpos[i] >= n_pos) return -1;
        }
    }
    int64_t* lp = NULL;
    if (window > 0 && kind == OR_TREE) {
        lp = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_pos > 0 ? n_pos : 1));
        if (!lp || logical_positions(seg, n_pos, parent, n_seg, lp) != 0) { free(lp); return -1; }
    }
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t i = rows ? rows[r] : r;
            const double* o = O + (h * n_rows + r) * dv;
            const double* g = G + (h * n_rows + r) * dv;
            double* dq = dQ + (h * n_rows + r) * d;
            double l = L[h * n_rows + r];
            if (l == -INFINITY) continue;   /* the row saw no key at all: no gradient */
            double D = 0.0;
            for (int64_t c = 0; c < dv; ++c) D += g[c] * o[c];
            for (int64_t j = 0; j < nk; ++j) {
                if (!visible(kind, seg, parent, n_seg, qpos[i], kpos[j])) continue;
                if (window > 0) {
                    int64_t lq = lp ? lp[qpos[i]] : qpos[i], lk = lp ? lp[kpos[j]] : kpos[j];
                    if (lq - lk >= window) continue;
                }
                double s = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    s += widen(Q, dtype, h * q_sh + i * q_st + c) * widen(K, dtype, h * k_sh + j * k_st + c);
                double p = exp(s * scale - l);
                double gv = 0.0;
                for (int64_t c = 0; c < dv; ++c) gv += g[c] * widen(V, dtype, h * v_sh + j * v_st + c);
                double ds = p * (gv - D);
                for (int64_t c = 0; c < dv; ++c) dV[(h * nk + j) * dv + c] += p * g[c];
                for (int64_t c = 0; c < d; ++c) {
                    dq[c] += scale * ds * widen(K, dtype, h * k_sh + j * k_st + c);
                    dK[(h * nk + j) * d + c] += scale * ds * widen(Q, dtype, h * q_sh + i * q_st + c);
                }
            }
        }
    }
    free(lp);
    return 0;
}

/*
 * oracle_merge2_backward: adjoints of the two-way merge (same page, section
 * 04): with w_r = exp(L_r - L) for the merged (O, L), an incoming output
 * gradient G and LSE gradient gL,
 *     dO_r = w_r G,    dL_r = w_r (dot(G, o_r - o) + gL).
 * (The gL term is the derivative of L = log sum exp(L_r), i.e. w_r.)  Rows
 * whose merged L is -inf get zero adjoints.  All [n_rows][dv] / [n_rows].
 */
void oracle_merge_backward(int n_parts, const double* const* O_parts, const double* const* L_parts,
                           int64_t n_rows, int64_t dv, const double* O, const double* L,
                           const double* G, const double* gL, double* const* dO_parts, double* const* dL_parts) {
    for (int p = 0; p < n_parts; ++p) {
        for (int64_t r = 0; r < n_rows; ++r) {
            const double* o_r = O_parts[p] + r * dv;
            const double* o = O + r * dv;
            const double* g = G + r * dv;
            double w = (L[r] == -INFINITY || L_parts[p][r] == -INFINITY) ? 0.0 : exp(L_parts[p][r] - L[r]);
            double dot = 0.0;
            for (int64_t c = 0; c < dv; ++c) {
                dO_parts[p][r * dv + c] = w * g[c];
                dot += g[c] * (o_r[c] - o[c]);
            }
            dL_parts[p][r] = w * (dot + (gL ? gL[r] : 0.0));
        }
    }
}

/*
 * oracle_sink_backward: adjoints of the sink step (same page, section 06):
 * y = w o with w = exp(L - L_total), L_total = logaddexp(L, a); for an
 * incoming gradient g of y,
 *     dJ/do = w g,   dJ/dL = w (1 - w) dot(g, o),   dJ/da = -w (1 - w) dot(g, o)
 * summed over the rows of each head for a.  O is the output before the sink.
 * O, G, dO: [H][n_rows][dv]; L, dL: [H][n_rows]; a, da: [H].
 */
void oracle_sink_backward(int64_t n_heads, int64_t n_rows, int64_t dv, const double* O, const double* L,
                          const double* a, const double* G, double* dO, double* dL, double* da) {
    for (int64_t h = 0; h < n_heads; ++h) {
        da[h] = 0.0;
        for (int64_t r = 0; r < n_rows; ++r) {
            double l = L[h * n_rows + r];
            double m = l > a[h] ? l : a[h];
            double lt = (m == -INFINITY) ? -INFINITY : m + log(exp(l - m) + exp(a[h] - m));
            double w = (l == -INFINITY) ? 0.0 : exp(l - lt);
            const double* o = O + (h * n_rows + r) * dv;
            const double* g = G + (h * n_rows + r) * dv;
            double dot = 0.0;
            for (int64_t c = 0; c < dv; ++c) {
                dO[(h * n_rows + r) * dv + c] = w * g[c];
                dot += g[c] * o[c];
            }
            dL[h * n_rows + r] = w * (1.0 - w) * dot;
            da[h] += -w * (1.0 - w) * dot;
        }
    }
}

/*
 * oracle_merge2: (O_a, L_a) <- merge((O_a, L_a), (O_b, L_b)) for n_rows rows
 * of dv values each, in place on the first operand.
 */
void oracle_merge2(int64_t n_rows, int64_t dv, double* Oa, double* La,
                   const double* Ob, const double* Lb) {
    for (int64_t r = 0; r < n_rows; ++r) {
        double la = La[r], lb = Lb[r];
        double m = la > lb ? la : lb;
        double* oa = Oa + r * dv;
        const double* ob = Ob + r * dv;
        if (m == -INFINITY) { /* neither side saw a key */
            for (int64_t c = 0; c < dv; ++c) oa[c] = 0.0;
            La[r] = -INFINITY;
            continue;
        }
        double a = exp(la - m), b = exp(lb - m);
        for (int64_t c = 0; c < dv; ++c) oa[c] = (a * oa[c] + b * ob[c]) / (a + b);
        La[r] = m + log(a + b);
    }
}

/*
 * oracle_merge: left fold of oracle_merge2 over n_parts partials, starting
 * from part 0.  O_parts[p] is [n_rows][dv], L_parts[p] is [n_rows].
 */
void oracle_merge(int n_parts, const double* const* O_parts, const double* const* L_parts,
                  int64_t n_rows, int64_t dv, double* O, double* L) {
    if (n_parts <= 0) {
        for (int64_t r = 0; r < n_rows; ++r) {
            L[r] = -INFINITY;
            for (int64_t c = 0; c < dv; ++c) O[r * dv + c] = 0.0;
        }
        return;
    }
    memcpy(O, O_parts[0], sizeof(double) * (size_t)(n_rows * dv));
    memcpy(L, L_parts[0], sizeof(double) * (size_t)n_rows);
    for (int p = 1; p < n_parts; ++p) oracle_merge2(n_rows, dv, O, L, O_parts[p], L_parts[p]);
}

/*
 * oracle_apply_sink: a learned attention-sink logit a_h per head adds
 * probability mass with zero value to the softmax denominator, once per query
 * ("Context Parallelism in ART", section 06, the sink as probability mass:
 * L_total = logaddexp(L, a), w = exp(L - L_total), y = w o).  O is
 * [n_heads][n_rows][dv], L is [n_heads][n_rows], a is [n_heads]; in place.
 * logaddexp is taken in its max-shifted form.  A row with no visible key
 * (L = -inf) gets w = 0 and L_total = a (all of its mass is the sink's).
 */
void oracle_apply_sink(int64_t n_heads, int64_t n_rows, int64_t dv, double* O, double* L, const double* a) {
    for (int64_t h = 0; h < n_heads; ++h) {
        for (int64_t r = 0; r < n_rows; ++r) {
            double l = L[h * n_rows + r];
            double m = l > a[h] ? l : a[h];
            double lt = (m == -INFINITY) ? -INFINITY : m + log(exp(l - m) + exp(a[h] - m));
            double w = (l == -INFINITY) ? 0.0 : exp(l - lt);
            double* o = O + (h * n_rows + r) * dv;
            for (int64_t c = 0; c < dv; ++c) o[c] = w * o[c];
            L[h * n_rows + r] = lt;
        }
    }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
