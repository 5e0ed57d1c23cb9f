// Host-side checks run under the address and undefined-behaviour sanitizers
// (built and run by tests/test_host_sanitize.py with g++; no GPU):
//
//  * the descriptor's host code (context_blockwise_attention_amd/csrc/
//    host_tree.hpp): tree validation, subtree ends, ancestor lengths,
//    logical positions and visible-pair counting, on random depth-first
//    preorder trees, against brute force over an explicit visibility
//    predicate (a packed token sees its own segment up to itself and every
//    token of its strict ancestor segments; with a window, only keys whose
//    root-to-leaf position is within the window of the query's --
//    "Context Parallelism in ART", sections 02, 03 and 06);
//  * the rejection of malformed trees with the documented status codes;
//  * large trees (no brute force) for memory-error coverage;
//  * the fp64 reference in oracle/cpattn_oracle.c (linked in), called on
//    random trees, windows, row subsets and merges, for memory errors and
//    non-finite results.
//
// Prints one line per group of checks and exits non-zero on the first failure.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "../context_blockwise_attention_amd/csrc/host_tree.hpp"

extern "C" {
int oracle_attention(int64_t H, int64_t nq, int64_t nk, int64_t d, int64_t dv, int dtype, const void* Q,
                     int64_t q_sh, int64_t q_st, const void* K, int64_t k_sh, int64_t k_st, const void* V,
                     int64_t v_sh, int64_t v_st, const int64_t* qpos, const int64_t* kpos, int kind,
                     const int32_t* seg, int64_t n_pos, const int32_t* parent, int32_t n_seg, int64_t window,
                     double scale, const int64_t* rows, int64_t n_rows, double* O, double* L, int n_threads);
int oracle_attention_backward(int64_t H, int64_t nq, int64_t nk, int64_t d, int64_t dv, int dtype, const void* Q,
                              int64_t q_sh, int64_t q_st, const void* K, int64_t k_sh, int64_t k_st, const void* V,
                              int64_t v_sh, int64_t v_st, const int64_t* qpos, const int64_t* kpos, int kind,
                              const int32_t* seg, int64_t n_pos, const int32_t* parent, int32_t n_seg,
                              int64_t window, double scale, const int64_t* rows, int64_t n_rows, const double* O,
                              const double* L, const double* G, double* dQ, double* dK, double* dV);
void oracle_merge(int n_parts, const double* const* O_parts, const double* const* L_parts, int64_t n_rows,
                  int64_t dv, double* O, double* L);
void oracle_merge_backward(int n_parts, const double* const* O_parts, const double* const* L_parts,
                           int64_t n_rows, int64_t dv, const double* O, const double* L, const double* G,
                           const double* gL, double* const* dO_parts, double* const* dL_parts);
void oracle_apply_sink(int64_t n_heads, int64_t n_rows, int64_t dv, double* O, double* L, const double* a);
void oracle_sink_backward(int64_t n_heads, int64_t n_rows, int64_t dv, const double* O, const double* L,
                          const double* a, const double* G, double* dO, double* dL, double* da);
}

using namespace cpattn_host;

static std::string g_msg;
static int record(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_msg = buf;
    return code;
}

static int g_fail = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);             \
            std::fprintf(stderr, "\n");                    \
            std::exit(1);                                  \
        }                                                  \
    } while (0)

struct Tree {
    std::vector<int32_t> seg, parent;
};

// Random tree stored in depth-first preorder: random parent links, segments
// renumbered in preorder, random run lengths in [lo, hi].
static Tree random_tree(std::mt19937_64& rng, int n_seg, int lo, int hi) {
    std::vector<int> par(n_seg);
    for (int s = 0; s < n_seg; ++s) par[s] = s == 0 ? -1 : (int)(rng() % (uint64_t)(s + 1)) - 1;
    std::vector<std::vector<int>> kids(n_seg);
    std::vector<int> roots;
    for (int s = 0; s < n_seg; ++s) (par[s] < 0 ? roots : kids[par[s]]).push_back(s);
    std::vector<int> order;
    std::vector<int> st(roots.rbegin(), roots.rend());
    while (!st.empty()) {
        int s = st.back();
        st.pop_back();
        order.push_back(s);
        for (auto it = kids[s].rbegin(); it != kids[s].rend(); ++it) st.push_back(*it);
    }
    std::vector<int> idx(n_seg);
    for (int i = 0; i < n_seg; ++i) idx[order[i]] = i;
    Tree t;
    t.parent.resize(n_seg);
    for (int i = 0; i < n_seg; ++i) t.parent[i] = par[order[i]] < 0 ? -1 : idx[par[order[i]]];
    for (int i = 0; i < n_seg; ++i) {
        int len = lo + (int)(rng() % (uint64_t)(hi - lo + 1));
        for (int k = 0; k < len; ++k) t.seg.push_back(i);
    }
    return t;
}

static bool is_strict_ancestor(const std::vector<int32_t>& parent, int a, int s) {
    for (int p = parent[s]; p >= 0; p = parent[p])
        if (p == a) return true;
    return false;
}

// Brute force: logical positions and the visibility predicate.
struct Brute {
    std::vector<int64_t> lpos;
    const Tree* t;
    explicit Brute(const Tree& tr) : t(&tr) {
        const int n = (int)tr.seg.size(), n_seg = (int)tr.parent.size();
        std::vector<int64_t> len(n_seg, 0), first(n_seg, -1);
        for (int x = 0; x < n; ++x) {
            if (first[tr.seg[x]] < 0) first[tr.seg[x]] = x;
            ++len[tr.seg[x]];
        }
        lpos.resize(n);
        for (int x = 0; x < n; ++x) {
            int64_t l = x - first[tr.seg[x]];
            for (int p = tr.parent[tr.seg[x]]; p >= 0; p = tr.parent[p]) l += len[p];
            lpos[x] = l;
        }
    }
    bool visible(int64_t y, int64_t x, int64_t window) const {
        const int sy = t->seg[y], sx = t->seg[x];
        const bool v = (sx == sy && x <= y) || is_strict_ancestor(t->parent, sx, sy);
        return v && (window == 0 || lpos[y] - lpos[x] < window);
    }
};

static int64_t brute_pairs(const Brute& b, cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk, int64_t w) {
    int64_t c = 0;
    for (int64_t i = 0; i < nq; ++i)
        for (int64_t j = 0; j < nk; ++j) c += b.visible(qp.base + qp.stride * i, kp.base + kp.stride * j, w);
    return c;
}

static int64_t causal_pairs(cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk, int64_t w) {
    int64_t c = 0;
    for (int64_t i = 0; i < nq; ++i)
        for (int64_t j = 0; j < nk; ++j) {
            const int64_t y = qp.base + qp.stride * i, x = kp.base + kp.stride * j;
            c += x <= y && (w == 0 || y - x < w);
        }
    return c;
}

// A random block of positions inside [0, n): (posmap, rows).
static void random_block(std::mt19937_64& rng, int64_t n, cpattn_posmap* p, int64_t* rows) {
    const int kind = (int)(rng() % 3);
    if (kind == 0) {   // contiguous
        int64_t a = (int64_t)(rng() % (uint64_t)n), b = (int64_t)(rng() % (uint64_t)n);
        if (a > b) std::swap(a, b);
        *p = cpattn_posmap{a, 1};
        *rows = b - a + 1;
    } else {   // strided (stripes and ragged strides)
        const int64_t stride = 2 + (int64_t)(rng() % 6);
        const int64_t base = (int64_t)(rng() % (uint64_t)std::min<int64_t>(stride, n));
        const int64_t max_rows = (n - 1 - base) / stride + 1;
        *p = cpattn_posmap{base, stride};
        *rows = 1 + (int64_t)(rng() % (uint64_t)max_rows);
    }
}

static void check_tree_counts(std::mt19937_64& rng, int trials) {
    int64_t layouts = 0;
    for (int trial = 0; trial < trials; ++trial) {
        const int n_seg = 1 + (int)(rng() % 24);
        Tree tr = random_tree(rng, n_seg, 1, 90);
        const int64_t n = (int64_t)tr.seg.size();
        HostTree h;
        h.kind = kKindTree;
        h.n_pos = n;
        std::vector<int32_t> stack;
        int rc = tree_host(tr.seg.data(), n, tr.parent.data(), n_seg, "check", record, h.segs, h.run_order, stack,
                           h.anc_len);
        CHECK(rc == CPATTN_OK, "valid preorder tree rejected: %s", g_msg.c_str());
        Brute b(tr);
        // subtree ends: one past the last position of any descendant-or-self
        for (int s = 0; s < n_seg; ++s) {
            int64_t end = h.segs[s].run_end;
            for (int u = 0; u < n_seg; ++u)
                if (is_strict_ancestor(tr.parent, s, u)) end = std::max<int64_t>(end, h.segs[u].run_end);
            CHECK(h.segs[s].subtree_end == end, "segment %d subtree end %d, brute force %lld", s,
                  h.segs[s].subtree_end, (long long)end);
        }
        // horizon form of the predicate: x visible to y iff x <= y < end[seg x]
        for (int64_t y = 0; y < n; y += 1 + (int64_t)(rng() % 3))
            for (int64_t x = 0; x < n; x += 1 + (int64_t)(rng() % 3)) {
                const bool hz = x <= y && y < h.segs[tr.seg[x]].subtree_end;
                CHECK(hz == b.visible(y, x, 0), "horizon predicate differs at y=%lld x=%lld", (long long)y,
                      (long long)x);
            }
        std::vector<int32_t> lpos;
        tree_lpos(h, lpos);
        for (int64_t x = 0; x < n; ++x)
            CHECK(lpos[x] == b.lpos[x], "logical position of %lld: %d vs %lld", (long long)x, lpos[x],
                  (long long)b.lpos[x]);
        // pair counts on random layouts, without and with windows
        for (int rep = 0; rep < 6; ++rep) {
            cpattn_posmap qp, kp;
            int64_t nq, nk;
            random_block(rng, n, &qp, &nq);
            random_block(rng, n, &kp, &nk);
            const int64_t w = rep % 2 ? 0 : 1 + (int64_t)(rng() % (uint64_t)(n + 2));
            h.window = (int32_t)w;
            const int64_t got = pair_count(h, qp, nq, kp, nk, 1);
            const int64_t want = brute_pairs(b, qp, nq, kp, nk, w);
            CHECK(got == want, "tree pair count %lld vs brute force %lld (window %lld)", (long long)got,
                  (long long)want, (long long)w);
            if (w == 0)
                CHECK(pair_nonempty_nowin(h, qp, nq, kp, nk) == (want > 0), "tree non-empty test disagrees");
            const int64_t est = pair_count(h, qp, nq, kp, nk, 1 + (int64_t)(rng() % 7));
            CHECK(est >= 0, "negative estimate");
            ++layouts;
        }
        h.window = 0;
    }
    std::printf("trees: %d random preorder trees, %lld layouts: subtree ends, horizons, logical positions, "
                "pair counts match brute force\n", trials, (long long)layouts);
}

static void check_causal_counts(std::mt19937_64& rng, int trials) {
    for (int trial = 0; trial < trials; ++trial) {
        const int64_t n = 1 + (int64_t)(rng() % 700);
        HostTree h;
        h.kind = kKindCausal;
        h.n_pos = n;
        cpattn_posmap qp, kp;
        int64_t nq, nk;
        random_block(rng, n, &qp, &nq);
        random_block(rng, n, &kp, &nk);
        const int64_t w = trial % 2 ? 0 : 1 + (int64_t)(rng() % (uint64_t)(n + 2));
        h.window = (int32_t)w;
        const int64_t want = causal_pairs(qp, nq, kp, nk, w);
        CHECK(pair_count(h, qp, nq, kp, nk, 1) == want, "causal pair count differs");
        if (w == 0) CHECK(pair_nonempty_nowin(h, qp, nq, kp, nk) == (want > 0), "causal non-empty test disagrees");
    }
    std::printf("causal: %d random layouts match brute force\n", trials);
}

static void check_rejections() {
    struct Case {
        std::vector<int32_t> seg, parent;
        int code;
        const char* what;
    } cases[] = {
        {{0, 0, 1, 1, 2, 2}, {-1, -1, 0}, CPATTN_EUNSUPPORTED, "child outside its parent's subtree"},
        {{0, 1, 0}, {-1, 0}, CPATTN_EINVAL, "split segment"},
        {{0, 0, 3}, {-1, 0}, CPATTN_EINVAL, "segment id out of range"},
        {{0, -1}, {-1}, CPATTN_EINVAL, "negative segment id"},
        {{0, 1}, {1, 0}, CPATTN_EINVAL, "parent cycle"},
        {{0, 1, 2}, {2, 0, 1}, CPATTN_EINVAL, "longer parent cycle"},
        {{0, 1}, {-1, 5}, CPATTN_EINVAL, "parent out of range"},
        {{0, 1}, {-1, 1}, CPATTN_EINVAL, "segment its own parent"},
        {{0, 0}, {-1, 0}, CPATTN_EINVAL, "segment without a token"},
        {{0, 0, 1, 1}, {1, -1}, CPATTN_EUNSUPPORTED, "parent stored after its child"},
    };
    for (const Case& c : cases) {
        std::vector<SegInfo> segs;
        std::vector<int32_t> order, stack;
        std::vector<int64_t> anc;
        int rc = tree_host(c.seg.data(), (int64_t)c.seg.size(), c.parent.data(), (int32_t)c.parent.size(), "check",
                           record, segs, order, stack, anc);
        CHECK(rc == c.code, "%s: code %d, expected %d (%s)", c.what, rc, c.code, g_msg.c_str());
    }
    std::vector<SegInfo> segs;
    std::vector<int32_t> order, stack;
    std::vector<int64_t> anc;
    int32_t one = 0, root = -1;
    CHECK(tree_host(nullptr, 3, &root, 1, "check", record, segs, order, stack, anc) == CPATTN_EINVAL, "NULL seg");
    CHECK(tree_host(&one, 1, nullptr, 1, "check", record, segs, order, stack, anc) == CPATTN_EINVAL, "NULL parent");
    CHECK(tree_host(&one, -1, &root, 1, "check", record, segs, order, stack, anc) == CPATTN_EINVAL, "n_tok < 0");
    CHECK(tree_host(&one, 1, &root, 0, "check", record, segs, order, stack, anc) == CPATTN_EINVAL, "no segments");
    CHECK(tree_host(nullptr, 0, nullptr, 0, "check", record, segs, order, stack, anc) == CPATTN_OK, "empty tree");
    std::printf("rejections: %zu malformed trees and 5 argument errors return their codes\n",
                sizeof cases / sizeof cases[0]);
}

static void check_large(std::mt19937_64& rng) {
    for (int trial = 0; trial < 3; ++trial) {
        Tree tr = random_tree(rng, 3000 + trial * 1000, 1, 120);
        const int64_t n = (int64_t)tr.seg.size();
        HostTree h;
        h.kind = kKindTree;
        h.n_pos = n;
        std::vector<int32_t> stack, lpos;
        CHECK(tree_host(tr.seg.data(), n, tr.parent.data(), (int32_t)tr.parent.size(), "check", record, h.segs,
                        h.run_order, stack, h.anc_len) == CPATTN_OK,
              "large tree rejected: %s", g_msg.c_str());
        tree_lpos(h, lpos);
        int64_t total = 0;
        const int N = 4;
        const int64_t c = n / N;
        for (int r = 0; r < N; ++r)
            for (int b = 0; b < N; ++b) {
                h.window = trial == 1 ? 4096 : 0;
                total += pair_count(h, cpattn_posmap{r * c, 1}, c, cpattn_posmap{b * c, 1}, c, 1);
                (void)pair_count(h, cpattn_posmap{r * c, 1}, c, cpattn_posmap{b * c, 1}, c, 97);
                h.window = 0;
                (void)pair_nonempty_nowin(h, cpattn_posmap{r * c, 1}, c, cpattn_posmap{b * c, 1}, c);
            }
        CHECK(total > 0, "large tree has no visible pair");
    }
    std::printf("large: 3 trees of up to %d segments through validation, logical positions and counting\n", 5000);
}

static void check_oracle(std::mt19937_64& rng) {
    std::normal_distribution<double> nd(0.0, 1.0);
    int calls = 0;
    for (int trial = 0; trial < 6; ++trial) {
        Tree tr = random_tree(rng, 1 + (int)(rng() % 8), 1, 40);
        const int64_t n = (int64_t)tr.seg.size(), H = 2, d = trial % 2 ? 64 : 16, dv = d;
        std::vector<double> Q(H * n * d), K(H * n * d), V(H * n * dv), G(H * n * dv);
        for (auto* v : {&Q, &K, &V, &G})
            for (double& x : *v) x = nd(rng);
        std::vector<int64_t> pos(n);
        for (int64_t i = 0; i < n; ++i) pos[i] = i;
        std::vector<int64_t> rows;
        for (int64_t i = 0; i < n; i += 1 + (int64_t)(rng() % 3)) rows.push_back(i);
        const int64_t nr = (int64_t)rows.size();
        const int64_t window = trial % 3 == 0 ? 0 : 1 + (int64_t)(rng() % (uint64_t)n);
        std::vector<double> O(H * nr * dv), L(H * nr);
        int rc = oracle_attention(H, n, n, d, dv, 0, Q.data(), n * d, d, K.data(), n * d, d, V.data(), n * dv, dv,
                                  pos.data(), pos.data(), 1, tr.seg.data(), n, tr.parent.data(),
                                  (int32_t)tr.parent.size(), window, 1.0 / std::sqrt((double)d), rows.data(), nr,
                                  O.data(), L.data(), 1);
        CHECK(rc == 0, "oracle_attention rejected a valid tree");
        for (double x : L) CHECK(std::isfinite(x), "non-finite LSE (every row sees itself)");
        std::vector<double> Gr(H * nr * dv), dQ(H * nr * d, 0.0), dK(H * n * d, 0.0), dV(H * n * dv, 0.0);
        for (size_t i = 0; i < Gr.size(); ++i) Gr[i] = G[i % G.size()];
        rc = oracle_attention_backward(H, n, n, d, dv, 0, Q.data(), n * d, d, K.data(), n * d, d, V.data(), n * dv,
                                       dv, pos.data(), pos.data(), 1, tr.seg.data(), n, tr.parent.data(),
                                       (int32_t)tr.parent.size(), window, 1.0 / std::sqrt((double)d), rows.data(),
                                       nr, O.data(), L.data(), Gr.data(), dQ.data(), dK.data(), dV.data());
        CHECK(rc == 0, "oracle_attention_backward rejected a valid tree");
        for (auto* v : {&dQ, &dK, &dV})
            for (double x : *v) CHECK(std::isfinite(x), "non-finite gradient");
        // merge of three partials (one row empty in every part), its adjoint, the sink and its adjoint
        const int P = 3;
        const int64_t rws = H * nr;
        std::vector<std::vector<double>> Op(P, std::vector<double>(rws * dv)), Lp(P, std::vector<double>(rws));
        for (int p = 0; p < P; ++p) {
            for (double& x : Op[p]) x = nd(rng);
            for (int64_t r = 0; r < rws; ++r) Lp[p][r] = r == 0 ? -INFINITY : 3.0 * nd(rng);
        }
        std::vector<const double*> op, lp;
        for (int p = 0; p < P; ++p) {
            op.push_back(Op[p].data());
            lp.push_back(Lp[p].data());
        }
        std::vector<double> Om(rws * dv), Lm(rws), gL(rws, 0.5);
        oracle_merge(P, op.data(), lp.data(), rws, dv, Om.data(), Lm.data());
        std::vector<std::vector<double>> dO(P, std::vector<double>(rws * dv)), dL(P, std::vector<double>(rws));
        std::vector<double*> dop, dlp;
        for (int p = 0; p < P; ++p) {
            dop.push_back(dO[p].data());
            dlp.push_back(dL[p].data());
        }
        oracle_merge_backward(P, op.data(), lp.data(), rws, dv, Om.data(), Lm.data(), Gr.data(), gL.data(),
                              dop.data(), dlp.data());
        std::vector<double> a(H), da(H), dOs(rws * dv), dLs(rws);
        for (double& x : a) x = nd(rng);
        std::vector<double> Os = Om, Ls = Lm;
        oracle_apply_sink(H, nr, dv, Os.data(), Ls.data(), a.data());
        oracle_sink_backward(H, nr, dv, Om.data(), Lm.data(), a.data(), Gr.data(), dOs.data(), dLs.data(), da.data());
        for (double x : da) CHECK(std::isfinite(x), "non-finite sink gradient");
        calls += 6;
    }
    std::printf("oracle: %d calls (attention, backward, merge, merge adjoint, sink, sink adjoint) on random trees\n",
                calls);
}

int main() {
    std::mt19937_64 rng(20261202);
    check_rejections();
    check_tree_counts(rng, 60);
    check_causal_counts(rng, 200);
    check_large(rng);
    check_oracle(rng);
    std::printf("host checks passed\n");
    return g_fail;
}
