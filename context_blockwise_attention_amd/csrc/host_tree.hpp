// host_tree.hpp -- host-only part of the visibility descriptor (plain C++17,
// no HIP): validation of a packed prefix tree, its per-segment runs, subtree
// ends and ancestor lengths, logical (root-to-leaf) positions, and the
// counting of visible (query, key) pairs between two blocks of positions.
//
// A query at position y sees key x iff x is in y's own segment at or before y,
// or x belongs to a strict ancestor segment of y's ("Context Parallelism in
// ART", sections 02-03); with a sliding window the key's logical position must
// also be within `window` of the query's (same page, section 06).  With the
// row stored in depth-first preorder this is x <= y < end[x], where end[x] is
// one past the last position of the subtree of x's segment.
//
// Kept free of device code so that it can be built and checked on the host
// alone (tests/host_tree_check.cpp, under the address and undefined-behaviour
// sanitizers).
#pragma once

#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/cpattn.h"

namespace cpattn_host {

enum : int32_t { kKindCausal = 0, kKindTree = 1 };

struct SegInfo {
    int32_t run_start, run_end, parent, subtree_end;
};

// The host side of a descriptor.
struct HostTree {
    int32_t kind = kKindCausal;
    int64_t n_pos = 0;
    std::vector<SegInfo> segs;        // tree: per segment
    std::vector<int32_t> run_order;   // tree: segments by run start
    std::vector<int64_t> anc_len;     // tree: tokens of the strict ancestors of each segment
    int32_t window = 0;               // sliding window in logical positions (0 = none)
};

// printf-style error reporter: records the message, returns the code
typedef int (*FailFn)(int code, const char* fmt, ...);

// Validates a prefix tree stored in depth-first preorder and fills the host
// parts of its descriptor: for each segment its run [run_start, run_end), its
// parent and the end of its subtree (segs), the segments in storage order
// (order) and the token count of each segment's strict ancestors (anc_len).
// The vectors are only assigned within the capacity they already have when
// it suffices (the no-allocation builder reserves it once).
inline int tree_host(const int32_t* seg_id, int64_t n_tok, const int32_t* parent, int32_t n_seg, const char* who,
                     FailFn fail, std::vector<SegInfo>& segs, std::vector<int32_t>& order,
                     std::vector<int32_t>& stack, std::vector<int64_t>& anc_len) {
    if (n_tok < 0 || n_tok > INT32_MAX) return fail(CPATTN_EINVAL, "%s: n_tok %lld out of range", who, (long long)n_tok);
    if (n_seg < 0) return fail(CPATTN_EINVAL, "%s: n_seg < 0", who);
    if ((n_tok > 0 && !seg_id) || (n_seg > 0 && !parent)) return fail(CPATTN_EINVAL, "%s: NULL array", who);
    if (n_tok > 0 && n_seg == 0) return fail(CPATTN_EINVAL, "%s: tokens but no segments", who);

    segs.assign((size_t)n_seg, SegInfo{-1, -1, -1, -1});
    for (int32_t s = 0; s < n_seg; ++s) {
        if (parent[s] < -1 || parent[s] >= n_seg || parent[s] == s)
            return fail(CPATTN_EINVAL, "%s: parent[%d] = %d out of range", who, s, parent[s]);
        segs[s].parent = parent[s];
    }
    // runs: every segment must be one contiguous, non-empty run
    order.clear();   // segments in storage order
    for (int64_t x = 0; x < n_tok; ++x) {
        int32_t s = seg_id[x];
        if (s < 0 || s >= n_seg) return fail(CPATTN_EINVAL, "%s: seg_id[%lld] = %d out of range", who, (long long)x, s);
        if (x == 0 || seg_id[x - 1] != s) {
            if (segs[s].run_start >= 0)
                return fail(CPATTN_EINVAL, "%s: segment %d is split into several runs", who, s);
            segs[s].run_start = (int32_t)x;
            order.push_back(s);
        }
        segs[s].run_end = (int32_t)x + 1;
    }
    for (int32_t s = 0; s < n_seg; ++s)
        if (segs[s].run_start < 0) return fail(CPATTN_EINVAL, "%s: segment %d has no token", who, s);
    // cycles (a parent chain that never reaches a root)
    for (int32_t s = 0; s < n_seg; ++s) {
        int32_t cur = s;
        int32_t steps = 0;
        while (cur >= 0 && steps <= n_seg) {
            cur = segs[cur].parent;
            ++steps;
        }
        if (cur >= 0) return fail(CPATTN_EINVAL, "%s: parent links of segment %d form a cycle", who, s);
    }
    // depth-first preorder: walking segments in storage order, the parent of
    // each must be on the stack of open ancestors; a segment's subtree closes
    // when a segment that is not its descendant starts.
    stack.clear();
    for (size_t i = 0; i < order.size(); ++i) {
        int32_t s = order[i];
        int32_t p = segs[s].parent;
        while (!stack.empty() && stack.back() != p) {
            segs[stack.back()].subtree_end = segs[s].run_start;
            stack.pop_back();
        }
        if (p >= 0 && stack.empty())
            return fail(CPATTN_EUNSUPPORTED,
                        "%s: segment %d is not stored inside its parent %d's subtree "
                        "(the row must be in depth-first preorder)", who, s, p);
        stack.push_back(s);
    }
    while (!stack.empty()) {
        segs[stack.back()].subtree_end = (int32_t)n_tok;
        stack.pop_back();
    }
    anc_len.assign((size_t)n_seg, 0);
    for (int32_t sgi : order) {   // preorder: a parent's total is known before its children's
        const int32_t p = segs[sgi].parent;
        anc_len[sgi] = p < 0 ? 0 : anc_len[p] + (segs[p].run_end - segs[p].run_start);
    }
    return CPATTN_OK;
}

// Logical position of every physical position of a tree: the tokens of its
// strict ancestors plus its offset inside its own run.
inline void tree_lpos(const HostTree& t, std::vector<int32_t>& lpos) {
    lpos.resize((size_t)t.n_pos);
    for (int32_t sg : t.run_order)
        for (int32_t x = t.segs[sg].run_start; x < t.segs[sg].run_end; ++x)
            lpos[x] = (int32_t)(t.anc_len[sg] + x - t.segs[sg].run_start);
}

// Number of keys of a block (positions base + stride * j, j < n) inside the
// position range [a, b].
inline int64_t keys_in_range(cpattn_posmap kp, int64_t nk, int64_t a, int64_t b) {
    if (a > b || nk == 0) return 0;
    auto ceil_div = [](int64_t x, int64_t y) { return x >= 0 ? (x + y - 1) / y : -((-x) / y); };
    auto floor_div = [](int64_t x, int64_t y) { return x >= 0 ? x / y : -((-x + y - 1) / y); };
    const int64_t lo = std::max<int64_t>(0, ceil_div(a - kp.base, kp.stride));
    const int64_t hi = std::min<int64_t>(nk - 1, floor_div(b - kp.base, kp.stride));
    return hi >= lo ? hi - lo + 1 : 0;
}

// Visible (query, key) pairs of a block pair, counted on every step-th query
// row and scaled by step (exact for step = 1).  Positions must lie inside the
// descriptor (the callers check them).
inline int64_t pair_count(const HostTree& m, cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk,
                          int64_t step) {
    if (nq == 0 || nk == 0) return 0;
    int64_t sum = 0;
    for (int64_t i = 0; i < nq; i += step) {
        const int64_t y = qp.base + qp.stride * i;
        // keys of a run of segment s (positions [a, b]) whose logical position
        // (x - run_start + anc_len) is within the window of the query's
        const int64_t W = m.window;
        if (m.kind == kKindCausal) {
            sum += keys_in_range(kp, nk, W > 0 ? std::max<int64_t>(0, y - W + 1) : 0, y);
            continue;
        }
        // segment of position y: the last run starting at or before y
        auto it = std::upper_bound(m.run_order.begin(), m.run_order.end(), y,
                                   [&](int64_t v, int32_t seg) { return v < m.segs[seg].run_start; });
        int32_t sg = *(it - 1);
        const int64_t ly = m.anc_len[sg] + y - m.segs[sg].run_start;
        auto clip = [&](int32_t s2) {   // first position of s2's run inside the window
            const int64_t lbase = m.segs[s2].run_start - m.anc_len[s2];
            return W > 0 ? std::max<int64_t>(m.segs[s2].run_start, ly - W + 1 + lbase) : (int64_t)m.segs[s2].run_start;
        };
        int64_t c = keys_in_range(kp, nk, clip(sg), y);
        for (int32_t a = m.segs[sg].parent; a >= 0; a = m.segs[a].parent)
            c += keys_in_range(kp, nk, clip(a), m.segs[a].run_end - 1);
        sum += c;
    }
    return sum * step;
}

// Does any query of the block see any key of the block?  Exact without a
// window (per segment, the smallest key position gives the widest chance);
// with a window the answer is pair_count(..., 1) > 0.
inline bool pair_nonempty_nowin(const HostTree& m, cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk) {
    if (nq == 0 || nk == 0) return false;
    const int64_t qmax = qp.base + qp.stride * (nq - 1);
    auto first_query_at_or_after = [&](int64_t x) -> int64_t {
        if (x <= qp.base) return qp.base;
        int64_t i = (x - qp.base + qp.stride - 1) / qp.stride;
        return qp.base + qp.stride * i;
    };
    if (m.kind == kKindCausal) return kp.base <= qmax;
    const int64_t kmax = kp.base + kp.stride * (nk - 1);
    for (const SegInfo& s : m.segs) {
        int64_t lo = std::max<int64_t>(s.run_start, kp.base);
        int64_t hi = std::min<int64_t>(s.run_end - 1, kmax);
        if (lo > hi) continue;
        int64_t j = (lo - kp.base + kp.stride - 1) / kp.stride;   // first key of the block in the run
        int64_t xa = kp.base + kp.stride * j;
        if (xa > hi) continue;
        int64_t y = first_query_at_or_after(xa);
        if (y <= qmax && y < s.subtree_end) return true;
    }
    return false;
}

}  // namespace cpattn_host
