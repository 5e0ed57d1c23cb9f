// api.hip -- C ABI of the blockwise attention library (declared in cpattn.h).
//
// Host responsibilities: argument validation (fail fast, no fallback), the
// prefix-tree visibility descriptor, the ring schedule (which key/value block
// each rank visits in each round, which rounds are empty), and packing the
// work of one round into a single launch.  All arithmetic runs in the kernels
// of attn_kernel.hpp and merge_kernel.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/cpattn.h"
#include "host_tree.hpp"
#include "attn_bf16_kernel.hpp"
#include "attn_bwd_bf16_kernel.hpp"
#include "attn_bwd_kernel.hpp"
#include "attn_kernel.hpp"
#include "merge_kernel.hpp"
#include "probe_kernel.hpp"

using namespace cpattn;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

static int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

static int hip_fail(hipError_t e, const char* what) {
    return fail(CPATTN_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

extern "C" const char* cpattn_last_error(void) { return g_last_error.c_str(); }
extern "C" int cpattn_version(void) { return (CPATTN_VERSION_MAJOR << 16) | CPATTN_VERSION_MINOR; }

// ---------------------------------------------------------------------------
// visibility descriptor
// ---------------------------------------------------------------------------
using cpattn_host::HostTree;
using cpattn_host::SegInfo;
static_assert(cpattn_host::kKindCausal == kCausal && cpattn_host::kKindTree == kTree, "mask kinds");

// Host-side pair counts of a (query block, key block) layout, cached in the
// descriptor (it is immutable), so that repeated ring calls over the same
// layout do no per-row host work.
struct PairKey {
    int64_t v[6];   // q base, q stride, q rows, k base, k stride, k rows
    bool operator==(const PairKey& o) const { return std::memcmp(v, o.v, sizeof v) == 0; }
};
struct PairKeyHash {
    size_t operator()(const PairKey& k) const {
        uint64_t h = 1469598103934665603ull;   // FNV-1a over the six fields
        for (int i = 0; i < 6; ++i) {
            h ^= (uint64_t)k.v[i];
            h *= 1099511628211ull;
        }
        return (size_t)h;
    }
};
struct PairStats {
    int64_t exact = -1;       // visible pairs (-1: not computed yet)
    double estimate = -1.0;   // sampled estimate used to order a launch's jobs
};
constexpr size_t kPairCacheMax = 4096;

// host part (kind, positions, segment runs, window) plus the device arrays
struct cpattn_mask : HostTree {
    int32_t* d_seg = nullptr;     // [n_pos]
    int32_t* d_end = nullptr;     // [n_pos]
    int4* d_segtab = nullptr;     // [n_seg]
    int32_t* d_lpos = nullptr;    // [n_pos] logical positions (tree with a window)
    bool is_static = false;       // device arrays in the library's static buffer (cpattn_mask_tree_static)
    mutable std::mutex pair_mu;   // guards pair_cache (calls may come from several threads)
    mutable std::unordered_map<PairKey, PairStats, PairKeyHash> pair_cache;
};

extern "C" int cpattn_mask_causal(int64_t n_pos, cpattn_mask** out) {
    if (!out) return fail(CPATTN_EINVAL, "cpattn_mask_causal: out is NULL");
    if (n_pos < 0 || n_pos > INT32_MAX) return fail(CPATTN_EINVAL, "cpattn_mask_causal: n_pos %lld out of range", (long long)n_pos);
    cpattn_mask* m = new (std::nothrow) cpattn_mask();
    if (!m) return fail(CPATTN_ENOMEM, "cpattn_mask_causal: out of host memory");
    m->kind = kCausal;
    m->n_pos = n_pos;
    *out = m;
    return CPATTN_OK;
}

extern "C" int cpattn_mask_free(cpattn_mask* m) {
    if (!m || m->is_static) return CPATTN_OK;   // a static descriptor belongs to the library
    hipError_t e1 = m->d_seg ? hipFree(m->d_seg) : hipSuccess;
    hipError_t e2 = m->d_end ? hipFree(m->d_end) : hipSuccess;
    hipError_t e3 = m->d_segtab ? hipFree(m->d_segtab) : hipSuccess;
    hipError_t e4 = m->d_lpos ? hipFree(m->d_lpos) : hipSuccess;
    delete m;
    if (e1 != hipSuccess) return hip_fail(e1, "cpattn_mask_free");
    if (e2 != hipSuccess) return hip_fail(e2, "cpattn_mask_free");
    if (e3 != hipSuccess) return hip_fail(e3, "cpattn_mask_free");
    if (e4 != hipSuccess) return hip_fail(e4, "cpattn_mask_free");
    return CPATTN_OK;
}

extern "C" int64_t cpattn_mask_npos(const cpattn_mask* m) { return m ? m->n_pos : -1; }

// The device arrays of a tree descriptor, staged on the host: the subtree end
// of each position and the segment table.
static void tree_arrays(const int32_t* seg_id, int64_t n_tok, const std::vector<SegInfo>& segs,
                        std::vector<int32_t>& end, std::vector<int4>& tab) {
    end.resize((size_t)n_tok);
    for (int64_t x = 0; x < n_tok; ++x) end[x] = segs[seg_id[x]].subtree_end;
    tab.resize(segs.size());
    for (size_t s = 0; s < segs.size(); ++s)
        tab[s] = int4{segs[s].run_start, segs[s].run_end, segs[s].parent, segs[s].subtree_end};
}

// Uploads a tree descriptor's device arrays (enqueued on st, complete on return).
static hipError_t tree_upload(int32_t* d_seg, int32_t* d_end, int4* d_segtab, const int32_t* seg_id, int64_t n_tok,
                              const std::vector<int32_t>& end, const std::vector<int4>& tab, hipStream_t st) {
    hipError_t e = hipSuccess;
    if (n_tok > 0 &&
        ((e = hipMemcpyAsync(d_seg, seg_id, sizeof(int32_t) * n_tok, hipMemcpyHostToDevice, st)) != hipSuccess ||
         (e = hipMemcpyAsync(d_end, end.data(), sizeof(int32_t) * n_tok, hipMemcpyHostToDevice, st)) != hipSuccess))
        return e;
    if (!tab.empty() &&
        (e = hipMemcpyAsync(d_segtab, tab.data(), sizeof(int4) * tab.size(), hipMemcpyHostToDevice, st)) != hipSuccess)
        return e;
    // the host staging arrays are released or reused after this call
    return hipStreamSynchronize(st);
}

// Builds the horizon representation of a prefix tree stored in depth-first
// preorder: for each segment its run [run_start, run_end), its parent and the
// end of its subtree; for each position its segment and subtree end.
extern "C" int cpattn_mask_tree(const int32_t* seg_id, int64_t n_tok, const int32_t* parent, int32_t n_seg,
                                void* stream, cpattn_mask** out) {
    const char* who = "cpattn_mask_tree";
    if (!out) return fail(CPATTN_EINVAL, "%s: out is NULL", who);
    *out = nullptr;
    std::vector<SegInfo> segs;
    std::vector<int32_t> order, stack;
    std::vector<int64_t> anc_len;
    int rc = cpattn_host::tree_host(seg_id, n_tok, parent, n_seg, who, fail, segs, order, stack, anc_len);
    if (rc != CPATTN_OK) return rc;

    cpattn_mask* m = new (std::nothrow) cpattn_mask();
    if (!m) return fail(CPATTN_ENOMEM, "%s: out of host memory", who);
    m->kind = kTree;
    m->n_pos = n_tok;
    m->segs = std::move(segs);
    m->run_order = std::move(order);
    m->anc_len = std::move(anc_len);
    std::vector<int32_t> end;
    std::vector<int4> tab;
    tree_arrays(seg_id, n_tok, m->segs, end, tab);

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    size_t nb = sizeof(int32_t) * (size_t)std::max<int64_t>(n_tok, 1);
    size_t tb = sizeof(int4) * (size_t)std::max<int32_t>(n_seg, 1);
    hipError_t e;
    if ((e = hipMalloc(&m->d_seg, nb)) != hipSuccess || (e = hipMalloc(&m->d_end, nb)) != hipSuccess ||
        (e = hipMalloc(&m->d_segtab, tb)) != hipSuccess) {
        cpattn_mask_free(m);
        return fail(CPATTN_ENOMEM, "%s: hipMalloc: %s", who, hipGetErrorString(e));
    }
    if ((e = tree_upload(m->d_seg, m->d_end, m->d_segtab, seg_id, n_tok, end, tab, st)) != hipSuccess) {
        cpattn_mask_free(m);
        return hip_fail(e, "cpattn_mask_tree: upload");
    }
    *out = m;
    return CPATTN_OK;
}

// ---------------------------------------------------------------------------
// tree descriptor without device allocation (cpattn_mask_tree_static)
// ---------------------------------------------------------------------------
// The device arrays live in `scratch`, a static buffer of the library: one
// copy per GPU, which keeps the last call's descriptor until the process
// ends.  Host code never uses the array's name as an address (in host code it
// is only a handle): the device address is taken once per device with
// hipGetSymbolAddress and kept in the device's slot.
constexpr int64_t kStaticMaxTok = CPATTN_STATIC_MAX_TOK;
constexpr int32_t kStaticMaxSeg = CPATTN_STATIC_MAX_SEG;
constexpr size_t kStaticEndOff = sizeof(int32_t) * (size_t)kStaticMaxTok;       // seg at 0, end after it
constexpr size_t kStaticTabOff = 2 * sizeof(int32_t) * (size_t)kStaticMaxTok;   // segment table (int4)
constexpr size_t kStaticBytes = kStaticTabOff + sizeof(int4) * (size_t)kStaticMaxSeg;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

struct StaticMaskSlot {
    bool ready = false;
    unsigned char* dev = nullptr;   // this device's copy of `scratch`
    cpattn_mask mask;               // host side of the descriptor, reused call after call
    std::vector<int32_t> stack, end;
    std::vector<int4> tab;
};
static StaticMaskSlot g_static_slots[kMaxDevices];
static std::mutex g_static_init;

// Device address of `scratch` and host capacity for the largest tree, once
// per device (the only allocations of this path, on its first call).
static int static_slot(StaticMaskSlot** out, const char* who) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "cpattn_mask_tree_static: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CPATTN_EUNSUPPORTED, "%s: device %d out of range", who, dev);
    StaticMaskSlot& sl = g_static_slots[dev];
    std::lock_guard<std::mutex> lock(g_static_init);
    if (!sl.ready) {
        void* ptr = nullptr;
        if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_fail(e, "cpattn_mask_tree_static: hipGetSymbolAddress");
        sl.dev = static_cast<unsigned char*>(ptr);
        sl.mask.segs.reserve(kStaticMaxSeg);
        sl.mask.run_order.reserve(kStaticMaxSeg);
        sl.mask.anc_len.reserve(kStaticMaxSeg);
        sl.stack.reserve(kStaticMaxSeg);
        sl.end.reserve((size_t)kStaticMaxTok);
        sl.tab.reserve(kStaticMaxSeg);
        sl.ready = true;
    }
    *out = &sl;
    return CPATTN_OK;
}

extern "C" int cpattn_mask_tree_static(const int32_t* seg_id, int64_t n_tok, const int32_t* parent, int32_t n_seg,
                                       void* stream, cpattn_mask** out) {
    const char* who = "cpattn_mask_tree_static";
    if (!out) return fail(CPATTN_EINVAL, "%s: out is NULL", who);
    *out = nullptr;
    if (n_tok > kStaticMaxTok || n_seg > kStaticMaxSeg)
        return fail(CPATTN_EUNSUPPORTED, "%s: %lld tokens / %d segments exceed the static descriptor's capacity "
                    "(%lld tokens, %d segments); use cpattn_mask_tree", who, (long long)n_tok, n_seg,
                    (long long)kStaticMaxTok, kStaticMaxSeg);
    StaticMaskSlot* sl = nullptr;
    int rc = static_slot(&sl, who);
    if (rc != CPATTN_OK) return rc;
    cpattn_mask& m = sl->mask;
    // the previous descriptor of this device is replaced (also on failure)
    {
        std::lock_guard<std::mutex> lock(m.pair_mu);
        m.pair_cache.clear();   // no allocation: the map keeps its buckets
    }
    m.kind = kTree;
    m.n_pos = 0;
    m.is_static = true;
    m.window = 0;
    m.d_lpos = nullptr;
    rc = cpattn_host::tree_host(seg_id, n_tok, parent, n_seg, who, fail, m.segs, m.run_order, sl->stack, m.anc_len);
    if (rc != CPATTN_OK) return rc;
    tree_arrays(seg_id, n_tok, m.segs, sl->end, sl->tab);
    m.d_seg = reinterpret_cast<int32_t*>(sl->dev);
    m.d_end = reinterpret_cast<int32_t*>(sl->dev + kStaticEndOff);
    m.d_segtab = reinterpret_cast<int4*>(sl->dev + kStaticTabOff);
    hipError_t e = tree_upload(m.d_seg, m.d_end, m.d_segtab, seg_id, n_tok, sl->end, sl->tab,
                               reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cpattn_mask_tree_static: upload");
    m.n_pos = n_tok;
    *out = &m;
    return CPATTN_OK;
}

// A descriptor with the same visibility as m plus a sliding window on logical
// (root-to-leaf) positions.  The new descriptor owns copies of m's device
// arrays and, for a tree, the logical position of every physical position.
extern "C" int cpattn_mask_with_window(const cpattn_mask* m, int64_t window, void* stream, cpattn_mask** out) {
    const char* who = "cpattn_mask_with_window";
    if (!out) return fail(CPATTN_EINVAL, "%s: out is NULL", who);
    *out = nullptr;
    if (!m) return fail(CPATTN_EINVAL, "%s: mask is NULL", who);
    if (window < 1 || window > (1 << 30)) return fail(CPATTN_EINVAL, "%s: window %lld out of range [1, 2^30]", who,
                                                        (long long)window);
    cpattn_mask* w = new (std::nothrow) cpattn_mask();
    if (!w) return fail(CPATTN_ENOMEM, "%s: out of host memory", who);
    w->kind = m->kind;
    w->n_pos = m->n_pos;
    w->segs = m->segs;
    w->run_order = m->run_order;
    w->anc_len = m->anc_len;
    w->window = (int32_t)window;
    if (m->kind == kTree) {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        const size_t nb = sizeof(int32_t) * (size_t)std::max<int64_t>(m->n_pos, 1);
        const size_t tb = sizeof(int4) * std::max<size_t>(m->segs.size(), 1);
        std::vector<int32_t> lpos;
        cpattn_host::tree_lpos(*m, lpos);
        hipError_t e;
        if ((e = hipMalloc(&w->d_seg, nb)) != hipSuccess || (e = hipMalloc(&w->d_end, nb)) != hipSuccess ||
            (e = hipMalloc(&w->d_segtab, tb)) != hipSuccess || (e = hipMalloc(&w->d_lpos, nb)) != hipSuccess) {
            cpattn_mask_free(w);
            return fail(CPATTN_ENOMEM, "%s: hipMalloc: %s", who, hipGetErrorString(e));
        }
        if ((e = hipMemcpyAsync(w->d_seg, m->d_seg, nb, hipMemcpyDeviceToDevice, st)) != hipSuccess ||
            (e = hipMemcpyAsync(w->d_end, m->d_end, nb, hipMemcpyDeviceToDevice, st)) != hipSuccess ||
            (e = hipMemcpyAsync(w->d_segtab, m->d_segtab, tb, hipMemcpyDeviceToDevice, st)) != hipSuccess ||
            (m->n_pos > 0 &&
             (e = hipMemcpyAsync(w->d_lpos, lpos.data(), sizeof(int32_t) * (size_t)m->n_pos, hipMemcpyHostToDevice,
                                 st)) != hipSuccess) ||
            (e = hipStreamSynchronize(st)) != hipSuccess) {
            cpattn_mask_free(w);
            return hip_fail(e, "cpattn_mask_with_window: upload");
        }
    }
    *out = w;
    return CPATTN_OK;
}

// ---------------------------------------------------------------------------
// argument checks
// ---------------------------------------------------------------------------
static int check_tensor(const cpattn_tensor* t, const char* who, const char* name) {
    if (!t) return fail(CPATTN_EINVAL, "%s: %s is NULL", who, name);
    if (t->dtype != CPATTN_BF16 && t->dtype != CPATTN_F32)
        return fail(CPATTN_EUNSUPPORTED, "%s: %s dtype %d unsupported (bf16 or f32)", who, name, t->dtype);
    if (t->d != 64 && t->d != 128)
        return fail(CPATTN_EUNSUPPORTED, "%s: %s head dim %lld unsupported (64 or 128)", who, name, (long long)t->d);
    if (t->n_heads < 1 || t->n_tok < 0 || t->n_tok > INT32_MAX)
        return fail(CPATTN_EINVAL, "%s: %s has bad sizes (heads %lld, tokens %lld)", who, name,
                    (long long)t->n_heads, (long long)t->n_tok);
    const int64_t al = t->dtype == CPATTN_BF16 ? 8 : 4;
    if (t->n_tok > 0 && !t->data) return fail(CPATTN_EINVAL, "%s: %s data is NULL", who, name);
    if ((reinterpret_cast<uintptr_t>(t->data) & 15) != 0)
        return fail(CPATTN_EUNSUPPORTED, "%s: %s data is not 16-byte aligned", who, name);
    if (t->stride_tok % al != 0 || t->stride_head % al != 0 || t->stride_tok < t->d || t->stride_head < 0)
        return fail(CPATTN_EUNSUPPORTED, "%s: %s strides (%lld, %lld) unsupported", who, name,
                    (long long)t->stride_head, (long long)t->stride_tok);
    // the kernels address one head's rows with 32-bit byte offsets
    const int64_t esize = t->dtype == CPATTN_BF16 ? 2 : 4;
    if (t->n_tok > 0 && ((t->n_tok - 1) * t->stride_tok + t->d) * esize > INT32_MAX)
        return fail(CPATTN_EUNSUPPORTED, "%s: %s spans more than 2 GiB per head", who, name);
    return CPATTN_OK;
}

static int check_posmap(cpattn_posmap p, int64_t n, const cpattn_mask* m, const char* who, const char* name) {
    if (p.stride < 1) return fail(CPATTN_EINVAL, "%s: %s stride %lld < 1", who, name, (long long)p.stride);
    if (n == 0) return CPATTN_OK;
    const int64_t last = p.base + p.stride * (n - 1);
    if (p.base < 0 || last >= m->n_pos || last < p.base)
        return fail(CPATTN_EINVAL, "%s: %s positions [%lld, %lld] outside the mask's [0, %lld)", who, name,
                    (long long)p.base, (long long)last, (long long)m->n_pos);
    return CPATTN_OK;
}


// pair_count over every row, and the sampled estimate, remembered per layout
static int64_t pair_exact(const cpattn_mask* m, cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk) {
    const PairKey key{{qp.base, qp.stride, nq, kp.base, kp.stride, nk}};
    {
        std::lock_guard<std::mutex> lock(m->pair_mu);
        auto it = m->pair_cache.find(key);
        if (it != m->pair_cache.end() && it->second.exact >= 0) return it->second.exact;
    }
    const int64_t c = cpattn_host::pair_count(*m, qp, nq, kp, nk, 1);
    std::lock_guard<std::mutex> lock(m->pair_mu);
    if (m->pair_cache.size() >= kPairCacheMax) m->pair_cache.clear();
    m->pair_cache[key].exact = c;
    return c;
}

// Does any query of the block see any key of the block?  Exact for both masks.
static bool pair_nonempty(const cpattn_mask* m, cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk) {
    if (nq == 0 || nk == 0) return false;
    if (m->window > 0) return pair_exact(m, qp, nq, kp, nk) > 0;   // exact, per query row
    return cpattn_host::pair_nonempty_nowin(*m, qp, nq, kp, nk);
}

// Approximate visible pairs from about 256 evenly spaced query rows; orders
// the jobs of a launch.
static double pair_estimate(const cpattn_mask* m, cpattn_posmap qp, int64_t nq, cpattn_posmap kp, int64_t nk) {
    const PairKey key{{qp.base, qp.stride, nq, kp.base, kp.stride, nk}};
    {
        std::lock_guard<std::mutex> lock(m->pair_mu);
        auto it = m->pair_cache.find(key);
        if (it != m->pair_cache.end() && it->second.estimate >= 0.0) return it->second.estimate;
    }
    const double e = (double)cpattn_host::pair_count(*m, qp, nq, kp, nk, std::max<int64_t>(1, nq / 256));
    std::lock_guard<std::mutex> lock(m->pair_mu);
    if (m->pair_cache.size() >= kPairCacheMax) m->pair_cache.clear();
    m->pair_cache[key].estimate = e;
    return e;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
// Raises a kernel's dynamic LDS limit to `bytes` once per device, before its
// first launch there.  `done` is the kernel's set of devices already raised
// (bit d: device d); host threads may race here, which is harmless: the call
// is idempotent, and a device is marked only after it succeeded.  Devices
// past 63 are raised on every launch.
static hipError_t raise_lds_limit(const void* kern, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

template <typename T, int D, int BN, bool WIN>
static int launch_partial_t(LaunchArgs& a, hipStream_t st) {
    using TL = Tile<T, D, BN>;
    const int smem = 2 * TL::STAGE_BYTES;
    const auto kern = partial_attention_kernel<T, D, BN, WIN>;
    static std::atomic<uint64_t> lds_raised{0};   // per instantiation: the attribute is per function
    if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), smem, lds_raised); e != hipSuccess)
        return hip_fail(e, "hipFuncSetAttribute");
    const int grid = (a.total_wg + 7) / 8 * 8;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), smem, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "partial attention launch");
    return CPATTN_OK;
}

// bf16 partial attention: key-tile width and prefetch distance of the
// ping-pong kernel (see attn_bf16_kernel.hpp)
constexpr int kBf16BN = 64;
constexpr int kBf16PF = 2;

template <int D, bool WIN>
static int launch_bf16(LaunchArgs& a, hipStream_t st) {
    using TT = PPTile<D, kBf16BN, kBf16PF>;
    const auto kern = attn_bf16_pp_kernel<D, kBf16BN, kBf16PF, WIN>;
    const int smem = WIN ? TT::LDS_BYTES_WIN : TT::LDS_BYTES;
    static std::atomic<uint64_t> lds_raised{0};
    if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), smem, lds_raised); e != hipSuccess)
        return hip_fail(e, "hipFuncSetAttribute");
    const int grid = (a.total_wg + 7) / 8 * 8;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kPPThreads), smem, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "partial attention launch");
    return CPATTN_OK;
}

// one instantiation per (dtype, head dim, window or not); the windowed ones
// differ only in the tile walk and the elementwise mask
static int launch_partial(LaunchArgs& a, int dtype, int d, hipStream_t st) {
    if (a.total_wg == 0) return CPATTN_OK;
    const bool win = a.mask.window > 0;
    if (dtype == CPATTN_BF16) {
        if (d == 128) return win ? launch_bf16<128, true>(a, st) : launch_bf16<128, false>(a, st);
        return win ? launch_bf16<64, true>(a, st) : launch_bf16<64, false>(a, st);
    }
    if (d == 128) return win ? launch_partial_t<float, 128, 32, true>(a, st) : launch_partial_t<float, 128, 32, false>(a, st);
    return win ? launch_partial_t<float, 64, 32, true>(a, st) : launch_partial_t<float, 64, 32, false>(a, st);
}

static MaskArgs mask_args(const cpattn_mask* m) {
    MaskArgs ma{};
    ma.kind = m->kind;
    ma.n_pos = (int32_t)m->n_pos;
    ma.seg = m->d_seg;
    ma.end = m->d_end;
    ma.segtab = m->d_segtab;
    ma.lpos = m->d_lpos;
    ma.window = m->window;
    return ma;
}

// query rows per workgroup of the kernel that serves a dtype
static int rows_per_wg(int dtype) { return dtype == CPATTN_BF16 ? kPPBM : kBM; }

static JobArgs make_job(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, cpattn_posmap qp,
                        cpattn_posmap kp, float* o, float* lse, int accumulate) {
    JobArgs j{};
    j.q = q->data;
    j.k = k->data;
    j.v = v->data;
    j.o = o;
    j.lse = lse;
    j.q_sh = q->stride_head;
    j.k_sh = k->stride_head;
    j.v_sh = v->stride_head;
    j.q_st = (int32_t)q->stride_tok;
    j.k_st = (int32_t)k->stride_tok;
    j.v_st = (int32_t)v->stride_tok;
    j.qbase = (int32_t)qp.base;
    j.qstride = (int32_t)qp.stride;
    j.kbase = (int32_t)kp.base;
    j.kstride = (int32_t)kp.stride;
    j.n_q = (int32_t)q->n_tok;
    j.n_k = (int32_t)k->n_tok;
    j.accumulate = accumulate;
    const int bm = rows_per_wg(q->dtype);
    j.q_tiles = (int32_t)((q->n_tok + bm - 1) / bm);
    j.kv_group = (int32_t)(q->n_heads / k->n_heads);
    return j;
}

// Packs jobs into launches of at most kMaxJobs each.
static int run_jobs(std::vector<JobArgs>& jobs, const cpattn_mask* m, int heads, float scale, int dtype, int d,
                    hipStream_t st) {
    const float scale_log2 = scale * 1.4426950408889634f;
    for (size_t first = 0; first < jobs.size(); first += kMaxJobs) {
        LaunchArgs a{};
        a.mask = mask_args(m);
        a.heads = heads;
        a.scale_log2 = scale_log2;
        int n = 0;
        int64_t sum_qt = 0;
        for (size_t i = first; i < jobs.size() && n < kMaxJobs; ++i, ++n) {
            a.jobs[n] = jobs[i];
            sum_qt += jobs[i].q_tiles;
        }
        // work slots: see work_item() in attn_kernel.hpp
        a.heads_per_xcd = heads >= 8 ? (heads + 7) / 8 : 0;
        const int64_t slots = a.heads_per_xcd > 0 ? 8 * (int64_t)a.heads_per_xcd * sum_qt : (int64_t)heads * sum_qt;
        if (slots > INT32_MAX / 2) return fail(CPATTN_EUNSUPPORTED, "too many workgroups in one launch");
        a.n_jobs = n;
        a.sum_q_tiles = (int32_t)sum_qt;
        a.total_wg = (int32_t)slots;
        int rc = launch_partial(a, dtype, d, st);
        if (rc != CPATTN_OK) return rc;
    }
    return CPATTN_OK;
}

static int launch_fill(float* o, float* lse, int64_t rows, int64_t d, hipStream_t st) {
    if (rows == 0) return CPATTN_OK;
    const int64_t n = rows * d;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, st, o, lse, rows, d);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "fill launch");
}

static int check_qkv(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, const char* who) {
    int rc;
    if ((rc = check_tensor(q, who, "q")) || (rc = check_tensor(k, who, "k")) || (rc = check_tensor(v, who, "v"))) return rc;
    if (q->dtype != k->dtype || q->dtype != v->dtype)
        return fail(CPATTN_EUNSUPPORTED, "%s: q, k and v must share one dtype", who);
    if (q->d != k->d || q->d != v->d) return fail(CPATTN_EUNSUPPORTED, "%s: q, k and v must share one head dim", who);
    // grouped-query attention: every K/V head serves the same number of query heads
    if (k->n_heads != v->n_heads || q->n_heads % k->n_heads != 0)
        return fail(CPATTN_EINVAL, "%s: head counts (q %lld, k %lld, v %lld): k and v must match and divide q", who,
                    (long long)q->n_heads, (long long)k->n_heads, (long long)v->n_heads);
    if (k->n_tok != v->n_tok) return fail(CPATTN_EINVAL, "%s: k and v token counts differ", who);
    return CPATTN_OK;
}

static int check_scale(float scale, const char* who) {
    if (!(scale > 0.f) || !std::isfinite(scale))
        return fail(CPATTN_EUNSUPPORTED, "%s: scale must be finite and > 0", who);
    return CPATTN_OK;
}

static int check_out(const float* o, const float* lse, const char* who) {
    if (!o || !lse) return fail(CPATTN_EINVAL, "%s: output pointer is NULL", who);
    if ((reinterpret_cast<uintptr_t>(o) & 15) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3) != 0)
        return fail(CPATTN_EUNSUPPORTED, "%s: o must be 16-byte aligned and lse 4-byte aligned", who);
    return CPATTN_OK;
}

extern "C" int cpattn_partial(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                              const cpattn_mask* mask, cpattn_posmap q_pos, cpattn_posmap k_pos, float scale,
                              float* o_out, float* lse_out, int accumulate, void* stream) {
    const char* who = "cpattn_partial";
    int rc;
    if ((rc = check_qkv(q, k, v, who))) return rc;
    if (!mask) return fail(CPATTN_EINVAL, "%s: mask is NULL", who);
    if ((rc = check_scale(scale, who))) return rc;
    if (accumulate != 0 && accumulate != 1) return fail(CPATTN_EINVAL, "%s: accumulate must be 0 or 1", who);
    if (q->n_tok == 0) return CPATTN_OK;
    if ((rc = check_out(o_out, lse_out, who))) return rc;
    if ((rc = check_posmap(q_pos, q->n_tok, mask, who, "q_pos")) || (rc = check_posmap(k_pos, k->n_tok, mask, who, "k_pos")))
        return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (k->n_tok == 0 || !pair_nonempty(mask, q_pos, q->n_tok, k_pos, k->n_tok)) {
        if (accumulate) return CPATTN_OK;   // merging an empty partial is the identity
        return launch_fill(o_out, lse_out, q->n_heads * q->n_tok, q->d, st);
    }
    std::vector<JobArgs> jobs{make_job(q, k, v, q_pos, k_pos, o_out, lse_out, accumulate)};
    return run_jobs(jobs, mask, (int)q->n_heads, scale, q->dtype, (int)q->d, st);
}

// Ranks that run: all of them (ranks == NULL, n_ranks_run == N) or a list
// without repeats.
static int ranks_to_run(int N, const int* ranks, int n_ranks_run, std::vector<int>* run, const char* who) {
    if (!ranks) {
        if (n_ranks_run != N) return fail(CPATTN_EINVAL, "%s: ranks is NULL but n_ranks_run != N", who);
        for (int r = 0; r < N; ++r) run->push_back(r);
        return CPATTN_OK;
    }
    if (n_ranks_run < 0 || n_ranks_run > N) return fail(CPATTN_EINVAL, "%s: n_ranks_run out of range", who);
    std::vector<char> seen(N, 0);
    for (int i = 0; i < n_ranks_run; ++i) {
        if (ranks[i] < 0 || ranks[i] >= N) return fail(CPATTN_EINVAL, "%s: rank %d out of range", who, ranks[i]);
        if (seen[ranks[i]]) return fail(CPATTN_EINVAL, "%s: rank %d listed twice", who, ranks[i]);
        seen[ranks[i]] = 1;
        run->push_back(ranks[i]);
    }
    return CPATTN_OK;
}

// Ring of N ranks that hold C chunks each (chunk i = r * C + c); see
// cpattn_ring_emulate_chunks in cpattn.h.
static int ring_core(int N, int C, const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                     const cpattn_posmap* pos, const int* ranks, int n_ranks_run, const cpattn_mask* mask,
                     float scale, float* const* o_out, float* const* lse_out, void* stream, const char* who) {
    int rc;
    if (N < 1 || N > 64) return fail(CPATTN_EINVAL, "%s: N = %d out of range [1, 64]", who, N);
    if (C < 1 || C > 8) return fail(CPATTN_EINVAL, "%s: chunks per rank = %d out of range [1, 8]", who, C);
    if (!q || !k || !v || !pos || !o_out || !lse_out) return fail(CPATTN_EINVAL, "%s: NULL array argument", who);
    if (!mask) return fail(CPATTN_EINVAL, "%s: mask is NULL", who);
    if ((rc = check_scale(scale, who))) return rc;
    std::vector<int> run;
    if ((rc = ranks_to_run(N, ranks, n_ranks_run, &run, who))) return rc;
    const int NC = N * C;
    // every chunk's K/V is visited; only the chunks of ranks that run need queries
    const cpattn_tensor& ref = k[0];
    for (int i = 0; i < NC; ++i) {
        if ((rc = check_qkv(&k[i], &k[i], &v[i], who))) return rc;
        if (k[i].dtype != ref.dtype || k[i].d != ref.d || k[i].n_heads != ref.n_heads)
            return fail(CPATTN_EUNSUPPORTED, "%s: every block must share dtype, head dim and heads", who);
        if ((rc = check_posmap(pos[i], k[i].n_tok, mask, who, "pos"))) return rc;
    }
    for (int r : run)
        for (int c = 0; c < C; ++c) {
            const int i = r * C + c;
            if ((rc = check_qkv(&q[i], &k[i], &v[i], who))) return rc;
            if (q[i].n_tok != k[i].n_tok)
                return fail(CPATTN_EINVAL, "%s: chunk %d holds %lld queries but %lld keys at the same positions", who, i,
                            (long long)q[i].n_tok, (long long)k[i].n_tok);
            if (q[i].n_tok > 0 && (rc = check_out(o_out[i], lse_out[i], who))) return rc;
        }

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (run.empty()) return CPATTN_OK;
    const int heads = (int)q[run[0] * C].n_heads;   // query heads (K/V may have fewer: grouped-query attention)
    for (int r : run)
        for (int c = 0; c < C; ++c)
            if (q[r * C + c].n_heads != heads)
                return fail(CPATTN_EINVAL, "%s: every query chunk must have the same head count", who);
    const int dtype = ref.dtype;
    const int d = (int)ref.d;
    // Each query chunk's visits in ring order: in round k the key chunks of
    // rank (r - k) mod N, in chunk order, without the empty ones.  Launch l
    // runs the l-th visit of every query chunk: the chunks' outputs are
    // independent, and each chunk's partials still merge in ring order, so
    // this is the ring's result with fewer, fuller launches.
    std::vector<int> units;
    std::vector<std::vector<int>> visits(NC);
    size_t n_launch = 0;
    for (int r : run)
        for (int c = 0; c < C; ++c) {
            const int i = r * C + c;
            units.push_back(i);
            for (int kk = 0; kk < N; ++kk) {
                const int b = ((r - kk) % N + N) % N;
                for (int c2 = 0; c2 < C; ++c2) {
                    const int j = b * C + c2;
                    if (pair_nonempty(mask, pos[i], q[i].n_tok, pos[j], k[j].n_tok)) visits[i].push_back(j);
                }
            }
            n_launch = std::max(n_launch, visits[i].size());
        }
    for (size_t l = 0; l < n_launch; ++l) {
        std::vector<JobArgs> jobs;
        std::vector<double> work;
        for (int i : units) {
            if (l >= visits[i].size()) continue;
            const int j = visits[i][l];
            jobs.push_back(make_job(&q[i], &k[j], &v[j], pos[i], pos[j], o_out[i], lse_out[i], l > 0 ? 1 : 0));
            work.push_back(pair_estimate(mask, pos[i], q[i].n_tok, pos[j], k[j].n_tok));
        }
        // heaviest job first: the launch's last workgroups are its lightest
        std::vector<size_t> idx(jobs.size());
        for (size_t x = 0; x < idx.size(); ++x) idx[x] = x;
        std::stable_sort(idx.begin(), idx.end(), [&](size_t x, size_t y) { return work[x] > work[y]; });
        std::vector<JobArgs> sorted;
        for (size_t x : idx) sorted.push_back(jobs[x]);
        if ((rc = run_jobs(sorted, mask, heads, scale, dtype, d, st))) return rc;
    }
    for (int i : units)
        if (visits[i].empty() && (rc = launch_fill(o_out[i], lse_out[i], heads * q[i].n_tok, d, st))) return rc;
    return CPATTN_OK;
}

extern "C" int cpattn_ring_emulate(int N, const cpattn_tensor* q_blocks, const cpattn_tensor* k_blocks,
                                   const cpattn_tensor* v_blocks, const cpattn_posmap* pos, const int* ranks,
                                   int n_ranks_run, const cpattn_mask* mask, float scale, float* const* o_out,
                                   float* const* lse_out, void* stream) {
    return ring_core(N, 1, q_blocks, k_blocks, v_blocks, pos, ranks, n_ranks_run, mask, scale, o_out, lse_out, stream,
                     "cpattn_ring_emulate");
}

extern "C" int cpattn_ring_emulate_chunks(int N, int C, const cpattn_tensor* q_chunks, const cpattn_tensor* k_chunks,
                                          const cpattn_tensor* v_chunks, const cpattn_posmap* pos, const int* ranks,
                                          int n_ranks_run, const cpattn_mask* mask, float scale,
                                          float* const* o_out, float* const* lse_out, void* stream) {
    return ring_core(N, C, q_chunks, k_chunks, v_chunks, pos, ranks, n_ranks_run, mask, scale, o_out, lse_out,
                     stream, "cpattn_ring_emulate_chunks");
}

extern "C" int cpattn_ring_plan(int N, int C, const int64_t* n_tok, const cpattn_posmap* pos,
                                const cpattn_mask* mask, int64_t* work) {
    const char* who = "cpattn_ring_plan";
    int rc;
    if (N < 1 || N > 64) return fail(CPATTN_EINVAL, "%s: N = %d out of range [1, 64]", who, N);
    if (C < 1 || C > 8) return fail(CPATTN_EINVAL, "%s: chunks per rank = %d out of range [1, 8]", who, C);
    if (!n_tok || !pos || !work) return fail(CPATTN_EINVAL, "%s: NULL array argument", who);
    if (!mask) return fail(CPATTN_EINVAL, "%s: mask is NULL", who);
    for (int i = 0; i < N * C; ++i) {
        if (n_tok[i] < 0 || n_tok[i] > INT32_MAX) return fail(CPATTN_EINVAL, "%s: chunk %d size out of range", who, i);
        if ((rc = check_posmap(pos[i], n_tok[i], mask, who, "pos"))) return rc;
    }
    for (int r = 0; r < N; ++r)
        for (int kk = 0; kk < N; ++kk) {
            const int b = ((r - kk) % N + N) % N;
            int64_t w = 0;
            for (int c = 0; c < C; ++c)
                for (int c2 = 0; c2 < C; ++c2)
                    w += pair_exact(mask, pos[r * C + c], n_tok[r * C + c], pos[b * C + c2], n_tok[b * C + c2]);
            work[r * N + kk] = w;
        }
    return CPATTN_OK;
}

extern "C" int cpattn_merge(int n_parts, const float* const* o_parts, const float* const* lse_parts, int64_t n_rows,
                            int64_t d, float* o_out, float* lse_out, void* stream) {
    const char* who = "cpattn_merge";
    if (n_parts < 1 || n_parts > kMaxMergeParts)
        return fail(CPATTN_EINVAL, "%s: n_parts = %d out of range [1, %d]", who, n_parts, kMaxMergeParts);
    if (n_rows < 0 || d < 1 || d > (1 << 20)) return fail(CPATTN_EINVAL, "%s: bad sizes", who);
    if (!o_parts || !lse_parts) return fail(CPATTN_EINVAL, "%s: NULL part arrays", who);
    if (n_rows == 0) return CPATTN_OK;
    if (!o_out || !lse_out) return fail(CPATTN_EINVAL, "%s: NULL output", who);
    MergeArgs a{};
    const bool vec = d % 4 == 0 && (reinterpret_cast<uintptr_t>(o_out) & 15) == 0;
    for (int p = 0; p < n_parts; ++p) {
        if (!o_parts[p] || !lse_parts[p]) return fail(CPATTN_EINVAL, "%s: part %d is NULL", who, p);
        a.o[p] = o_parts[p];
        a.l[p] = lse_parts[p];
    }
    bool all_aligned = vec;
    for (int p = 0; p < n_parts; ++p) all_aligned = all_aligned && (reinterpret_cast<uintptr_t>(o_parts[p]) & 15) == 0;
    const int unit = all_aligned ? 4 : 1;
    a.o_out = o_out;
    a.l_out = lse_out;
    a.rows = n_rows;
    a.n = n_parts;
    a.d = (int32_t)d;
    const int64_t units = d / unit;
    a.tpr = (int32_t)std::min<int64_t>(256, std::max<int64_t>(1, units));
    // round threads-per-row down to a divisor of 256 so rows never straddle workgroups
    while (256 % a.tpr) --a.tpr;
    const int64_t rows_per_block = 256 / a.tpr;
    const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many rows", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    using MergeFn = void (*)(MergeArgs);
    static const MergeFn vec4[9] = {merge_kernel<0, 4>, merge_kernel<1, 4>, merge_kernel<2, 4>,
                                    merge_kernel<3, 4>, merge_kernel<4, 4>, merge_kernel<5, 4>,
                                    merge_kernel<6, 4>, merge_kernel<7, 4>, merge_kernel<8, 4>};
    static const MergeFn vec1[9] = {merge_kernel<0, 1>, merge_kernel<1, 1>, merge_kernel<2, 1>,
                                    merge_kernel<3, 1>, merge_kernel<4, 1>, merge_kernel<5, 1>,
                                    merge_kernel<6, 1>, merge_kernel<7, 1>, merge_kernel<8, 1>};
    const int np = n_parts <= 8 ? n_parts : 0;
    hipLaunchKernelGGL(unit == 4 ? vec4[np] : vec1[np], dim3((unsigned)blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "merge launch");
}

extern "C" int cpattn_apply_sink(float* o, float* lse, const float* sink_logits, int64_t n_heads, int64_t n_rows,
                                 int64_t d, void* stream) {
    const char* who = "cpattn_apply_sink";
    if (n_heads < 1 || n_rows < 0 || d < 4 || d > (1 << 20)) return fail(CPATTN_EINVAL, "%s: bad sizes", who);
    if (d % 4 != 0) return fail(CPATTN_EUNSUPPORTED, "%s: d must be a multiple of 4", who);
    if (n_rows == 0) return CPATTN_OK;
    if (!o || !lse || !sink_logits) return fail(CPATTN_EINVAL, "%s: NULL pointer", who);
    if ((reinterpret_cast<uintptr_t>(o) & 15) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3) != 0 ||
        (reinterpret_cast<uintptr_t>(sink_logits) & 3) != 0)
        return fail(CPATTN_EUNSUPPORTED, "%s: o must be 16-byte aligned, lse and sink_logits 4-byte aligned", who);
    SinkArgs a{};
    a.o = o;
    a.lse = lse;
    a.sink = sink_logits;
    a.rows = n_heads * n_rows;
    a.rows_per_head = n_rows;
    a.d = (int32_t)d;
    a.tpr = (int32_t)std::min<int64_t>(256, d / 4);
    while (256 % a.tpr) --a.tpr;
    const int64_t rows_per_block = 256 / a.tpr;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many rows", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(sink_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "sink launch");
}

// threads per row for the row kernels of the merge and sink adjoints: a power
// of two <= 64, so that a row's lanes lie in one wave
static int32_t row_threads(int64_t d) {
    int32_t t = 1;
    while (t < 64 && 2 * t <= d / 4) t *= 2;
    return t;
}

extern "C" int cpattn_merge_backward(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                                     int64_t n_rows, int64_t d, const float* o, const float* lse, const float* g_o,
                                     const float* g_lse, float* const* g_o_parts, float* const* g_lse_parts,
                                     void* stream) {
    const char* who = "cpattn_merge_backward";
    if (n_parts < 1 || n_parts > kMaxMergeParts)
        return fail(CPATTN_EINVAL, "%s: n_parts = %d out of range [1, %d]", who, n_parts, kMaxMergeParts);
    if (n_rows < 0 || d < 4 || d > (1 << 20)) return fail(CPATTN_EINVAL, "%s: bad sizes", who);
    if (d % 4 != 0) return fail(CPATTN_EUNSUPPORTED, "%s: d must be a multiple of 4", who);
    if (!o_parts || !lse_parts || !g_o_parts || !g_lse_parts) return fail(CPATTN_EINVAL, "%s: NULL part arrays", who);
    if (n_rows == 0) return CPATTN_OK;
    if (!o || !lse || !g_o) return fail(CPATTN_EINVAL, "%s: NULL pointer", who);
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    MergeBwdArgs a{};
    bool aligned = al16(o) && al16(g_o);
    for (int p = 0; p < n_parts; ++p) {
        if (!o_parts[p] || !lse_parts[p] || !g_o_parts[p] || !g_lse_parts[p])
            return fail(CPATTN_EINVAL, "%s: part %d has a NULL pointer", who, p);
        aligned = aligned && al16(o_parts[p]) && al16(g_o_parts[p]);
        a.o[p] = o_parts[p];
        a.l[p] = lse_parts[p];
        a.go[p] = g_o_parts[p];
        a.gl[p] = g_lse_parts[p];
    }
    if (!aligned) return fail(CPATTN_EUNSUPPORTED, "%s: O arrays must be 16-byte aligned", who);
    a.o_m = o;
    a.l_m = lse;
    a.g = g_o;
    a.g_l = g_lse;
    a.rows = n_rows;
    a.n = n_parts;
    a.d = (int32_t)d;
    a.tpr = row_threads(d);
    const int64_t rows_per_block = 256 / a.tpr;
    const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many rows", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(merge_backward_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "merge backward launch");
}

extern "C" int cpattn_sink_backward(const float* o, const float* lse, const float* sink_logits, int64_t n_heads,
                                    int64_t n_rows, int64_t d, const float* g_o, float* g_o_in, float* g_lse_in,
                                    float* g_sink, void* stream) {
    const char* who = "cpattn_sink_backward";
    if (n_heads < 1 || n_rows < 0 || d < 4 || d > (1 << 20)) return fail(CPATTN_EINVAL, "%s: bad sizes", who);
    if (d % 4 != 0) return fail(CPATTN_EUNSUPPORTED, "%s: d must be a multiple of 4", who);
    if (n_heads > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many heads", who);
    if (!sink_logits || !g_sink) return fail(CPATTN_EINVAL, "%s: NULL pointer", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (n_rows > 0) {
        if (!o || !lse || !g_o || !g_o_in || !g_lse_in) return fail(CPATTN_EINVAL, "%s: NULL pointer", who);
        auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
        if (!al16(o) || !al16(g_o) || !al16(g_o_in))
            return fail(CPATTN_EUNSUPPORTED, "%s: O arrays must be 16-byte aligned", who);
        SinkBwdArgs a{};
        a.y = o;
        a.lse = lse;
        a.sink = sink_logits;
        a.g = g_o;
        a.go = g_o_in;
        a.gl = g_lse_in;
        a.rows = n_heads * n_rows;
        a.rows_per_head = n_rows;
        a.d = (int32_t)d;
        a.tpr = row_threads(d);
        const int64_t rows_per_block = 256 / a.tpr;
        const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
        if (blocks > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many rows", who);
        hipLaunchKernelGGL(sink_backward_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    }
    // with no rows the sink gradient is zero (the reduction over nothing)
    hipLaunchKernelGGL(sink_grad_kernel, dim3((unsigned)n_heads), dim3(256), 0, st, g_lse_in, n_rows, g_sink);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "sink backward launch");
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
template <typename T, int D, bool WIN>
static int launch_bwd_t(BwdArgs& a, bool dkv, hipStream_t st) {
    using S = BwdStage<T, D>;
    // bf16: tiles loaded straight into LDS, transposed operands read with
    // ds_read_b64_tr_b16; fp32: register-staged tiles
    void (*kq)(BwdArgs);
    void (*kkv)(BwdArgs);
    int smem_dq, smem_dkv;
    if constexpr (sizeof(T) == 2) {
        kq = attn_bwd_dq_bf16_kernel<D, WIN>;
        kkv = attn_bwd_dkv_bf16_kernel<D, WIN>;
        smem_dq = BwdDqBf16Smem<D, WIN ? 1 : kBwdDqKeyTile / kBwdTile>::BYTES;
        smem_dkv = BwdDkvBf16Smem<D>::BYTES;
    } else {
        kq = attn_bwd_dq_kernel<T, D, WIN>;
        kkv = attn_bwd_dkv_kernel<T, D, WIN>;
        smem_dq = (2 * S::ROW_ELEMS + S::T_ELEMS) * (int)sizeof(T) + 2 * kBwdTile * 4;
        smem_dkv = (2 * S::ROW_ELEMS + 2 * S::T_ELEMS) * (int)sizeof(T) + 3 * kBwdTile * 4;
    }
    static std::atomic<uint64_t> raised_dq{0}, raised_dkv{0};
    hipError_t ea = raise_lds_limit(reinterpret_cast<const void*>(kq), smem_dq, raised_dq);
    if (ea == hipSuccess) ea = raise_lds_limit(reinterpret_cast<const void*>(kkv), smem_dkv, raised_dkv);
    if (ea != hipSuccess) return hip_fail(ea, "hipFuncSetAttribute");
    if (a.total_wg == 0) return CPATTN_OK;
    if (dkv) hipLaunchKernelGGL(kkv, dim3(a.total_wg), dim3(kBwdThreads), smem_dkv, st, a);
    else hipLaunchKernelGGL(kq, dim3(a.total_wg), dim3(kBwdThreads), smem_dq, st, a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "backward launch");
}

template <bool WIN>
static int launch_bwd_w(BwdArgs& a, bool dkv, int dtype, int d, hipStream_t st) {
    if (dtype == CPATTN_BF16)
        return d == 128 ? launch_bwd_t<__bf16, 128, WIN>(a, dkv, st) : launch_bwd_t<__bf16, 64, WIN>(a, dkv, st);
    return d == 128 ? launch_bwd_t<float, 128, WIN>(a, dkv, st) : launch_bwd_t<float, 64, WIN>(a, dkv, st);
}

static int launch_bwd(BwdArgs& a, bool dkv, int dtype, int d, hipStream_t st) {
    return a.mask.window > 0 ? launch_bwd_w<true>(a, dkv, dtype, d, st) : launch_bwd_w<false>(a, dkv, dtype, d, st);
}

struct BwdPair {
    const cpattn_tensor *q, *k, *v, *dout;
    cpattn_posmap qp, kp;
    const float *lse, *delta;
    float *dq, *dk, *dv;
};

// One dQ launch and one dK/dV launch for a set of pairs (`which`: 1 = dQ
// only, 2 = dK/dV only, 3 = both); the pairs of one call must not share a
// query block (dQ) or a key block (dK/dV).
static int run_bwd(const std::vector<BwdPair>& pairs, const cpattn_mask* m, float scale, hipStream_t st,
                   int which = 3) {
    for (size_t first = 0; first < pairs.size(); first += kMaxJobs) {
        const size_t n = std::min<size_t>(kMaxJobs, pairs.size() - first);
        for (int dkv = 0; dkv < 2; ++dkv) {
            if (!(which & (1 << dkv))) continue;
            BwdArgs a{};
            a.mask = mask_args(m);
            a.scale = scale;
            a.scale_log2 = scale * 1.4426950408889634f;
            a.n_jobs = (int32_t)n;
            int64_t sum_tiles = 0;
            int dtype = 0, d = 0;
            for (size_t i = 0; i < n; ++i) {
                const BwdPair& P = pairs[first + i];
                BwdJob& j = a.jobs[i];
                j.q = P.q->data;
                j.k = P.k->data;
                j.v = P.v->data;
                j.dout = P.dout->data;
                j.lse = P.lse;
                j.delta = P.delta;
                j.dq = P.dq;
                j.dk = P.dk;
                j.dv = P.dv;
                j.q_sh = P.q->stride_head;
                j.k_sh = P.k->stride_head;
                j.v_sh = P.v->stride_head;
                j.do_sh = P.dout->stride_head;
                j.q_st = (int32_t)P.q->stride_tok;
                j.k_st = (int32_t)P.k->stride_tok;
                j.v_st = (int32_t)P.v->stride_tok;
                j.do_st = (int32_t)P.dout->stride_tok;
                j.qbase = (int32_t)P.qp.base;
                j.qstride = (int32_t)P.qp.stride;
                j.kbase = (int32_t)P.kp.base;
                j.kstride = (int32_t)P.kp.stride;
                j.n_q = (int32_t)P.q->n_tok;
                j.n_k = (int32_t)P.k->n_tok;
                j.kv_group = (int32_t)(P.q->n_heads / P.k->n_heads);
                const int64_t rows = dkv ? P.k->n_tok : P.q->n_tok;
                j.tiles = (int32_t)((rows + kBwdRows - 1) / kBwdRows);
                a.heads = (int32_t)(dkv ? P.k->n_heads : P.q->n_heads);
                sum_tiles += j.tiles;
                dtype = P.q->dtype;
                d = (int)P.q->d;
            }
            // (all pairs of a call have the same head counts: checked by the callers)
            a.heads_per_xcd = a.heads >= 8 ? (a.heads + 7) / 8 : 0;
            a.last_first = dkv ? 0 : 1;
            const int64_t wg = sum_tiles * (a.heads_per_xcd > 0 ? 8 * (int64_t)a.heads_per_xcd : (int64_t)a.heads);
            if (wg > INT32_MAX / 2) return fail(CPATTN_EUNSUPPORTED, "too many workgroups in one launch");
            a.total_wg = (int32_t)wg;
            int rc = launch_bwd(a, dkv == 1, dtype, d, st);
            if (rc != CPATTN_OK) return rc;
        }
    }
    return CPATTN_OK;
}

static int check_bwd_common(const cpattn_tensor* q, const cpattn_tensor* dout, const cpattn_mask* mask,
                            const float* lse, const float* delta, const char* who) {
    int rc;
    if (!mask) return fail(CPATTN_EINVAL, "%s: mask is NULL", who);
    if ((rc = check_tensor(dout, who, "dout"))) return rc;
    if (dout->dtype != q->dtype || dout->d != q->d || dout->n_heads != q->n_heads || dout->n_tok != q->n_tok)
        return fail(CPATTN_EINVAL, "%s: dout must match q in dtype, heads, tokens and head dim", who);
    if (q->n_tok > 0 && (!lse || !delta)) return fail(CPATTN_EINVAL, "%s: lse or delta is NULL", who);
    return CPATTN_OK;
}

extern "C" int cpattn_stream_probe(int kind, const void* src, void* dst, int64_t bytes, int grid, void* stream) {
    const char* who = "cpattn_stream_probe";
    if (kind != 0 && kind != 1) return fail(CPATTN_EINVAL, "%s: kind must be 0 (read) or 1 (copy)", who);
    if (bytes < 0 || bytes % 16 != 0) return fail(CPATTN_EINVAL, "%s: bytes must be a non-negative multiple of 16", who);
    if (grid > (1 << 20)) return fail(CPATTN_EINVAL, "%s: grid above 2^20 workgroups", who);
    if (bytes == 0) return CPATTN_OK;
    if (!src || !dst) return fail(CPATTN_EINVAL, "%s: NULL pointer", who);
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
        return fail(CPATTN_EUNSUPPORTED, "%s: src and dst must be 16-byte aligned", who);
    const int64_t units = bytes / 16;
    const int64_t full = (units + 255) / 256;
    const int64_t blocks = grid > 0 ? std::min<int64_t>(grid, full) : full;
    if (blocks > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many bytes", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const float4* s4 = reinterpret_cast<const float4*>(src);
    float4* d4 = reinterpret_cast<float4*>(dst);
    if (kind == 0)
        hipLaunchKernelGGL(stream_probe_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, units);
    else
        hipLaunchKernelGGL(stream_probe_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, units);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "stream probe launch");
}

extern "C" int cpattn_backward_delta(const float* o, const cpattn_tensor* dout, float* delta, void* stream) {
    const char* who = "cpattn_backward_delta";
    int rc;
    if ((rc = check_tensor(dout, who, "dout"))) return rc;
    if (dout->n_tok == 0) return CPATTN_OK;
    if (!o || !delta) return fail(CPATTN_EINVAL, "%s: NULL pointer", who);
    if ((reinterpret_cast<uintptr_t>(o) & 15) != 0 || (reinterpret_cast<uintptr_t>(delta) & 3) != 0)
        return fail(CPATTN_EUNSUPPORTED, "%s: o must be 16-byte aligned and delta 4-byte aligned", who);
    const int64_t rows = dout->n_heads * dout->n_tok;
    const int64_t rows_per_block = 256 / (dout->d / 4);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > INT32_MAX) return fail(CPATTN_EUNSUPPORTED, "%s: too many rows", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dout->dtype == CPATTN_BF16)
        hipLaunchKernelGGL(bwd_delta_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st, o,
                           reinterpret_cast<const __bf16*>(dout->data), dout->stride_head, (int32_t)dout->stride_tok,
                           delta, rows, (int32_t)dout->n_tok, (int32_t)dout->d);
    else
        hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, o,
                           reinterpret_cast<const float*>(dout->data), dout->stride_head, (int32_t)dout->stride_tok,
                           delta, rows, (int32_t)dout->n_tok, (int32_t)dout->d);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CPATTN_OK : hip_fail(e, "delta launch");
}

extern "C" int cpattn_partial_backward(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                       const cpattn_mask* mask, cpattn_posmap q_pos, cpattn_posmap k_pos, float scale,
                                       const float* lse, const float* delta, const cpattn_tensor* dout, float* dq,
                                       float* dk, float* dv, void* stream) {
    const char* who = "cpattn_partial_backward";
    int rc;
    if ((rc = check_qkv(q, k, v, who))) return rc;
    if ((rc = check_scale(scale, who))) return rc;
    if ((rc = check_bwd_common(q, dout, mask, lse, delta, who))) return rc;
    if (q->n_tok == 0 || k->n_tok == 0) return CPATTN_OK;
    if ((rc = check_out(dq, lse, who)) || (rc = check_out(dk, delta, who)) || (rc = check_out(dv, delta, who))) return rc;
    if ((rc = check_posmap(q_pos, q->n_tok, mask, who, "q_pos")) || (rc = check_posmap(k_pos, k->n_tok, mask, who, "k_pos")))
        return rc;
    if (!pair_nonempty(mask, q_pos, q->n_tok, k_pos, k->n_tok)) return CPATTN_OK;
    std::vector<BwdPair> pairs{BwdPair{q, k, v, dout, q_pos, k_pos, lse, delta, dq, dk, dv}};
    return run_bwd(pairs, mask, scale, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int cpattn_ring_backward_chunks(int N, int C, const cpattn_tensor* q_chunks,
                                           const cpattn_tensor* k_chunks, const cpattn_tensor* v_chunks,
                                           const cpattn_posmap* pos, const cpattn_mask* mask, float scale,
                                           const float* const* lse, const float* const* delta,
                                           const cpattn_tensor* dout_chunks, float* const* dq, float* const* dk,
                                           float* const* dv, void* stream) {
    const char* who = "cpattn_ring_backward_chunks";
    int rc;
    if (N < 1 || N > 64) return fail(CPATTN_EINVAL, "%s: N = %d out of range [1, 64]", who, N);
    if (C < 1 || C > 8) return fail(CPATTN_EINVAL, "%s: C = %d out of range [1, 8]", who, C);
    if (!q_chunks || !k_chunks || !v_chunks || !pos || !lse || !delta || !dout_chunks || !dq || !dk || !dv)
        return fail(CPATTN_EINVAL, "%s: NULL array argument", who);
    if ((rc = check_scale(scale, who))) return rc;
    const int NC = N * C;
    for (int i = 0; i < NC; ++i) {
        if ((rc = check_qkv(&q_chunks[i], &k_chunks[i], &v_chunks[i], who))) return rc;
        if ((rc = check_bwd_common(&q_chunks[i], &dout_chunks[i], mask, lse[i], delta[i], who))) return rc;
        if (q_chunks[i].n_tok != k_chunks[i].n_tok)
            return fail(CPATTN_EINVAL, "%s: chunk %d holds %lld queries but %lld keys", who, i,
                        (long long)q_chunks[i].n_tok, (long long)k_chunks[i].n_tok);
        if (q_chunks[i].dtype != q_chunks[0].dtype || q_chunks[i].d != q_chunks[0].d ||
            q_chunks[i].n_heads != q_chunks[0].n_heads || k_chunks[i].n_heads != k_chunks[0].n_heads)
            return fail(CPATTN_EUNSUPPORTED, "%s: every chunk must share dtype, head dim and heads", who);
        if ((rc = check_posmap(pos[i], k_chunks[i].n_tok, mask, who, "pos"))) return rc;
        if (q_chunks[i].n_tok > 0 &&
            ((rc = check_out(dq[i], lse[i], who)) || (rc = check_out(dk[i], delta[i], who)) ||
             (rc = check_out(dv[i], delta[i], who))))
            return rc;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    auto pair = [&](int qi, int ki) {
        return BwdPair{&q_chunks[qi], &k_chunks[ki], &v_chunks[ki], &dout_chunks[qi], pos[qi], pos[ki], lse[qi],
                       delta[qi], dq[qi], dk[ki], dv[ki]};
    };
    // Round k: every chunk a of rank r meets every key chunk c of rank
    // b = (r - k) mod N.  A launch may hold one pair per query chunk (dQ)
    // and, separately, one per key chunk (dK/dV): the dQ launches of a round
    // take one key chunk index c at a time (query chunks (r, a) all differ),
    // the dK/dV launches one query chunk index a (key chunks (b, c) all differ).
    for (int k = 0; k < N; ++k) {
        for (int c = 0; c < C; ++c) {
            std::vector<BwdPair> pairs;
            for (int r = 0; r < N; ++r) {
                const int b = ((r - k) % N + N) % N;
                for (int a = 0; a < C; ++a) {
                    const int qi = r * C + a, ki = b * C + c;
                    if (pair_nonempty(mask, pos[qi], q_chunks[qi].n_tok, pos[ki], k_chunks[ki].n_tok))
                        pairs.push_back(pair(qi, ki));
                }
            }
            if ((rc = run_bwd(pairs, mask, scale, st, 1))) return rc;
        }
        for (int a = 0; a < C; ++a) {
            std::vector<BwdPair> pairs;
            for (int r = 0; r < N; ++r) {
                const int b = ((r - k) % N + N) % N;
                for (int c = 0; c < C; ++c) {
                    const int qi = r * C + a, ki = b * C + c;
                    if (pair_nonempty(mask, pos[qi], q_chunks[qi].n_tok, pos[ki], k_chunks[ki].n_tok))
                        pairs.push_back(pair(qi, ki));
                }
            }
            if ((rc = run_bwd(pairs, mask, scale, st, 2))) return rc;
        }
    }
    return CPATTN_OK;
}

extern "C" int cpattn_ring_backward(int N, const cpattn_tensor* q_blocks, const cpattn_tensor* k_blocks,
                                    const cpattn_tensor* v_blocks, const cpattn_posmap* pos, const cpattn_mask* mask,
                                    float scale, const float* const* lse, const float* const* delta,
                                    const cpattn_tensor* dout_blocks, float* const* dq, float* const* dk,
                                    float* const* dv, void* stream) {
    const char* who = "cpattn_ring_backward";
    int rc;
    if (N < 1 || N > 64) return fail(CPATTN_EINVAL, "%s: N = %d out of range [1, 64]", who, N);
    if (!q_blocks || !k_blocks || !v_blocks || !pos || !lse || !delta || !dout_blocks || !dq || !dk || !dv)
        return fail(CPATTN_EINVAL, "%s: NULL array argument", who);
    if ((rc = check_scale(scale, who))) return rc;
    for (int r = 0; r < N; ++r) {
        if ((rc = check_qkv(&q_blocks[r], &k_blocks[r], &v_blocks[r], who))) return rc;
        if ((rc = check_bwd_common(&q_blocks[r], &dout_blocks[r], mask, lse[r], delta[r], who))) return rc;
        if (q_blocks[r].n_tok != k_blocks[r].n_tok)
            return fail(CPATTN_EINVAL, "%s: rank %d holds %lld queries but %lld keys", who, r,
                        (long long)q_blocks[r].n_tok, (long long)k_blocks[r].n_tok);
        if (q_blocks[r].dtype != q_blocks[0].dtype || q_blocks[r].d != q_blocks[0].d ||
            q_blocks[r].n_heads != q_blocks[0].n_heads || k_blocks[r].n_heads != k_blocks[0].n_heads)
            return fail(CPATTN_EUNSUPPORTED, "%s: every block must share dtype, head dim and heads", who);
        if ((rc = check_posmap(pos[r], k_blocks[r].n_tok, mask, who, "pos"))) return rc;
        if (q_blocks[r].n_tok > 0 &&
            ((rc = check_out(dq[r], lse[r], who)) || (rc = check_out(dk[r], delta[r], who)) ||
             (rc = check_out(dv[r], delta[r], who))))
            return rc;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // Round k: rank r's queries against the keys of rank (r - k) mod N.  Each
    // round is a permutation of the blocks, so its pairs share neither a
    // query block (dQ) nor a key block (dK, dV: the contributions that would
    // travel back to the key's owner are added in place).
    for (int k = 0; k < N; ++k) {
        std::vector<BwdPair> pairs;
        for (int r = 0; r < N; ++r) {
            const int b = ((r - k) % N + N) % N;
            if (!pair_nonempty(mask, pos[r], q_blocks[r].n_tok, pos[b], k_blocks[b].n_tok)) continue;
            pairs.push_back(BwdPair{&q_blocks[r], &k_blocks[b], &v_blocks[b], &dout_blocks[r], pos[r], pos[b], lse[r],
                                    delta[r], dq[r], dk[b], dv[b]});
        }
        if ((rc = run_bwd(pairs, mask, scale, st))) return rc;
    }
    return CPATTN_OK;
}
