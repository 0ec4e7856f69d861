// C ABI of libbh.so: context, argument checks, launch sequencing, status.
//
// bh_build runs the steps of [Tree] 实现步骤 in order on one stream with no
// host synchronisation: bounding box -> Morton keys -> stable sort (with the
// sorted copy of the sources gathered in its last pass) -> octree -> centre
// of mass.  bh_gravity runs the walk.  Every scalar one step hands to the next
// (the root cube, node counts, the status word) stays in device memory.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <type_traits>

#include "bh_internal.h"

using namespace bh;

struct bh_ctx {
    int device = 0;
    int64_t max_src = 0, max_tgt = 0;
    int key_bits = 63, bits = 21, leaf_cap = 16, curve = 0;
    uint64_t node_cap = 0;

    DevParams *prm = nullptr;
    DevParams *host_prm = nullptr;   // pinned, for synchronous read-back
    float *bbox_part = nullptr;
    uint64_t *keys = nullptr, *keys_alt = nullptr;
    uint32_t *vals = nullptr, *vals_alt = nullptr;
    uint16_t *hlut = nullptr;         // Hilbert key tables (kHilbertLutEntries)
    uint32_t *spine = nullptr;
    float4 *spos = nullptr;
    uint64_t *keys_sorted = nullptr;  // aliases keys or keys_alt after a build
    uint32_t *perm = nullptr;         // aliases vals or vals_alt after a build
    uint32_t *inv = nullptr;          // Morton rank of each caller index (unsorted walks)
    double *diag = nullptr;           // partial sums of bh_diagnostics
    unsigned long long *icount = nullptr;   // interactions of the last counted walk
    bool counting = false;            // bh_set_counting: walks count into icount
    bool last_counted = false;        // the last walk counted into icount

    // lock-based dense build (allocated on first use)
    int32_t *lk_child = nullptr, *lk_level = nullptr, *lk_next = nullptr, *lk_counter = nullptr;
    int32_t lk_cap = 0;
    uint32_t lk_n = 0;
    BuildScratch bw = {};
    Node *nodes = nullptr;
    Node *wnodes = nullptr;           // per-call walk records (see launch_walk)
    uint32_t wn_cap = 0;              // records wnodes holds
    uint32_t *wbal = nullptr;         // the walk's XCD runs and per-group times
    int *bal_want = nullptr;          // pinned, written by the device: the last walk's
    int *bal_want_dev = nullptr;      //   times call for uneven XCD runs (its device address)
    uint32_t *clustered = nullptr;    // the word after it: a sort found long runs of equal
    uint32_t *clustered_dev = nullptr; //   top key bits clustered in tiles (sticky)
    uint32_t hist_groups = 0;         // groups wbal holds times for (0: none)
    int hist_kind = -1;               // 0: self-gravity, 1: separate targets
    bool hist_new = false;            // those times are not yet looked at
    uint32_t runs_groups = 0;         // groups wbal holds runs for
    int runs_kind = -1;
    uint32_t walk_calls = 0;          // per-target walks so far (times kept every 4th)
    int last_runs = -1;               // the last per-target walk used uneven runs (-1: none yet)
    int last_split = 0;               // ... and split its heaviest groups

    uint64_t *tkeys = nullptr, *tkeys_alt = nullptr;
    uint32_t *tvals = nullptr, *tvals_alt = nullptr;
    uint32_t *tspine = nullptr;
    float4 *tpos = nullptr;

    uint32_t n_src = 0;
    bool built = false;
    hipStream_t last_stream = nullptr;

    bool prof = false;
    hipEvent_t ev[8] = {};
};

namespace {

// particle and target counts must fit 31 bits
constexpr int64_t kMaxCount = ((int64_t)1 << 31) - 1;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <typename T>
hipError_t dalloc(T **p, size_t count)
{
    if (count == 0) count = 1;
    return hipMalloc((void **)p, count * sizeof(T));
}

void free_all(bh_ctx *c)
{
    void *ptrs[] = {c->prm, c->hlut, c->bbox_part, c->keys, c->keys_alt, c->vals, c->vals_alt, c->spine,
                    c->spos, c->bw.dc, c->bw.tile_counts, c->bw.tile_sums, c->bw.chunk_tot, c->bw.tile_scan,
                    c->bw.first_node, c->bw.P, c->nodes, c->wnodes, c->wbal,
                    c->tkeys, c->tkeys_alt, c->tvals,
                    c->tvals_alt, c->tspine, c->tpos, c->inv, c->diag, c->icount, c->lk_child,
                    c->lk_level, c->lk_next, c->lk_counter};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
    if (c->host_prm) (void)hipHostFree(c->host_prm);
    if (c->bal_want) (void)hipHostFree(c->bal_want);
    for (hipEvent_t &e : c->ev)
        if (e) (void)hipEventDestroy(e);
}

void record(bh_ctx *c, int k, hipStream_t s)
{
    if (c->prof) (void)hipEventRecord(c->ev[k], s);
}

bh_status launch_status()
{
    return hipGetLastError() == hipSuccess ? BH_OK : BH_ERR_HIP;
}

// Nodes a tree over n sources can need: at each of the levels 0 .. bits-1 the
// cells holding more than B sources are disjoint, so at most n / (B + 1) of
// them are split (internal), and leaves are disjoint non-empty cells, at most
// n; plus the end record.
uint64_t node_bound(uint64_t n, int bits, int leaf_cap)
{
    return (uint64_t)bits * (n / (uint64_t)(leaf_cap + 1)) + n + 1;
}

// Walk records a context keeps: one per node of the largest tree it can
// build, the end record included, up to the assembly loop's limit.
uint32_t walk_records(uint64_t max_src, int bits, int leaf_cap, uint64_t node_cap)
{
    uint64_t k = node_bound(max_src, bits, leaf_cap);
    k = k < node_cap + 1 ? k : node_cap + 1;
    return (uint32_t)(k < (uint64_t)kAsmMaxNodes ? k : (uint64_t)kAsmMaxNodes);
}

}  // namespace

// ---- the allocation-free step -------------------------------------------
//
// bh_gravity_static runs bh_build + bh_gravity (self-gravity) on a context
// whose buffers are carved out of one static device array, so the call never
// allocates.  The array's host-side name is not a device address: the
// device's copy is located once per device with hipGetSymbolAddress and only
// that address is used.  Every buffer the kernels read is written by an
// earlier kernel of the same call (the bounding-box kernel resets the status
// word), so nothing needs clearing between calls; calls that overlap on one
// device race for the array.

namespace {

constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
constexpr int kStaticMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct StaticDevice {
    unsigned char *base = nullptr;   // this device's copy of `scratch`
    bool ready = false;
};
StaticDevice g_static[kStaticMaxDevices];
std::mutex g_static_mu;


// Lays the buffers of a static context for n sources out from `base` (256-byte
// aligned pieces); returns the bytes used.  base == nullptr only measures.
size_t static_layout(bh_ctx *c, unsigned char *base, uint32_t n)
{
    size_t off = 0;
    auto take = [&](auto **p, size_t count) {
        using T = typename std::remove_pointer<typename std::remove_pointer<decltype(p)>::type>::type;
        if (count == 0) count = 1;
        if (base) *p = reinterpret_cast<T *>(base + off);
        off += ((count * sizeof(T) + 255) / 256) * 256;
    };
    const size_t ns = n, tiles = build_blocks(n);
    take(&c->prm, 1);
    take(&c->hlut, (size_t)kHilbertLutEntries);
    take(&c->bbox_part, 8 * 1024);
    take(&c->keys, ns);
    take(&c->keys_alt, ns);
    take(&c->vals, ns);
    take(&c->vals_alt, ns);
    take(&c->spine, sort_spine_entries(n));
    take(&c->spos, ns + kSourcePad);
    take(&c->bw.dc, ns);
    take(&c->bw.tile_counts, tiles);
    take(&c->bw.tile_sums, tiles);
    take(&c->bw.chunk_tot, tiles + 1);
    take(&c->bw.tile_scan, tiles + 1);
    take(&c->bw.first_node, ns + 1);
    take(&c->bw.P, ns + 1);
    take(&c->nodes, (size_t)c->node_cap + 1);
    c->wn_cap = walk_records(n, c->bits, c->leaf_cap, c->node_cap);
    take(&c->wnodes, (size_t)c->wn_cap);
    return off;
}

// The device's copy of `scratch`, located (and the Hilbert key tables copied
// into it) on the first call on that device.
bh_status static_base(int dev, unsigned char **out)
{
    if (dev < 0 || dev >= kStaticMaxDevices) return BH_ERR_INVALID;
    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticDevice &d = g_static[dev];
    if (!d.ready) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BH_ERR_HIP;
        bh_ctx probe;
        static_layout(&probe, (unsigned char *)p, 0);
        uint16_t host_lut[kHilbertLutEntries];
        if (!hilbert_lut_host(host_lut)) return BH_ERR_HIP;
        if (hipMemcpy(probe.hlut, host_lut, sizeof(host_lut), hipMemcpyHostToDevice) !=
            hipSuccess)
            return BH_ERR_HIP;
        d.base = (unsigned char *)p;
        d.ready = true;
    }
    *out = d.base;
    return BH_OK;
}

}  // namespace

extern "C" {

const char *bh_status_string(int status)
{
    switch (status) {
    case BH_OK: return "ok";
    case BH_ERR_INVALID: return "invalid argument";
    case BH_ERR_OOM: return "device allocation failed";
    case BH_ERR_HIP: return "HIP runtime error";
    case BH_ERR_CAPACITY: return "tree node capacity exceeded";
    case BH_ERR_NONFINITE: return "non-finite source coordinate or mass";
    case BH_ERR_NOT_BUILT: return "no successful build";
    case BH_ERR_CONTENTION: return "lock-based build: an insertion ran out of retries";
    default: return "unknown status";
    }
}

bh_status bh_create(bh_ctx **out, int64_t max_sources, int64_t max_targets,
                    const bh_build_params *params)
{
    if (!out) return BH_ERR_INVALID;
    *out = nullptr;
    if (max_sources < 0 || max_targets < 0 || max_sources > kMaxCount || max_targets > kMaxCount)
        return BH_ERR_INVALID;
    bh_build_params p = {63, 16, 0, 0, 0};
    if (params) p = *params;
    if ((p.key_bits != 63 && p.key_bits != 30) || p.leaf_cap < 1 || p.leaf_cap > kMaxLeafCap ||
        p.node_capacity < 0 || (p.key_curve != BH_CURVE_MORTON && p.key_curve != BH_CURVE_HILBERT) ||
        p.reserved != 0)
        return BH_ERR_INVALID;

    bh_ctx *c = new (std::nothrow) bh_ctx();
    if (!c) return BH_ERR_OOM;
    if (hipGetDevice(&c->device) != hipSuccess) {
        delete c;
        return BH_ERR_HIP;
    }
    c->max_src = max_sources;
    c->max_tgt = max_targets;
    c->key_bits = p.key_bits;
    c->bits = p.key_bits / 3;
    c->leaf_cap = p.leaf_cap;
    c->curve = p.key_curve;
    c->node_cap = p.node_capacity ? (uint64_t)p.node_capacity
                                  : node_bound((uint64_t)max_sources, c->bits, c->leaf_cap);
    if (c->node_cap > 0xfffffff0ull) c->node_cap = 0xfffffff0ull;

    const size_t ns = (size_t)max_sources, nt = (size_t)max_targets;
    const size_t tiles = build_blocks((uint32_t)ns);
    bool ok = true;
    ok &= dalloc(&c->prm, 1) == hipSuccess;
    {
        uint16_t host_lut[kHilbertLutEntries];
        ok &= hilbert_lut_host(host_lut);
        ok &= dalloc(&c->hlut, (size_t)kHilbertLutEntries) == hipSuccess;
        if (ok)
            ok &= hipMemcpy(c->hlut, host_lut, sizeof(host_lut), hipMemcpyHostToDevice) ==
                  hipSuccess;
    }
    ok &= hipHostMalloc((void **)&c->host_prm, sizeof(DevParams), hipHostMallocDefault) == hipSuccess;
    if (hipHostMalloc((void **)&c->bal_want, 2 * sizeof(int), hipHostMallocMapped) ==
        hipSuccess) {
        c->bal_want[0] = c->bal_want[1] = 0;
        ok &= hipHostGetDevicePointer((void **)&c->bal_want_dev, c->bal_want, 0) == hipSuccess;
        c->clustered = reinterpret_cast<uint32_t *>(c->bal_want + 1);
        c->clustered_dev = reinterpret_cast<uint32_t *>(c->bal_want_dev + 1);
    } else {
        c->bal_want = nullptr;
        ok = false;
    }
    ok &= dalloc(&c->bbox_part, 8 * 1024) == hipSuccess;
    ok &= dalloc(&c->keys, ns) == hipSuccess;
    ok &= dalloc(&c->keys_alt, ns) == hipSuccess;
    ok &= dalloc(&c->vals, ns) == hipSuccess;
    ok &= dalloc(&c->vals_alt, ns) == hipSuccess;
    ok &= dalloc(&c->spine, sort_spine_entries((uint32_t)ns)) == hipSuccess;
    // the walk reads up to 7 sources past a leaf and one node record past the last
    ok &= dalloc(&c->spos, ns + kSourcePad) == hipSuccess;
    ok &= dalloc(&c->bw.dc, ns) == hipSuccess;
    ok &= dalloc(&c->bw.tile_counts, tiles) == hipSuccess;
    ok &= dalloc(&c->bw.tile_sums, tiles) == hipSuccess;
    ok &= dalloc(&c->bw.chunk_tot, tiles + 1) == hipSuccess;
    ok &= dalloc(&c->bw.tile_scan, tiles + 1) == hipSuccess;
    ok &= dalloc(&c->bw.first_node, ns + 1) == hipSuccess;
    ok &= dalloc(&c->bw.P, ns + 1) == hipSuccess;
    ok &= dalloc(&c->nodes, (size_t)c->node_cap + 1) == hipSuccess;
    c->wn_cap = walk_records((uint64_t)ns, c->bits, c->leaf_cap, c->node_cap);
    ok &= dalloc(&c->wnodes, (size_t)c->wn_cap) == hipSuccess;
    ok &= dalloc(&c->wbal,
                 (size_t)kWalkBalanceHead + 3 * (size_t)walk_groups((uint32_t)(ns > nt ? ns : nt))) ==
          hipSuccess;
    ok &= dalloc(&c->inv, ns) == hipSuccess;
    ok &= dalloc(&c->diag, (size_t)kDiagMaxPartials * kDiagTerms) == hipSuccess;
    ok &= dalloc(&c->icount, 1) == hipSuccess;
    if (nt) {
        ok &= dalloc(&c->tkeys, nt) == hipSuccess;
        ok &= dalloc(&c->tkeys_alt, nt) == hipSuccess;
        ok &= dalloc(&c->tvals, nt) == hipSuccess;
        ok &= dalloc(&c->tvals_alt, nt) == hipSuccess;
        ok &= dalloc(&c->tspine, sort_spine_entries((uint32_t)nt)) == hipSuccess;
        ok &= dalloc(&c->tpos, nt) == hipSuccess;
    }
    for (hipEvent_t &e : c->ev) ok &= hipEventCreate(&e) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        free_all(c);
        delete c;
        return BH_ERR_OOM;
    }
    *out = c;
    return BH_OK;
}

bh_status bh_destroy(bh_ctx *c)
{
    if (!c) return BH_OK;
    (void)hipDeviceSynchronize();
    free_all(c);
    delete c;
    return BH_OK;
}

bh_status bh_build(bh_ctx *c, const float *src_pos_mass, int64_t n, void *stream)
{
    if (!c || n < 0 || n > c->max_src) return BH_ERR_INVALID;
    if (n > 0 && (!src_pos_mass || !aligned16(src_pos_mass))) return BH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    c->last_stream = s;
    c->built = false;
    const uint32_t un = (uint32_t)n;
    const float4 *src = (const float4 *)src_pos_mass;

    record(c, 0, s);
    launch_bbox(src, un, c->bbox_part, bbox_partials(un), c->prm, c->bits, s);
    if (un > 0) {
        launch_morton(src, un, c->prm, c->bits, c->curve, c->hlut, c->keys, c->vals, s);
        record(c, 1, s);
        // Once a sort of this context has found runs of equal top key bits
        // clustered in tiles (the device's flag, read without waiting, so
        // perhaps a few builds late), its later builds sort every bit in LSD
        // passes: the runs' kernel would wait on its busiest tiles.
        SortRuns sr;
        if (c->clustered) {
            sr.clustered = c->clustered_dev;
            sr.all_passes = __atomic_load_n(c->clustered, __ATOMIC_RELAXED) != 0;
        }
        radix_sort(c->keys, c->vals, c->keys_alt, c->vals_alt, &c->keys_sorted, &c->perm, un,
                   c->key_bits, 0, c->spine, src, c->spos, sr, s);
        record(c, 2, s);
        build_tree(c->keys_sorted, c->spos, un, c->bits, c->leaf_cap, c->node_cap, c->bw,
                   c->nodes, c->prm, s);
        record(c, 3, s);
    } else {
        for (int k = 1; k <= 3; ++k) record(c, k, s);
    }
    bh_status st = launch_status();
    if (st != BH_OK) return st;
    c->n_src = un;
    c->built = true;
    return BH_OK;
}

// Keys of separate targets on the sources' root cube (clamped) with `bits`
// bits per axis on the tree's curve, their stable sort, and the sorted copy in
// c->tpos; returns the caller index of each sorted target.
// Separate targets keyed on the sources' root cube (`bits` per axis) and
// sorted by the key bits from skip_bits up, stable; their positions gathered
// into tpos in that order.
static const uint32_t *sort_targets(bh_ctx *c, const float *targets, uint32_t nt, int bits,
                                    int skip_bits, hipStream_t s)
{
    uint64_t *ko;
    uint32_t *vo;
    launch_morton((const float4 *)targets, nt, c->prm, bits, c->curve, c->hlut, c->tkeys,
                  c->tvals, s);
    radix_sort(c->tkeys, c->tvals, c->tkeys_alt, c->tvals_alt, &ko, &vo, nt, 3 * bits,
               skip_bits, c->tspine, (const float4 *)targets, c->tpos, SortRuns(), s);
    return vo;
}

// The walk's order of separate targets only groups nearby targets into waves
// (every target's result is independent of its wave), so 30-bit keys (a 1024^3
// grid on the root cube) serve as well as the tree's own, and so do their top
// bits alone while the cells they name hold about a wave of targets or fewer:
// up to 2^20 targets the top 14 bits (the low two of the four sort passes
// skipped), up to 2^28 the top 22; targets in one such cell keep the caller's
// order.  (Measured on the surface workloads, 10^6 queries: the query call
// 4-12% faster with 14 bits than with 30, 3-8% with 22.)
constexpr int kTargetOrderBits = 10;
static int target_order_skip(uint32_t nt)
{
    return nt <= (1u << 20) ? 16 : nt <= (1u << 28) ? 8 : 0;
}

// every this many per-target walks of one context store their per-group times
constexpr uint32_t kWalkTimedEvery = 4;

static bh_status gravity_impl(bh_ctx *c, const float *targets, int64_t n_targets, float theta,
                              float G, float eps, uint32_t flags, float *out, uint64_t *count,
                              void *stream)
{
    if (!c) return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    if (n_targets < 0 || n_targets > kMaxCount || !(theta >= 0.f) || !(eps >= 0.f) ||
        !__builtin_isfinite(G))
        return BH_ERR_INVALID;
    if (flags & ~(uint32_t)(BH_WALK_VOTE | BH_WALK_UNSORTED)) return BH_ERR_INVALID;
    if (n_targets > 0 && (!out || !aligned16(out))) return BH_ERR_INVALID;
    if (targets) {
        if (n_targets > c->max_tgt || !aligned16(targets)) return BH_ERR_INVALID;
    } else if ((uint32_t)n_targets != c->n_src) {
        return BH_ERR_INVALID;
    }
    hipStream_t s = (hipStream_t)stream;
    c->last_stream = s;
    const uint32_t nt = (uint32_t)n_targets;
    // with counting on, a walk without a caller's counter counts into the
    // context's own (from zero), for bh_get_interactions
    c->last_counted = !count && c->counting;
    if (c->last_counted) {
        launch_zero_u64(c->icount, s);
        count = (uint64_t *)c->icount;
    }
    if (nt == 0) return launch_status();
    if (c->n_src == 0) {
        launch_fill_zero((float4 *)out, nt, s);
        return launch_status();
    }
    WalkArgs a;
    a.nodes = c->nodes;
    a.wnodes = c->wnodes;
    a.wn_cap = c->wn_cap;
    a.src = c->spos;
    a.prm = c->prm;
    a.n_targets = nt;
    a.theta = theta;
    a.G = G;
    a.eps = eps;
    a.out = (float4 *)out;
    a.count = (unsigned long long *)count;
    a.vote = (flags & BH_WALK_VOTE) != 0;
    a.unsorted = (flags & BH_WALK_UNSORTED) != 0;
    // the per-target walk in key order balances its XCD runs on the previous
    // such walk's per-group times when that walk had the same groups
    const bool balanced = !a.vote && !a.unsorted && c->wn_cap > 0 && c->bal_want;
    const int kind = targets ? 1 : 0;
    const uint32_t groups = walk_groups(nt);
    // Balance of the XCD runs: every kWalkTimedEvery-th walk of the same
    // groups stores its per-group times (each wave reads the clock twice);
    // the walk after it chooses runs from them and the ones between keep
    // those runs.  The device's verdict (read without waiting, so it may lag
    // a call behind) says whether they are uneven, which needs a grid with
    // room for them.
    const bool same_hist = c->hist_groups == groups && c->hist_kind == kind;
    const bool same_runs = c->runs_groups == groups && c->runs_kind == kind;
    a.balance = balanced ? c->wbal : nullptr;
    a.balance_eval = balanced && same_hist && c->hist_new;
    a.balance_fresh = balanced && !same_runs && !a.balance_eval;
    const int want = c->bal_want ? __atomic_load_n(c->bal_want, __ATOMIC_RELAXED) : 0;
    // heavy groups split into waves of their own, in front of the grid and
    // dealt to every XCD in turn (so they also even out the XCDs' work), in
    // preference to uneven runs
    a.balance_split = balanced && !a.balance_fresh && (want & 2) && walk_split_max(groups) > 0;
    a.balance_runs = balanced && (same_runs || a.balance_eval) && (want & 1) && !a.balance_split;
    a.balance_record = balanced && (!same_hist || c->walk_calls < 2 ||
                                    c->walk_calls % kWalkTimedEvery == 0);
    a.balance_want = balanced ? c->bal_want_dev : nullptr;
    if (a.unsorted) {
        a.self = targets == nullptr;
        if (targets) {
            a.tpos = (const float4 *)targets;
            a.tmap = nullptr;
        } else {
            launch_invert(c->perm, nt, c->inv, s);
            a.tpos = c->spos;
            a.tmap = c->inv;
        }
    } else if (targets) {
        a.tpos = c->tpos;
        // the vote's groups are 64 consecutive targets of the tree's key
        // order; the per-target walk's results do not depend on the grouping
        a.tmap = a.vote ? sort_targets(c, targets, nt, c->bits, 0, s)
                        : sort_targets(c, targets, nt, kTargetOrderBits, target_order_skip(nt), s);
        a.self = 0;
    } else {
        a.tpos = c->spos;
        a.tmap = c->perm;
        a.self = 1;
    }
    record(c, 5, s);
    launch_walk(a, s);
    record(c, 6, s);
    if (balanced) {
        if (a.balance_eval || a.balance_fresh) {
            c->runs_groups = groups;
            c->runs_kind = kind;
        }
        if (a.balance_eval) c->hist_new = false;
        c->last_runs = a.balance_runs ? 1 : 0;
        c->last_split = a.balance_split ? 1 : 0;
        if (a.balance_record) {
            c->hist_groups = groups;
            c->hist_kind = kind;
            c->hist_new = true;
        }
        ++c->walk_calls;
    }
    return launch_status();
}

bh_status bh_gravity(bh_ctx *c, const float *targets, int64_t n_targets, float theta, float G,
                     float eps, float *out_acc_pot, void *stream)
{
    return gravity_impl(c, targets, n_targets, theta, G, eps, 0u, out_acc_pot, nullptr, stream);
}

bh_status bh_gravity_counted(bh_ctx *c, const float *targets, int64_t n_targets, float theta,
                             float G, float eps, float *out_acc_pot, uint64_t *interactions,
                             void *stream)
{
    if (!interactions) return BH_ERR_INVALID;
    return gravity_impl(c, targets, n_targets, theta, G, eps, 0u, out_acc_pot, interactions,
                        stream);
}

bh_status bh_gravity_ex(bh_ctx *c, const float *targets, int64_t n_targets, float theta, float G,
                        float eps, uint32_t flags, float *out_acc_pot, uint64_t *interactions,
                        void *stream)
{
    return gravity_impl(c, targets, n_targets, theta, G, eps, flags, out_acc_pot, interactions,
                        stream);
}

bh_status bh_direct(const float *src_pos_mass, int64_t n_src, const float *targets,
                    int64_t n_targets, float G, float eps, float *out_acc_pot, void *stream)
{
    if (n_src < 0 || n_targets < 0 || n_src > kMaxCount || n_targets > kMaxCount)
        return BH_ERR_INVALID;
    if (!(eps >= 0.f) || !__builtin_isfinite(G)) return BH_ERR_INVALID;
    if (n_src > 0 && (!src_pos_mass || !aligned16(src_pos_mass))) return BH_ERR_INVALID;
    if (n_targets > 0 && (!out_acc_pot || !aligned16(out_acc_pot))) return BH_ERR_INVALID;
    if (targets) {
        if (!aligned16(targets)) return BH_ERR_INVALID;
    } else if (n_targets != n_src) {
        return BH_ERR_INVALID;
    }
    hipStream_t s = (hipStream_t)stream;
    const uint32_t nt = (uint32_t)n_targets;
    if (nt == 0) return BH_OK;
    if (n_src == 0)
        launch_fill_zero((float4 *)out_acc_pot, nt, s);
    else
        launch_direct((const float4 *)src_pos_mass, (uint32_t)n_src, (const float4 *)targets, nt,
                      targets == nullptr, G, eps, (float4 *)out_acc_pot, s);
    return launch_status();
}

bh_status bh_sbh(bh_ctx *c, const float *targets, int64_t n_targets, int d, int samples,
                 uint64_t seed, float G, float eps, float *out_acc_pot, void *stream)
{
    if (!c) return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    if (c->leaf_cap != 1 || (d != 2 && d != 4) || samples < 1) return BH_ERR_INVALID;
    if (n_targets < 0 || n_targets > c->max_tgt || !(eps >= 0.f) || !__builtin_isfinite(G))
        return BH_ERR_INVALID;
    if (n_targets > 0 && (!targets || !out_acc_pot || !aligned16(targets) ||
                          !aligned16(out_acc_pot)))
        return BH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    c->last_stream = s;
    const uint32_t nt = (uint32_t)n_targets;
    if (nt == 0) return BH_OK;
    if (c->n_src == 0) {
        launch_fill_zero((float4 *)out_acc_pot, nt, s);
        return launch_status();
    }
    SbhArgs a;
    a.nodes = c->nodes;
    a.tperm = sort_targets(c, targets, nt, c->bits, 0, s);
    a.tpos = c->tpos;
    a.prm = c->prm;
    a.n_targets = nt;
    a.d = d;
    a.samples = samples;
    a.seed = seed;
    a.G = G;
    a.eps = eps;
    a.out = (float4 *)out_acc_pot;
    launch_sbh(a, s);
    return launch_status();
}

bh_status bh_build_locked(bh_ctx *c, const float *src_pos_mass, int64_t n, void *stream)
{
    if (!c || n < 0 || n > c->max_src) return BH_ERR_INVALID;
    if (n > 0 && (!src_pos_mass || !aligned16(src_pos_mass))) return BH_ERR_INVALID;
    if (!c->lk_child) {   // first use: cells for the worst case of the key depth
        const uint64_t cap = (uint64_t)c->max_src * (uint64_t)(c->bits - 1) + 1;
        if (cap > 0x7ffffff0ull) return BH_ERR_INVALID;
        c->lk_cap = (int32_t)cap;
        bool ok = dalloc(&c->lk_child, (size_t)cap * 8) == hipSuccess;
        ok &= dalloc(&c->lk_level, (size_t)cap) == hipSuccess;
        ok &= dalloc(&c->lk_next, (size_t)c->max_src) == hipSuccess;
        ok &= dalloc(&c->lk_counter, 1) == hipSuccess;
        if (!ok) return BH_ERR_OOM;
    }
    hipStream_t s = (hipStream_t)stream;
    c->last_stream = s;
    c->built = false;   // the keys and the root cube are replaced below
    const uint32_t un = (uint32_t)n;
    const float4 *src = (const float4 *)src_pos_mass;
    launch_bbox(src, un, c->bbox_part, bbox_partials(un), c->prm, c->bits, s);
    // the dense build indexes slots by octant: Morton keys whatever the curve
    if (un > 0) launch_morton(src, un, c->prm, c->bits, 0, c->hlut, c->keys, c->vals, s);
    launch_lock_build(c->keys, un, c->bits, c->lk_child, c->lk_level, c->lk_next, c->lk_cap,
                      c->lk_counter, c->prm, s);
    c->lk_n = un;
    return launch_status();
}

bh_status bh_get_locked_tree(bh_ctx *c, int64_t *n_cells, int64_t *cap, int32_t *child,
                             int32_t *level, int32_t *next, void *stream)
{
    if (!c || !n_cells || !cap || !c->lk_child) return BH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    int32_t counter = 0;
    if (hipMemcpyAsync(&counter, c->lk_counter, sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return BH_ERR_HIP;
    const int32_t first = counter < 0 ? 0 : counter;
    *cap = c->lk_cap;
    *n_cells = c->lk_cap - first;
    const size_t nc = (size_t)(c->lk_cap - first);
    bool ok = true;
    if (child)
        ok &= hipMemcpyAsync(child, c->lk_child + (size_t)first * 8, nc * 8 * sizeof(int32_t),
                             hipMemcpyDeviceToDevice, s) == hipSuccess;
    if (level)
        ok &= hipMemcpyAsync(level, c->lk_level + first, nc * sizeof(int32_t),
                             hipMemcpyDeviceToDevice, s) == hipSuccess;
    if (next && c->lk_n)
        ok &= hipMemcpyAsync(next, c->lk_next, (size_t)c->lk_n * sizeof(int32_t),
                             hipMemcpyDeviceToDevice, s) == hipSuccess;
    return ok ? BH_OK : BH_ERR_HIP;
}

bh_status bh_kick_drift(float *pos_mass, float *vel, const float *acc_pot, int64_t n,
                        float dt_kick, float dt_drift, void *stream)
{
    if (n < 0 || n > kMaxCount || !__builtin_isfinite(dt_kick) || !__builtin_isfinite(dt_drift))
        return BH_ERR_INVALID;
    if (n == 0) return BH_OK;
    if (!vel || !aligned16(vel)) return BH_ERR_INVALID;
    if (dt_kick != 0.f && (!acc_pot || !aligned16(acc_pot))) return BH_ERR_INVALID;
    if (dt_drift != 0.f && (!pos_mass || !aligned16(pos_mass))) return BH_ERR_INVALID;
    launch_kick_drift((float4 *)pos_mass, (float4 *)vel, (const float4 *)acc_pot, (uint32_t)n,
                      dt_kick, dt_drift, (hipStream_t)stream);
    return launch_status();
}

bh_status bh_leapfrog_step(bh_ctx *c, float *pos_mass, float *vel, float *acc_pot, int64_t n,
                           float dt, float theta, float G, float eps, void *stream)
{
    if (!c || n < 0 || n > c->max_src || !__builtin_isfinite(dt)) return BH_ERR_INVALID;
    if (!(theta >= 0.f) || !(eps >= 0.f) || !__builtin_isfinite(G)) return BH_ERR_INVALID;
    if (n > 0 && (!pos_mass || !vel || !acc_pot || !aligned16(pos_mass) || !aligned16(vel) ||
                  !aligned16(acc_pot)))
        return BH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t un = (uint32_t)n;
    launch_kick_drift((float4 *)pos_mass, (float4 *)vel, (const float4 *)acc_pot, un, 0.5f * dt,
                      dt, s);
    bh_status st = bh_build(c, pos_mass, n, stream);
    if (st != BH_OK) return st;
    st = gravity_impl(c, nullptr, n, theta, G, eps, 0u, acc_pot, nullptr, stream);
    if (st != BH_OK) return st;
    launch_kick_drift((float4 *)pos_mass, (float4 *)vel, (const float4 *)acc_pot, un, 0.5f * dt,
                      0.f, s);
    return launch_status();
}

bh_status bh_diagnostics(bh_ctx *c, const float *pos_mass, const float *vel,
                         const float *acc_pot, int64_t n, double *out, void *stream)
{
    if (!c || n < 0 || n > kMaxCount || !out) return BH_ERR_INVALID;
    if (n > 0 && (!pos_mass || !vel || !acc_pot || !aligned16(pos_mass) || !aligned16(vel) ||
                  !aligned16(acc_pot)))
        return BH_ERR_INVALID;
    launch_diagnostics((const float4 *)pos_mass, (const float4 *)vel, (const float4 *)acc_pot,
                       (uint32_t)n, c->diag, out, (hipStream_t)stream);
    return launch_status();
}

static bh_status read_params(bh_ctx *c, hipStream_t s)
{
    if (hipMemcpyAsync(c->host_prm, c->prm, sizeof(DevParams), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return BH_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return BH_ERR_HIP;
    return BH_OK;
}

bh_status bh_sync(bh_ctx *c)
{
    if (!c) return BH_ERR_INVALID;
    bh_status st = read_params(c, c->last_stream);
    if (st != BH_OK) return st;
    const uint32_t w = c->host_prm->status;
    if (w & kStatusNonFinite) {
        c->built = false;
        return BH_ERR_NONFINITE;
    }
    if (w & kStatusCapacity) {
        c->built = false;
        return BH_ERR_CAPACITY;
    }
    if (w & kStatusLockRetry) return BH_ERR_CONTENTION;
    return BH_OK;
}

bh_status bh_get_keys(bh_ctx *c, uint64_t *keys_sorted, uint32_t *perm, void *stream)
{
    if (!c || !c->built) return c ? BH_ERR_NOT_BUILT : BH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    const size_t n = c->n_src;
    if (n == 0) return BH_OK;
    if (keys_sorted &&
        hipMemcpyAsync(keys_sorted, c->keys_sorted, n * 8, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return BH_ERR_HIP;
    if (perm && hipMemcpyAsync(perm, c->perm, n * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return BH_ERR_HIP;
    return BH_OK;
}

bh_status bh_get_node_count(bh_ctx *c, int64_t *n_nodes, void *stream)
{
    if (!c || !n_nodes) return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    if (c->n_src == 0) {
        *n_nodes = 0;
        return BH_OK;
    }
    bh_status st = read_params(c, (hipStream_t)stream);
    if (st != BH_OK) return st;
    *n_nodes = c->host_prm->n_nodes;
    return BH_OK;
}

bh_status bh_node_hmax(bh_ctx *c, const float *h, int64_t n, float *node_hmax,
                       int64_t n_nodes_max, void *stream)
{
    if (!c || n < 0 || n_nodes_max < 0) return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    if ((uint64_t)n != c->n_src || (n > 0 && (!h || !node_hmax))) return BH_ERR_INVALID;
    if (n == 0) return BH_OK;
    hipStream_t s = (hipStream_t)stream;
    c->last_stream = s;
    bh_status st = read_params(c, s);   // the node count (and the build's status)
    if (st != BH_OK) return st;
    if (c->host_prm->status != 0) return BH_ERR_NOT_BUILT;
    const uint32_t nn = c->host_prm->n_nodes;
    if ((uint64_t)nn > (uint64_t)n_nodes_max) return BH_ERR_INVALID;
    launch_node_hmax(c->nodes, c->perm, h, nn, c->prm, c->node_cap, c->bits, node_hmax, s);
    return launch_status();
}

bh_status bh_get_nodes(bh_ctx *c, bh_node *nodes, int64_t n_nodes, void *stream)
{
    if (!c || n_nodes < 0 || (uint64_t)n_nodes > c->node_cap || (n_nodes && !nodes))
        return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    if (n_nodes == 0) return BH_OK;
    if (hipMemcpyAsync(nodes, c->nodes, (size_t)n_nodes * sizeof(Node), hipMemcpyDeviceToDevice,
                       (hipStream_t)stream) != hipSuccess)
        return BH_ERR_HIP;
    return BH_OK;
}

bh_status bh_get_bbox(bh_ctx *c, double *lo, double *hi, double *L, void *stream)
{
    if (!c || !lo || !hi || !L) return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    bh_status st = read_params(c, (hipStream_t)stream);
    if (st != BH_OK) return st;
    for (int a = 0; a < 3; ++a) {
        lo[a] = c->host_prm->lo[a];
        hi[a] = c->host_prm->hi[a];
    }
    *L = c->host_prm->L;
    return BH_OK;
}

bh_status bh_set_counting(bh_ctx *c, int enable)
{
    if (!c) return BH_ERR_INVALID;
    c->counting = enable != 0;
    return BH_OK;
}

bh_status bh_get_walk_runs(bh_ctx *c, uint32_t *starts, int32_t *uneven, int32_t *split)
{
    if (!c || !uneven || c->last_runs < 0) return BH_ERR_INVALID;
    *uneven = c->last_runs;
    if (split) *split = 0;
    if (!starts && !(split && c->last_split)) return BH_OK;
    uint32_t head[kWalkSplitCount + 1];
    if (hipMemcpyAsync(head, c->wbal, sizeof(head), hipMemcpyDeviceToHost, c->last_stream) !=
            hipSuccess ||
        hipStreamSynchronize(c->last_stream) != hipSuccess)
        return BH_ERR_HIP;
    if (starts) memcpy(starts, head, 9 * sizeof(uint32_t));
    if (split && c->last_split) *split = (int32_t)head[kWalkSplitCount];
    return BH_OK;
}

bh_status bh_get_interactions(bh_ctx *c, uint64_t *host_total)
{
    if (!c || !host_total) return BH_ERR_INVALID;
    if (!c->last_counted) return BH_ERR_INVALID;
    unsigned long long v = 0;
    if (hipMemcpyAsync(&v, c->icount, sizeof(v), hipMemcpyDeviceToHost, c->last_stream) !=
            hipSuccess ||
        hipStreamSynchronize(c->last_stream) != hipSuccess)
        return BH_ERR_HIP;
    *host_total = (uint64_t)v;
    return BH_OK;
}

bh_status bh_get_cells(bh_ctx *c, int64_t *n_nodes, uint8_t *level, uint64_t *prefix,
                       uint32_t *count, void *stream)
{
    if (!c || !n_nodes) return BH_ERR_INVALID;
    if (!c->built) return BH_ERR_NOT_BUILT;
    *n_nodes = 0;
    if (c->n_src == 0) return BH_OK;
    hipStream_t s = (hipStream_t)stream;
    bh_status st = read_params(c, s);   // the node count (and the build's status)
    if (st != BH_OK) return st;
    if (c->host_prm->status & (kStatusNonFinite | kStatusCapacity)) return BH_ERR_NOT_BUILT;
    const uint32_t nn = c->host_prm->n_nodes;
    *n_nodes = nn;
    launch_cells(c->nodes, c->spos, nn, c->bits, c->prm, level, prefix, count, s);
    return launch_status();
}

bh_status bh_set_profiling(bh_ctx *c, int enable)
{
    if (!c) return BH_ERR_INVALID;
    c->prof = enable != 0;
    return BH_OK;
}

bh_status bh_get_profile(bh_ctx *c, float *ms, int n)
{
    if (!c || !ms || n < 0) return BH_ERR_INVALID;
    if (!c->prof) return BH_ERR_INVALID;
    const int pairs[4][2] = {{0, 1}, {1, 2}, {2, 3}, {5, 6}};
    for (int k = 0; k < n && k < 4; ++k) {
        if (hipEventSynchronize(c->ev[pairs[k][1]]) != hipSuccess) return BH_ERR_HIP;
        float t = 0.f;
        if (hipEventElapsedTime(&t, c->ev[pairs[k][0]], c->ev[pairs[k][1]]) != hipSuccess)
            return BH_ERR_HIP;
        ms[k] = t;
    }
    return BH_OK;
}


bh_status bh_gravity_static(const float *src_pos_mass, int64_t n, const bh_build_params *params,
                            float theta, float G, float eps, float *out_acc_pot, void *stream)
{
    bh_build_params p = {63, 16, 0, 0, 0};
    if (params) p = *params;
    if ((p.key_bits != 63 && p.key_bits != 30) || p.leaf_cap < 1 || p.leaf_cap > kMaxLeafCap ||
        p.node_capacity != 0 || (p.key_curve != BH_CURVE_MORTON && p.key_curve != BH_CURVE_HILBERT) ||
        p.reserved != 0)
        return BH_ERR_INVALID;
    if (n < 0 || n > kMaxCount || !(theta >= 0.f) || !(eps >= 0.f) || !__builtin_isfinite(G))
        return BH_ERR_INVALID;
    if (n > 0 && (!src_pos_mass || !out_acc_pot || !aligned16(src_pos_mass) ||
                  !aligned16(out_acc_pot)))
        return BH_ERR_INVALID;
    bh_ctx c;   // host-side description only: no allocation, no events
    c.max_src = n;
    c.key_bits = p.key_bits;
    c.bits = p.key_bits / 3;
    c.leaf_cap = p.leaf_cap;
    c.curve = p.key_curve;
    c.node_cap = node_bound((uint64_t)n, c.bits, c.leaf_cap);
    if (static_layout(&c, nullptr, (uint32_t)n) > kStaticScratchBytes) return BH_ERR_CAPACITY;
    if (n == 0) return BH_OK;
    if (hipGetDevice(&c.device) != hipSuccess) return BH_ERR_HIP;
    unsigned char *base = nullptr;
    bh_status st = static_base(c.device, &base);
    if (st != BH_OK) return st;
    static_layout(&c, base, (uint32_t)n);
    st = bh_build(&c, src_pos_mass, n, stream);
    if (st != BH_OK) return st;
    return gravity_impl(&c, nullptr, n, theta, G, eps, 0u, out_acc_pot, nullptr, stream);
}

}  // extern "C"
