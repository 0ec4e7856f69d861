// Internal declarations shared by the HIP translation units of libbh.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bh.h"

namespace bh {

constexpr int kMaxLevels = 22;      // levels 0..21 for 63-bit keys
constexpr int kMaxLeafCap = 256;
constexpr int kSourcePad = 8;       // readable slack after the sorted sources

// Device status bits (a word in DevParams; 0 = fine).
constexpr uint32_t kStatusNonFinite = 1u;
constexpr uint32_t kStatusCapacity = 2u;
constexpr uint32_t kStatusLockRetry = 4u;   // lock-based build: an insertion ran out of retries

// Per-build scalars kept in device memory, so that no step needs the host to
// read back an intermediate value.
struct DevParams {
    double lo[3];        // min corner of the sources
    double hi[3];        // max corner
    double L;            // root cube side = largest extent
    double scale;        // 2^bits / L, or 0 when L == 0
    uint32_t status;     // kStatus* bits
    uint32_t n_nodes;    // nodes emitted by the build
    uint32_t n_src;      // sources of this build
    uint32_t pad;
};

// fp64 (mass, mass-weighted offsets) used for centre-of-mass prefix sums.
struct alignas(16) D4 {
    double m, x, y, z;
};
__host__ __device__ inline D4 operator+(D4 a, D4 b) { return D4{a.m + b.m, a.x + b.x, a.y + b.y, a.z + b.z}; }
__host__ __device__ inline D4 operator-(D4 a, D4 b) { return D4{a.m - b.m, a.x - b.x, a.y - b.y, a.z - b.z}; }

// Exclusive per-tile prefix of node counts and particle sums.  Node counts
// are 32-bit (a chunk of tiles holds at most 2^21 positions, so fewer than
// 2^26 nodes); the scan over chunks also sums them in 64 bits and sets
// `wrapped` in the totals entry when the whole tree has 2^32 nodes or more.
struct alignas(16) TileScan {
    D4 sums;
    uint32_t nodes, wrapped, leaves, pad;
};

// Pre-order node record; the public bh_node has the same layout.
struct alignas(16) Node {
    float cx, cy, cz, m;
    uint32_t start, count, skip, meta;
};
static_assert(sizeof(Node) == 32, "node is 32 bytes");
static_assert(sizeof(Node) == sizeof(bh_node), "node matches the public record");

constexpr uint32_t kLeafBit = 1u << 8;
__host__ __device__ inline uint32_t node_level(uint32_t meta) { return meta & 0xffu; }

// Radix sort geometry: a tile of 2048 keys per workgroup of 256 threads, or
// 4096 from kSortLargeN keys on (the spine is sized for the smaller tile).
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr int kSortItemsLarge = 16;
constexpr uint32_t kSortLargeN = 1u << 22;
constexpr int kSortTile = kSortThreads * kSortItems;
constexpr int kRadix = 256;

// Workgroups are dispatched to the 8 XCDs round-robin (block b to XCD b mod 8).
// xcd_block(b, nb) renumbers them so each XCD takes one contiguous run of the
// nb work items, and work items that share data share that XCD's L2.
__device__ inline uint32_t xcd_block(uint32_t b, uint32_t nb)
{
    const uint32_t x = b & 7u, k = b >> 3, q = nb >> 3, r = nb & 7u;
    return x * q + min(x, r) + k;
}

// Tree build geometry: 1024 key positions per workgroup of 256 threads.
constexpr int kBuildThreads = 256;
constexpr int kBuildTile = 1024;
constexpr int kTileScanThreads = 1024;

// Quantised coordinate of x on the root cube: floor((x - lo) * scale) in fp64,
// each step one correctly rounded IEEE operation, clamped to [0, top] (below the
// cube and NaN give 0, the max face and beyond the top cell).
__device__ inline uint64_t quantise(float x, double lo, double scale, uint64_t top)
{
#pragma clang fp contract(off)
    const double d = (double)x - lo;
    const double u = d * scale;
    const double f = floor(u);
    if (!(f >= 0.0)) return 0;
    if (f >= (double)top) return top;
    return (uint64_t)f;
}

// ---- launchers (each defined in its own .hip file) ------------------------

// bbox.hip
void launch_bbox(const float4 *src, uint32_t n, float *partials, uint32_t n_partials,
                 DevParams *prm, int bits, hipStream_t s);
uint32_t bbox_partials(uint32_t n);
// curve 0: Morton keys, 1: Hilbert keys (hilbert_lut: the device copy of the
// tables hilbert_lut_host fills, kHilbertLutEntries entries; unused for Morton)
constexpr int kHilbertStates = 48;
constexpr int kHilbertLutEntries = kHilbertStates * 64 + kHilbertStates * 8;
bool hilbert_lut_host(uint16_t *out);
void launch_morton(const float4 *pts, uint32_t n, const DevParams *prm, int bits, int curve,
                   const uint16_t *hilbert_lut,
                   uint64_t *keys, uint32_t *idx, hipStream_t s);

// radix_sort.hip
size_t sort_spine_entries(uint32_t n);
// The 63-bit key sort with a gather sorts the top 40 bits in five passes and
// then orders each run of equal top bits in one kernel, whose workgroups sort
// the runs of more than 64 members that start in their tile one after another.
// clustered (host-mapped, may be null) is set to 1 when some tile starts
// several; all_passes sorts all 64 bits in eight passes instead (the same
// order), with no such kernel.
struct SortRuns {
    uint32_t *clustered = nullptr;
    bool all_passes = false;
};
// Stable LSD sort of (keys, vals) over the key bits [skip_bits, key_bits)
// (skip_bits a multiple of 8; 0: every bit below key_bits): keys equal in
// those bits keep their input order.  Ping-pongs between the two buffer
// pairs; the result ends in (keys_out, vals_out).  With gather_src != NULL the
// last pass also writes gather_dst[i] = gather_src[vals[i]].
void radix_sort(uint64_t *keys, uint32_t *vals, uint64_t *keys_alt, uint32_t *vals_alt,
                uint64_t **keys_out, uint32_t **vals_out, uint32_t n, int key_bits,
                int skip_bits, uint32_t *spine, const float4 *gather_src, float4 *gather_dst,
                const SortRuns &sr, hipStream_t s);

// Exclusive scan of each row of a [rows][len] table, one workgroup per row:
// pref[r][t] = sum(in[r][0..t)), tot[r] = row total.
void launch_scan_rows(const uint32_t *in, uint32_t *pref, uint32_t *tot, uint32_t rows,
                      uint32_t len, hipStream_t s);

// build.hip
uint32_t build_blocks(uint32_t n);
// Device scratch of the tree build (owned by the context).
struct BuildScratch {
    uint16_t *dc;           // per position: d + 1 (low byte), nodes starting there (high byte)
    uint2 *tile_counts;     // per tile: nodes and leaves starting in the tile
    D4 *tile_sums;          // per tile: particle sums
    TileScan *chunk_tot;    // per chunk of tiles: node count and particle sums
    TileScan *tile_scan;    // per chunk: exclusive prefix; [n_chunks] = totals
    uint2 *first_node;      // per leaf start (and n): pre-order index of the first node
                            // there, and the number of leaves before it
    D4 *P;                  // per leaf in pre-order (and one past the last): prefix sums
                            // of (m, m (x - lo)) over the sources before the leaf
};
void build_tree(const uint64_t *keys_sorted, const float4 *spos, uint32_t n, int bits,
                int leaf_cap, uint64_t node_capacity, BuildScratch &w, Node *nodes,
                DevParams *prm, hipStream_t s);

// per node: level, key prefix of the cell's place on its level's grid, count
// (any output may be NULL)
void launch_cells(const Node *nodes, const float4 *spos, uint32_t nn, int bits,
                  const DevParams *prm, uint8_t *level, uint64_t *prefix, uint32_t *count,
                  hipStream_t s);

// *p = 0 by a one-thread kernel (no memset node under stream capture)
void launch_zero_u64(unsigned long long *p, hipStream_t s);

// hmax.hip: per-node maximum of h (caller order) over the node's sources
void launch_node_hmax(const Node *nodes, const uint32_t *perm, const float *h, uint32_t n_nodes,
                      const DevParams *prm, uint64_t cap, int bits, float *out, hipStream_t s);

// traverse.hip
// node count up to which the walk's assembly loop runs: its 32-bit node byte
// offsets (X * 32 for X <= the end record's index) cannot wrap
constexpr uint32_t kAsmMaxNodes = (1u << 27) - 1;
struct WalkArgs {
    const Node *nodes;
    Node *wnodes;               // per-call walk records (skips in bytes, thresholds in place)
    uint32_t wn_cap;            // records wnodes holds (0: none; the compiled loop walks)
    const float4 *src;          // sources in Morton order
    const float4 *tpos;         // target positions (Morton order, or as given when unsorted)
    const uint32_t *tmap;       // sorted: caller index of each target; unsorted self: Morton rank
    const DevParams *prm;
    uint32_t n_targets;
    int self;                   // targets are the sources (exclude i == j)
    int vote;                   // wave-wide vote instead of the per-lane walk
    int unsorted;               // walk the targets in the caller's order
    float theta, G, eps;
    float4 *out;
    unsigned long long *count;  // optional interaction counter
    // XCD balance of the sorted per-target walk (layout of the buffer at
    // kWalkBalanceHead; null: none).  balance_eval: the buffer holds times of
    // a recent walk of the same groups not yet looked at, from which to choose
    // the runs (and set *balance_want, host-mapped, may be null); else keep
    // the runs it holds (balance_fresh: none for these groups, write the equal
    // runs).  balance_runs: walk those runs (a grid with room for uneven
    // runs), else the equal runs of xcd_block.  balance_record: store this
    // walk's per-group times.
    // balance_split: the launch also walks the heaviest groups (listed in the
    // buffer) as kWalkSplitParts waves of their own, ahead of the rest.
    uint32_t *balance;
    int balance_eval;
    int balance_fresh;
    int balance_runs;
    int balance_split;
    int balance_record;
    int *balance_want;
};
void launch_walk(const WalkArgs &a, hipStream_t s);
// walk groups of 64 targets, and the most groups one XCD's run may take
__host__ __device__ inline uint32_t walk_groups(uint32_t n_targets) { return (n_targets + 63) / 64; }
__host__ __device__ inline uint32_t walk_xcd_cap(uint32_t groups) { return (groups + 7) / 8 + (groups + 31) / 32; }
// The walk's balance buffer (kWalkBalanceHead + 3 groups entries): entries
// 0-8 the first group of each XCD's run (the ninth = groups), entry
// kWalkSplitCount the number of split groups; from kWalkBalanceHead on one
// time per group, then the split groups (walk_split_max(groups) entries),
// then one split flag per group.
constexpr uint32_t kWalkBalanceHead = 32;
constexpr uint32_t kWalkSplitCount = 9;
// A group whose recorded time stands far above the mean is walked as
// kWalkSplitParts waves of 64 / kWalkSplitParts targets each (every target's
// result is its own walk, so the same bits): its waves then end sooner, and
// they start first.  At most one group in 32 is split (none below 512).
constexpr uint32_t kWalkSplitParts = 4;
__host__ __device__ inline uint32_t walk_split_max(uint32_t groups)
{
    return groups < 512 ? 0u : 2 * ((groups + 63) / 64);
}
// inv[perm[k]] = k
void launch_invert(const uint32_t *perm, uint32_t n, uint32_t *inv, hipStream_t s);
void launch_fill_zero(float4 *out, uint32_t n, hipStream_t s);

// sbh.hip: stochastic Barnes-Hut at separate targets (sorted; leaf capacity 1)
struct SbhArgs {
    const Node *nodes;
    const float4 *tpos;         // targets in Morton order
    const uint32_t *tperm;      // caller index of each sorted target
    const DevParams *prm;
    uint32_t n_targets;
    int d;                      // 2 or 4
    int samples;
    uint64_t seed;
    float G, eps;
    float4 *out;
};
void launch_sbh(const SbhArgs &a, hipStream_t s);

// lockbuild.hip: the pages' lock-based dense build (cells allocated downward
// from cap - 1, the root; slots: -1 empty, -2 locked, particle, n + cell id)
void launch_lock_build(const uint64_t *keys, uint32_t n, int bits, int32_t *child,
                       int32_t *level, int32_t *next, int32_t cap, int32_t *counter,
                       DevParams *prm, hipStream_t s);

// integrate.hip: leapfrog kick/drift and conserved-quantity sums
constexpr int kDiagTerms = 10;           // mass, kinetic, potential, p xyz, L xyz, count
constexpr uint32_t kDiagMaxPartials = 1024;
void launch_kick_drift(float4 *pos, float4 *vel, const float4 *acc, uint32_t n, float dt_kick,
                       float dt_drift, hipStream_t s);
uint32_t diag_partials(uint32_t n);
void launch_diagnostics(const float4 *pos, const float4 *vel, const float4 *acc, uint32_t n,
                        double *partials, double *out, hipStream_t s);

// direct.hip: all-pairs sum over the caller's sources (self: tgt is ignored,
// the sources are the targets and each excludes itself)
void launch_direct(const float4 *src, uint32_t n, const float4 *tgt, uint32_t nt, bool self,
                   float G, float eps, float4 *out, hipStream_t s);

}  // namespace bh
