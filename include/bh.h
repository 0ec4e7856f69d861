/*
 * bh.h — Barnes-Hut octree self-gravity on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbh.so.  Plain pointers and sizes only.  All device pointers are
 * HIP device memory on the current device; every `stream` argument is a
 * hipStream_t passed as void* (NULL = the default stream).
 *
 * The operations follow these pages (cited by title and section):
 *   [GASPHiA]  "GASPHiA中的自引力树代码效率与优化分析"
 *   [Tree]     "树结构（基于根据 Burtscher 和 Pingali 的研究）" and its embedded
 *              article "基于稠密存储的并行树构建实现方案"
 *   [SBH]      notes on "Stochastic Barnes-Hut Approximation for Fast Summation
 *              on the GPU"
 *
 * Conventions
 *   Particles are float4 rows (x, y, z, m), 16 bytes each, 16-byte aligned
 *   ([Tree] 构建树结构: the w component carries the mass).
 *   Every call is stream-ordered and asynchronous unless stated otherwise;
 *   pointers must stay valid until the stream reaches the call.
 *   Argument errors are returned synchronously.  Conditions found on the
 *   device (non-finite coordinates, node-capacity overflow) are recorded in a
 *   device status word and returned by bh_sync; a build that failed on the
 *   device leaves the context unbuilt for the next bh_gravity.
 *   A context is not thread-safe: use one per host thread / stream.
 *   Limits: n < 2^31 particles.
 */
#ifndef BH_H
#define BH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bh_ctx bh_ctx;

typedef enum bh_status {
    BH_OK = 0,
    BH_ERR_INVALID = -1,    /* bad argument: NULL, negative or too-large size, misaligned pointer, bad parameter */
    BH_ERR_OOM = -2,        /* device allocation failed in bh_create */
    BH_ERR_HIP = -3,        /* a HIP runtime call or kernel launch failed */
    BH_ERR_CAPACITY = -4,   /* the tree needed more nodes than node_capacity */
    BH_ERR_NONFINITE = -5,  /* a source coordinate or mass is NaN or infinite */
    BH_ERR_NOT_BUILT = -6,  /* bh_gravity before a successful bh_build */
    BH_ERR_CONTENTION = -7  /* bh_build_locked: an insertion ran out of retries */
} bh_status;

/* Key curves: the order in which sources are sorted and siblings appear in the
 * node array.  Morton is the Z-order of [Tree] 实现步骤; Hilbert visits the same
 * cells (each still one contiguous run of the order) with every step between
 * neighbouring cells, so the 64 consecutive targets of a wave are more compact
 * and the walk visits fewer nodes.  Results differ only by rounding (the same
 * cells, summed in another order). */
#define BH_CURVE_MORTON 0
#define BH_CURVE_HILBERT 1

/* Build parameters, fixed for the life of a context.
 *   key_bits      63 (21 bits per axis) or 30 (10 bits per axis): the depth of
 *                 the Morton key of [Tree] 实现步骤 and the deepest tree level.
 *   leaf_cap      B >= 1: a cell holding more than B particles is split into its
 *                 octants unless it is at the deepest level ([Tree] 实现步骤: a
 *                 leaf holds a few particles).  At most 256.
 *   node_capacity maximum number of tree nodes; 0 selects the bound
 *                 (key_bits/3) * floor(max_sources / (B + 1)) + max_sources + 1,
 *                 which no tree exceeds: the split cells of one level are
 *                 disjoint and hold more than B sources each, and leaves are
 *                 disjoint non-empty cells.
 *   key_curve     BH_CURVE_MORTON (default) or BH_CURVE_HILBERT (keys after
 *                 Skilling, "Programming the Hilbert curve", 2004); bh_get_keys
 *                 returns keys of this curve.  Separate targets are ordered by
 *                 the same curve (for the per-target walk on a 1024^3 grid of
 *                 the root cube, which groups nearby targets as well; its
 *                 results do not depend on the order). */
typedef struct bh_build_params {
    int32_t key_bits;
    int32_t leaf_cap;
    int64_t node_capacity;
    int32_t key_curve;
    int32_t reserved;   /* must be 0 */
} bh_build_params;

/* One tree node as stored on the device (32 bytes), in pre-order: a node's
 * subtree is the index range [self, skip).  Children follow their parent in
 * key order: octant order 0..7 for Morton keys (the octant numbering of [Tree]
 * 构建树结构: x upper half = 1, y = 2, z = 4), the curve's order for Hilbert
 * keys.  com_x..mass follow [GASPHiA] 计算节点质心. */
typedef struct bh_node {
    float com_x, com_y, com_z;  /* centre of mass (cell centre when mass is 0) */
    float mass;                 /* total mass of the cell */
    uint32_t start;             /* first particle, as an index into the Morton-sorted order */
    uint32_t count;             /* number of particles in the cell */
    uint32_t skip;              /* pre-order index just past this subtree */
    uint32_t meta;              /* bits 0-7: level (root = 0); bit 8: leaf */
} bh_node;

/* Create a context owning all device scratch for up to max_sources sources
 * and max_targets separate targets (0 if only self-gravity is needed).
 * Allocates device memory (synchronous).  *out is NULL on failure. */
bh_status bh_create(bh_ctx **out, int64_t max_sources, int64_t max_targets,
                    const bh_build_params *params);

/* Build the tree over n sources, steps of [Tree] 实现步骤 in order:
 * bounding box (确定粒子空间范围), Morton keys and their stable sort (粒子空间
 * 排序, the gather index of [GASPHiA] 排序算法), the octree (构建树结构) and the
 * centre of mass of every node ([GASPHiA] 计算节点质心).
 *   src_pos_mass  device, n float4 rows (x, y, z, m), read only, 16-byte aligned.
 * The sources are copied in sorted order; src_pos_mass is not needed after
 * the stream passes this call.  n = 0 builds an empty tree.  With 63-bit keys
 * the sort orders the top 40 bits in passes and then each run of keys equal
 * in those bits; once a build of the context has found many long such runs
 * (sources clustered far below the root cube's scale), its later builds sort
 * all bits in passes instead.  Either way the order, and every result, is the
 * same. */
bh_status bh_build(bh_ctx *ctx, const float *src_pos_mass, int64_t n, void *stream);

/* Accelerations and potentials by the tree walk of [GASPHiA] 计算自引力 /
 * 性能瓶颈分析: a node is used whole when (w/theta)^2 < r^2 (w the node's cell
 * edge, r the distance from the target to its centre of mass), otherwise its
 * children are visited; an opened leaf is summed particle by particle.
 * Every interaction uses Plummer softening:
 *   a += G m d / (|d|^2 + eps^2)^(3/2),  phi -= G m / (|d|^2 + eps^2)^(1/2),
 * with d = x_source - x_target; a pair with |d|^2 + eps^2 = 0 adds nothing.
 *   targets       NULL: the built sources are the targets and each excludes
 *                 itself; else device, n_targets float4 rows (w ignored), at
 *                 most max_targets ([SBH] 实验结果 evaluates separate queries).
 *   out_acc_pot   device, n_targets float4 rows (ax, ay, az, phi) in the
 *                 caller's order of the targets (for targets == NULL,
 *                 n_targets must equal the n given to bh_build).
 *   theta >= 0 (0 = exact direct sum), eps >= 0, G any finite value.
 * The context remembers each walk's time per group of 64 targets; when the
 * next walk has the same groups (the same target count, self-gravity or not)
 * and those times show the eight XCDs' equal runs of groups out of balance,
 * it moves the runs' ends, and when a few groups take far longer than the
 * mean, it walks each of them as four waves of 16 targets, started first.
 * That changes only where and how each target's walk runs: the results are
 * the same bits either way. */
bh_status bh_gravity(bh_ctx *ctx, const float *targets, int64_t n_targets, float theta,
                     float G, float eps, float *out_acc_pot, void *stream);

/* Same as bh_gravity, and adds the number of interactions (accepted nodes plus
 * particle pairs, self excluded) to *interactions (device, uint64) — slower,
 * for measurement and tests. */
bh_status bh_gravity_counted(bh_ctx *ctx, const float *targets, int64_t n_targets,
                             float theta, float G, float eps, float *out_acc_pot,
                             uint64_t *interactions, void *stream);

/* Walk variants for measuring the pages' design choices (flags, OR-ed):
 *   BH_WALK_VOTE      the warp vote of [GASPHiA] 性能瓶颈分析: the 64 targets of a
 *                     wave walk together, and when the opening test fails for any
 *                     of them, every one of them uses the node's children (or,
 *                     for a leaf, its particles).  Results depend on which
 *                     targets share a wave (64 consecutive targets in the
 *                     order of the tree's keys) and are at least as accurate as
 *                     the per-target walk.
 *   BH_WALK_UNSORTED  walk the targets in the caller's order instead of their
 *                     Morton order ([GASPHiA] 排序算法 measures what this order
 *                     buys).  Without BH_WALK_VOTE the results are bit-identical
 *                     to the default walk; only the speed changes. */
#define BH_WALK_VOTE 1u
#define BH_WALK_UNSORTED 2u

/* bh_gravity with walk variant flags (0 = bh_gravity) and an optional
 * interaction counter (NULL = none; else as bh_gravity_counted).  Unknown
 * flag bits are rejected with BH_ERR_INVALID. */
bh_status bh_gravity_ex(bh_ctx *ctx, const float *targets, int64_t n_targets, float theta,
                        float G, float eps, uint32_t flags, float *out_acc_pot,
                        uint64_t *interactions, void *stream);

/* The lock-based dense build of [Tree] 构建树结构 / 核心代码片段 / 并发与同步 and
 * its embedded article on dense storage, kept to measure that design against
 * bh_build on the same device.  One thread per source walks down from the
 * root; at the first slot that is not a cell it takes the slot with a
 * compare-and-swap (empty -> locked); an empty slot receives the source, a
 * slot holding another source is subdivided into new cells (allocated
 * downward by an atomic decrement) until the two separate, and the slot is
 * released after a fence.  Octants come from the Morton keys, so the result
 * is the leaf-capacity-1 octree; sources with identical keys are chained at
 * the finest level.  The walk does not use this tree; bh_get_locked_tree
 * returns it.  Replaces the context's tree (bh_gravity needs bh_build again).
 * Allocates its arrays on first use (synchronous): max_sources * (key_bits/3
 * - 1) + 1 cells of 36 bytes.  Device status (bh_sync): BH_ERR_NONFINITE,
 * BH_ERR_CAPACITY, BH_ERR_CONTENTION (an insertion gave up after 4096
 * steps; the tree is then incomplete). */
bh_status bh_build_locked(bh_ctx *ctx, const float *src_pos_mass, int64_t n, void *stream);

/* The tree of the last bh_build_locked (synchronous).  Cells have ids
 * cap - n_cells .. cap - 1 (the root is cap - 1); row r of the copies is cell
 * cap - n_cells + r.  child: n_cells * 8 slots (-1 empty, 0..n-1 a source, the
 * head of its chain, n + id a cell), in octant order; level: n_cells levels;
 * next: n entries, the next source with the same key or -1.  Device buffers;
 * any may be NULL. */
bh_status bh_get_locked_tree(bh_ctx *ctx, int64_t *n_cells, int64_t *cap, int32_t *child,
                             int32_t *level, int32_t *next, void *stream);

/* Stochastic Barnes-Hut ([SBH] 方法, 关键设计): an unbiased Monte-Carlo estimate
 * of the sum at separate query points, on the context's tree, which must be
 * built with leaf_cap = 1 (paths end at single sources).  Per sample, one path
 * per stratum (the children of the root in the d-ary tree): the path index I
 * is uniform over the stratum's sources, the path length is set by Russian
 * roulette with continuation probability min(1, max(1, b_k) / b_{k+1}),
 * b = |q - centre of mass| / cell edge, and each step adds the children's
 * monopoles minus the cell's, divided by P(I in cell) P(K >= k).
 *   d        2: one octree level per step; 4: two (a leaf child stands for itself).
 *   samples  S >= 1 samples are averaged.
 *   seed     Philox4x32-10 key (low, high word); counter = (group, sample,
 *            stratum, j), j = 0 for I, j = k + 1 for the roulette at depth k;
 *            a group is the 64 consecutive queries of the queries' Morton
 *            order, which share their random numbers (so a wave follows one
 *            path).  I = start + floor(r count / 2^32) and u = (r >> 8) 2^-24 from
 *            the first output word r.
 *   targets  device, n_targets float4 rows (w ignored), at most max_targets.
 *   out_acc_pot as for bh_gravity.
 * Errors: BH_ERR_INVALID (leaf_cap != 1, bad d or samples, bad arguments),
 * BH_ERR_NOT_BUILT.  Asynchronous. */
bh_status bh_sbh(bh_ctx *ctx, const float *targets, int64_t n_targets, int d, int samples,
                 uint64_t seed, float G, float eps, float *out_acc_pot, void *stream);

/* Per-node maximum smoothing length: node_hmax[X] = the largest h among the
 * sources of node X of the last bh_build, the hmax the pages' tree keeps beside
 * the centre of mass for its SPH neighbour search ([Tree] 树结构 粒子领域搜索;
 * the d_node_hmax array of 重置树结构).  Leaves take the maximum over their
 * sources, internal nodes over their children.
 *   h            device, n floats in the caller's order of the built sources
 *                (n must equal the n of bh_build); finite values.
 *   node_hmax    device, at least as many floats as the tree has nodes, in
 *                node order (the order of bh_get_nodes).
 *   n_nodes_max  capacity of node_hmax in floats.
 * Waits for `stream` to finish the build (it reads the node count), then
 * runs asynchronously on `stream`.  Errors: BH_ERR_NOT_BUILT (no build, or
 * the build failed on the device), BH_ERR_INVALID (bad arguments, n other
 * than the built n, n_nodes_max below the node count). */
bh_status bh_node_hmax(bh_ctx *ctx, const float *h, int64_t n, float *node_hmax,
                       int64_t n_nodes_max, void *stream);

/* All-pairs direct sum, no tree and no context: every target against every
 * source with the interaction of bh_gravity.  This is the brute-force
 * reference that [GASPHiA] 精度与加速比验证 measures the walk's speed-up and
 * relative error against, and the theta = 0 limit of the walk.
 *   src_pos_mass  device, n_src float4 rows (x, y, z, m), 16-byte aligned.
 *   targets       NULL: the sources are the targets and each excludes itself
 *                 (n_targets must equal n_src); else device, n_targets float4
 *                 rows (w ignored), 16-byte aligned.
 *   out_acc_pot   device, n_targets float4 rows (ax, ay, az, phi), in the
 *                 order of the targets; must not overlap the inputs.
 *   eps >= 0, G finite; n_src, n_targets < 2^31.
 * fp32 pair terms summed in fp32 over runs of 512 sources, the runs summed in
 * fp64.  Non-finite inputs give non-finite outputs (no status word).
 * Asynchronous on `stream`; allocates nothing. */
bh_status bh_direct(const float *src_pos_mass, int64_t n_src, const float *targets,
                    int64_t n_targets, float G, float eps, float *out_acc_pot, void *stream);

/* ---- time stepping ------------------------------------------------------
 * The pages advance their 5M-particle galaxy collision in time ([GASPHiA],
 * page header) without naming the integrator; these calls give the
 * kick-drift-kick leapfrog, with the tree rebuilt every step.  Velocities are
 * float4 rows (vx, vy, vz, unused), 16-byte aligned, in the order of the
 * positions. */

/* vel += acc_pot.xyz * dt_kick, then pos_mass.xyz += vel * dt_drift, per
 * particle (the mass in pos_mass.w is untouched).  A zero dt skips its half:
 * acc_pot may be NULL when dt_kick == 0, pos_mass when dt_drift == 0.  dt
 * values must be finite.  Asynchronous; no context needed. */
bh_status bh_kick_drift(float *pos_mass, float *vel, const float *acc_pot, int64_t n,
                        float dt_kick, float dt_drift, void *stream);

/* One leapfrog step of the n particles:
 *   vel += a dt/2; pos += vel dt; bh_build(pos); a = bh_gravity(self);
 *   vel += a dt/2.
 * acc_pot must hold the accelerations and potentials at the current positions
 * on entry (from bh_gravity or the previous step) and holds those at the new
 * positions on return.  n <= max_sources.  Asynchronous; device errors of the
 * build (non-finite positions) are reported by bh_sync as for bh_build. */
bh_status bh_leapfrog_step(bh_ctx *ctx, float *pos_mass, float *vel, float *acc_pot, int64_t n,
                           float dt, float theta, float G, float eps, void *stream);

/* Conserved quantities of the state, summed in fp64 in a fixed order
 * (deterministic), into out[10] (device): total mass, kinetic energy
 * sum m |v|^2 / 2, potential energy sum m phi / 2 (phi = acc_pot.w, each
 * particle's potential from all others, G included), momentum sum m v (3),
 * angular momentum sum m x cross v (3), and the particle count.  Uses the
 * context's scratch: calls on one context must not overlap.  Asynchronous. */
bh_status bh_diagnostics(bh_ctx *ctx, const float *pos_mass, const float *vel,
                         const float *acc_pot, int64_t n, double *out, void *stream);

/* For callers that cannot allocate device memory (code under HIP stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * self-gravity step, bh_build followed by bh_gravity with targets == NULL,
 * with no context.  Every scratch buffer (keys, sort buffers, the sorted
 * sources, the tree and its walk records) lives in one static device array
 * of the library, 64 MiB on each GPU the library runs on, held until the
 * process ends.  The tree's node capacity is the bound
 * bits * floor(n / (leaf_cap + 1)) + n + 1, which no input can exceed, so a
 * step fits when about 225 bytes per source (63-bit keys, leaf_cap 16; about
 * 825 with leaf_cap 1) fit the array: up to roughly 300000 sources at
 * leaf_cap 16, 81000 at leaf_cap 1.
 *   src_pos_mass  device, n float4 rows (x, y, z, m), 16-byte aligned.
 *   params        key_bits, leaf_cap and key_curve as for bh_create
 *                 (node_capacity and reserved must be 0); NULL = 63-bit
 *                 Morton keys, leaf_cap 16.
 *   out_acc_pot   device, n float4 rows (ax, ay, az, phi), caller order.
 *   theta, G, eps as for bh_gravity.
 * Results are bit-identical to bh_build + bh_gravity on a context with the
 * same parameters.  Errors: BH_ERR_INVALID (bad argument), BH_ERR_CAPACITY
 * (the step needs more than the static array holds: use a context), both
 * before anything is launched; BH_ERR_HIP.  Non-finite sources give NaN
 * outputs (there is no status word to read back).  The first call on a
 * device locates that device's array and copies 7 KB of key-curve tables
 * into it (synchronous; make it outside stream capture); later calls only
 * launch kernels on `stream`.  Calls on one device share its array, which
 * keeps the last call's contents: calls that overlap on one device race
 * (serialise them, e.g. on one stream).  Calls no hipMalloc or hipFree. */
bh_status bh_gravity_static(const float *src_pos_mass, int64_t n, const bh_build_params *params,
                            float theta, float G, float eps, float *out_acc_pot, void *stream);

/* Wait for the context's last stream and return the device status word
 * (BH_OK, BH_ERR_NONFINITE or BH_ERR_CAPACITY).  Synchronous. */
bh_status bh_sync(bh_ctx *ctx);

/* Free the context (synchronous).  NULL is accepted. */
bh_status bh_destroy(bh_ctx *ctx);

/* Static text for a status code. */
const char *bh_status_string(int status);

/* ---- introspection, used by the parity tests ---------------------------- */

/* Copy the Morton keys in sorted order and the sorted permutation (perm[i] =
 * the caller's index of the i-th sorted source) of the last build into
 * device buffers of n entries.  Either pointer may be NULL. */
bh_status bh_get_keys(bh_ctx *ctx, uint64_t *keys_sorted, uint32_t *perm, void *stream);

/* Number of nodes of the last build (synchronous: waits for the stream). */
bh_status bh_get_node_count(bh_ctx *ctx, int64_t *n_nodes, void *stream);

/* Copy the first n_nodes nodes (bh_node records) into a device buffer. */
bh_status bh_get_nodes(bh_ctx *ctx, bh_node *nodes, int64_t n_nodes, void *stream);

/* The tree of the last bh_build described cell by cell, in pre-order, as the
 * octree of [Tree] 构建树结构 defines its cells (synchronous for the count,
 * then asynchronous on `stream` for the arrays):
 *   *n_nodes  host: the number of nodes (0 for an empty build);
 *   level     device, n_nodes bytes: the cell's level (root = 0);
 *   prefix    device, n_nodes uint64: the cell's place on its level's grid,
 *             the top `level` bits of each quantised coordinate interleaved
 *             with x in bit 3k, y in 3k + 1, z in 3k + 2 (the octant
 *             numbering of [Tree] 构建树结构), for either key curve;
 *   count     device, n_nodes uint32: the number of sources in the cell.
 * Any of the three arrays may be NULL.  The caller sizes them from a first
 * call with all three NULL, or from bh_get_node_count.  Errors:
 * BH_ERR_NOT_BUILT (no build, or the build failed on the device). */
bh_status bh_get_cells(bh_ctx *ctx, int64_t *n_nodes, uint8_t *level, uint64_t *prefix,
                       uint32_t *count, void *stream);

/* Interaction counting for measurement ([GASPHiA] 性能瓶颈分析 counts one
 * interaction per node used whole and one per source of an opened leaf).
 * With counting enabled, every bh_gravity / bh_gravity_ex call made without a
 * caller's counter adds its interactions (accepted nodes plus particle pairs,
 * self excluded) to the context's own counter, cleared at the start of that
 * call; the walk is then slower.  bh_get_interactions waits for the stream of
 * the last such call and returns that call's total; BH_ERR_INVALID if the
 * context's last walk did not count. */
bh_status bh_set_counting(bh_ctx *ctx, int enable);
bh_status bh_get_interactions(bh_ctx *ctx, uint64_t *host_total);

/* Root cube of the last build (synchronous): lo[3] = min corner, hi[3] = max
 * corner of the sources, *L = the cube side (largest extent), all fp64. */
bh_status bh_get_bbox(bh_ctx *ctx, double *lo, double *hi, double *L, void *stream);

/* Per-phase device times of the last bh_build and bh_gravity in ms, when
 * enabled with bh_set_profiling (events add a little overhead).
 * ms[0] bbox + keys, ms[1] sort, ms[2] tree with centres of mass,
 * ms[3] walk (the last bh_gravity).  Up to n (<= 4) entries.  Synchronous. */
bh_status bh_set_profiling(bh_ctx *ctx, int enable);
bh_status bh_get_profile(bh_ctx *ctx, float *ms, int n);

/* How the last per-target walk (bh_gravity, bh_gravity_counted) shared its
 * groups of 64 targets among the eight XCDs (synchronous): *uneven = 1 when it
 * walked runs balanced on an earlier walk's times, and then starts[0..8] are
 * the first group of each XCD's run (starts[8] = the group count); *uneven = 0
 * when it walked the equal runs (starts then unspecified).  *split = the number
 * of groups it walked as four waves of 16 targets each (its heaviest, by an
 * earlier walk's times), 0 for none.  starts and split may be NULL.  For
 * measurement and tests; BH_ERR_INVALID if the context has not yet walked that
 * way. */
bh_status bh_get_walk_runs(bh_ctx *ctx, uint32_t *starts, int32_t *uneven, int32_t *split);

#ifdef __cplusplus
}
#endif
#endif /* BH_H */
