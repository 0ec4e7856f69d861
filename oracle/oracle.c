/*
 * Barnes-Hut oracle: a plain, slow, obviously-correct CPU implementation of
 * the octree self-gravity path, in IEEE fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library; the product path (the HIP
 * library under barnes_hut_tree_amd/) never does.  It shares no code, header,
 * table or helper with the HIP path.
 *
 * Pages followed (cited by title and section):
 *   [GASPHiA]  "GASPHiA中的自引力树代码效率与优化分析"
 *   [Tree]     "树结构（基于根据 Burtscher 和 Pingali 的研究）", including the
 *              embedded article "基于稠密存储的并行树构建实现方案"
 *   [SBH]      notes on "Stochastic Barnes-Hut Approximation for Fast
 *              Summation on the GPU"
 *
 * The steps are taken in the order the pages give them ([Tree] 实现步骤):
 * bounding box -> spatial key -> tree by recursive subdivision -> centre of
 * mass per cell ([GASPHiA] 计算节点质心) -> per-target walk with the opening
 * test ([GASPHiA] 性能瓶颈分析).  Readings taken where the pages are silent are
 * stated at each step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Data                                                                      */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t level;       /* 0 = root */
    int32_t is_leaf;
    int64_t corner[3];   /* integer corner on the level-l grid, in [0, 2^l) */
    int64_t off;         /* first member in the partitioned index array */
    int64_t count;       /* number of member particles */
    int64_t child[8];    /* cell index per key digit (the octant for Morton keys), -1 if empty */
    int32_t n_children;
    double mass;         /* M_c = sum of member masses */
    double com[3];       /* X_c = sum(m x) / M_c, or the cell centre if M_c = 0 */
} orc_cell;

typedef struct {
    int64_t n;
    int bits;            /* bits per axis: 21 (63-bit keys) or 10 (30-bit keys) */
    int leaf_cap;        /* B: a cell with more than B particles is split */
    int curve;           /* key order: 0 Morton (Z), 1 Hilbert */
    const float *src;    /* caller's float4 array (x, y, z, m), not owned */
    double lo[3], hi[3], L;
    uint64_t *q;         /* 3 integer coordinates per particle */
    uint64_t *keys;      /* Morton key per particle, input order */
    int64_t *perm;       /* stable argsort of keys */
    int64_t *idx;        /* particle indices partitioned cell by cell */
    orc_cell *cells;     /* pre-order: parent first, children by octant 0..7 */
    int64_t n_cells, cap_cells;
} orc_tree;

/* ------------------------------------------------------------------------ */
/* Step 1: bounding box.  [Tree] 确定粒子空间范围: the min and max of x, y, z  */
/* over all particles give the root's extent.  Reading: the root cube is     */
/* anchored at the min corner and its side is the largest extent, L.         */
/* ------------------------------------------------------------------------ */
static void step_bbox(orc_tree *t)
{
    for (int a = 0; a < 3; ++a) {
        t->lo[a] = INFINITY;
        t->hi[a] = -INFINITY;
    }
    for (int64_t i = 0; i < t->n; ++i) {
        for (int a = 0; a < 3; ++a) {
            double x = (double)t->src[4 * i + a];
            if (x < t->lo[a]) t->lo[a] = x;
            if (x > t->hi[a]) t->hi[a] = x;
        }
    }
    t->L = 0.0;
    if (t->n == 0) {
        for (int a = 0; a < 3; ++a) t->lo[a] = t->hi[a] = 0.0;
        return;
    }
    for (int a = 0; a < 3; ++a) {
        double ext = t->hi[a] - t->lo[a];
        if (ext > t->L) t->L = ext;
    }
}

/* ------------------------------------------------------------------------ */
/* Step 2: Morton key.  [Tree] 实现步骤 names Morton (Z-order) encoding for   */
/* the spatial sort.  Each axis is quantised to `bits` bits on the root cube  */
/* (scale S = 2^bits / L, fp64, one IEEE op per step), the top cell clamps,  */
/* and the bits are interleaved with x lowest: bit 3k <- x bit k,            */
/* 3k+1 <- y bit k, 3k+2 <- z bit k.  That order is the octant numbering of   */
/* [Tree] 构建树结构 (childIndex = 1 for the upper x half, +2 for y, +4 for z). */
/* ------------------------------------------------------------------------ */
/* Hilbert index of integer coordinates (x, y, z) of `bits` bits each, after
   Skilling, "Programming the Hilbert curve" (AIP Conf. Proc. 707, 2004): the
   coordinates are turned into the transposed index in place (undo excess
   work from the top bit down, then Gray-encode), and the transposed index is
   read out one bit level at a time, x bit first, so that each 3-bit digit
   names a child cell of the cell above it, in the curve's order. */
static uint64_t hilbert_key(uint64_t x, uint64_t y, uint64_t z, int bits)
{
    uint64_t X[3] = {x, y, z};
    const uint64_t M = (uint64_t)1 << (bits - 1);
    for (uint64_t Q = M; Q > 1; Q >>= 1) {
        const uint64_t P = Q - 1;
        for (int i = 0; i < 3; ++i) {
            if (X[i] & Q) {
                X[0] ^= P;
            } else {
                const uint64_t t = (X[0] ^ X[i]) & P;
                X[0] ^= t;
                X[i] ^= t;
            }
        }
    }
    for (int i = 1; i < 3; ++i) X[i] ^= X[i - 1];
    uint64_t t = 0;
    for (uint64_t Q = M; Q > 1; Q >>= 1)
        if (X[2] & Q) t ^= Q - 1;
    for (int i = 0; i < 3; ++i) X[i] ^= t;
    uint64_t key = 0;
    for (int b = bits - 1; b >= 0; --b)
        for (int i = 0; i < 3; ++i) key = (key << 1) | ((X[i] >> b) & 1u);
    return key;
}

static void step_keys(orc_tree *t)
{
    const uint64_t top = ((uint64_t)1 << t->bits) - 1;
    const double S = (t->L > 0.0) ? ldexp(1.0, t->bits) / t->L : 0.0;
    for (int64_t i = 0; i < t->n; ++i) {
        uint64_t key = 0;
        for (int a = 0; a < 3; ++a) {
            double d = (double)t->src[4 * i + a] - t->lo[a];
            double u = d * S;
            double f = floor(u);
            uint64_t qa = (f >= (double)top) ? top : (uint64_t)f;
            t->q[3 * i + a] = qa;
            for (int k = 0; k < t->bits; ++k)
                key |= ((qa >> k) & 1u) << (3 * k + a);
        }
        if (t->curve == 1)
            key = hilbert_key(t->q[3 * i], t->q[3 * i + 1], t->q[3 * i + 2], t->bits);
        t->keys[i] = key;
    }
}

/* ------------------------------------------------------------------------ */
/* Step 3: order.  [GASPHiA] 排序算法 sorts an index array (a gather index,   */
/* particle data stays put) into tree order; [Tree] 实现步骤 sorts by Morton  */
/* key.  Both give the same cell order; within equal keys the input index    */
/* decides (stable).                                                         */
/* ------------------------------------------------------------------------ */
static const uint64_t *g_sort_keys; /* qsort has no context argument */

static int cmp_by_key_then_index(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    uint64_t ka = g_sort_keys[a], kb = g_sort_keys[b];
    if (ka != kb) return ka < kb ? -1 : 1;
    return (a > b) - (a < b);
}

static void step_order(orc_tree *t)
{
    for (int64_t i = 0; i < t->n; ++i) t->perm[i] = i;
    g_sort_keys = t->keys;
    qsort(t->perm, (size_t)t->n, sizeof(int64_t), cmp_by_key_then_index);
}

/* ------------------------------------------------------------------------ */
/* Step 4: tree by recursive subdivision.  [Tree] 实现步骤 / 构建树结构: a     */
/* cell that holds too many particles is divided into its 8 octants, and     */
/* each leaf holds a few particles ("若干粒子") or has reached the smallest   */
/* division.  Readings: a cell with more than B particles is split unless it  */
/* is at the finest level (bits); membership of an octant is decided by the  */
/* integer coordinates, the upper half of each axis taking the set bit;      */
/* empty octants produce no cell; children are visited in the order of the   */
/* key digit that names them: octant order 0..7 for Morton keys, the curve's */
/* order for Hilbert keys (the same cells, in another order).                */
/* ------------------------------------------------------------------------ */
static int64_t new_cell(orc_tree *t)
{
    if (t->n_cells == t->cap_cells) {
        t->cap_cells = t->cap_cells ? 2 * t->cap_cells : 1024;
        t->cells = (orc_cell *)realloc(t->cells, (size_t)t->cap_cells * sizeof(orc_cell));
    }
    memset(&t->cells[t->n_cells], 0, sizeof(orc_cell));
    return t->n_cells++;
}

static int octant_of(const orc_tree *t, int64_t p, int child_level)
{
    /* The octant of the level-(child_level-1) cell that particle p falls in,
       read from bit (bits - child_level) of each integer coordinate. */
    int shift = t->bits - child_level;
    int ox = (int)((t->q[3 * p + 0] >> shift) & 1u);
    int oy = (int)((t->q[3 * p + 1] >> shift) & 1u);
    int oz = (int)((t->q[3 * p + 2] >> shift) & 1u);
    return ox + 2 * oy + 4 * oz;
}

/* the key digit naming the level-child_level cell that holds particle p */
static int digit_of(const orc_tree *t, int64_t p, int child_level)
{
    return (int)((t->keys[p] >> (3 * (t->bits - child_level))) & 7u);
}

static int64_t subdivide(orc_tree *t, int level, const int64_t corner[3],
                         int64_t off, int64_t count, int64_t *scratch)
{
    int64_t c = new_cell(t);
    t->cells[c].level = level;
    for (int a = 0; a < 3; ++a) t->cells[c].corner[a] = corner[a];
    t->cells[c].off = off;
    t->cells[c].count = count;
    for (int k = 0; k < 8; ++k) t->cells[c].child[k] = -1;

    if (count <= t->leaf_cap || level == t->bits) {
        t->cells[c].is_leaf = 1;
        return c;
    }

    /* Stable partition of the members by the key digit of their child cell
       (for Morton keys the digit is the octant). */
    int64_t digit_count[8] = {0};
    for (int64_t k = 0; k < count; ++k)
        digit_count[digit_of(t, t->idx[off + k], level + 1)]++;
    int64_t digit_off[8];
    digit_off[0] = 0;
    for (int o = 1; o < 8; ++o) digit_off[o] = digit_off[o - 1] + digit_count[o - 1];
    int64_t fill[8];
    memcpy(fill, digit_off, sizeof(fill));
    for (int64_t k = 0; k < count; ++k) {
        int64_t p = t->idx[off + k];
        scratch[fill[digit_of(t, p, level + 1)]++] = p;
    }
    memcpy(&t->idx[off], scratch, (size_t)count * sizeof(int64_t));

    for (int o = 0; o < 8; ++o) {
        if (digit_count[o] == 0) continue;
        /* the child's place on the level+1 grid, from its members' coordinates */
        const int oct = octant_of(t, t->idx[off + digit_off[o]], level + 1);
        int64_t child_corner[3];
        child_corner[0] = 2 * corner[0] + (oct & 1);
        child_corner[1] = 2 * corner[1] + ((oct >> 1) & 1);
        child_corner[2] = 2 * corner[2] + ((oct >> 2) & 1);
        int64_t ch = subdivide(t, level + 1, child_corner, off + digit_off[o],
                               digit_count[o], scratch);
        /* t->cells may have moved during the recursion: index, not pointer. */
        t->cells[c].child[o] = ch;
        t->cells[c].n_children++;
    }
    return c;
}

static void step_tree(orc_tree *t)
{
    for (int64_t i = 0; i < t->n; ++i) t->idx[i] = i;
    if (t->n == 0) return;
    int64_t *scratch = (int64_t *)malloc((size_t)t->n * sizeof(int64_t));
    int64_t root_corner[3] = {0, 0, 0};
    subdivide(t, 0, root_corner, 0, t->n, scratch);
    free(scratch);
}

/* ------------------------------------------------------------------------ */
/* Step 5: centre of mass.  [GASPHiA] 计算节点质心 and the tree-code idea of  */
/* the same page (a far cluster acts as one point mass at its centre of      */
/* mass): M_c = sum m, X_c = sum(m x) / M_c over the cell's members.          */
/* Reading: a massless cell takes its geometric centre.                      */
/* ------------------------------------------------------------------------ */
static void step_com(orc_tree *t)
{
    for (int64_t c = 0; c < t->n_cells; ++c) {
        orc_cell *cell = &t->cells[c];
        double m = 0.0, s[3] = {0.0, 0.0, 0.0};
        for (int64_t k = 0; k < cell->count; ++k) {
            int64_t p = t->idx[cell->off + k];
            double mp = (double)t->src[4 * p + 3];
            m += mp;
            for (int a = 0; a < 3; ++a) s[a] += mp * (double)t->src[4 * p + a];
        }
        cell->mass = m;
        for (int a = 0; a < 3; ++a) {
            if (m != 0.0) {
                cell->com[a] = s[a] / m;
            } else {
                double w = ldexp(t->L, -cell->level);
                cell->com[a] = t->lo[a] + w * ((double)cell->corner[a] + 0.5);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Public: build                                                             */
/* ------------------------------------------------------------------------ */
orc_tree *orc_build_curve(const float *pos_mass, int64_t n, int key_bits, int leaf_cap,
                          int curve)
{
    if (n < 0 || leaf_cap < 1 || (key_bits != 30 && key_bits != 63) || (curve != 0 && curve != 1))
        return NULL;
    orc_tree *t = (orc_tree *)calloc(1, sizeof(orc_tree));
    t->n = n;
    t->curve = curve;
    t->bits = key_bits / 3;
    t->leaf_cap = leaf_cap;
    t->src = pos_mass;
    size_t nn = (size_t)(n > 0 ? n : 1);
    t->q = (uint64_t *)malloc(3 * nn * sizeof(uint64_t));
    t->keys = (uint64_t *)malloc(nn * sizeof(uint64_t));
    t->perm = (int64_t *)malloc(nn * sizeof(int64_t));
    t->idx = (int64_t *)malloc(nn * sizeof(int64_t));
    step_bbox(t);
    step_keys(t);
    step_order(t);
    step_tree(t);
    step_com(t);
    return t;
}

orc_tree *orc_build(const float *pos_mass, int64_t n, int key_bits, int leaf_cap)
{
    return orc_build_curve(pos_mass, n, key_bits, leaf_cap, 0);
}

void orc_free(orc_tree *t)
{
    if (!t) return;
    free(t->q);
    free(t->keys);
    free(t->perm);
    free(t->idx);
    free(t->cells);
    free(t);
}

void orc_bbox(const orc_tree *t, double *lo3, double *hi3, double *L)
{
    for (int a = 0; a < 3; ++a) {
        lo3[a] = t->lo[a];
        hi3[a] = t->hi[a];
    }
    *L = t->L;
}

void orc_keys(const orc_tree *t, uint64_t *keys) { memcpy(keys, t->keys, (size_t)t->n * sizeof(uint64_t)); }
void orc_perm(const orc_tree *t, int64_t *perm) { memcpy(perm, t->perm, (size_t)t->n * sizeof(int64_t)); }
int64_t orc_ncells(const orc_tree *t) { return t->n_cells; }

/* Per cell, in pre-order: level, leaf flag, key prefix (the top 3*level key
   bits, from the integer corner), start (= offset in sorted order), count,
   number of children, mass and centre of mass. */
void orc_cells(const orc_tree *t, int32_t *level, int32_t *is_leaf, uint64_t *prefix,
               int64_t *start, int64_t *count, int32_t *n_children, double *mass, double *com)
{
    for (int64_t c = 0; c < t->n_cells; ++c) {
        const orc_cell *cell = &t->cells[c];
        uint64_t pre = 0;
        for (int a = 0; a < 3; ++a)
            for (int k = 0; k < cell->level; ++k)
                pre |= (((uint64_t)cell->corner[a] >> k) & 1u) << (3 * k + a);
        if (level) level[c] = cell->level;
        if (is_leaf) is_leaf[c] = cell->is_leaf;
        if (prefix) prefix[c] = pre;
        if (start) start[c] = cell->off;
        if (count) count[c] = cell->count;
        if (n_children) n_children[c] = cell->n_children;
        if (mass) mass[c] = cell->mass;
        if (com)
            for (int a = 0; a < 3; ++a) com[3 * c + a] = cell->com[a];
    }
}

/* ------------------------------------------------------------------------ */
/* Step 6: walk.  [GASPHiA] 性能瓶颈分析 gives the opening test of the        */
/* gravity kernel: a node is used whole when w_sq / theta_sq < r_sq, and a    */
/* particle child is always used directly.  Readings: w is the full cell     */
/* edge L / 2^level; r is the unsoftened distance from the target to the     */
/* cell's centre of mass; the test is strict; the root is tested too and no  */
/* cell is excluded for containing the target.  A leaf that is opened is     */
/* summed particle by particle, skipping the target itself.                  */
/*                                                                           */
/* Interaction (Plummer softening eps, reading for the softened kernel):     */
/*   d = X_src - x, r2 = |d|^2 + eps^2, a += G m d / r2^(3/2),               */
/*   phi -= G m / r2^(1/2); a pair with r2 == 0 contributes nothing.          */
/* ------------------------------------------------------------------------ */
typedef struct {
    const orc_tree *t;
    double x[3];
    int64_t self;        /* source index of the target, or -1 */
    double theta_sq, G, eps_sq;
    int tie_mode;        /* 0: as computed, 1: near-ties opened, 2: near-ties accepted */
    double acc[3], phi;
    int64_t n_inter, n_ties;
} walker;

static void interact(walker *w, double m, const double *xs)
{
    double d[3], r2 = w->eps_sq;
    for (int a = 0; a < 3; ++a) {
        d[a] = xs[a] - w->x[a];
        r2 += d[a] * d[a];
    }
    if (r2 == 0.0) return;
    double inv_r = 1.0 / sqrt(r2);
    double inv_r3 = inv_r * inv_r * inv_r;
    for (int a = 0; a < 3; ++a) w->acc[a] += w->G * m * d[a] * inv_r3;
    w->phi -= w->G * m * inv_r;
}

static void walk(walker *w, int64_t c)
{
    const orc_tree *t = w->t;
    const orc_cell *cell = &t->cells[c];
    double r_sq = 0.0;
    for (int a = 0; a < 3; ++a) {
        double d = cell->com[a] - w->x[a];
        r_sq += d * d;
    }
    double width = ldexp(t->L, -cell->level);
    double w_sq = width * width;
    double threshold = w_sq / w->theta_sq;
    int accept = threshold < r_sq;
    /* near-tie: within 2^-20 of the threshold on the softened scale
       (r_sq + eps_sq against threshold + eps_sq, the scale on which an fp32
       walk may evaluate the same test) */
    if (isfinite(threshold) &&
        fabs(r_sq - threshold) <= ldexp(threshold + w->eps_sq, -20)) {
        w->n_ties++;
        if (w->tie_mode == 1) accept = 0;
        if (w->tie_mode == 2) accept = 1;
    }
    if (accept) {
        interact(w, cell->mass, cell->com);
        w->n_inter++;
        return;
    }
    if (!cell->is_leaf) {
        for (int o = 0; o < 8; ++o)
            if (cell->child[o] >= 0) walk(w, cell->child[o]);
        return;
    }
    for (int64_t k = 0; k < cell->count; ++k) {
        int64_t p = t->idx[cell->off + k];
        if (p == w->self) continue;
        double xs[3] = {(double)t->src[4 * p + 0], (double)t->src[4 * p + 1],
                        (double)t->src[4 * p + 2]};
        interact(w, (double)t->src[4 * p + 3], xs);
        w->n_inter++;
    }
}

/* targets == NULL: the targets are the sources themselves (self excluded);
   which[k] (or k when which == NULL) names the k-th target.  out holds
   (ax, ay, az, phi) per target; n_inter and n_ties are per target and may be
   NULL. */
void orc_bh(const orc_tree *t, const float *targets, const int64_t *which, int64_t nt,
            double theta, double G, double eps, int tie_mode, double *out,
            int64_t *n_inter, int64_t *n_ties)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t k = 0; k < nt; ++k) {
        int64_t i = which ? which[k] : k;
        const float *p = targets ? &targets[4 * i] : &t->src[4 * i];
        walker w;
        memset(&w, 0, sizeof(w));
        w.t = t;
        for (int a = 0; a < 3; ++a) w.x[a] = (double)p[a];
        w.self = targets ? -1 : i;
        w.theta_sq = theta * theta;
        w.G = G;
        w.eps_sq = eps * eps;
        w.tie_mode = tie_mode;
        if (t->n_cells > 0) walk(&w, 0);
        out[4 * k + 0] = w.acc[0];
        out[4 * k + 1] = w.acc[1];
        out[4 * k + 2] = w.acc[2];
        out[4 * k + 3] = w.phi;
        if (n_inter) n_inter[k] = w.n_inter;
        if (n_ties) n_ties[k] = w.n_ties;
    }
}

/* ------------------------------------------------------------------------ */
/* The warp vote of [GASPHiA] 性能瓶颈分析: the threads of one warp walk the   */
/* tree together, and when the opening test fails for any of them, all of    */
/* them descend.  Here a group is `group` consecutive targets in the order    */
/* of the stable Morton-key sort (not the tree's partition order, which      */
/* keeps input order inside a leaf); the targets are the sources, self       */
/* excluded.  At a cell, each member applies the test of walk(); if no       */
/* member fails, every member uses the cell whole; otherwise every member    */
/* uses its children, or, for a leaf, its particles.  A member therefore     */
/* never uses a cell that the per-particle walk would open, and may use the  */
/* children of one it would accept.  Near-ties (as in walk()) are counted    */
/* for every member of the group.                                            */
/* ------------------------------------------------------------------------ */
typedef struct {
    const orc_tree *t;
    int64_t m;               /* members */
    walker *w;               /* one walker (position, self, sums) per member */
    int *accept;             /* scratch, per member */
} group_walker;

static void walk_group(group_walker *g, int64_t c)
{
    const orc_tree *t = g->t;
    const orc_cell *cell = &t->cells[c];
    const double width = ldexp(t->L, -cell->level);
    const double threshold = width * width / g->w[0].theta_sq;
    int any_open = 0, tie = 0;
    for (int64_t k = 0; k < g->m; ++k) {
        walker *w = &g->w[k];
        double r_sq = 0.0;
        for (int a = 0; a < 3; ++a) {
            double d = cell->com[a] - w->x[a];
            r_sq += d * d;
        }
        int accept = threshold < r_sq;
        if (isfinite(threshold) && fabs(r_sq - threshold) <= ldexp(threshold, -20)) {
            tie = 1;
            if (w->tie_mode == 1) accept = 0;
            if (w->tie_mode == 2) accept = 1;
        }
        g->accept[k] = accept;
        if (!accept) any_open = 1;
    }
    if (tie)
        for (int64_t k = 0; k < g->m; ++k) g->w[k].n_ties++;
    if (!any_open) {
        for (int64_t k = 0; k < g->m; ++k) {
            interact(&g->w[k], cell->mass, cell->com);
            g->w[k].n_inter++;
        }
        return;
    }
    if (!cell->is_leaf) {
        for (int o = 0; o < 8; ++o)
            if (cell->child[o] >= 0) walk_group(g, cell->child[o]);
        return;
    }
    for (int64_t k = 0; k < g->m; ++k) {
        walker *w = &g->w[k];
        for (int64_t q = 0; q < cell->count; ++q) {
            int64_t p = t->idx[cell->off + q];
            if (p == w->self) continue;
            double xs[3] = {(double)t->src[4 * p + 0], (double)t->src[4 * p + 1],
                            (double)t->src[4 * p + 2]};
            interact(w, (double)t->src[4 * p + 3], xs);
            w->n_inter++;
        }
    }
}

/* Self-gravity by the warp vote, groups of `group` >= 1 consecutive sorted
   sources.  groups[k] (or k when groups == NULL) names the k-th group to
   evaluate, n_groups of them; out (n x 4, the caller's order of the sources)
   and the per-source n_inter / n_ties (may be NULL) are written for the
   members of those groups only. */
int orc_bh_vote(const orc_tree *t, int64_t group, const int64_t *groups, int64_t n_groups,
                double theta, double G, double eps, int tie_mode, double *out,
                int64_t *n_inter, int64_t *n_ties)
{
    if (group < 1 || n_groups < 0) return -1;
    const int64_t total = (t->n + group - 1) / group;
    if (!groups) n_groups = total;
    for (int64_t k = 0; k < n_groups; ++k)
        if (groups && (groups[k] < 0 || groups[k] >= total)) return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : failed)
    for (int64_t k = 0; k < n_groups; ++k) {
        const int64_t gi = groups ? groups[k] : k;
        const int64_t first = gi * group;
        const int64_t m = (t->n - first < group) ? t->n - first : group;
        group_walker g;
        g.t = t;
        g.m = m;
        g.w = (walker *)calloc((size_t)m, sizeof(walker));
        g.accept = (int *)calloc((size_t)m, sizeof(int));
        if (!g.w || !g.accept) {
            free(g.w);
            free(g.accept);
            failed = 1;
            continue;
        }
        for (int64_t q = 0; q < m; ++q) {
            walker *w = &g.w[q];
            const int64_t i = t->perm[first + q];
            w->t = t;
            for (int a = 0; a < 3; ++a) w->x[a] = (double)t->src[4 * i + a];
            w->self = i;
            w->theta_sq = theta * theta;
            w->G = G;
            w->eps_sq = eps * eps;
            w->tie_mode = tie_mode;
        }
        if (t->n_cells > 0) walk_group(&g, 0);
        for (int64_t q = 0; q < m; ++q) {
            const walker *w = &g.w[q];
            const int64_t i = w->self;
            for (int a = 0; a < 3; ++a) out[4 * i + a] = w->acc[a];
            out[4 * i + 3] = w->phi;
            if (n_inter) n_inter[i] = w->n_inter;
            if (n_ties) n_ties[i] = w->n_ties;
        }
        free(g.w);
        free(g.accept);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and    */
/* Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): ten rounds; */
/* each multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 (full  */
/* 64-bit products), xors the high halves with words 1 and 3 and the key,    */
/* and the key is bumped by 0x9E3779B9 and 0xBB67AE85 after every round.     */
/* ------------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out)
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* Separate query points are ordered by their Morton keys on the sources'   */
/* root cube (the quantisation of step 2, clamped to the cube on both sides) */
/* and stably sorted; consecutive runs of that order form the groups that    */
/* share random numbers below.                                               */
int orc_target_order(const orc_tree *t, const float *targets, int64_t nt, int64_t *order)
{
    uint64_t *keys = (uint64_t *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(uint64_t));
    if (!keys) return -2;
    const uint64_t top = ((uint64_t)1 << t->bits) - 1;
    const double S = (t->L > 0.0) ? ldexp(1.0, t->bits) / t->L : 0.0;
    for (int64_t i = 0; i < nt; ++i) {
        uint64_t key = 0, qq[3];
        for (int a = 0; a < 3; ++a) {
            double f = floor(((double)targets[4 * i + a] - t->lo[a]) * S);
            uint64_t qa = !(f >= 0.0) ? 0 : (f >= (double)top) ? top : (uint64_t)f;
            for (int k = 0; k < t->bits; ++k) key |= ((qa >> k) & 1u) << (3 * k + a);
            qq[a] = qa;
        }
        keys[i] = (t->curve == 1) ? hilbert_key(qq[0], qq[1], qq[2], t->bits) : key;
        order[i] = i;
    }
    g_sort_keys = keys;
    qsort(order, (size_t)nt, sizeof(int64_t), cmp_by_key_then_index);
    free(keys);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stochastic Barnes-Hut ([SBH] 方法, 关键设计).  Each source's contribution  */
/* is written as a telescoping sum along its root-to-leaf path, every step   */
/* replacing a cell's monopole by its children's.  A sample picks a path     */
/* index I uniformly among the sources and a path length by Russian roulette */
/* (continuing from depth k with probability                                 */
/* p_k = min(1, max(1, b_k) / b_{k+1}), b = |q - centre of mass| / box edge), */
/* and adds for each step taken the exchange term                            */
/*   Delta_T = sum over children c of m_c f(c, q) - m_T f(T, q)              */
/* divided by P(I in T) * P(K >= k).  Strata: the children of the root, one  */
/* path per stratum with I uniform over its sources, plus each stratum's     */
/* monopole.  Readings: the tree is the octree with single-source leaves     */
/* (B = 1; a leaf of coincident sources at the finest level has Delta = 0    */
/* and ends the path); branching d = 2 per axis steps one octree level, d = 4 */
/* two (a child that is a leaf stands for itself); the random numbers are    */
/* shared by a group of consecutive targets (the same seed across a warp),   */
/* drawn from Philox4x32-10 with key = seed and counter = (group, sample,    */
/* stratum, j), j = 0 for the path index and j = k + 1 for the roulette at   */
/* depth k; I = start + floor(r * count / 2^32) on the first output word r,  */
/* u = (r >> 8) 2^-24.  S samples are averaged.                              */
/* ------------------------------------------------------------------------ */
static int64_t dchildren(const orc_tree *t, int64_t c, int d, int64_t *out)
{
    const orc_cell *cell = &t->cells[c];
    int64_t n = 0;
    for (int o = 0; o < 8; ++o) {
        const int64_t ch = cell->child[o];
        if (ch < 0) continue;
        if (d == 2 || t->cells[ch].is_leaf) {
            out[n++] = ch;
            continue;
        }
        for (int o2 = 0; o2 < 8; ++o2)
            if (t->cells[ch].child[o2] >= 0) out[n++] = t->cells[ch].child[o2];
    }
    return n;
}

static void kernel_f(const double *q, double m, const double *p, double eps_sq, double *f)
{
    double d[3], r2 = eps_sq;
    for (int a = 0; a < 3; ++a) {
        d[a] = p[a] - q[a];
        r2 += d[a] * d[a];
    }
    if (r2 == 0.0) {
        f[0] = f[1] = f[2] = f[3] = 0.0;
        return;
    }
    const double inv = 1.0 / sqrt(r2);
    for (int a = 0; a < 3; ++a) f[a] = m * d[a] * inv * inv * inv;
    f[3] = -m * inv;
}

static double far_ratio(const orc_tree *t, const orc_cell *c, const double *q)
{
    double r2 = 0.0;
    for (int a = 0; a < 3; ++a) {
        double d = q[a] - c->com[a];
        r2 += d * d;
    }
    return sqrt(r2) / ldexp(t->L, -c->level);
}

int orc_sbh(const orc_tree *t, const float *targets, const int64_t *which, int64_t nt,
            const int64_t *group, int d, int samples, uint64_t seed, double G, double eps,
            double *out, double *pot_sq, int64_t *n_near)
{
    if ((d != 2 && d != 4) || samples < 1) return -1;
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const double eps_sq = eps * eps;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nt; ++k) {
        const int64_t i = which ? which[k] : k;
        const double q[3] = {(double)targets[4 * i], (double)targets[4 * i + 1],
                             (double)targets[4 * i + 2]};
        double sum[4] = {0.0, 0.0, 0.0, 0.0}, sq = 0.0, f[4];
        int64_t near = 0;
        int64_t strata[64], kids[64];
        int64_t n_strata = 0;
        if (t->n_cells > 0 && !t->cells[0].is_leaf) n_strata = dchildren(t, 0, d, strata);
        for (int s = 0; s < samples; ++s) {
            double est[4] = {0.0, 0.0, 0.0, 0.0};
            if (t->n_cells > 0 && t->cells[0].is_leaf) {   /* one leaf: the exact sum */
                const orc_cell *leaf = &t->cells[0];
                for (int64_t j = 0; j < leaf->count; ++j) {
                    const int64_t p = t->idx[leaf->off + j];
                    const double xs[3] = {t->src[4 * p], t->src[4 * p + 1], t->src[4 * p + 2]};
                    kernel_f(q, (double)t->src[4 * p + 3], xs, eps_sq, f);
                    for (int a = 0; a < 4; ++a) est[a] += f[a];
                }
            }
            for (int64_t ci = 0; ci < n_strata; ++ci) {
                const orc_cell *c = &t->cells[strata[ci]];
                kernel_f(q, c->mass, c->com, eps_sq, f);
                for (int a = 0; a < 4; ++a) est[a] += f[a];
                if (c->is_leaf) continue;
                uint32_t ctr[4] = {(uint32_t)group[k], (uint32_t)s, (uint32_t)ci, 0u}, r[4];
                orc_philox4x32_10(ctr, key, r);
                const int64_t I = c->off + (int64_t)(((uint64_t)r[0] * (uint64_t)c->count) >> 32);
                int64_t T = strata[ci];
                double w = 1.0;
                for (uint32_t depth = 0; !t->cells[T].is_leaf; ++depth) {
                    const orc_cell *cell = &t->cells[T];
                    const int64_t nk = dchildren(t, T, d, kids);
                    int64_t next = -1;
                    for (int64_t j = 0; j < nk; ++j) {
                        const orc_cell *ch = &t->cells[kids[j]];
                        if (I >= ch->off && I < ch->off + ch->count) next = kids[j];
                    }
                    const double b0 = far_ratio(t, cell, q);
                    const double b1 = far_ratio(t, &t->cells[next], q);
                    const double pk = (b1 > 0.0) ? fmin(1.0, fmax(1.0, b0) / b1) : 1.0;
                    ctr[3] = depth + 1;
                    orc_philox4x32_10(ctr, key, r);
                    const double u = ldexp((double)(r[0] >> 8), -24);
                    if (fabs(u - pk) <= 1e-5) near++;
                    if (!(u < pk)) break;
                    w /= pk;
                    const double scale = w * (double)c->count / (double)cell->count;
                    for (int64_t j = 0; j < nk; ++j) {
                        const orc_cell *ch = &t->cells[kids[j]];
                        kernel_f(q, ch->mass, ch->com, eps_sq, f);
                        for (int a = 0; a < 4; ++a) est[a] += scale * f[a];
                    }
                    kernel_f(q, cell->mass, cell->com, eps_sq, f);
                    for (int a = 0; a < 4; ++a) est[a] -= scale * f[a];
                    T = next;
                }
            }
            for (int a = 0; a < 4; ++a) sum[a] += est[a];
            sq += est[3] * est[3];
        }
        for (int a = 0; a < 4; ++a) out[4 * k + a] = G * sum[a] / samples;
        if (pot_sq) pot_sq[k] = G * G * sq / samples;
        if (n_near) n_near[k] = near;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Direct sum, the plain definition the tree approximates ([GASPHiA]          */
/* 如何计算自引力: every pair of particles attracts; O(N^2)):                   */
/*   a_i = G sum_{j != i} m_j d_ij / (|d_ij|^2 + eps^2)^(3/2),                */
/*   phi_i = -G sum_{j != i} m_j / (|d_ij|^2 + eps^2)^(1/2).                  */
/* ------------------------------------------------------------------------ */
void orc_direct(const float *src, int64_t n, const float *targets, const int64_t *which,
                int64_t nt, double G, double eps, double *out)
{
    const double eps_sq = eps * eps;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nt; ++k) {
        int64_t i = which ? which[k] : k;
        const float *p = targets ? &targets[4 * i] : &src[4 * i];
        int64_t self = targets ? -1 : i;
        double x[3] = {(double)p[0], (double)p[1], (double)p[2]};
        double acc[3] = {0.0, 0.0, 0.0}, phi = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            if (j == self) continue;
            double d[3], r2 = eps_sq;
            for (int a = 0; a < 3; ++a) {
                d[a] = (double)src[4 * j + a] - x[a];
                r2 += d[a] * d[a];
            }
            if (r2 == 0.0) continue;
            double m = (double)src[4 * j + 3];
            double inv_r = 1.0 / sqrt(r2);
            double inv_r3 = inv_r * inv_r * inv_r;
            for (int a = 0; a < 3; ++a) acc[a] += G * m * d[a] * inv_r3;
            phi -= G * m * inv_r;
        }
        out[4 * k + 0] = acc[0];
        out[4 * k + 1] = acc[1];
        out[4 * k + 2] = acc[2];
        out[4 * k + 3] = phi;
    }
}

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
