// Octree from Morton-sorted keys, and the bottom-up centre-of-mass pass.
//
// The pages build the tree top-down by inserting particles one at a time
// under atomic child-slot locks ([Tree] 构建树结构 / 基于稠密存储的并行树构建实现方案,
// [GASPHiA] 自顶向下建立树).  The cells such a build produces are determined by
// the particle set alone: a cell of level l is a run of sorted keys sharing
// their top 3l bits, and it is split when it holds more than B particles
// and l is above the deepest level.  This file derives every node of that
// tree in parallel from the sorted keys, with no locks and no atomics on
// tree slots, and stores it in pre-order (a subtree is a contiguous index
// range [node, skip)), the node order used by the walk.
//
// For sorted position a, let d(a) be the number of leading octal digits that
// keys a-1 and a share (d(0) = -1).  The level-l cell containing a starts at a
// exactly when d(a) < l.  A leaf starts at a iff the level-d(a) cell holding a
// has more than B particles; the leaf's level is then
//     ell(a) = min(bits, 1 + max(d(a), min_{1<=t<=B} d(a+t)))
// (the smallest level whose cell starting at a holds at most B particles),
// and the nodes starting at a are the cells of levels d(a)+1 .. ell(a): c(a)
// of them, ancestors first.  So the pre-order index of node (a, l) is
// sum_{a'<a} c(a') + l - d(a) - 1, one prefix sum over positions.
//
// Kernels: count (d, c, per-tile totals per column) -> a scan of each column
// over the tiles -> emit (node start/level, level lists, index of
// the first node at each position) -> ranges (cell end by galloping search,
// skip = first node at the end, leaf centres of mass).  The centre of mass of
// internal nodes ([GASPHiA] 计算节点质心) is then combined level by level from
// the deepest level up, each node summing its children.
#include "bh_internal.h"

namespace bh {
namespace {

__device__ inline int lcp_digits(uint64_t k1, uint64_t k2, int bits)
{
    const uint64_t x = k1 ^ k2;
    if (x == 0) return bits;
    const int h = 63 - __clzll((long long)x);
    return (3 * bits - 1 - h) / 3;
}

// d(j) over [0, n]; outside (1..n-1) it is -1 (a boundary at every level).
__device__ inline int d_at(const uint64_t *keys, int64_t j, uint32_t n, int bits)
{
    if (j <= 0 || j >= (int64_t)n) return -1;
    return lcp_digits(keys[j - 1], keys[j], bits);
}

__global__ __launch_bounds__(kBuildThreads) void k_count(const uint64_t *__restrict__ keys,
                                                         uint32_t n, int bits, int B,
                                                         uint16_t *__restrict__ dc,
                                                         uint32_t *__restrict__ block_counts,
                                                         uint32_t n_tiles)
{
    __shared__ int8_t sd[kBuildTile + 2 * kMaxLeafCap + 2];
    __shared__ uint32_t lc[kBuildCols];
    const int64_t t0 = (int64_t)blockIdx.x * kBuildTile;
    const int64_t w0 = t0 - B;   // window covers positions [t0 - B, t0 + tile + B]
    const int wlen = kBuildTile + 2 * B + 1;
    for (int k = threadIdx.x; k < wlen; k += kBuildThreads)
        sd[k] = (int8_t)d_at(keys, w0 + k, n, bits);
    if (threadIdx.x < kBuildCols) lc[threadIdx.x] = 0;
    __syncthreads();

    for (int k = 0; k < kBuildTile / kBuildThreads; ++k) {
        const int off = k * kBuildThreads + threadIdx.x;
        const int64_t a = t0 + off;
        if (a >= (int64_t)n) break;
        const int ia = off + B;  // index of a in the window
        const int da = sd[ia];
        int c = 0;
        bool leaf_start;
        if (a == 0) {
            leaf_start = true;
        } else if (da >= bits) {
            leaf_start = false;
        } else {
            // size of the level-d(a) cell around a, capped above B
            int cnt = 1;
            for (int t = 0; t < B && cnt <= B; ++t) {
                if (sd[ia - t] >= da) ++cnt; else break;
            }
            for (int t = 1; t <= B && cnt <= B; ++t) {
                if (sd[ia + t] >= da) ++cnt; else break;
            }
            leaf_start = cnt > B;
        }
        if (leaf_start) {
            int rm = bits;
            for (int t = 1; t <= B; ++t) rm = min(rm, (int)sd[ia + t]);
            const int ell = min(bits, 1 + max(da, rm));
            c = ell - da;
            for (int l = da + 1; l <= ell; ++l) atomicAdd(&lc[1 + l], 1u);
            atomicAdd(&lc[0], (uint32_t)c);
        }
        dc[a] = (uint16_t)((da + 1) | (c << 8));
    }
    __syncthreads();
    if (threadIdx.x < kBuildCols) block_counts[threadIdx.x * n_tiles + blockIdx.x] = lc[threadIdx.x];
}

__device__ inline uint32_t wave_incl_scan(uint32_t v)
{
    const uint32_t lane = threadIdx.x & 63;
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(v, o, 64);
        if (lane >= (uint32_t)o) v += t;
    }
    return v;
}

// pref[c][t] / tot[c]: per-column scan over tiles of the k_count table
// (column 0: nodes, column 1 + l: nodes of level l).
__global__ __launch_bounds__(kBuildThreads) void k_emit(const uint16_t *__restrict__ dc, uint32_t n,
                                                        const uint32_t *__restrict__ pref,
                                                        const uint32_t *__restrict__ tot,
                                                        uint32_t n_tiles, uint64_t cap,
                                                        uint32_t *__restrict__ first_node,
                                                        uint32_t *__restrict__ level_list,
                                                        Node *__restrict__ nodes,
                                                        DevParams *__restrict__ prm)
{
    constexpr int per = kBuildTile / kBuildThreads;  // consecutive positions per thread
    __shared__ uint32_t wtot[kBuildThreads / 64];
    __shared__ uint32_t lrank[kBuildCols];
    __shared__ uint32_t lbase[kBuildCols];   // this tile's first slot in each level list
    const uint32_t blk = blockIdx.x;
    const uint32_t total = tot[0];           // all nodes
    if (threadIdx.x < kBuildCols) lrank[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        uint32_t off = 0;
        for (int l = 0; l < kMaxLevels; ++l) {
            lbase[1 + l] = off + pref[(1 + l) * n_tiles + blk];
            off += tot[1 + l];
        }
    }

    const int64_t a0 = (int64_t)blk * kBuildTile + per * threadIdx.x;
    int dd[per], cc[per];
    uint32_t s = 0;
    for (int k = 0; k < per; ++k) {
        const int64_t a = a0 + k;
        uint16_t v = a < (int64_t)n ? dc[a] : (uint16_t)0;
        dd[k] = (int)(v & 0xffu) - 1;
        cc[k] = v >> 8;
        s += cc[k];
    }
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(s);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t run = pref[blk];
    for (uint32_t w = 0; w < wave; ++w) run += wtot[w];
    run += incl - s;

    for (int k = 0; k < per; ++k) {
        const int64_t a = a0 + k;
        if (a >= (int64_t)n) break;
        first_node[a] = run;
        for (int j = 0; j < cc[k]; ++j) {
            const int l = dd[k] + 1 + j;
            const uint32_t X = run + j;
            const uint32_t r = atomicAdd(&lrank[1 + l], 1u);
            const uint32_t pos = lbase[1 + l] + r;
            if (X < cap) {
                nodes[X].start = (uint32_t)a;
                nodes[X].meta = (uint32_t)l | (j == cc[k] - 1 ? kLeafBit : 0u);
            }
            if (pos < cap) level_list[pos] = X;
        }
        run += cc[k];
    }
    if (blk == n_tiles - 1 && threadIdx.x == 0) first_node[n] = total;
    if (blk == 0 && threadIdx.x == 0) {
        prm->n_nodes = total;
        if (total > cap) prm->status |= kStatusCapacity;
        uint32_t off = 0;
        for (int l = 0; l < kMaxLevels; ++l) {
            prm->level_offset[l] = off;
            prm->level_count[l] = tot[1 + l];
            off += tot[1 + l];
        }
        prm->level_offset[kMaxLevels] = off;
    }
}

// Integer coordinate of axis `axis` from a Morton key (inverse interleave).
__device__ inline uint32_t compact3(uint64_t k)
{
    k &= 0x1249249249249249ull;
    k = (k ^ (k >> 2)) & 0x10c30c30c30c30c3ull;
    k = (k ^ (k >> 4)) & 0x100f00f00f00f00full;
    k = (k ^ (k >> 8)) & 0x001f0000ff0000ffull;
    k = (k ^ (k >> 16)) & 0x001f00000000ffffull;
    k = (k ^ (k >> 32)) & 0x00000000001fffffull;
    return (uint32_t)k;
}

// Geometric centre of the level-l cell holding `key` (for massless cells).
__device__ inline float3 cell_centre(uint64_t key, int level, int bits, const DevParams *prm)
{
    float c[3];
    for (int a = 0; a < 3; ++a) {
        const uint32_t corner = compact3(key >> a) >> (bits - level);
        const double w = __builtin_ldexp(prm->L, -level);
        c[a] = (float)(prm->lo[a] + w * ((double)corner + 0.5));
    }
    return make_float3(c[0], c[1], c[2]);
}

__global__ __launch_bounds__(256) void k_ranges(const uint64_t *__restrict__ keys,
                                                const float4 *__restrict__ spos, uint32_t n,
                                                int bits, uint64_t cap,
                                                const uint32_t *__restrict__ first_node,
                                                Node *__restrict__ nodes,
                                                const DevParams *__restrict__ prm)
{
    const uint32_t nn = (uint32_t)min((uint64_t)prm->n_nodes, cap);
    for (uint32_t X = blockIdx.x * blockDim.x + threadIdx.x; X < nn; X += gridDim.x * blockDim.x) {
        const uint32_t a = nodes[X].start;
        const uint32_t meta = nodes[X].meta;
        const int l = (int)node_level(meta);
        const int shift = 3 * (bits - l);
        const uint64_t p = keys[a] >> shift;
        // galloping search for the first sorted position past the cell
        uint32_t lo = a, hi = n;
        for (uint32_t step = 1;; step <<= 1) {
            const uint64_t j = (uint64_t)a + step;
            if (j >= n) break;
            if ((keys[j] >> shift) != p) { hi = (uint32_t)j; break; }
            lo = (uint32_t)j;
        }
        while (hi - lo > 1) {
            const uint32_t mid = lo + (hi - lo) / 2;
            if ((keys[mid] >> shift) == p) lo = mid; else hi = mid;
        }
        const uint32_t e = hi;
        nodes[X].count = e - a;
        nodes[X].skip = first_node[e];
        if (meta & kLeafBit) {
            const float4 r = spos[a];
            float m = 0.f, sx = 0.f, sy = 0.f, sz = 0.f;
            for (uint32_t j = a; j < e; ++j) {
                const float4 q = spos[j];
                m += q.w;
                sx = fmaf(q.w, q.x - r.x, sx);
                sy = fmaf(q.w, q.y - r.y, sy);
                sz = fmaf(q.w, q.z - r.z, sz);
            }
            float4 com;
            if (m != 0.f) {
                com = make_float4(r.x + sx / m, r.y + sy / m, r.z + sz / m, m);
            } else {
                const float3 c = cell_centre(keys[a], l, bits, prm);
                com = make_float4(c.x, c.y, c.z, 0.f);
            }
            *reinterpret_cast<float4 *>(&nodes[X]) = com;
        }
    }
}

// Internal nodes of one level: mass and centre of mass from their children,
// which follow the node in pre-order (first child = node + 1, next = skip).
__global__ __launch_bounds__(256) void k_com_level(const uint64_t *__restrict__ keys,
                                                   Node *__restrict__ nodes,
                                                   const uint32_t *__restrict__ level_list,
                                                   int level, int bits, uint64_t cap,
                                                   const DevParams *__restrict__ prm)
{
    if (prm->n_nodes > cap) return;
    const uint32_t cnt = prm->level_count[level];
    const uint32_t off = prm->level_offset[level];
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += gridDim.x * blockDim.x) {
        const uint32_t X = level_list[off + i];
        const Node nd = nodes[X];
        if (nd.meta & kLeafBit) continue;
        const float4 r = *reinterpret_cast<const float4 *>(&nodes[X + 1]);
        float m = 0.f, sx = 0.f, sy = 0.f, sz = 0.f;
        for (uint32_t c = X + 1; c < nd.skip; c = nodes[c].skip) {
            const float4 q = *reinterpret_cast<const float4 *>(&nodes[c]);
            m += q.w;
            sx = fmaf(q.w, q.x - r.x, sx);
            sy = fmaf(q.w, q.y - r.y, sy);
            sz = fmaf(q.w, q.z - r.z, sz);
        }
        float4 com;
        if (m != 0.f) {
            com = make_float4(r.x + sx / m, r.y + sy / m, r.z + sz / m, m);
        } else {
            const float3 c = cell_centre(keys[nd.start], level, bits, prm);
            com = make_float4(c.x, c.y, c.z, 0.f);
        }
        *reinterpret_cast<float4 *>(&nodes[X]) = com;
    }
}

uint32_t grid_for(uint64_t items, uint32_t max_blocks)
{
    uint64_t b = (items + 255) / 256;
    if (b < 1) b = 1;
    return (uint32_t)(b < max_blocks ? b : max_blocks);
}

}  // namespace

uint32_t build_blocks(uint32_t n)
{
    uint32_t t = (n + kBuildTile - 1) / kBuildTile;
    return t ? t : 1;
}

void build_tree(const uint64_t *keys_sorted, const float4 *spos, uint32_t n, int bits,
                int leaf_cap, uint64_t node_capacity, uint16_t *dc, uint32_t *block_counts,
                uint32_t *block_pref, uint32_t *block_tot, uint32_t *first_node,
                uint32_t *level_list, Node *nodes, DevParams *prm, hipStream_t s)
{
    const uint32_t tiles = build_blocks(n);
    hipLaunchKernelGGL(k_count, dim3(tiles), dim3(kBuildThreads), 0, s, keys_sorted, n, bits,
                       leaf_cap, dc, block_counts, tiles);
    launch_scan_rows(block_counts, block_pref, block_tot, kBuildCols, tiles, s);
    hipLaunchKernelGGL(k_emit, dim3(tiles), dim3(kBuildThreads), 0, s, dc, n,
                       (const uint32_t *)block_pref, (const uint32_t *)block_tot, tiles,
                       node_capacity, first_node, level_list, nodes, prm);
    hipLaunchKernelGGL(k_ranges, dim3(grid_for(n, 2048)), dim3(256), 0, s, keys_sorted, spos, n,
                       bits, node_capacity, first_node, nodes, (const DevParams *)prm);
}

void com_levels(const uint64_t *keys_sorted, Node *nodes, const uint32_t *level_list, uint32_t n,
                uint64_t node_capacity, int bits, DevParams *prm, hipStream_t s)
{
    const uint32_t grid = grid_for(n / 2 + 1, 1024);
    for (int l = bits - 1; l >= 0; --l)
        hipLaunchKernelGGL(k_com_level, dim3(grid), dim3(256), 0, s, keys_sorted, nodes,
                           level_list, l, bits, node_capacity, (const DevParams *)prm);
}

}  // namespace bh
