// Octree from Morton-sorted keys, and the centre of mass of every node.
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
// Centre of mass ([GASPHiA] 计算节点质心): M = sum m and X = sum(m x) / M over
// the cell's particles, which are the contiguous sorted range [start, end).
// The same tile pass keeps fp64 prefix sums P of (m, m (x - lo)) over the
// sorted particles, so every node, leaf or internal, takes
// (P[end] - P[start]) in one step; with fp64 sums the difference keeps about
// 1e-10 relative accuracy even at N = 2^26, far below the fp32 result.  Node
// ranges start and end only where leaves start, so P is kept at leaf starts,
// stored by leaf number (consecutive leaves, consecutive entries).
//
// Kernels: count (d, c, per-tile node and leaf totals and particle sums) ->
// one scan over the tiles -> emit (node start, leaf number and level; per
// leaf start the first node there and its leaf number; P per leaf) -> ranges
// (a leaf ends where the next node starts; an internal cell's end by
// galloping search in the keys; skip = first node at the end; mass and
// centre of mass from P).
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

// Per-particle summand of the centre-of-mass prefix: (m, m (x - lo)).
__device__ inline D4 mass_moment(float4 q, const DevParams *prm)
{
    const double m = (double)q.w;
    return D4{m, m * ((double)q.x - prm->lo[0]), m * ((double)q.y - prm->lo[1]),
              m * ((double)q.z - prm->lo[2])};
}

__device__ inline D4 shfl_up_d4(D4 v, int o)
{
    return D4{__shfl_up(v.m, o, 64), __shfl_up(v.x, o, 64), __shfl_up(v.y, o, 64),
              __shfl_up(v.z, o, 64)};
}

__device__ inline D4 wave_incl_scan_d4(D4 v)
{
    const uint32_t lane = threadIdx.x & 63;
    for (int o = 1; o < 64; o <<= 1) {
        const D4 t = shfl_up_d4(v, o);
        if (lane >= (uint32_t)o) v = v + t;
    }
    return v;
}

// Lowest set bit at or above bit s of the 128-bit value hi:lo (s <= 64), as
// an offset from s; 128 when there is none.
__device__ inline int first_from(uint64_t lo, uint64_t hi, int s)
{
    const uint64_t x = s < 64 ? (lo >> s) : 0ull;
    if (x != 0) return __builtin_ctzll(x);
    if (hi != 0) return (64 - s) + __builtin_ctzll(hi);
    return 128;
}

// Per position a of the tile: d(a), whether a leaf starts at a, and the
// number c(a) of nodes starting there (see the file comment).
//
// With B <= 64 (WAVE_ROWS), the searches of a position reach at most one
// 64-position row either side, so they are answered with ballots: each wave
// takes one row of 64 positions at a time, and for a depth threshold v the
// masks of d < v over the previous, current and next rows give every lane
// the nearest cell boundary shallower than v on either side (the level-d(a)
// cell around a is [last boundary < d(a) before a, first one after a)), and
// whether (a, a + B] holds one.  The loops run over the distinct values in
// the row only.  Larger B scans the window position by position.
template <bool WAVE_ROWS>
__global__ __launch_bounds__(kBuildThreads) void k_count(const uint64_t *__restrict__ keys,
                                                         const float4 *__restrict__ spos,
                                                         uint32_t n, int bits, int B,
                                                         uint16_t *__restrict__ dc,
                                                         uint2 *__restrict__ block_counts,
                                                         D4 *__restrict__ block_sums,
                                                         const DevParams *__restrict__ prm)
{
    __shared__ int8_t sd[kBuildTile + 2 * kMaxLeafCap + 2];
    __shared__ uint32_t lc, ll;
    const int W = WAVE_ROWS ? 64 : B;   // window margin either side of the tile
    const int64_t t0 = (int64_t)blockIdx.x * kBuildTile;
    const int64_t w0 = t0 - W;   // window covers positions [t0 - W, t0 + tile + W]
    const int wlen = kBuildTile + 2 * W + 1;
    for (int k = threadIdx.x; k < wlen; k += kBuildThreads)
        sd[k] = (int8_t)d_at(keys, w0 + k, n, bits);
    if (threadIdx.x == 0) {
        lc = 0;
        ll = 0;
    }
    __syncthreads();

    uint32_t my_nodes = 0, my_leaves = 0;
    for (int k = 0; k < kBuildTile / kBuildThreads; ++k) {
        const int off = k * kBuildThreads + threadIdx.x;
        const int64_t a = t0 + off;
        if (WAVE_ROWS) {
            if (t0 + k * kBuildThreads + (threadIdx.x & ~63) >= (int64_t)n) break;   // whole row past n
        } else if (a >= (int64_t)n) {
            break;
        }
        const bool valid = a < (int64_t)n;
        const int ia = off + W;  // index of a in the window
        const int da = sd[ia];
        bool leaf_start = false;
        int ell = bits;
        if (WAVE_ROWS) {
            const int l = (int)(threadIdx.x & 63);
            const int dp = sd[ia - 64], dn = sd[ia + 64];
            // leaf start: the level-d(a) cell around a holds more than B
            const bool need = valid && a > 0 && da < bits;
            leaf_start = valid && a == 0;
            uint64_t pending = __ballot(need);
            while (pending) {
                const int v = __builtin_amdgcn_readlane(da, __builtin_ctzll(pending));
                const uint64_t mp = __ballot(dp < v), mc = __ballot(da < v), mn = __ballot(dn < v);
                if (need && da == v) {
                    const uint64_t below = mc & ((1ull << l) - 1ull);
                    const int g = below ? l - (63 - __builtin_clzll(below))
                                        : (mp ? l + 1 + __builtin_clzll(mp) : 1000);
                    const int f = 1 + first_from(mc, mn, l + 1);
                    leaf_start = f + g > B;
                }
                pending &= ~__ballot(da == v);
            }
            // level of the leaf starting at a: the smallest level above d(a)
            // whose cell starting at a ends within (a, a + B], else bits
            uint64_t open = __ballot(leaf_start);
            if (open) {
                int lmin = leaf_start ? da + 1 : 1000;
                for (int o = 32; o > 0; o >>= 1) lmin = min(lmin, __shfl_xor(lmin, o, 64));
                const uint64_t wmask = B >= 64 ? ~0ull : ((1ull << B) - 1ull);
                for (int lv = lmin; lv < bits && open; ++lv) {
                    const uint64_t mc = __ballot(da < lv), mn = __ballot(dn < lv);
                    bool hit = false;
                    if (leaf_start && ell == bits && lv >= da + 1) {
                        const int s = l + 1;
                        const uint64_t win = s < 64 ? ((mc >> s) | (s > 0 ? mn << (64 - s) : 0ull))
                                                    : mn;
                        hit = (win & wmask) != 0;
                        if (hit) ell = lv;
                    }
                    open &= ~__ballot(hit);
                }
            }
        } else {
            if (a == 0) {
                leaf_start = true;
            } else if (da < bits) {
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
                ell = min(bits, 1 + max(da, rm));
            }
        }
        const int c = leaf_start ? ell - da : 0;
        my_nodes += (uint32_t)c;
        my_leaves += c > 0 ? 1u : 0u;
        if (valid) dc[a] = (uint16_t)((da + 1) | (c << 8));
    }
    for (int o = 32; o > 0; o >>= 1) {
        my_nodes += __shfl_xor(my_nodes, o, 64);
        my_leaves += __shfl_xor(my_leaves, o, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&lc, my_nodes);
        atomicAdd(&ll, my_leaves);
    }
    __syncthreads();
    // the tile's particle sums, each thread over 4 consecutive positions in
    // the order the emit kernel scans them
    {
        constexpr int per = kBuildTile / kBuildThreads;
        __shared__ D4 wsum[kBuildThreads / 64];
        D4 acc = {0.0, 0.0, 0.0, 0.0};
        for (int k = 0; k < per; ++k) {
            const int64_t a = t0 + per * threadIdx.x + k;
            if (a < (int64_t)n) acc = acc + mass_moment(spos[a], prm);
        }
        const D4 incl = wave_incl_scan_d4(acc);
        if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = incl;
        __syncthreads();
        if (threadIdx.x == 0) {
            D4 tot = wsum[0];
            for (int w = 1; w < kBuildThreads / 64; ++w) tot = tot + wsum[w];
            block_sums[blockIdx.x] = tot;
            block_counts[blockIdx.x] = make_uint2(lc, ll);
        }
    }
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

__device__ inline uint2 wave_incl_scan_u2(uint2 v)
{
    return make_uint2(wave_incl_scan(v.x), wave_incl_scan(v.y));
}

__device__ inline uint2 operator+(uint2 a, uint2 b) { return make_uint2(a.x + b.x, a.y + b.y); }
__device__ inline uint2 operator-(uint2 a, uint2 b) { return make_uint2(a.x - b.x, a.y - b.y); }

// The exclusive scan over tiles of (node count, leaf count, particle sums) is split so
// that every access is coalesced and no single workgroup walks all tiles.
// Tiles are grouped in chunks of chunk_tiles(n_tiles) consecutive tiles (a
// multiple of 64, at most kTileScanThreads chunks).  k_chunk_totals reduces
// each chunk with one wave (64 consecutive tiles per load); k_scan_chunks,
// one workgroup, scans the chunk totals: out[c] = the sum of the chunks
// before c, out[n_chunks] = the totals.  Each emit workgroup then adds the
// tiles before its own within its chunk.
__device__ inline void wave_sum_tiles(const uint2 *__restrict__ counts,
                                      const D4 *__restrict__ sums, uint32_t b, uint32_t e,
                                      uint2 &c, D4 &m)
{
    const uint32_t lane = threadIdx.x & 63;
    c = make_uint2(0u, 0u);
    m = D4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
    for (uint32_t t = b + lane; t < e; t += 64) {
        c += counts[t];
        m = m + sums[t];
    }
    for (int o = 32; o > 0; o >>= 1) {
        c = c + make_uint2(__shfl_xor(c.x, o, 64), __shfl_xor(c.y, o, 64));
        m = m + D4{__shfl_xor(m.m, o, 64), __shfl_xor(m.x, o, 64), __shfl_xor(m.y, o, 64),
                   __shfl_xor(m.z, o, 64)};
    }
}

// one wave per chunk
__global__ __launch_bounds__(64) void k_chunk_totals(const uint2 *__restrict__ counts,
                                                     const D4 *__restrict__ sums,
                                                     uint32_t n_tiles, uint32_t chunk,
                                                     TileScan *__restrict__ tot)
{
    const uint32_t k = blockIdx.x;
    uint2 c;
    D4 m;
    wave_sum_tiles(counts, sums, k * chunk, min(n_tiles, (k + 1) * chunk), c, m);
    if (threadIdx.x == 0) {
        tot[k].nodes = c.x;
        tot[k].leaves = c.y;
        tot[k].sums = m;
    }
}

__global__ __launch_bounds__(kTileScanThreads) void k_scan_chunks(
    const TileScan *__restrict__ tot, uint32_t n_chunks, TileScan *__restrict__ out)
{
    constexpr int kWavesScan = kTileScanThreads / 64;
    __shared__ D4 wsum[kWavesScan + 1];
    __shared__ uint2 wcnt[kWavesScan + 1];
    __shared__ unsigned long long wide[kWavesScan];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t k = threadIdx.x;
    const uint2 c = k < n_chunks ? make_uint2(tot[k].nodes, tot[k].leaves) : make_uint2(0u, 0u);
    const D4 m = k < n_chunks ? tot[k].sums : D4{0.0, 0.0, 0.0, 0.0};
    const uint2 ic = wave_incl_scan_u2(c);
    const D4 im = wave_incl_scan_d4(m);
    // the same node total in 64 bits, to detect a 32-bit wrap
    unsigned long long c64 = c.x;
    for (int o = 32; o > 0; o >>= 1) c64 += __shfl_xor(c64, o, 64);
    if (lane == 63) {
        wcnt[wave] = ic;
        wsum[wave] = im;
        wide[wave] = c64;
    }
    __syncthreads();
    // the first wave turns the wave totals into exclusive prefixes
    if (wave == 0) {
        const uint2 c2 = lane < kWavesScan ? wcnt[lane] : make_uint2(0u, 0u);
        const D4 m2 = lane < kWavesScan ? wsum[lane] : D4{0.0, 0.0, 0.0, 0.0};
        const uint2 ic2 = wave_incl_scan_u2(c2);
        const D4 im2 = wave_incl_scan_d4(m2);
        if (lane < kWavesScan) {
            wcnt[lane] = ic2 - c2;
            wsum[lane] = im2 - m2;
        }
        if (lane == kWavesScan - 1) {
            wcnt[kWavesScan] = ic2;
            wsum[kWavesScan] = im2;
        }
    }
    __syncthreads();
    const uint2 rc = (ic - c) + wcnt[wave], tc = wcnt[kWavesScan];
    const D4 rm = (im - m) + wsum[wave], tm = wsum[kWavesScan];
    if (k < n_chunks) {
        out[k].nodes = rc.x;
        out[k].leaves = rc.y;
        out[k].sums = rm;
    }
    if (k == 0) {
        unsigned long long all = 0;
        for (int w = 0; w < kWavesScan; ++w) all += wide[w];
        out[n_chunks].nodes = tc.x;
        out[n_chunks].leaves = tc.y;
        out[n_chunks].wrapped = all > 0xffffffffull ? 1u : 0u;
        out[n_chunks].sums = tm;
    }
}

// chunk_pref: the exclusive scan over chunks of the tiles' node and leaf
// counts and particle sums ([n_chunks] = the totals); the tiles before this
// one in its chunk are added here.  Outputs: per node its start, the number
// of leaves before it in pre-order and its level/leaf word, in the second
// half of its record (the ranges kernel completes the record); per leaf the
// prefix P of the particle sums at its start, stored by leaf number so the
// ranges kernel reads it in order; per leaf start position the first node
// there and its leaf number (for the ends of internal cells).
__global__ __launch_bounds__(kBuildThreads) void k_emit(const uint16_t *__restrict__ dc,
                                                        const float4 *__restrict__ spos, uint32_t n,
                                                        const uint2 *__restrict__ tile_counts,
                                                        const D4 *__restrict__ tile_sums,
                                                        const TileScan *__restrict__ chunk_pref,
                                                        uint32_t n_tiles, uint32_t chunk,
                                                        uint64_t cap,
                                                        uint2 *__restrict__ first_node,
                                                        D4 *__restrict__ P,
                                                        Node *__restrict__ nodes,
                                                        DevParams *__restrict__ prm)
{
    constexpr int per = kBuildTile / kBuildThreads;  // consecutive positions per thread
    static_assert(per == 4, "the LDS layout below assumes 4 positions per thread");
    __shared__ uint2 wtot[kBuildThreads / 64];
    __shared__ D4 wsum[kBuildThreads / 64];
    __shared__ uint32_t tile_nodes, tile_leaves;
    __shared__ D4 tile_mass;
    const uint32_t blk = blockIdx.x;
    const uint32_t n_chunks = (n_tiles + chunk - 1) / chunk;
    const uint32_t total = chunk_pref[n_chunks].nodes;   // all nodes
    if (threadIdx.x < 64) {
        const uint32_t c0 = blk / chunk;
        uint2 c;
        D4 m;
        wave_sum_tiles(tile_counts, tile_sums, c0 * chunk, blk, c, m);
        if (threadIdx.x == 0) {
            tile_nodes = chunk_pref[c0].nodes + c.x;
            tile_leaves = chunk_pref[c0].leaves + c.y;
            tile_mass = chunk_pref[c0].sums + m;
        }
    }

    // Coalesced loads into LDS: per position its (d, c) word and its mass
    // moment.  Each thread then works on 4 consecutive positions; their four
    // moments are stored at a stride of 9 16-byte units per thread (one unit
    // of padding), so the threads' 16-byte LDS accesses fall in distinct banks.
    // (fn and sdc are also accessed as 16- and 8-byte words)
    __shared__ double2 mom[kBuildThreads * 9];                // moments, then the prefix P
    __shared__ __attribute__((aligned(16))) uint32_t fn[kBuildTile];   // first node per position
    __shared__ __attribute__((aligned(16))) uint32_t flr[kBuildTile];  // leaves before it
    __shared__ __attribute__((aligned(16))) uint16_t sdc[kBuildTile];
    auto unit = [](int j) { return (j >> 2) * 9 + (j & 3) * 2; };
    const int64_t t0 = (int64_t)blk * kBuildTile;
    for (int k = 0; k < per; ++k) {
        const int j = k * kBuildThreads + threadIdx.x;
        const int64_t a = t0 + j;
        sdc[j] = a < (int64_t)n ? dc[a] : (uint16_t)0;
        const D4 m = a < (int64_t)n ? mass_moment(spos[a], prm) : D4{0.0, 0.0, 0.0, 0.0};
        mom[unit(j)] = make_double2(m.m, m.x);
        mom[unit(j) + 1] = make_double2(m.y, m.z);
    }
    __syncthreads();

    // each thread: 4 consecutive positions
    const int j0 = per * threadIdx.x;
    const int64_t a0 = t0 + j0;
    int dd[per], cc[per];
    D4 mk[per];
    uint32_t s = 0, sl = 0;
    D4 ms = {0.0, 0.0, 0.0, 0.0};
    {
        const uint2 w = reinterpret_cast<const uint2 *>(sdc)[threadIdx.x];
        const uint32_t v4[per] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
        for (int k = 0; k < per; ++k) {
            dd[k] = (int)(v4[k] & 0xffu) - 1;
            cc[k] = (int)(v4[k] >> 8);
            s += cc[k];
            sl += cc[k] > 0 ? 1u : 0u;
            const double2 u0 = mom[unit(j0 + k)], u1 = mom[unit(j0 + k) + 1];
            mk[k] = D4{u0.x, u0.y, u1.x, u1.y};
            ms = ms + mk[k];
        }
    }
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint2 incl = wave_incl_scan_u2(make_uint2(s, sl));
    const D4 mincl = wave_incl_scan_d4(ms);
    if (lane == 63) {
        wtot[wave] = incl;
        wsum[wave] = mincl;
    }
    __syncthreads();
    uint32_t run = tile_nodes, lrun = tile_leaves;
    D4 mrun = tile_mass;
    for (uint32_t w = 0; w < wave; ++w) {
        run += wtot[w].x;
        lrun += wtot[w].y;
        mrun = mrun + wsum[w];
    }
    run += incl.x - s;
    lrun += incl.y - sl;
    mrun = mrun + (mincl - ms);

    uint32_t fn4[per], lr4[per];
    for (int k = 0; k < per; ++k) {
        const int64_t a = a0 + k;
        fn4[k] = run;
        lr4[k] = lrun;
        mom[unit(j0 + k)] = make_double2(mrun.m, mrun.x);
        mom[unit(j0 + k) + 1] = make_double2(mrun.y, mrun.z);
        mrun = mrun + mk[k];
        if (a < (int64_t)n) {
            for (int j = 0; j < cc[k]; ++j) {
                const int l = dd[k] + 1 + j;
                const uint32_t X = run + j;
                if (X < cap)
                    reinterpret_cast<uint4 *>(&nodes[X])[1] =
                        make_uint4((uint32_t)a, lrun, 0u,
                                   (uint32_t)l | (j == cc[k] - 1 ? kLeafBit : 0u));
            }
        }
        run += cc[k];
        lrun += cc[k] > 0 ? 1u : 0u;
    }
    reinterpret_cast<uint4 *>(fn)[threadIdx.x] = make_uint4(fn4[0], fn4[1], fn4[2], fn4[3]);
    reinterpret_cast<uint4 *>(flr)[threadIdx.x] = make_uint4(lr4[0], lr4[1], lr4[2], lr4[3]);
    __syncthreads();
    // coalesced stores; nodes start and end only where a leaf starts, so the
    // prefix and the first node are needed only there (the prefix stored at
    // the leaf's number, dense in the leaves)
    for (int k = 0; k < per; ++k) {
        const int j = k * kBuildThreads + threadIdx.x;
        const int64_t a = t0 + j;
        if (a < (int64_t)n && (sdc[j] >> 8) != 0) {
            first_node[a] = make_uint2(fn[j], flr[j]);
            const double2 u0 = mom[unit(j)], u1 = mom[unit(j) + 1];
            P[flr[j]] = D4{u0.x, u0.y, u1.x, u1.y};
        }
    }
    if (blk == n_tiles - 1 && threadIdx.x == 0) {
        const uint32_t leaves = chunk_pref[n_chunks].leaves;
        first_node[n] = make_uint2(total, leaves);
        P[leaves] = chunk_pref[n_chunks].sums;
    }
    if (blk == 0 && threadIdx.x == 0) {
        prm->n_nodes = total;
        if (total > cap || chunk_pref[n_chunks].wrapped) prm->status |= kStatusCapacity;
    }
}

// Geometric centre of the level-l cell holding the source at p (for massless
// cells), from its quantised coordinates: valid for either key curve.
__device__ inline float3 cell_centre(float4 p, int level, int bits, const DevParams *prm)
{
    const uint64_t top = (1ull << bits) - 1;
    const float xyz[3] = {p.x, p.y, p.z};
    float c[3];
    for (int a = 0; a < 3; ++a) {
        const uint64_t corner = quantise(xyz[a], prm->lo[a], prm->scale, top) >> (bits - level);
        const double w = __builtin_ldexp(prm->L, -level);
        c[a] = (float)(prm->lo[a] + w * ((double)corner + 0.5));
    }
    return make_float3(c[0], c[1], c[2]);
}

// First sorted position past the level-l cell that holds position a: the
// first j > a whose key has another level-l prefix (or n).  Keys sharing the
// prefix are one contiguous run, so the positions inside form a prefix of
// any increasing set of probes; each round issues eight independent probes:
// a + step * {1..8} with step growing eightfold while all are inside, then
// seven evenly spaced probes in the remaining bracket.
__device__ inline uint32_t cell_end(const uint64_t *__restrict__ keys, uint32_t n, uint32_t a,
                                    int shift)
{
    const uint64_t p = keys[a] >> shift;
    uint64_t lo = a, hi = n;   // keys[lo] inside; hi outside (or n)
    for (uint64_t step = 1;; step *= 8) {
        uint64_t j[8];
        bool in[8];
        uint64_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            j[k] = (uint64_t)a + (uint64_t)(k + 1) * step;
            v[k] = keys[min(j[k], (uint64_t)n - 1)];   // unconditional: all eight in flight
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) in[k] = j[k] < n && (v[k] >> shift) == p;
        int m = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) m += in[k] ? 1 : 0;
        if (m == 8) {
            lo = j[7];
            continue;
        }
        if (m > 0) lo = j[m - 1];
        hi = min((uint64_t)n, j[m]);
        break;
    }
    while (hi - lo > 1) {
        uint64_t j[7];
        bool in[7];
        const uint64_t w = hi - lo;
        uint64_t v[7];
#pragma unroll
        for (int k = 0; k < 7; ++k) {
            j[k] = lo + 1 + ((w - 1) * (uint64_t)(k + 1)) / 8;   // in (lo, hi)
            v[k] = keys[j[k]];
        }
#pragma unroll
        for (int k = 0; k < 7; ++k) in[k] = (v[k] >> shift) == p;
        int m = 0;
#pragma unroll
        for (int k = 0; k < 7; ++k) m += in[k] ? 1 : 0;
        const uint64_t nlo = m > 0 ? j[m - 1] : lo;
        const uint64_t nhi = m < 7 ? j[m] : hi;
        lo = nlo;
        hi = nhi;
    }
    return (uint32_t)hi;
}

// Per node: its particle range, skip, mass and centre of mass, written as one
// 32-byte record.  A leaf ends where the next node in pre-order starts (its
// skip is the next node, and the next leaf's prefix closes its sums); an
// internal cell's end is searched in the keys, and the first node at the end
// gives its skip and the leaf whose prefix closes its sums.
__global__ __launch_bounds__(256) void k_ranges(const uint64_t *__restrict__ keys,
                                                const float4 *__restrict__ spos,
                                                const D4 *__restrict__ P, uint32_t n,
                                                int bits, uint64_t cap,
                                                const uint2 *__restrict__ first_node,
                                                Node *__restrict__ nodes,
                                                const DevParams *__restrict__ prm)
{
    const uint32_t nn = (uint32_t)min((uint64_t)prm->n_nodes, cap);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // the record after the last node (the array holds cap + 1): an empty
        // leaf at an undefined (NaN) centre, which every target still walking
        // opens, so the walk needs no bound check on its common path
        reinterpret_cast<float4 *>(&nodes[nn])[0] = make_float4(NAN, NAN, NAN, 0.f);
        reinterpret_cast<uint4 *>(&nodes[nn])[1] = make_uint4(n, 0u, nn, kLeafBit);
    }
    for (uint32_t X = blockIdx.x * blockDim.x + threadIdx.x; X < nn; X += gridDim.x * blockDim.x) {
        const uint4 rec = reinterpret_cast<const uint4 *>(&nodes[X])[1];
        const uint32_t a = rec.x, lr = rec.y, meta = rec.w;
        const int l = (int)node_level(meta);
        const bool leaf = (meta & kLeafBit) != 0;
        const D4 pa = P[lr];
        uint32_t e, skip, le;
        if (leaf) {
            // the next record's start is rewritten with the same value
            e = X + 1 < nn ? nodes[X + 1].start : n;
            skip = X + 1;
            le = lr + 1;
        } else {
            e = cell_end(keys, n, a, 3 * (bits - l));
            const uint2 f = first_node[e];
            skip = f.x;
            le = f.y;
        }
        const D4 sum = P[le] - pa;
        float4 com;
        if (sum.m != 0.0) {
            com = make_float4((float)(prm->lo[0] + sum.x / sum.m),
                              (float)(prm->lo[1] + sum.y / sum.m),
                              (float)(prm->lo[2] + sum.z / sum.m), (float)sum.m);
        } else {
            const float3 c = cell_centre(spos[a], l, bits, prm);
            com = make_float4(c.x, c.y, c.z, 0.f);
        }
        reinterpret_cast<float4 *>(&nodes[X])[0] = com;
        reinterpret_cast<uint4 *>(&nodes[X])[1] = make_uint4(a, e - a, skip, meta);
    }
}

// Per node in pre-order, the canonical description of its cell: level,
// count, and the key prefix naming the cell's place on its level's grid (the
// top `level` bits of each integer coordinate, interleaved x into bit 3k, y
// into 3k + 1, z into 3k + 2, the octant numbering of [Tree] 构建树结构).  The
// place comes from the quantised coordinates of the cell's first sorted
// source, so it is the same for either key curve.
__global__ __launch_bounds__(256) void k_cells(const Node *__restrict__ nodes,
                                               const float4 *__restrict__ spos, uint32_t nn,
                                               int bits, const DevParams *__restrict__ prm,
                                               uint8_t *__restrict__ level,
                                               uint64_t *__restrict__ prefix,
                                               uint32_t *__restrict__ count)
{
    const uint64_t top = (1ull << bits) - 1;
    for (uint32_t X = blockIdx.x * blockDim.x + threadIdx.x; X < nn; X += gridDim.x * blockDim.x) {
        const uint4 rec = reinterpret_cast<const uint4 *>(&nodes[X])[1];
        const int l = (int)node_level(rec.w);
        if (level) level[X] = (uint8_t)l;
        if (count) count[X] = rec.y;
        if (prefix) {
            const float4 p = spos[rec.x];
            const float xyz[3] = {p.x, p.y, p.z};
            uint64_t pre = 0;
            for (int a = 0; a < 3; ++a) {
                const uint64_t c = quantise(xyz[a], prm->lo[a], prm->scale, top) >> (bits - l);
                for (int k = 0; k < l; ++k) pre |= ((c >> k) & 1ull) << (3 * k + a);
            }
            prefix[X] = pre;
        }
    }
}

__global__ void k_zero_u64(unsigned long long *p) { *p = 0ull; }

uint32_t grid_for(uint64_t items, uint32_t max_blocks)
{
    uint64_t b = (items + 255) / 256;
    if (b < 1) b = 1;
    return (uint32_t)(b < max_blocks ? b : max_blocks);
}

}  // namespace

// Tiles per chunk of the tile scan: a multiple of 64, with at most
// kTileScanThreads chunks.
static uint32_t chunk_tiles(uint32_t tiles)
{
    const uint32_t per = (tiles + kTileScanThreads - 1) / kTileScanThreads;
    return ((per + 63) / 64) * 64;
}

uint32_t build_blocks(uint32_t n)
{
    uint32_t t = (n + kBuildTile - 1) / kBuildTile;
    return t ? t : 1;
}

void build_tree(const uint64_t *keys_sorted, const float4 *spos, uint32_t n, int bits,
                int leaf_cap, uint64_t node_capacity, BuildScratch &w, Node *nodes,
                DevParams *prm, hipStream_t s)
{
    const uint32_t tiles = build_blocks(n);
    if (leaf_cap <= 64)
        hipLaunchKernelGGL(k_count<true>, dim3(tiles), dim3(kBuildThreads), 0, s, keys_sorted,
                           spos, n, bits, leaf_cap, w.dc, w.tile_counts, w.tile_sums,
                           (const DevParams *)prm);
    else
        hipLaunchKernelGGL(k_count<false>, dim3(tiles), dim3(kBuildThreads), 0, s, keys_sorted,
                           spos, n, bits, leaf_cap, w.dc, w.tile_counts, w.tile_sums,
                           (const DevParams *)prm);
    const uint32_t chunk = chunk_tiles(tiles);
    const uint32_t n_chunks = (tiles + chunk - 1) / chunk;
    hipLaunchKernelGGL(k_chunk_totals, dim3(n_chunks), dim3(64), 0, s,
                       (const uint2 *)w.tile_counts, (const D4 *)w.tile_sums, tiles, chunk,
                       w.chunk_tot);
    hipLaunchKernelGGL(k_scan_chunks, dim3(1), dim3(kTileScanThreads), 0, s,
                       (const TileScan *)w.chunk_tot, n_chunks, w.tile_scan);
    hipLaunchKernelGGL(k_emit, dim3(tiles), dim3(kBuildThreads), 0, s, (const uint16_t *)w.dc, spos,
                       n, (const uint2 *)w.tile_counts, (const D4 *)w.tile_sums,
                       (const TileScan *)w.tile_scan, tiles, chunk, node_capacity, w.first_node,
                       w.P, nodes, prm);
    // about one node per thread: n / 2 threads (a tree of leaf capacity 16
    // has about n / 3 nodes; the grid-stride loop covers any excess)
    hipLaunchKernelGGL(k_ranges, dim3(grid_for(n / 2 + 1, 65535)), dim3(256), 0, s, keys_sorted, spos,
                       (const D4 *)w.P, n, bits, node_capacity, (const uint2 *)w.first_node,
                       nodes, (const DevParams *)prm);
}

void launch_zero_u64(unsigned long long *p, hipStream_t s)
{
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(1), 0, s, p);
}

void launch_cells(const Node *nodes, const float4 *spos, uint32_t nn, int bits,
                  const DevParams *prm, uint8_t *level, uint64_t *prefix, uint32_t *count,
                  hipStream_t s)
{
    if (nn == 0) return;
    hipLaunchKernelGGL(k_cells, dim3(grid_for(nn, 4096)), dim3(256), 0, s, nodes, spos, nn, bits,
                       prm, level, prefix, count);
}

}  // namespace bh
