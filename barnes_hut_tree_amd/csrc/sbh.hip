// Stochastic Barnes-Hut ([SBH] 方法, 关键设计): an unbiased Monte-Carlo
// estimate of the sum over sources built on the same octree.
//
// Every source's contribution is a telescoping sum along its root-to-leaf
// path, each step replacing a cell's monopole by its children's.  One sample
// per stratum (the children of the root in the d-ary tree) draws a path index
// I uniformly among the stratum's sources and a path length by Russian
// roulette: from depth k the walk continues with probability
// p_k = min(1, max(1, b_k) / b_{k+1}), b = |q - centre of mass| / cell edge,
// and each step taken adds the exchange term
//   Delta_T = sum over children c of m_c f(c, q) - m_T f(T, q)
// divided by P(I in T) P(K >= k).  The tree has single-source leaves; d = 2
// steps one octree level, d = 4 two (a child that is a leaf stands for
// itself).
//
// GPU mapping: the 64 queries of a wave share the random numbers (one
// Philox4x32-10 stream keyed by the seed, counter = (wave, sample, stratum,
// j)), so all lanes follow the same path: node records are wave-uniform and
// come through scalar loads, as in the walk; each lane keeps its own
// roulette outcome, weight and sums.
#include "bh_internal.h"
#include "interaction.h"

namespace bh {
namespace {

constexpr int kSbhThreads = 64;

__device__ inline uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011), first output word:
// ten rounds of two 32x32 -> 64-bit products by 0xD2511F53 and 0xCD9E8D57,
// the key bumped by 0x9E3779B9 and 0xBB67AE85 after each round.
__device__ inline uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

struct Rec {
    float cx, cy, cz, m;
    uint32_t start, count, skip, meta;
};

__device__ inline Rec load_node(const Node *__restrict__ nodes, uint32_t x)
{
    const uint4 *r = reinterpret_cast<const uint4 *>(nodes + x);
    const uint4 lo = r[0], hi = r[1];
    return Rec{__uint_as_float(lo.x), __uint_as_float(lo.y), __uint_as_float(lo.z),
               __uint_as_float(lo.w), hi.x, hi.y, hi.z, hi.w};
}

__device__ inline bool is_leaf(const Rec &r) { return (r.meta & kLeafBit) != 0; }

// Visit the d-ary children of node x (record rx) in pre-order: the octree
// children (D = 2), or their children with leaf children standing for
// themselves (D = 4).  fn(index, record) is called wave-uniformly.
template <int D, typename F>
__device__ inline void for_children(const Node *__restrict__ nodes, uint32_t x, const Rec &rx,
                                    F &&fn)
{
    for (uint32_t c = x + 1; c < rx.skip;) {
        const Rec rc = load_node(nodes, c);
        if (D == 2 || is_leaf(rc)) {
            fn(c, rc);
        } else {
            for (uint32_t g = c + 1; g < rc.skip;) {
                const Rec rg = load_node(nodes, g);
                fn(g, rg);
                g = rg.skip;
            }
        }
        c = rc.skip;
    }
}

// |q - centre of mass| / cell edge
__device__ inline float far_ratio(const Rec &r, float4 q, float L)
{
    const float dx = q.x - r.cx, dy = q.y - r.cy, dz = q.z - r.cz;
    const float edge = ldexpf(L, -(int)node_level(r.meta));
    return sqrtf(fmaf(dz, dz, fmaf(dy, dy, dx * dx))) / edge;
}

template <int D, bool SOFT>
__global__ __launch_bounds__(kSbhThreads) void k_sbh(const Node *__restrict__ nodes,
                                                     const float4 *__restrict__ tpos,
                                                     const uint32_t *__restrict__ tperm,
                                                     const DevParams *__restrict__ prm,
                                                     uint32_t n, int samples, uint32_t key0,
                                                     uint32_t key1, float G, float eps2,
                                                     float4 *__restrict__ out)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t group = blockIdx.x;   // one wave per workgroup: the wave's index
    const uint32_t i = group * kSbhThreads + lane;
    const bool valid = i < n;
    if (prm->status != 0) {
        if (valid) out[tperm[i]] = make_float4(NAN, NAN, NAN, NAN);
        return;
    }
    const float4 q = valid ? tpos[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float L = (float)prm->L;
    const Rec root = load_node(nodes, 0);

    float sx = 0.f, sy = 0.f, sz = 0.f, sp = 0.f;
    for (int s = 0; s < samples; ++s) {
        float ex = 0.f, ey = 0.f, ez = 0.f, ep = 0.f;
        if (is_leaf(root)) {
            // a single leaf (one source, or coincident ones): its monopole is exact
            pair<SOFT>(make_float4(root.cx, root.cy, root.cz, root.m), q.x, q.y, q.z, eps2, ex,
                       ey, ez, ep);
        }
        uint32_t stratum = 0;
        for_children<D>(nodes, 0, root, [&](uint32_t cidx, const Rec &rc) {
            const uint32_t ci = stratum++;
            pair<SOFT>(make_float4(rc.cx, rc.cy, rc.cz, rc.m), q.x, q.y, q.z, eps2, ex, ey, ez,
                       ep);
            if (is_leaf(rc)) return;
            const uint32_t r = sgpr(philox_word0(group, (uint32_t)s, ci, 0u, key0, key1));
            const uint32_t I = rc.start + __umulhi(r, rc.count);
            uint32_t t = cidx;
            Rec rt = rc;
            float w = 1.f;
            bool alive = valid;
            for (uint32_t depth = 0; !is_leaf(rt); ++depth) {
                // the child on the path (the one holding source I)
                uint32_t nxt = 0;
                Rec rn = rt;
                for_children<D>(nodes, t, rt, [&](uint32_t k, const Rec &rk) {
                    if (I >= rk.start && I - rk.start < rk.count) {
                        nxt = k;
                        rn = rk;
                    }
                });
                const float b0 = far_ratio(rt, q, L), b1 = far_ratio(rn, q, L);
                const float pk = b1 > 0.f ? fminf(1.f, fmaxf(1.f, b0) / b1) : 1.f;
                const uint32_t ru = sgpr(philox_word0(group, (uint32_t)s, ci, depth + 1u, key0,
                                                      key1));
                const float u = (float)(ru >> 8) * 0x1p-24f;
                alive = alive && u < pk;
                if (__ballot(alive) == 0) break;
                w = alive ? w / pk : w;
                // exchange term: the children's monopoles minus the cell's
                float dx = 0.f, dy = 0.f, dz = 0.f, dp = 0.f;
                for_children<D>(nodes, t, rt, [&](uint32_t, const Rec &rk) {
                    pair<SOFT>(make_float4(rk.cx, rk.cy, rk.cz, rk.m), q.x, q.y, q.z, eps2, dx,
                               dy, dz, dp);
                });
                pair<SOFT>(make_float4(rt.cx, rt.cy, rt.cz, -rt.m), q.x, q.y, q.z, eps2, dx, dy,
                           dz, dp);
                const float scale = alive ? w * ((float)rc.count / (float)rt.count) : 0.f;
                ex = fmaf(scale, dx, ex);
                ey = fmaf(scale, dy, ey);
                ez = fmaf(scale, dz, ez);
                ep = fmaf(scale, dp, ep);
                t = nxt;
                rt = rn;
            }
        });
        sx += ex;
        sy += ey;
        sz += ez;
        sp += ep;
    }
    if (valid) {
        const float g = G / (float)samples;
        out[tperm[i]] = make_float4(g * sx, g * sy, g * sz, g * sp);
    }
}

template <int D>
void launch_d(const SbhArgs &a, hipStream_t s)
{
    const uint32_t grid = (a.n_targets + kSbhThreads - 1) / kSbhThreads;
    const float eps2 = a.eps * a.eps;
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    if (eps2 > 0.f)
        hipLaunchKernelGGL((k_sbh<D, true>), dim3(grid), dim3(kSbhThreads), 0, s, a.nodes, a.tpos,
                           a.tperm, a.prm, a.n_targets, a.samples, k0, k1, a.G, eps2, a.out);
    else
        hipLaunchKernelGGL((k_sbh<D, false>), dim3(grid), dim3(kSbhThreads), 0, s, a.nodes,
                           a.tpos, a.tperm, a.prm, a.n_targets, a.samples, k0, k1, a.G, eps2,
                           a.out);
}

}  // namespace

void launch_sbh(const SbhArgs &a, hipStream_t s)
{
    if (a.n_targets == 0) return;
    if (a.d == 4) launch_d<4>(a, s); else launch_d<2>(a, s);
}

}  // namespace bh
