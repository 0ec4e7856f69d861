// The tree walk: accelerations and potentials of a Morton-ordered batch of
// targets ([GASPHiA] 计算自引力, 性能瓶颈分析).
//
// One wavefront walks the tree for 64 consecutive sorted targets.  The node it
// visits is wave-uniform, so node records come through scalar loads and are
// broadcast to all lanes for free.  The walk is stackless: nodes sit in
// pre-order, a subtree spans [node, skip), and each lane keeps a cursor, the
// next node it must see (initially the root).  At node X the lanes whose
// cursor equals X apply the opening test of the pages, (w/theta)^2 < r^2 with
// w the cell edge and r the distance to the centre of mass.  Lanes that pass
// add one monopole term and move their cursor to skip(X).  The others open X;
// a 64-lane ballot of them decides the wave's next node: X + 1 (the first
// child) if any lane opened an internal node, else skip(X).  An opened leaf
// is summed particle by particle by the lanes that opened it.
//
// A lane that accepted an ancestor of the current node holds a cursor at that
// ancestor's skip, which is at or beyond skip(X); the wave reaches it exactly
// when it leaves that subtree.  So every lane sees exactly the nodes its own
// particle-by-particle walk would visit (the pages' warp vote instead makes
// all lanes descend when any lane must; here the ballot only decides where
// the wave goes, and the per-lane cursor keeps each lane's result its own).
#include "bh_internal.h"

namespace bh {
namespace {

constexpr int kWalkThreads = 256;

// Blocks are dispatched to the 8 XCDs round-robin; give each XCD a contiguous
// run of the Morton order so the nodes and particles its waves share stay in
// that XCD's L2.
__device__ inline uint32_t xcd_block(uint32_t b, uint32_t nb)
{
    const uint32_t x = b & 7u, k = b >> 3, q = nb >> 3, r = nb & 7u;
    return x * q + min(x, r) + k;
}

template <bool SOFT>
__device__ inline void pair(float4 s, float px, float py, float pz, float eps2, float &ax,
                            float &ay, float &az, float &pot)
{
    const float dx = s.x - px, dy = s.y - py, dz = s.z - pz;
    const float r2 = fmaf(dz, dz, fmaf(dy, dy, fmaf(dx, dx, eps2)));
    float inv = __builtin_amdgcn_rsqf(r2);
    if (!SOFT) inv = r2 > 0.f ? inv : 0.f;
    const float mi = s.w * inv;
    const float f = mi * inv * inv;
    ax = fmaf(f, dx, ax);
    ay = fmaf(f, dy, ay);
    az = fmaf(f, dz, az);
    pot -= mi;
}

template <bool SOFT, bool SELF, bool COUNT>
__global__ __launch_bounds__(kWalkThreads) void k_walk(const Node *__restrict__ nodes,
                                                       const float4 *__restrict__ src,
                                                       const float4 *__restrict__ tpos,
                                                       const uint32_t *__restrict__ tperm,
                                                       const DevParams *__restrict__ prm,
                                                       uint32_t n, float theta, float G,
                                                       float eps2, float4 *__restrict__ out,
                                                       unsigned long long *__restrict__ count)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t blk = xcd_block(blockIdx.x, gridDim.x);
    const uint32_t wave_base = blk * kWalkThreads + (threadIdx.x & ~63u);
    const uint32_t i = wave_base + lane;
    const bool valid = i < n;
    if (wave_base >= n) return;

    if (prm->status != 0) {
        if (valid) out[tperm[i]] = make_float4(NAN, NAN, NAN, NAN);
        return;
    }
    const uint32_t nn = prm->n_nodes;
    const float4 p = valid ? tpos[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const double L = prm->L;
    const float T0 = (float)(L * L / ((double)theta * (double)theta));

    uint32_t cur = valid ? 0u : 0xffffffffu;
    float ax = 0.f, ay = 0.f, az = 0.f, pot = 0.f;
    uint32_t n_int = 0;

    uint32_t X = 0;
    while (X < nn) {
        X = __builtin_amdgcn_readfirstlane(X);
        const Node nd = nodes[X];
        const uint32_t level = node_level(nd.meta);
        const bool leaf = (nd.meta & kLeafBit) != 0;
        const float T = ldexpf(T0, -2 * (int)level);
        const float dx = nd.cx - p.x, dy = nd.cy - p.y, dz = nd.cz - p.z;
        const float r2 = fmaf(dz, dz, fmaf(dy, dy, dx * dx));
        const bool active = cur == X;
        const bool acc = active && (T < r2);
        const bool open = active && !acc;
        if (acc) {
            const float r2s = r2 + eps2;
            const float inv = __builtin_amdgcn_rsqf(r2s);
            const float mi = nd.m * inv;
            const float f = mi * inv * inv;
            ax = fmaf(f, dx, ax);
            ay = fmaf(f, dy, ay);
            az = fmaf(f, dz, az);
            pot -= mi;
            if (COUNT) ++n_int;
        }
        const uint64_t omask = __ballot(open);
        if (leaf) {
            if (omask != 0) {
                const uint32_t b = nd.start, e = nd.start + nd.count;
                // a leaf holding some of this wave's own targets needs the
                // self pair removed; others take the plain loop
                const bool mine = SELF && b < wave_base + 64 && e > wave_base;
                if (open) {
                    if (mine) {
                        for (uint32_t j = b; j < e; ++j) {
                            float4 s = src[j];
                            s.w = (j == i) ? 0.f : s.w;
                            pair<SOFT>(s, p.x, p.y, p.z, eps2, ax, ay, az, pot);
                        }
                    } else {
                        for (uint32_t j = b; j < e; ++j)
                            pair<SOFT>(src[j], p.x, p.y, p.z, eps2, ax, ay, az, pot);
                    }
                    if (COUNT) n_int += (e - b) - ((SELF && i >= b && i < e) ? 1u : 0u);
                }
            }
            if (active) cur = nd.skip;
            X = nd.skip;
        } else {
            if (acc) cur = nd.skip;
            if (open) cur = X + 1;
            X = omask ? X + 1 : nd.skip;
        }
    }
    if (valid) out[tperm[i]] = make_float4(G * ax, G * ay, G * az, G * pot);
    if (COUNT) {
        unsigned long long c = n_int;
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
        if (lane == 0) atomicAdd(count, c);
    }
}

__global__ void k_fill_zero(float4 *out, uint32_t n)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <bool SOFT, bool SELF, bool COUNT>
void launch3(const WalkArgs &a, hipStream_t s)
{
    const uint32_t grid = (a.n_targets + kWalkThreads - 1) / kWalkThreads;
    hipLaunchKernelGGL((k_walk<SOFT, SELF, COUNT>), dim3(grid), dim3(kWalkThreads), 0, s, a.nodes,
                       a.src, a.tpos, a.tperm, a.prm, a.n_targets, a.theta, a.G, a.eps * a.eps,
                       a.out, a.count);
}

template <bool SOFT, bool SELF>
void launch2(const WalkArgs &a, hipStream_t s)
{
    if (a.count) launch3<SOFT, SELF, true>(a, s); else launch3<SOFT, SELF, false>(a, s);
}

template <bool SOFT>
void launch1(const WalkArgs &a, hipStream_t s)
{
    if (a.self) launch2<SOFT, true>(a, s); else launch2<SOFT, false>(a, s);
}

}  // namespace

void launch_walk(const WalkArgs &a, hipStream_t s)
{
    if (a.n_targets == 0) return;
    // Plummer softening with eps^2 > 0 never meets r^2 + eps^2 == 0
    if (a.eps * a.eps > 0.f) launch1<true>(a, s); else launch1<false>(a, s);
}

void launch_fill_zero(float4 *out, uint32_t n, hipStream_t s)
{
    if (n == 0) return;
    hipLaunchKernelGGL(k_fill_zero, dim3((n + 255) / 256), dim3(256), 0, s, out, n);
}

}  // namespace bh
