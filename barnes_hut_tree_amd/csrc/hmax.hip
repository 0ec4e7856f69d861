// Per-node maximum smoothing length: the hmax field that the pages' tree keeps
// next to the centre of mass for the SPH neighbour search of [Tree] (树结构,
// 粒子领域搜索; d_node_hmax in 重置树结构): the largest h among a cell's
// particles.  Leaves take the maximum over their particles (read through the
// sort permutation); an internal cell takes the maximum over its children,
// which are one level deeper, so the levels are done from the deepest up, one
// launch each.  Children of X are X + 1, then each child's skip, up to X's
// skip (pre-order).  Maxima are exact, so the result does not depend on order.
#include <algorithm>

#include "bh_internal.h"

namespace bh {
namespace {

constexpr int kHmaxThreads = 256;

__global__ __launch_bounds__(kHmaxThreads) void k_hmax_leaves(const Node *__restrict__ nodes,
                                                              const uint32_t *__restrict__ perm,
                                                              const float *__restrict__ h,
                                                              const DevParams *__restrict__ prm,
                                                              uint64_t cap, float *__restrict__ out)
{
    const uint32_t nn = (uint32_t)min((uint64_t)prm->n_nodes, cap);
    for (uint32_t X = blockIdx.x * blockDim.x + threadIdx.x; X < nn; X += gridDim.x * blockDim.x) {
        const uint4 rec = reinterpret_cast<const uint4 *>(&nodes[X])[1];   // start, count, skip, meta
        if (!(rec.w & kLeafBit)) continue;
        float m = -INFINITY;
        for (uint32_t j = rec.x; j < rec.x + rec.y; ++j) m = fmaxf(m, h[perm[j]]);
        out[X] = m;
    }
}

__global__ __launch_bounds__(kHmaxThreads) void k_hmax_level(const Node *__restrict__ nodes,
                                                             const DevParams *__restrict__ prm,
                                                             uint64_t cap, uint32_t level,
                                                             float *__restrict__ out)
{
    const uint32_t nn = (uint32_t)min((uint64_t)prm->n_nodes, cap);
    for (uint32_t X = blockIdx.x * blockDim.x + threadIdx.x; X < nn; X += gridDim.x * blockDim.x) {
        const uint4 rec = reinterpret_cast<const uint4 *>(&nodes[X])[1];
        if ((rec.w & kLeafBit) || node_level(rec.w) != level) continue;
        float m = -INFINITY;
        for (uint32_t c = X + 1; c < rec.z && c < nn; c = nodes[c].skip) m = fmaxf(m, out[c]);
        out[X] = m;
    }
}

}  // namespace

void launch_node_hmax(const Node *nodes, const uint32_t *perm, const float *h, uint32_t n_nodes,
                      const DevParams *prm, uint64_t cap, int bits, float *out, hipStream_t s)
{
    if (n_nodes == 0) return;
    const uint32_t grid = (uint32_t)std::min<uint64_t>((n_nodes + kHmaxThreads - 1) / kHmaxThreads,
                                                       65535);
    hipLaunchKernelGGL(k_hmax_leaves, dim3(grid), dim3(kHmaxThreads), 0, s, nodes, perm, h, prm,
                       cap, out);
    for (int l = bits - 1; l >= 0; --l)
        hipLaunchKernelGGL(k_hmax_level, dim3(grid), dim3(kHmaxThreads), 0, s, nodes, prm, cap,
                           (uint32_t)l, out);
}

}  // namespace bh
