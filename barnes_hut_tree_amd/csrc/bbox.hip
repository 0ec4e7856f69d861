// Bounding box and Morton keys.
//
// Bounding box: [Tree] 确定粒子空间范围 takes x/y/z min and max of all
// particles by a reduction; they fix the root cell.  The root cube is
// anchored at the min corner with side L = the largest extent.
//
// Keys: [Tree] 实现步骤 orders particles by Morton (Z-order) code; a Hilbert
// key is the other curve a context can choose (same cells, sibling order of
// the curve).  Each axis
// is quantised on the root cube in fp64, q = floor((x - lo) * 2^bits / L),
// clamped to [0, 2^bits - 1], and the bits are interleaved x, y, z from the
// least significant end, which matches the octant numbering of [Tree]
// 构建树结构 (x upper half = 1, y = 2, z = 4).  Each fp64 step is a single
// correctly rounded IEEE operation, so the keys are reproducible bit for bit.
#include "bh_internal.h"

namespace bh {
namespace {

constexpr int kBboxThreads = 256;
constexpr int kBboxMaxBlocks = 1024;
constexpr int kPartial = 8;   // min xyz, max xyz, non-finite flag, pad

__device__ inline float wave_min(float v)
{
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ inline float wave_max(float v)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// One pass over the float4 rows: each workgroup reduces a grid-strided share
// to six extrema and a non-finite flag.  Coalesced 16-byte loads.
__global__ __launch_bounds__(kBboxThreads) void k_bbox_partial(const float4 *__restrict__ src,
                                                               uint32_t n,
                                                               float *__restrict__ partials)
{
    float mn[3] = {INFINITY, INFINITY, INFINITY};
    float mx[3] = {-INFINITY, -INFINITY, -INFINITY};
    float bad = 0.0f;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float4 p = src[i];
        if (!(isfinite(p.x) && isfinite(p.y) && isfinite(p.z) && isfinite(p.w))) bad = 1.0f;
        mn[0] = fminf(mn[0], p.x); mn[1] = fminf(mn[1], p.y); mn[2] = fminf(mn[2], p.z);
        mx[0] = fmaxf(mx[0], p.x); mx[1] = fmaxf(mx[1], p.y); mx[2] = fmaxf(mx[2], p.z);
    }
    __shared__ float red[kBboxThreads / 64][kPartial];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float v[7];
    for (int a = 0; a < 3; ++a) {
        v[a] = wave_min(mn[a]);
        v[3 + a] = wave_max(mx[a]);
    }
    v[6] = wave_max(bad);
    if (lane == 0)
        for (int k = 0; k < 7; ++k) red[wave][k] = v[k];
    __syncthreads();
    if (threadIdx.x < 7) {
        const int k = threadIdx.x;
        float r = red[0][k];
        for (int w = 1; w < kBboxThreads / 64; ++w)
            r = (k < 3) ? fminf(r, red[w][k]) : fmaxf(r, red[w][k]);
        partials[blockIdx.x * kPartial + k] = r;
    }
}

// Combines the partials and derives the root cube in fp64.
__global__ __launch_bounds__(kBboxThreads) void k_bbox_final(const float *__restrict__ partials,
                                                             uint32_t n_partials, uint32_t n,
                                                             int bits, DevParams *prm)
{
    __shared__ float red[kBboxThreads / 64][kPartial];
    float v[7] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY, 0.0f};
    for (uint32_t b = threadIdx.x; b < n_partials; b += blockDim.x) {
        for (int k = 0; k < 3; ++k) v[k] = fminf(v[k], partials[b * kPartial + k]);
        for (int k = 3; k < 7; ++k) v[k] = fmaxf(v[k], partials[b * kPartial + k]);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int k = 0; k < 3; ++k) v[k] = wave_min(v[k]);
    for (int k = 3; k < 7; ++k) v[k] = wave_max(v[k]);
    if (lane == 0)
        for (int k = 0; k < 7; ++k) red[wave][k] = v[k];
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kBboxThreads / 64; ++w) {
            for (int k = 0; k < 3; ++k) v[k] = fminf(v[k], red[w][k]);
            for (int k = 3; k < 7; ++k) v[k] = fmaxf(v[k], red[w][k]);
        }
        double L = 0.0;
        for (int a = 0; a < 3; ++a) {
            double lo = n ? (double)v[a] : 0.0;
            double hi = n ? (double)v[3 + a] : 0.0;
            prm->lo[a] = lo;
            prm->hi[a] = hi;
            double ext = hi - lo;
            if (ext > L) L = ext;
        }
        prm->L = L;
        // 2^bits / L as one IEEE division
        prm->scale = (L > 0.0) ? __builtin_ldexp(1.0, bits) / L : 0.0;
        prm->status = (v[6] != 0.0f) ? kStatusNonFinite : 0u;
        prm->n_nodes = 0;
        prm->n_src = n;
    }
}

__device__ inline uint64_t spread3(uint64_t v)
{
    // insert two zero bits between consecutive bits of a 21-bit value
    v &= 0x1fffffull;
    v = (v | (v << 32)) & 0x001f00000000ffffull;
    v = (v | (v << 16)) & 0x001f0000ff0000ffull;
    v = (v | (v << 8)) & 0x100f00f00f00f00full;
    v = (v | (v << 4)) & 0x10c30c30c30c30c3ull;
    v = (v | (v << 2)) & 0x1249249249249249ull;
    return v;
}


// Hilbert index of BITS-bit integer coordinates, after Skilling,
// "Programming the Hilbert curve" (AIP Conf. Proc. 707, 2004): the transposed
// index is formed in place (undo excess work from the top bit down, then Gray
// encoding) and its bits are interleaved x, y, z from the most significant
// end, so each 3-bit digit names a child cell in the curve's order.  Every
// cell is still one contiguous key range: the tree is the same, only the
// order of siblings changes.
//
// The level loop is unrolled for the two key widths, each level's choices
// are selects rather than branches, and the final correction (bit i of t is
// the parity of the bits of z above i) is a suffix-parity of z >> 1 in five
// shift-xor steps.
template <int BITS>
__device__ inline uint64_t hilbert3(uint32_t x, uint32_t y, uint32_t z)
{
#pragma unroll
    for (int q = BITS - 1; q >= 1; --q) {
        const uint32_t P = (1u << q) - 1u;
        x ^= ((x >> q) & 1u) ? P : 0u;
        {
            const uint32_t t = (x ^ y) & P;
            const bool set = (y >> q) & 1u;
            x ^= set ? P : t;
            y ^= set ? 0u : t;
        }
        {
            const uint32_t t = (x ^ z) & P;
            const bool set = (z >> q) & 1u;
            x ^= set ? P : t;
            z ^= set ? 0u : t;
        }
    }
    y ^= x;
    z ^= y;
    uint32_t t = z >> 1;
    t ^= t >> 1;
    t ^= t >> 2;
    t ^= t >> 4;
    t ^= t >> 8;
    t ^= t >> 16;
    x ^= t;
    y ^= t;
    z ^= t;
    return spread3(z) | (spread3(y) << 1) | (spread3(x) << 2);
}

template <bool HILBERT, int BITS>
__global__ __launch_bounds__(256) void k_morton(const float4 *__restrict__ pts, uint32_t n,
                                                const DevParams *__restrict__ prm,
                                                uint64_t *__restrict__ keys,
                                                uint32_t *__restrict__ idx)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float4 p = pts[i];
    const uint64_t top = (1ull << BITS) - 1;
    const double s = prm->scale;
    const uint64_t qx = quantise(p.x, prm->lo[0], s, top);
    const uint64_t qy = quantise(p.y, prm->lo[1], s, top);
    const uint64_t qz = quantise(p.z, prm->lo[2], s, top);
    keys[i] = HILBERT ? hilbert3<BITS>((uint32_t)qx, (uint32_t)qy, (uint32_t)qz)
                      : spread3(qx) | (spread3(qy) << 1) | (spread3(qz) << 2);
    idx[i] = i;
}

template <bool HILBERT>
void launch_keys(const float4 *pts, uint32_t n, const DevParams *prm, int bits, uint64_t *keys,
                 uint32_t *idx, hipStream_t s)
{
    const dim3 grid((n + 255) / 256), block(256);
    if (bits == 21)
        hipLaunchKernelGGL((k_morton<HILBERT, 21>), grid, block, 0, s, pts, n, prm, keys, idx);
    else
        hipLaunchKernelGGL((k_morton<HILBERT, 10>), grid, block, 0, s, pts, n, prm, keys, idx);
}

}  // namespace

uint32_t bbox_partials(uint32_t n)
{
    uint32_t b = (n + kBboxThreads * 4 - 1) / (kBboxThreads * 4);
    if (b < 1) b = 1;
    if (b > kBboxMaxBlocks) b = kBboxMaxBlocks;
    return b;
}

void launch_bbox(const float4 *src, uint32_t n, float *partials, uint32_t n_partials,
                 DevParams *prm, int bits, hipStream_t s)
{
    hipLaunchKernelGGL(k_bbox_partial, dim3(n_partials), dim3(kBboxThreads), 0, s, src, n,
                       partials);
    hipLaunchKernelGGL(k_bbox_final, dim3(1), dim3(kBboxThreads), 0, s, partials, n_partials,
                       n, bits, prm);
}

void launch_morton(const float4 *pts, uint32_t n, const DevParams *prm, int bits, int curve,
                   uint64_t *keys, uint32_t *idx, hipStream_t s)
{
    if (n == 0) return;
    // bits is 21 (63-bit keys) or 10 (30-bit keys); bh_create admits no other
    if (curve == 1) launch_keys<true>(pts, n, prm, bits, keys, idx, s);
    else launch_keys<false>(pts, n, prm, bits, keys, idx, s);
}

}  // namespace bh
