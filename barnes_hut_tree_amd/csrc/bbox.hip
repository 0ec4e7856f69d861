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

#include <algorithm>

namespace bh {
constexpr int kHilbertMaxStates = 64;
}

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
// "Programming the Hilbert curve" (AIP Conf. Proc. 707, 2004): from the top
// bit down, each level's bits of (x, y, z) decide operations on all lower
// bits (invert the low bits of x, or exchange them with those of y or z);
// Gray encoding and a parity correction then give the transposed index,
// whose bits interleaved x, y, z from the most significant end are the key,
// so each 3-bit digit names a child cell in the curve's order.  Every cell is
// still one contiguous key range: the tree is the same, only the order of
// siblings changes.
//
// The lower-bit operations compose into one signed permutation of the three
// axes, the same at every lower level, and the parity correction of a level
// is the parity of the Gray-coded z bits above it.  So the transform is a
// finite automaton over the levels: state = (accumulated permutation, parity),
// input = the level's raw bits, output = the level's key digit.  The host
// derives its table once from the operations above (48 states reachable); the
// kernel runs one table lookup (in LDS) per level instead of the level's
// selects and exchanges.
struct HilbertTable {
    uint16_t e[kHilbertMaxStates * 8];   // digit | next state << 3
};

HilbertTable build_hilbert_table()
{
    // a state: map of the 3-bit vectors (x << 2 | y << 1 | z) of a lower level
    // under the operations so far, and the parity of the Gray-coded z bits
    struct State {
        uint8_t T[8];
        int p;
    };
    auto same = [](const State &a, const State &b) {
        for (int v = 0; v < 8; ++v)
            if (a.T[v] != b.T[v]) return false;
        return a.p == b.p;
    };
    State st[kHilbertMaxStates];
    int ns = 1;
    for (int v = 0; v < 8; ++v) st[0].T[v] = (uint8_t)v;
    st[0].p = 0;
    HilbertTable tab{};
    for (int i = 0; i < ns; ++i) {
        for (int r = 0; r < 8; ++r) {
            const int tv = st[i].T[r];   // this level's bits after the operations above
            const int tx = (tv >> 2) & 1, ty = (tv >> 1) & 1, tz = tv & 1;
            // Gray encoding (y ^= x, z ^= y), then the parity correction
            const int gx = tx, gy = ty ^ gx, gz = tz ^ gy;
            const int g = (gx << 2) | (gy << 1) | gz;
            const int digit = st[i].p ? (g ^ 7) : g;
            // this level's operations on the lower bits
            uint8_t U[8];
            for (int v = 0; v < 8; ++v) {
                int x = (v >> 2) & 1, y = (v >> 1) & 1, z = v & 1;
                if (tx) x ^= 1;
                if (ty) x ^= 1; else { const int t = x; x = y; y = t; }
                if (tz) x ^= 1; else { const int t = x; x = z; z = t; }
                U[v] = (uint8_t)((x << 2) | (y << 1) | z);
            }
            State nx;
            for (int v = 0; v < 8; ++v) nx.T[v] = U[st[i].T[v]];
            nx.p = st[i].p ^ gz;
            int id = 0;
            while (id < ns && !same(st[id], nx)) ++id;
            if (id == ns) {
                if (ns == kHilbertMaxStates) return HilbertTable{};   // cannot happen (48 states)
                st[ns++] = nx;
            }
            tab.e[i * 8 + r] = (uint16_t)(digit | (id << 3));
        }
    }
    return tab;
}

}  // namespace

// The automaton's tables indexed by Morton triples (z << 2 | y << 1 | x, the
// triples of the interleaved code): [0, 48 * 64) two levels per entry,
// (digit_hi << 3 | digit_lo) | next state << 6; then [48 * 64, + 48 * 8) one level,
// digit | next state << 3.  False if the automaton does not have the expected
// 48 states (it always does).
bool hilbert_lut_host(uint16_t *out)
{
    const HilbertTable t = build_hilbert_table();
    auto rev3 = [](uint32_t v) { return ((v & 1u) << 2) | (v & 2u) | ((v >> 2) & 1u); };
    uint32_t states = 1;
    for (int k = 0; k < kHilbertMaxStates * 8; ++k) states = std::max(states, (uint32_t)(t.e[k] >> 3) + 1);
    if (states != (uint32_t)kHilbertStates) return false;
    for (uint32_t st = 0; st < (uint32_t)kHilbertStates; ++st) {
        for (uint32_t mt = 0; mt < 8; ++mt)
            out[kHilbertStates * 64 + st * 8 + mt] = t.e[st * 8 + rev3(mt)];
        for (uint32_t hi = 0; hi < 8; ++hi)
            for (uint32_t lo = 0; lo < 8; ++lo) {
                const uint32_t e1 = t.e[st * 8 + rev3(hi)];
                const uint32_t e2 = t.e[(e1 >> 3) * 8 + rev3(lo)];
                out[st * 64 + (hi << 3 | lo)] =
                    (uint16_t)(((e1 & 7u) << 3) | (e2 & 7u) | ((e2 >> 3) << 6));
            }
    }
    return true;
}

namespace {

// Keys of KPT consecutive points per thread.  Hilbert keys: the quantised
// coordinates are interleaved into the Morton code first (z y x in each 3-bit
// triple), and the automaton then reads two levels per lookup, a 6-bit field of
// that code, from the two-level table (copied into LDS); an odd level count
// ends with one one-level lookup.
constexpr int kKeyThreads = 256;
constexpr int kKeysPerThread = 2;

template <bool HILBERT, int BITS>
__global__ __launch_bounds__(kKeyThreads) void k_morton(const float4 *__restrict__ pts, uint32_t n,
                                                        const DevParams *__restrict__ prm,
                                                        const uint16_t *__restrict__ hlut,
                                                        uint64_t *__restrict__ keys,
                                                        uint32_t *__restrict__ idx)
{
    __shared__ __attribute__((aligned(16))) uint16_t lut[HILBERT ? kHilbertLutEntries : 8];
    if (HILBERT) {
        const uint4 *g = reinterpret_cast<const uint4 *>(hlut);
        uint4 *l = reinterpret_cast<uint4 *>(lut);
        for (int k = threadIdx.x; k < kHilbertLutEntries / 8; k += kKeyThreads) l[k] = g[k];
        __syncthreads();
    }
    const uint16_t *lut2 = lut, *lut1 = lut + kHilbertStates * 64;
    const uint64_t top = (1ull << BITS) - 1;
    // 2^BITS / L as one IEEE division: the tree's own scale when BITS is the
    // tree's depth, and a coarser grid on the same cube for ordering targets
    const double L = prm->L;
    const double s = (L > 0.0) ? __builtin_ldexp(1.0, BITS) / L : 0.0;
    const uint32_t base = blockIdx.x * (kKeyThreads * kKeysPerThread) + threadIdx.x;
#pragma unroll
    for (int t = 0; t < kKeysPerThread; ++t) {
        const uint32_t i = base + t * kKeyThreads;
        if (i >= n) break;
        const float4 p = pts[i];
        const uint64_t qx = quantise(p.x, prm->lo[0], s, top);
        const uint64_t qy = quantise(p.y, prm->lo[1], s, top);
        const uint64_t qz = quantise(p.z, prm->lo[2], s, top);
        const uint64_t m = spread3(qx) | (spread3(qy) << 1) | (spread3(qz) << 2);
        uint64_t key = m;
        if (HILBERT) {
            uint32_t state = 0;
            key = 0;
#pragma unroll
            for (int q = BITS - 1; q >= 1; q -= 2) {
                const uint32_t f = (uint32_t)(m >> (3 * (q - 1))) & 63u;
                const uint32_t e = lut2[state * 64 + f];
                key = (key << 6) | (e & 63u);
                state = e >> 6;
            }
            if (BITS & 1) {
                const uint32_t e = lut1[state * 8 + ((uint32_t)m & 7u)];
                key = (key << 3) | (e & 7u);
            }
        }
        keys[i] = key;
        idx[i] = i;
    }
}

template <bool HILBERT>
void launch_keys(const float4 *pts, uint32_t n, const DevParams *prm, int bits,
                 const uint16_t *hlut, uint64_t *keys, uint32_t *idx, hipStream_t s)
{
    const dim3 grid((n + kKeyThreads * kKeysPerThread - 1) / (kKeyThreads * kKeysPerThread));
    const dim3 block(kKeyThreads);
    if (bits == 21)
        hipLaunchKernelGGL((k_morton<HILBERT, 21>), grid, block, 0, s, pts, n, prm, hlut, keys, idx);
    else
        hipLaunchKernelGGL((k_morton<HILBERT, 10>), grid, block, 0, s, pts, n, prm, hlut, keys, idx);
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
                   const uint16_t *hilbert_lut, uint64_t *keys, uint32_t *idx, hipStream_t s)
{
    if (n == 0) return;
    // bits is 21 (63-bit keys) or 10 (30-bit keys); bh_create admits no other
    if (curve == 1) launch_keys<true>(pts, n, prm, bits, hilbert_lut, keys, idx, s);
    else launch_keys<false>(pts, n, prm, bits, hilbert_lut, keys, idx, s);
}

}  // namespace bh
