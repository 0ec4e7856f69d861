// The all-pairs direct sum: every target against every source with the same
// softened interaction as the tree walk.  It is the brute-force reference the
// walk's speed and accuracy are measured against ([GASPHiA] 精度与加速比验证)
// and the theta -> 0 limit of the walk.
//
// One lane per target.  All lanes of a wave need the same source at the same
// time, so sources come through scalar loads, 16 (256 bytes) per batch, and
// feed the vector instructions as scalar operands: 13 vector instructions and
// one reciprocal square root per pair.  (Copying each source into vector
// registers and reusing it for several targets per lane measured slower: the
// scalar operand spares a vector-register read.)  Each lane sums in fp32 over
// runs of kChunk sources and folds every run into fp64 totals, so a
// million-term sum keeps the rounding error of a few-hundred-term one.
#include "bh_internal.h"
#include "interaction.h"

namespace bh {
namespace {

constexpr int kDirectThreads = 256;
constexpr uint32_t kBatch = 16;    // sources per batch of scalar loads
constexpr uint32_t kChunk = 512;   // sources per fp32 partial sum
static_assert(kChunk % kBatch == 0, "runs hold whole batches");

// Sources [c, ce) (a multiple of kBatch long) against the lane's target.
// MASK: the run may hold the lane's own particle i, whose mass is masked out
// (the self pair).
template <bool SOFT, bool MASK>
__device__ __attribute__((always_inline)) inline void run(const float4 *__restrict__ src,
                                                          uint32_t c, uint32_t ce, uint32_t i,
                                                          float4 p, float eps2, float &ax,
                                                          float &ay, float &az, float &pot)
{
    for (uint32_t j = c; j < ce; j += kBatch) {
        const float4 *q = src + j;
        float4 s[kBatch];
#pragma unroll
        for (uint32_t k = 0; k < kBatch; ++k) s[k] = q[k];
        asm volatile("" ::: "memory");   // issue the whole batch of loads first
#pragma unroll
        for (uint32_t k = 0; k < kBatch; ++k) {
            float4 t = s[k];
            if (MASK) t.w = (j + k == i) ? 0.f : t.w;
            pair<SOFT>(t, p.x, p.y, p.z, eps2, ax, ay, az, pot);
        }
    }
}

template <bool SOFT, bool SELF>
__global__ __launch_bounds__(kDirectThreads) void k_direct(const float4 *__restrict__ src,
                                                           uint32_t n,
                                                           const float4 *__restrict__ tgt,
                                                           uint32_t nt, float G, float eps2,
                                                           float4 *__restrict__ out)
{
    const uint32_t base = __builtin_amdgcn_readfirstlane(blockIdx.x * kDirectThreads +
                                                         (threadIdx.x & ~63u));
    if (base >= nt) return;
    const uint32_t i = base + (threadIdx.x & 63u);
    const float4 p = tgt[min(i, nt - 1u)];

    double sx = 0.0, sy = 0.0, sz = 0.0, sp = 0.0;
    const uint32_t nb = n & ~(kBatch - 1);
    for (uint32_t c = 0; c < nb; c += kChunk) {
        const uint32_t ce = min(c + kChunk, nb);
        float ax = 0.f, ay = 0.f, az = 0.f, pot = 0.f;
        if (SELF && SOFT && c < base + 64u && base < ce)
            run<SOFT, true>(src, c, ce, i, p, eps2, ax, ay, az, pot);
        else
            run<SOFT, false>(src, c, ce, i, p, eps2, ax, ay, az, pot);
        sx += ax;
        sy += ay;
        sz += az;
        sp += pot;
    }

    // the last n mod kBatch sources, one at a time
    float ax = 0.f, ay = 0.f, az = 0.f, pot = 0.f;
    for (uint32_t j = nb; j < n; ++j) {
        float4 t = src[j];
        if (SELF && SOFT) t.w = (j == i) ? 0.f : t.w;
        pair<SOFT>(t, p.x, p.y, p.z, eps2, ax, ay, az, pot);
    }
    const double g = G;
    if (i < nt)
        out[i] = make_float4((float)(g * (sx + ax)), (float)(g * (sy + ay)),
                             (float)(g * (sz + az)), (float)(g * (sp + pot)));
}

template <bool SOFT, bool SELF>
void launch2(const float4 *src, uint32_t n, const float4 *tgt, uint32_t nt, float G, float eps2,
             float4 *out, hipStream_t s)
{
    const uint32_t grid = (nt + kDirectThreads - 1) / kDirectThreads;
    hipLaunchKernelGGL((k_direct<SOFT, SELF>), dim3(grid), dim3(kDirectThreads), 0, s, src, n,
                       tgt, nt, G, eps2, out);
}

}  // namespace

void launch_direct(const float4 *src, uint32_t n, const float4 *tgt, uint32_t nt, bool self,
                   float G, float eps, float4 *out, hipStream_t s)
{
    if (nt == 0) return;
    const float eps2 = eps * eps;
    const float4 *t = self ? src : tgt;
    if (eps2 > 0.f) {
        if (self) launch2<true, true>(src, n, t, nt, G, eps2, out, s);
        else launch2<true, false>(src, n, t, nt, G, eps2, out, s);
    } else {
        // without softening the self pair (distance zero) adds nothing by itself
        launch2<false, false>(src, n, t, nt, G, eps2, out, s);
    }
}

}  // namespace bh
