// Time stepping around the gravity step.  The pages advance their 5M-particle
// galaxy collision in time ([GASPHiA], page header) without naming the
// integrator; this is the kick-drift-kick leapfrog with the tree rebuilt
// from the new positions every step, plus the conserved quantities used to
// watch it (mass, kinetic and potential energy, momentum, angular momentum).
#include "bh_internal.h"

namespace bh {
namespace {

constexpr int kStepThreads = 256;
constexpr int kDiagThreads = 256;

// v += a dt_kick, then x += v dt_drift (the mass in x.w is untouched).
template <bool KICK, bool DRIFT>
__global__ __launch_bounds__(kStepThreads) void k_kick_drift(float4 *__restrict__ pos,
                                                             float4 *__restrict__ vel,
                                                             const float4 *__restrict__ acc,
                                                             uint32_t n, float dtk, float dtd)
{
    const uint32_t i = blockIdx.x * kStepThreads + threadIdx.x;
    if (i >= n) return;
    float4 v = vel[i];
    if (KICK) {
        const float4 a = acc[i];
        v.x = fmaf(a.x, dtk, v.x);
        v.y = fmaf(a.y, dtk, v.y);
        v.z = fmaf(a.z, dtk, v.z);
        vel[i] = v;
    }
    if (DRIFT) {
        float4 p = pos[i];
        p.x = fmaf(v.x, dtd, p.x);
        p.y = fmaf(v.y, dtd, p.y);
        p.z = fmaf(v.z, dtd, p.z);
        pos[i] = p;
    }
}

__device__ inline double wave_sum(double v)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum of kDiagTerms per-particle terms over a workgroup; thread 0 gets the totals.
__device__ inline void block_sum(double (&t)[kDiagTerms], double (*lds)[kDiagTerms])
{
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kDiagTerms; ++q) t[q] = wave_sum(t[q]);
    if (lane == 0)
#pragma unroll
        for (int q = 0; q < kDiagTerms; ++q) lds[wave][q] = t[q];
    __syncthreads();
    if (threadIdx.x == 0)
        for (uint32_t w = 1; w < kDiagThreads / 64; ++w)
#pragma unroll
            for (int q = 0; q < kDiagTerms; ++q) t[q] += lds[w][q];
}

// Per-workgroup fp64 partial sums (grid-stride over the particles):
// mass, kinetic, potential (phi m / 2), momentum xyz, angular momentum xyz, count.
__global__ __launch_bounds__(kDiagThreads) void k_diag_partial(const float4 *__restrict__ pos,
                                                               const float4 *__restrict__ vel,
                                                               const float4 *__restrict__ acc,
                                                               uint32_t n,
                                                               double *__restrict__ partials)
{
    __shared__ double lds[kDiagThreads / 64][kDiagTerms];
    double t[kDiagTerms] = {};
    for (uint32_t i = blockIdx.x * kDiagThreads + threadIdx.x; i < n;
         i += gridDim.x * kDiagThreads) {
        const float4 p = pos[i], v = vel[i];
        const double m = p.w, vx = v.x, vy = v.y, vz = v.z, x = p.x, y = p.y, z = p.z;
        t[0] += m;
        t[1] += 0.5 * m * (vx * vx + vy * vy + vz * vz);
        t[2] += 0.5 * m * (double)acc[i].w;
        t[3] += m * vx;
        t[4] += m * vy;
        t[5] += m * vz;
        t[6] += m * (y * vz - z * vy);
        t[7] += m * (z * vx - x * vz);
        t[8] += m * (x * vy - y * vx);
        t[9] += 1.0;
    }
    block_sum(t, lds);
    if (threadIdx.x == 0)
#pragma unroll
        for (int q = 0; q < kDiagTerms; ++q) partials[blockIdx.x * kDiagTerms + q] = t[q];
}

// One workgroup adds the partials in a fixed order.
__global__ __launch_bounds__(kDiagThreads) void k_diag_final(const double *__restrict__ partials,
                                                             uint32_t n_partials,
                                                             double *__restrict__ out)
{
    __shared__ double lds[kDiagThreads / 64][kDiagTerms];
    double t[kDiagTerms] = {};
    for (uint32_t k = threadIdx.x; k < n_partials; k += kDiagThreads)
#pragma unroll
        for (int q = 0; q < kDiagTerms; ++q) t[q] += partials[k * kDiagTerms + q];
    block_sum(t, lds);
    if (threadIdx.x == 0)
#pragma unroll
        for (int q = 0; q < kDiagTerms; ++q) out[q] = t[q];
}

}  // namespace

void launch_kick_drift(float4 *pos, float4 *vel, const float4 *acc, uint32_t n, float dt_kick,
                       float dt_drift, hipStream_t s)
{
    if (n == 0) return;
    const dim3 grid((n + kStepThreads - 1) / kStepThreads), block(kStepThreads);
    const bool kick = dt_kick != 0.f, drift = dt_drift != 0.f;
    if (kick && drift)
        hipLaunchKernelGGL((k_kick_drift<true, true>), grid, block, 0, s, pos, vel, acc, n, dt_kick,
                           dt_drift);
    else if (kick)
        hipLaunchKernelGGL((k_kick_drift<true, false>), grid, block, 0, s, pos, vel, acc, n, dt_kick,
                           dt_drift);
    else if (drift)
        hipLaunchKernelGGL((k_kick_drift<false, true>), grid, block, 0, s, pos, vel, acc, n,
                           dt_kick, dt_drift);
}

uint32_t diag_partials(uint32_t n)
{
    const uint32_t b = (n + kDiagThreads - 1) / kDiagThreads;
    return b < 1 ? 1 : (b > kDiagMaxPartials ? kDiagMaxPartials : b);
}

void launch_diagnostics(const float4 *pos, const float4 *vel, const float4 *acc, uint32_t n,
                        double *partials, double *out, hipStream_t s)
{
    const uint32_t nb = diag_partials(n);
    hipLaunchKernelGGL(k_diag_partial, dim3(nb), dim3(kDiagThreads), 0, s, pos, vel, acc, n,
                       partials);
    hipLaunchKernelGGL(k_diag_final, dim3(1), dim3(kDiagThreads), 0, s, partials, nb, out);
}

}  // namespace bh
