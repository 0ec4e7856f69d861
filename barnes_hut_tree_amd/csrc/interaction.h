// One softened gravitational interaction, shared by the tree walk and the
// direct sum ([GASPHiA] 计算自引力): the source (x, y, z, m) pulls the target
// at p with acceleration m d / (|d|^2 + eps^2)^(3/2) and adds -m /
// (|d|^2 + eps^2)^(1/2) to its potential, d = source - target (G is applied
// once, to the finished sums).  Without softening (SOFT = false) a pair at
// distance zero adds nothing.
#pragma once

#include <hip/hip_runtime.h>

namespace bh {

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

}  // namespace bh
