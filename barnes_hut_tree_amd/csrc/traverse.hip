// The tree walk: accelerations and potentials of a Morton-ordered batch of
// targets ([GASPHiA] 计算自引力, 性能瓶颈分析).
//
// One wavefront walks the tree for 64 consecutive sorted targets.  The node it
// visits is wave-uniform, so node records come through scalar loads and are
// broadcast to all lanes for free.  The walk is stackless: nodes sit in
// pre-order, a subtree spans [node, skip), and each lane keeps a rejoin index,
// the next node it must see (initially the root).  At node X the lanes with
// rejoin <= X apply the opening test of the pages, (w/theta)^2 < r^2 with w
// the cell edge and r the distance to the centre of mass.  Lanes that pass
// add one monopole term and set rejoin = skip(X).  The others open X;
// a 64-lane ballot of them decides the wave's next node: X + 1 (the first
// child) if any lane opened an internal node, else skip(X).  An opened leaf
// is summed particle by particle by the lanes that opened it.
//
// A lane that accepted an ancestor of the current node waits for that
// ancestor's skip, which is at or beyond skip(X); the wave reaches it exactly
// when it leaves that subtree.  So every lane sees exactly the nodes its own
// particle-by-particle walk would visit (the pages' warp vote instead makes
// all lanes descend when any lane must; here the ballot only decides where
// the wave goes, and the per-lane rejoin index keeps each lane's result its
// own).
//
// The walk is a loop written in assembly: node visits, descents and the sums
// of opened leaves, with each next node record requested before the current
// visit's arithmetic.  The build writes an end record after the last node,
// which every lane still walking opens, so the loop needs no bound check; it
// returns to C++ at that record and at leaves that may hold the wave's own
// targets, where the self pair is masked.
#include <algorithm>

#include "bh_internal.h"
#include "interaction.h"

namespace bh {
namespace {

constexpr int kWalkThreads = 64;

// One source of an opened leaf: the interaction of pair() (interaction.h),
// with eps2 taken from a vector register and the potential term subtracted
// after rounding instead of fused.  A vector op with a scalar-register
// operand issues at about 0.9 wave instructions per cycle per CU, one with
// register operands only at 1.3-1.9, and this keeps two of the thirteen ops
// register-only.
template <bool SOFT>
__device__ __attribute__((always_inline)) inline void leaf_pair(float4 s, float px, float py,
                                                                float pz, float eps2v, float &ax,
                                                                float &ay, float &az, float &pot)
{
#pragma clang fp contract(off)
    const float dx = s.x - px, dy = s.y - py, dz = s.z - pz;
    const float r2 = fmaf(dz, dz, fmaf(dy, dy, fmaf(dx, dx, eps2v)));
    float inv = __builtin_amdgcn_rsqf(r2);
    if (!SOFT) inv = r2 > 0.f ? inv : 0.f;
    const float mi = s.w * inv;
    const float f = mi * inv * inv;
    ax = fmaf(f, dx, ax);
    ay = fmaf(f, dy, ay);
    az = fmaf(f, dz, az);
    pot = pot - mi;
}

// Direct sum over the sources [b, e) of an opened leaf, eight at a time (one
// batch of scalar loads per eight).  MINE: the leaf may hold this lane's own
// particle i, whose mass is masked out.
template <bool SOFT, bool MINE>
__device__ __attribute__((always_inline)) inline void leaf_tile(
    const float4 *__restrict__ src, uint32_t b, uint32_t e, uint32_t i, float4 p, float eps2,
    float &ax, float &ay, float &az, float &pot)
{
    for (uint32_t j = b; j < e; j += 8) {
        const float4 *q = src + j;
        float4 s[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] = q[k];
        asm volatile("" ::: "memory");   // issue all eight loads first
        const uint32_t left = e - j;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if ((uint32_t)k < left) {
                if (MINE) s[k].w = (j + k == i) ? 0.f : s[k].w;
                leaf_pair<SOFT>(s[k], p.x, p.y, p.z, eps2, ax, ay, az, pot);
            }
        }
    }
}

__device__ inline uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// The assembly loop of the walk.  Register use: the node records of two
// consecutive visits land in s[32:39] and s[40:47] (x, y, z, m, start, count,
// skip, meta), so the next visit's node index is the previous record's skip
// field where it lies; a leaf's sources are loaded six at a time into
// s[16:31] and the leaf's own record slot, their address formed in
// s[48:49].  These fixed registers sit low: a kernel's scalar register count
// is its highest register used, and the walk keeps eight waves per SIMD only
// up to about 76 (measured: 70 registers gave 8 resident waves, 90 gave 7, 96
// gave 6, and the walk ran 7% faster at 68 than at 90 with the same code).
//
// The loop is bound by the latency of each visit's scalar load of its node
// record together with the vector issue, so the record of the next visit is
// requested as early as its index is known.  Moves to
// the skip are the common case (a wave descends into about one node in five
// it visits), so when a record arrives the loop at once requests the record
// at its skip into the other slot, before any arithmetic; the wave moves
// there when no lane opens the node, a descent waits for that request and
// then requests X + 1 instead, and an opened leaf (whose skip is X + 1) keeps
// it while its sources pass through the leaf's own slot.  Only in-bounds
// records are requested: skips point at most at the end record, whose own
// skip is itself.
//
// One visit of node XR (record slot R0..R7, the other slot OTHER):
//   act  = rejoin <= X                         (vcc, then exec)
//   s    = r^2 + eps^2, accumulated from eps^2 by three fused steps
//   far  = T + eps^2 < s (the record holds T + eps^2), by a compare that also
//          narrows exec to act & far: the opening test T < r^2 on the softened
//          scale, whose s is also the monopole's argument
//   open = act & ~exec                          (SCC: some lane opens X)
//   lanes in act & far add the monopole (their rejoin moves to the node's
//   skip only where the wave descends into the node or returns, below)
// The monopole is inv = rsq(s), f = m inv^3, a += f d, pot -= m inv, with
// eps^2 in a vector register and the potential term unfused, so that all but
// the node-field operands are register-only.  At least one instruction
// sits between the reciprocal square root and the first use of its result,
// which the hardware requires.  %[off] holds X + 1 from the head on.
// CNT: the interaction count update, if any.
#define BH_HEAD(R0, R1, R2, R6, R7, XR, OTHER)                                         \
    "v_cmp_ge_u32_e32 vcc, " XR ", %[rej]\n"                                           \
    "s_add_u32 %[off], " XR ", 32\n"                                                   \
    "s_waitcnt lgkmcnt(0)\n"                                                           \
    "s_load_dwordx8 " OTHER ", %[nb], " R6 "\n"                                        \
    "v_sub_f32_e32 %[dx], " R0 ", %[px]\n"                                             \
    "v_sub_f32_e32 %[dy], " R1 ", %[py]\n"                                             \
    "v_fma_f32 %[r2], %[dx], %[dx], %[eps2]\n"                                         \
    "v_sub_f32_e32 %[dz], " R2 ", %[pz]\n"                                             \
    "v_fmac_f32_e32 %[r2], %[dy], %[dy]\n"                                             \
    "v_fmac_f32_e32 %[r2], %[dz], %[dz]\n"                                             \
    "s_and_saveexec_b64 %[save], vcc\n"                                                \
    "v_cmpx_lt_f32_e64 %[far], |" R7 "|, %[r2]\n"                                      \
    "v_rsq_f32_e32 %[w], %[r2]\n"                                                      \
    "s_andn2_b64 %[open], vcc, exec\n"
#define BH_MONO(R3, CNT)                                                               \
    "v_mul_f32_e32 %[f], " R3 ", %[w]\n"                                               \
    "v_sub_f32_e32 %[pot], %[pot], %[f]\n"                                             \
    "v_mul_f32_e32 %[f], %[w], %[f]\n"                                                 \
    "v_mul_f32_e32 %[f], %[w], %[f]\n"                                                 \
    "v_fmac_f32_e32 %[ax], %[f], %[dx]\n"                                              \
    "v_fmac_f32_e32 %[ay], %[f], %[dy]\n"                                              \
    "v_fmac_f32_e32 %[az], %[f], %[dz]\n"                                              \
    CNT
#define BH_FETCH(NX, OTHER)                                                            \
    "s_load_dwordx8 " OTHER ", %[nb], " NX "\n"

// One source of a leaf opened in the assembly loop, in the order of
// leaf_pair(): X, Y, Z, M name the source's scalar registers.  GUARD is the
// r^2 > 0 test of the unsoftened interaction (with softening, a nop keeps
// the reciprocal square root one instruction from its first use).
#define BH_PAIR(X, Y, Z, M, GUARD, NEXT)                                               \
    "v_sub_f32_e32 %[dx], " X ", %[px]\n"                                              \
    "v_sub_f32_e32 %[dy], " Y ", %[py]\n"                                              \
    "v_fma_f32 %[r2], %[dx], %[dx], %[eps2]\n"                                         \
    "v_sub_f32_e32 %[dz], " Z ", %[pz]\n"                                              \
    "v_fmac_f32_e32 %[r2], %[dy], %[dy]\n"                                             \
    "v_fmac_f32_e32 %[r2], %[dz], %[dz]\n"                                             \
    "v_rsq_f32_e32 %[w], %[r2]\n"                                                      \
    GUARD(NEXT)                                                                        \
    "v_mul_f32_e32 %[f], " M ", %[w]\n"                                                \
    "v_sub_f32_e32 %[pot], %[pot], %[f]\n"                                             \
    "v_mul_f32_e32 %[f], %[w], %[f]\n"                                                 \
    "v_mul_f32_e32 %[f], %[w], %[f]\n"                                                 \
    "v_fmac_f32_e32 %[ax], %[f], %[dx]\n"                                              \
    "v_fmac_f32_e32 %[ay], %[f], %[dy]\n"                                              \
    "v_fmac_f32_e32 %[az], %[f], %[dz]\n"
#define BH_GUARD_SOFT(NEXT) NEXT
#define BH_GUARD_HARD(NEXT)                                                            \
    NEXT                                                                               \
    "v_cmp_lt_f32_e32 vcc, 0, %[r2]\n"                                                 \
    "v_cndmask_b32_e32 %[w], 0, %[w], vcc\n"
// NEXT, the instruction that fills the slot after the reciprocal square root,
// is the bounds compare of the batch's next source (a scalar instruction;
// the vector ops between it and its branch leave SCC alone), or a nop after
// the last source
#define BH_NEXT(K) "s_cmp_lt_u32 %[left], " #K "\n"
#define BH_LAST "s_nop 0\n"

// Visits from node X on, two per loop turn (slots A and B).  A node no lane
// opens moves the wave to its skip, whose record is already on its way into
// the other slot; an opened internal node (meta without the leaf bit) to
// X + 1; an opened leaf is summed by its openers, six sources per batch (one
// 64-byte and one 32-byte scalar load; the batch address, in s[48:49], is
// formed in 64 bits), and the wave moves on to its skip, the record already
// in the other slot.  The loop returns to the caller at the end record (count
// 0) and at a leaf that may hold the wave's own targets ([first, first +
// count) meets [wb, wbe)), whose self pairs the caller masks; X and the
// leaf's start, count and skip are then the outputs, and nothing is left in
// flight into the fixed registers.  Every step moves X forward, and the end
// record ends the loop at the latest.
// The lanes that used the node just visited (act & ~open, with act still in
// vcc) sit out its subtree: rejoin = its skip.  Needed only when the wave
// descends into that subtree or returns to the caller; when it moves to the
// skip itself, or past an opened leaf (skip = X + 1), they are active there.
#define BH_SIT_OUT(SKIP)                                                               \
    "s_andn2_b64 exec, vcc, %[open]\n"                                                 \
    "v_mov_b32_e32 %[rej], " SKIP "\n"                                                 \
    "s_mov_b64 exec, %[save]\n"

#define BH_RUN(CNT, LEAF_CNT, G)                                                       \
    "s_mov_b32 s46, %[X]\n"                                                            \
    BH_FETCH("s46", "s[32:39]")                                                        \
    "BH_A%=:\n"                                                                        \
    BH_HEAD("s32", "s33", "s34", "s38", "s39", "s46", "s[40:47]")                      \
    "s_cbranch_scc1 BH_OA%=\n"                                                         \
    BH_MONO("s35", CNT)                                                                \
    "s_mov_b64 exec, %[save]\n"                                                        \
    "BH_B%=:\n"                                                                        \
    BH_HEAD("s40", "s41", "s42", "s46", "s47", "s38", "s[32:39]")                      \
    "s_cbranch_scc1 BH_OB%=\n"                                                         \
    BH_MONO("s43", CNT)                                                                \
    "s_mov_b64 exec, %[save]\n"                                                        \
    "s_branch BH_A%=\n"                                                                \
    "BH_OA%=:\n"                                                                       \
    "s_bitcmp1_b32 s39, 31\n"                                                           \
    "s_cbranch_scc1 BH_KA%=\n"                                                         \
    "s_waitcnt lgkmcnt(0)\n"                                                           \
    BH_FETCH("%[off]", "s[40:47]")                                                     \
    "s_cbranch_execz BH_NA%=\n"                                                        \
    BH_MONO("s35", CNT)                                                                \
    "BH_NA%=:\n"                                                                       \
    BH_SIT_OUT("s38")                                                                  \
    "s_mov_b32 s38, %[off]\n"                                                          \
    "s_branch BH_B%=\n"                                                                \
    "BH_OB%=:\n"                                                                       \
    "s_bitcmp1_b32 s47, 31\n"                                                           \
    "s_cbranch_scc1 BH_KB%=\n"                                                         \
    "s_waitcnt lgkmcnt(0)\n"                                                           \
    BH_FETCH("%[off]", "s[32:39]")                                                     \
    "s_cbranch_execz BH_NB%=\n"                                                        \
    BH_MONO("s43", CNT)                                                                \
    "BH_NB%=:\n"                                                                       \
    BH_SIT_OUT("s46")                                                                  \
    "s_mov_b32 s46, %[off]\n"                                                          \
    "s_branch BH_A%=\n"                                                                \
    "BH_KA%=:\n"                                                                       \
    "s_lshl_b32 s48, s36, 4\n"                                                           \
    "s_lshr_b32 s49, s36, 28\n"                                                          \
    "s_add_u32 s48, s48, %[srclo]\n"                                                   \
    "s_addc_u32 s49, s49, %[srchi]\n"                                                  \
    "s_load_dwordx16 s[16:31], s[48:49], 0x0\n"                                        \
    "s_cbranch_execz BH_MA%=\n"                                                        \
    BH_MONO("s35", CNT)                                                                \
    "BH_MA%=:\n"                                                                       \
    "s_mov_b64 exec, %[save]\n"                                                        \
    "s_sub_u32 %[X], %[off], 32\n"                                                      \
    "s_mov_b32 %[first], s36\n"                                                        \
    "s_mov_b32 %[cnt], s37\n"                                                          \
    "s_mov_b32 %[skip], s38\n"                                                         \
    "BH_LA%=:\n"                                                                       \
    "s_cmp_eq_u32 %[cnt], 0\n"                                                         \
    "s_cbranch_scc1 BH_E%=\n"                                                          \
    "s_add_u32 %[le], %[first], %[cnt]\n"                                              \
    "s_cmp_lt_u32 %[first], %[wbe]\n"                                                  \
    "s_cbranch_scc0 BH_LNA%=\n"                                                        \
    "s_cmp_gt_u32 %[le], %[wb]\n"                                                      \
    "s_cbranch_scc1 BH_E%=\n"                                                          \
    "BH_LNA%=:\n"                                                                      \
    "s_and_saveexec_b64 %[save], %[open]\n"                                            \
    "s_mov_b32 %[j], %[first]\n"                                                       \
    "s_branch BH_LFA%=\n"                                                               \
    "BH_LTA%=:\n"                                                                      \
    "s_lshl_b32 s48, %[j], 4\n"                                                        \
    "s_lshr_b32 s49, %[j], 28\n"                                                       \
    "s_add_u32 s48, s48, %[srclo]\n"                                                   \
    "s_addc_u32 s49, s49, %[srchi]\n"                                                  \
    "s_load_dwordx16 s[16:31], s[48:49], 0x0\n"                                        \
    "BH_LFA%=:\n"                                                                      \
    "s_load_dwordx8 s[32:39], s[48:49], 0x40\n"                                        \
    "s_sub_u32 %[left], %[le], %[j]\n"                                                 \
    "s_waitcnt lgkmcnt(0)\n"                                                           \
    BH_PAIR("s16", "s17", "s18", "s19", G, BH_NEXT(2)) "s_cbranch_scc1 BH_LDA%=\n"     \
    BH_PAIR("s20", "s21", "s22", "s23", G, BH_NEXT(3)) "s_cbranch_scc1 BH_LDA%=\n"     \
    BH_PAIR("s24", "s25", "s26", "s27", G, BH_NEXT(4)) "s_cbranch_scc1 BH_LDA%=\n"     \
    BH_PAIR("s28", "s29", "s30", "s31", G, BH_NEXT(5)) "s_cbranch_scc1 BH_LDA%=\n"     \
    BH_PAIR("s32", "s33", "s34", "s35", G, BH_NEXT(6)) "s_cbranch_scc1 BH_LDA%=\n"     \
    BH_PAIR("s36", "s37", "s38", "s39", G, BH_LAST)                                    \
    "s_add_u32 %[j], %[j], 6\n"                                                        \
    "s_cmp_lt_u32 %[j], %[le]\n"                                                       \
    "s_cbranch_scc1 BH_LTA%=\n"                                                        \
    "BH_LDA%=:\n"                                                                      \
    LEAF_CNT                                                                           \
    "s_mov_b64 exec, %[save]\n"                                                        \
    "s_mov_b32 s38, %[skip]\n"                                                         \
    "s_branch BH_B%=\n"                                                                \
    "BH_KB%=:\n"                                                                       \
    "s_lshl_b32 s48, s44, 4\n"                                                           \
    "s_lshr_b32 s49, s44, 28\n"                                                          \
    "s_add_u32 s48, s48, %[srclo]\n"                                                   \
    "s_addc_u32 s49, s49, %[srchi]\n"                                                  \
    "s_load_dwordx16 s[16:31], s[48:49], 0x0\n"                                        \
    "s_cbranch_execz BH_MB%=\n"                                                        \
    BH_MONO("s43", CNT)                                                                \
    "BH_MB%=:\n"                                                                       \
    "s_mov_b64 exec, %[save]\n"                                                        \
    "s_sub_u32 %[X], %[off], 32\n"                                                      \
    "s_mov_b32 %[first], s44\n"                                                        \
    "s_mov_b32 %[cnt], s45\n"                                                          \
    "s_mov_b32 %[skip], s46\n"                                                         \
    "BH_LB%=:\n"                                                                       \
    "s_cmp_eq_u32 %[cnt], 0\n"                                                         \
    "s_cbranch_scc1 BH_E%=\n"                                                          \
    "s_add_u32 %[le], %[first], %[cnt]\n"                                              \
    "s_cmp_lt_u32 %[first], %[wbe]\n"                                                  \
    "s_cbranch_scc0 BH_LNB%=\n"                                                        \
    "s_cmp_gt_u32 %[le], %[wb]\n"                                                      \
    "s_cbranch_scc1 BH_E%=\n"                                                          \
    "BH_LNB%=:\n"                                                                      \
    "s_and_saveexec_b64 %[save], %[open]\n"                                            \
    "s_mov_b32 %[j], %[first]\n"                                                       \
    "s_branch BH_LFB%=\n"                                                               \
    "BH_LTB%=:\n"                                                                      \
    "s_lshl_b32 s48, %[j], 4\n"                                                        \
    "s_lshr_b32 s49, %[j], 28\n"                                                       \
    "s_add_u32 s48, s48, %[srclo]\n"                                                   \
    "s_addc_u32 s49, s49, %[srchi]\n"                                                  \
    "s_load_dwordx16 s[16:31], s[48:49], 0x0\n"                                        \
    "BH_LFB%=:\n"                                                                      \
    "s_load_dwordx8 s[40:47], s[48:49], 0x40\n"                                        \
    "s_sub_u32 %[left], %[le], %[j]\n"                                                 \
    "s_waitcnt lgkmcnt(0)\n"                                                           \
    BH_PAIR("s16", "s17", "s18", "s19", G, BH_NEXT(2)) "s_cbranch_scc1 BH_LDB%=\n"     \
    BH_PAIR("s20", "s21", "s22", "s23", G, BH_NEXT(3)) "s_cbranch_scc1 BH_LDB%=\n"     \
    BH_PAIR("s24", "s25", "s26", "s27", G, BH_NEXT(4)) "s_cbranch_scc1 BH_LDB%=\n"     \
    BH_PAIR("s28", "s29", "s30", "s31", G, BH_NEXT(5)) "s_cbranch_scc1 BH_LDB%=\n"     \
    BH_PAIR("s40", "s41", "s42", "s43", G, BH_NEXT(6)) "s_cbranch_scc1 BH_LDB%=\n"     \
    BH_PAIR("s44", "s45", "s46", "s47", G, BH_LAST)                                    \
    "s_add_u32 %[j], %[j], 6\n"                                                        \
    "s_cmp_lt_u32 %[j], %[le]\n"                                                       \
    "s_cbranch_scc1 BH_LTB%=\n"                                                        \
    "BH_LDB%=:\n"                                                                      \
    LEAF_CNT                                                                           \
    "s_mov_b64 exec, %[save]\n"                                                        \
    "s_mov_b32 s46, %[skip]\n"                                                         \
    "s_branch BH_A%=\n"                                                                \
    "BH_E%=:\n"                                                                        \
    "s_waitcnt lgkmcnt(0)\n"                                                           \
    BH_SIT_OUT("%[skip]")

#define BH_RUN_OUTS                                                                    \
    [X] "+s"(X), [ax] "+v"(ax), [ay] "+v"(ay), [az] "+v"(az), [pot] "+v"(pot),        \
        [rej] "+v"(rejoin), [first] "=&s"(first), [cnt] "=&s"(cnt), [skip] "=&s"(skip), \
        [dx] "=&v"(dx), [dy] "=&v"(dy), [dz] "=&v"(dz), [r2] "=&v"(r2), [w] "=&v"(w),    \
        [f] "=&v"(f), [off] "=&s"(off), [t] "=&s"(t), [far] "=&s"(far),                   \
        [save] "=&s"(save), [open] "=&s"(open), [le] "=&s"(le), [j] "=&s"(jj),          \
        [left] "=&s"(left)
#define BH_RUN_INS                                                                     \
    [nb] "s"(nb), [srclo] "s"(sb_lo), [srchi] "s"(sb_hi), [eps2] "v"(eps2v), [px] "v"(p.x),  \
        [py] "v"(p.y), [pz] "v"(p.z), [wb] "s"(wb), [wbe] "s"(wbe)
#define BH_RUN_CLOBBERS                                                                \
    "s16", "s17", "s18", "s19", "s20", "s21", "s22", "s23", "s24", "s25", "s26", "s27", \
        "s28", "s29", "s30", "s31", "s32", "s33", "s34", "s35", "s36", "s37", "s38",    \
        "s39", "s40", "s41", "s42", "s43", "s44", "s45", "s46", "s47", "s48", "s49",    \
        "vcc", "scc", "memory"

// Walk of one wave (see the file comment).  EXACT_T selects ldexp for the
// level thresholds (w_l / theta)^2 = T0 * 4^-l; otherwise 4^-l is an exponent
// decrement on the scalar unit (exact whenever T0 * 4^-21 stays normal), or,
// with FIXED_T, T0 itself (T0 = 0, inf or NaN is the same at every level).
//
// The walk is bound by the latency of its dependent node-record loads, with
// instruction issue second: a wave's vector and scalar instructions share its
// issue slots, and a vector op with a scalar-register operand issues at about
// two thirds the rate of one with register operands only.  The assembly loop
// (above) keeps the path of a visit that moves to the skip to 17 vector ops,
// 6 of them with a scalar operand, 9 scalar instructions and 1 branch, with
// the next record's load issued before the first vector op; the compiled
// form of the loop had 18 vector ops with 9 scalar operands, 13 scalar
// instructions and 3 branches, because the compiler re-derives the lane masks
// and the loop exit on every node, and it copied the accumulators several
// times around every opened leaf.  The two rarer thresholds keep the compiled
// loop.
// ASM: the assembly loop over the walk records (wnodes), else the compiled
// loop over the nodes with thresholds by ldexp.
template <bool SOFT, bool SELF, bool COUNT, bool ASM, bool ANY_MINE>
__device__ __attribute__((always_inline)) inline void walk_wave(
    const Node *__restrict__ nodes, const Node *__restrict__ wnodes,
    const float4 *__restrict__ src, uint32_t nn, float4 p, uint32_t i, uint32_t wave_base,
    bool valid, float T0, float eps2, float &ax, float &ay, float &az, float &pot,
    uint32_t &n_int)
{
    const char *node_bytes = reinterpret_cast<const char *>(ASM ? wnodes : nodes);
    // Lane state: a lane takes part at node X when rejoin <= X (both as byte
    // offsets into the walk records in the assembly loop).  A lane that
    // uses a node whole sets rejoin = skip(node) and so sits out the node's
    // subtree; lanes that open a node keep theirs.  (The wave lands on every
    // such skip on its way out, so `<=` and `==` select the same lanes.)  After
    // the visit of X, the lanes with rejoin <= X are exactly those that opened
    // it.
    uint32_t rejoin = valid ? 0u : 0xffffffffu;
    uint32_t X = 0;
    // a leaf opened by some lane: its openers sum its particles; a leaf
    // holding some of this wave's own targets needs the self pair removed
    auto open_leaf = [&](uint32_t b, uint32_t e, float e2) {
        if (rejoin <= X) {
            if (SELF && (ANY_MINE || (b < wave_base + 64 && e > wave_base)))
                leaf_tile<SOFT, true>(src, b, e, i, p, e2, ax, ay, az, pot);
            else
                leaf_tile<SOFT, false>(src, b, e, i, p, e2, ax, ay, az, pot);
            if (COUNT) n_int += (e - b) - ((SELF && i >= b && i < e) ? 1u : 0u);
        }
    };
    if constexpr (ASM) {
        const uint64_t nb = (uint64_t)node_bytes;
        const uint32_t sb_lo = sgpr((uint32_t)(uint64_t)src);
        const uint32_t sb_hi = sgpr((uint32_t)((uint64_t)src >> 32));
        // the loop sums a leaf unless it may hold this wave's own targets
        // (self-gravity in key order: [wave_base, wave_base + 64)); with
        // unsorted self-gravity every leaf may, with separate targets none
        const uint32_t wb = SELF ? (ANY_MINE ? 0u : wave_base) : 0xffffffffu;
        const uint32_t wbe = SELF ? (ANY_MINE ? 0xffffffffu : wave_base + 64) : 0u;
        float eps2v = eps2;
        asm volatile("" : "+v"(eps2v));   // held in a vector register
        for (;;) {
            X = sgpr(X);
            uint32_t first, cnt, skip, off, t, le, jj, left;
            float dx, dy, dz, r2, w, f;
            uint64_t far, save, open;
            if constexpr (COUNT) {
                uint32_t ni = n_int;
                if constexpr (SOFT)
                    asm volatile(BH_RUN("v_add_u32_e32 %[ni], 1, %[ni]\n",
                                        "v_add_u32_e32 %[ni], %[cnt], %[ni]\n", BH_GUARD_SOFT)
                                 : BH_RUN_OUTS, [ni] "+v"(ni)
                                 : BH_RUN_INS
                                 : BH_RUN_CLOBBERS);
                else
                    asm volatile(BH_RUN("v_add_u32_e32 %[ni], 1, %[ni]\n",
                                        "v_add_u32_e32 %[ni], %[cnt], %[ni]\n", BH_GUARD_HARD)
                                 : BH_RUN_OUTS, [ni] "+v"(ni)
                                 : BH_RUN_INS
                                 : BH_RUN_CLOBBERS);
                n_int = ni;
            } else {
                if constexpr (SOFT)
                    asm volatile(BH_RUN("", "", BH_GUARD_SOFT)
                                 : BH_RUN_OUTS
                                 : BH_RUN_INS
                                 : BH_RUN_CLOBBERS);
                else
                    asm volatile(BH_RUN("", "", BH_GUARD_HARD)
                                 : BH_RUN_OUTS
                                 : BH_RUN_INS
                                 : BH_RUN_CLOBBERS);
            }
            // the outputs are scalar registers; the compiler takes asm
            // outputs for per-lane values unless told
            X = sgpr(X);
            first = sgpr(first);
            cnt = sgpr(cnt);
            skip = sgpr(skip);
            if (cnt == 0) break;   // the end record (every other leaf holds a source)
            open_leaf(first, first + cnt, eps2v);
            X = skip;   // leave the leaf (skip == X + 1, as a byte offset)
        }
        return;
    }
    while (X < nn) {
        const uint4 *rec = reinterpret_cast<const uint4 *>(node_bytes + (size_t)X * sizeof(Node));
        const uint4 lo = rec[0], hi = rec[1];
        uint32_t mbits = lo.w;
        asm volatile("" : "+s"(mbits));   // keep the mass in a register, not reloaded
        const float cx = __uint_as_float(lo.x), cy = __uint_as_float(lo.y);
        const float cz = __uint_as_float(lo.z), m = __uint_as_float(mbits);
        const uint32_t skip = hi.z, meta = hi.w;
        const uint32_t level = node_level(meta);
        // the opening test on the softened scale: T + eps^2 < r^2 + eps^2
        const float T = ldexpf(T0, -2 * (int)level) + eps2;
        const float dx = cx - p.x, dy = cy - p.y, dz = cz - p.z;
        const float r2 = fmaf(dz, dz, fmaf(dy, dy, fmaf(dx, dx, eps2)));
        const uint64_t act_m = __ballot(rejoin <= X);
        const uint64_t far_m = __ballot(T < r2);
        const uint64_t open_m = act_m & ~far_m;
        if (rejoin <= X && T < r2) {
            const float inv = __builtin_amdgcn_rsqf(r2);
            const float mi = m * inv;
            const float f = mi * inv * inv;
            ax = fmaf(f, dx, ax);
            ay = fmaf(f, dy, ay);
            az = fmaf(f, dz, az);
            pot -= mi;
            rejoin = skip;
            if (COUNT) ++n_int;
        }
        if (open_m == 0) {   // every active lane used X whole
            X = skip;
            continue;
        }
        if ((meta & kLeafBit) == 0) {   // descend into an opened internal node
            X = X + 1;
            continue;
        }
        open_leaf(hi.x, hi.x + hi.y, eps2);
        X = skip;   // leave an opened leaf (skip == X + 1)
    }
}

// The warp vote of [GASPHiA] 性能瓶颈分析, kept for comparison: the wave
// moves as one, and when the opening test fails for any of its valid lanes,
// every lane uses the node's children (or, for a leaf, its particles);
// otherwise every lane uses the node whole.  Results then depend on which
// targets share a wave; every lane sees at least the nodes of its own walk.
template <bool SOFT, bool SELF, bool COUNT, bool EXACT_T, bool ANY_MINE>
__device__ __attribute__((always_inline)) inline void walk_vote(
    const Node *__restrict__ nodes, const float4 *__restrict__ src, uint32_t nn, float4 p,
    uint32_t i, uint32_t wave_base, bool valid, float T0, uint32_t T0_bits, uint32_t T_step,
    float eps2, float &ax, float &ay, float &az, float &pot, uint32_t &n_int)
{
    const char *node_bytes = reinterpret_cast<const char *>(nodes);
    uint32_t X = 0;
    while (X < nn) {
        const uint4 *rec = reinterpret_cast<const uint4 *>(node_bytes + (size_t)X * sizeof(Node));
        const uint4 lo = rec[0], hi = rec[1];
        const float cx = __uint_as_float(lo.x), cy = __uint_as_float(lo.y);
        const float cz = __uint_as_float(lo.z), m = __uint_as_float(lo.w);
        const uint32_t skip = hi.z, meta = hi.w;
        const uint32_t level = node_level(meta);
        const float T = EXACT_T ? ldexpf(T0, -2 * (int)level)
                                : __uint_as_float(sgpr(T0_bits - level * T_step));
        const float dx = cx - p.x, dy = cy - p.y, dz = cz - p.z;
        const float r2 = fmaf(dz, dz, fmaf(dy, dy, dx * dx));
        if (__ballot(valid && !(T < r2)) == 0) {   // no lane opens: all use X whole
            const float inv = __builtin_amdgcn_rsqf(r2 + eps2);
            const float mi = m * inv;
            const float f = mi * inv * inv;
            ax = fmaf(f, dx, ax);
            ay = fmaf(f, dy, ay);
            az = fmaf(f, dz, az);
            pot -= mi;
            if (COUNT) ++n_int;
            X = skip;
            continue;
        }
        if (meta & kLeafBit) {   // every lane sums the leaf's particles
            const uint32_t b = hi.x, e = hi.x + hi.y;
            if (SELF && (ANY_MINE || (b < wave_base + 64 && e > wave_base)))
                leaf_tile<SOFT, true>(src, b, e, i, p, eps2, ax, ay, az, pot);
            else
                leaf_tile<SOFT, false>(src, b, e, i, p, eps2, ax, ay, az, pot);
            if (COUNT) n_int += (e - b) - ((SELF && i >= b && i < e) ? 1u : 0u);
            X = skip;
            continue;
        }
        X = X + 1;
    }
}

// One wave per 64 consecutive targets of the walk order.  Sorted order (the
// product path): lane position c is the target's Morton rank, its position
// is tpos[c] and its result goes to tmap[c], the caller's index.  Unsorted
// order (kept to measure what the Morton order of targets buys, [GASPHiA]
// 排序算法): c is the caller's index and the output slot; for self-gravity
// tmap[c] is the target's Morton rank, which locates it (tpos is then the
// sorted sources) and identifies the self pair; separate targets are read
// from tpos[c] as given.
template <bool SOFT, bool SELF, bool COUNT, bool VOTE, bool UNSORTED>
__global__ __launch_bounds__(kWalkThreads) void k_walk(const Node *__restrict__ nodes,
                                                       const Node *__restrict__ wnodes,
                                                       uint32_t wn_cap,
                                                       const float4 *__restrict__ src,
                                                       const float4 *__restrict__ tpos,
                                                       const uint32_t *__restrict__ tmap,
                                                       const DevParams *__restrict__ prm,
                                                       uint32_t n, float theta, float G,
                                                       float eps2, float4 *__restrict__ out,
                                                       unsigned long long *__restrict__ count,
                                                       uint32_t *__restrict__ balance,
                                                       int runs, int record)
{
    const uint32_t lane = threadIdx.x & 63;
    // the group this wave walks: each XCD (workgroups are dealt to the eight
    // XCDs in turn) takes one contiguous run of groups, so the waves that run
    // together share the nodes near their targets in that XCD's L2; with
    // a balance buffer the runs are the ones balanced on the previous walk's times
    uint32_t blk;
    uint32_t part = 0;   // 0: the whole group; p > 0: its targets' p-th share
    // (the vote and caller-order walks keep the equal runs: mode 0)
    if (VOTE || UNSORTED) {
        blk = xcd_block(blockIdx.x, gridDim.x);
    } else if (runs & 1) {
        // the grid holds 8 cap workgroups, cap per XCD; an XCD whose run is
        // shorter lets its first ones return, while every XCD still has free
        // slots (at the end of the dispatch they would hold up the others)
        const uint32_t x = blockIdx.x & 7u, k = blockIdx.x >> 3;
        const uint32_t b0 = sgpr(balance[x]), b1 = sgpr(balance[x + 1]);
        const uint32_t idle = (gridDim.x >> 3) - (b1 - b0);
        if (k < idle) return;
        blk = b0 + (k - idle);
    } else if (runs & 2) {
        // the first kWalkSplitParts * smax workgroups walk the listed heavy
        // groups a share each; the rest the equal runs, less those groups
        const uint32_t ng = walk_groups(n), smax = walk_split_max(ng);
        const uint32_t extra = kWalkSplitParts * smax;
        if (blockIdx.x < extra) {
            const uint32_t si = blockIdx.x / kWalkSplitParts;
            if (si >= sgpr(balance[kWalkSplitCount])) return;
            blk = sgpr(balance[kWalkBalanceHead + ng + si]);
            part = 1 + blockIdx.x % kWalkSplitParts;
        } else {
            blk = xcd_block(blockIdx.x - extra, gridDim.x - extra);
            if (sgpr(balance[kWalkBalanceHead + ng + smax + blk])) return;
        }
    } else {
        blk = xcd_block(blockIdx.x, gridDim.x);
    }
    const uint32_t wave_base = sgpr(blk * kWalkThreads + (threadIdx.x & ~63u));
    constexpr uint32_t kShare = 64 / kWalkSplitParts;
    const uint32_t c = part ? wave_base + (part - 1) * kShare + lane : wave_base + lane;
    const bool valid = c < n && (part == 0 || lane < kShare);
    if (wave_base + (part ? (part - 1) * kShare : 0u) >= n) return;
    // the group's start time, kept in vector registers (scalar registers
    // decide how many waves stay resident)
    uint64_t t_start = record ? __builtin_amdgcn_s_memrealtime() : 0;
    asm volatile("" : "+v"(t_start));
    uint32_t i = c, slot = c;   // self index (Morton rank) and output slot
    if (valid) {
        if (!UNSORTED) slot = tmap[c];
        else if (SELF) i = tmap[c];
    }

    if (prm->status != 0) {
        if (valid) out[slot] = make_float4(NAN, NAN, NAN, NAN);
        return;
    }
    const uint32_t nn = prm->n_nodes;
    const float4 p = valid ? tpos[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const double L = prm->L;
    const float T0 = (float)(L * L / ((double)theta * (double)theta));
    // the assembly loop walks the per-call records (thresholds in place, any
    // T0) while they exist and their byte offsets fit 32 bits; otherwise the
    // compiled loop walks the nodes
    const bool use_asm = nn < kAsmMaxNodes && nn < wn_cap;
    // the warp vote: zero, inf and NaN thresholds are the same at every level
    // (step 0); a normal T0 with T0 * 4^-21 normal steps the exponent by 2 per
    // level; anything else takes ldexp
    const uint32_t T0_bits = sgpr(__float_as_uint(T0));
    const uint32_t T0_exp = (T0_bits >> 23) & 0xffu;
    const bool fixed = (T0_bits & 0x7fffffffu) == 0u || T0_exp == 255u;
    const bool exact = !fixed && T0_exp <= 44u;
    const uint32_t T_step = fixed ? 0u : (1u << 24);

    // wait for the target's position here: a first use inside the walk loop
    // would put the wait on every iteration
    asm volatile("" ::"v"(p.x), "v"(p.y), "v"(p.z));
    float ax = 0.f, ay = 0.f, az = 0.f, pot = 0.f;
    uint32_t n_int = 0;
    if (VOTE) {
        if (exact)
            walk_vote<SOFT, SELF, COUNT, true, UNSORTED>(nodes, src, nn, p, i, wave_base, valid, T0,
                                                         T0_bits, T_step, eps2, ax, ay, az, pot,
                                                         n_int);
        else
            walk_vote<SOFT, SELF, COUNT, false, UNSORTED>(nodes, src, nn, p, i, wave_base, valid,
                                                          T0, T0_bits, T_step, eps2, ax, ay, az,
                                                          pot, n_int);
    } else {
        if (use_asm)
            walk_wave<SOFT, SELF, COUNT, true, UNSORTED>(nodes, wnodes, src, nn, p, i, wave_base,
                                                         valid, T0, eps2, ax, ay, az, pot, n_int);
        else
            walk_wave<SOFT, SELF, COUNT, false, UNSORTED>(nodes, wnodes, src, nn, p, i, wave_base,
                                                          valid, T0, eps2, ax, ay, az, pot, n_int);
    }

    if (valid) out[slot] = make_float4(G * ax, G * ay, G * az, G * pot);
    // this group's time (one plain store: the per-wave device atomic this
    // replaced serialised on its few addresses)
    if (record && lane == 0 && part == 0)
        balance[kWalkBalanceHead + (wave_base >> 6)] =
            (uint32_t)(__builtin_amdgcn_s_memrealtime() - t_start);
    if (COUNT) {
        unsigned long long cnt = valid ? n_int : 0u;
        for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
        if (lane == 0) atomicAdd(count, cnt);
    }
}

// The walk records of one call: per node X <= n_nodes (the end record
// included) {com, mass, start, count, skip * 32, (T + eps^2) | leaf << 31},
// with the opening threshold T = (L / theta)^2 4^-level by ldexp (exact
// wherever it is representable) shifted by eps^2 in one fp32 addition, the
// value every per-target walk form compares r^2 + eps^2 with, and the skip as
// a byte offset, so the assembly loop uses both without arithmetic.  Written
// only when the loop will use them (see k_walk).
// The XCD balance before a walk, from the previous walk's per-group times
// (xb[kWalkBalanceHead + g], every kWalkBalanceSample-th read); xb[0..8]
// receive the first group of each XCD's run (xb[8] = ng).  The sampled times
// are summed over 256 chunks of consecutive groups (chunk c starts at
// ceil(c ng / 256); chunks 32x..32x+31 are the eighth x of the groups, the
// equal runs of xcd_block).  When the largest
// eighth is more than kWalkRebalance above their mean and the waves lived
// longer than kWalkBalanceMinTicks on average, *want = 1 (the host then
// launches the next walks with room for uneven runs), else 0.  With `runs`
// (such a walk) and *want = 1, the runs become eight contiguous ranges, ending
// on chunk boundaries, whose sums of the previous times are as equal as the
// cap of `cap` groups per run allows; otherwise the equal runs.  (Equal runs
// of a centrally symmetric input coincide with its root octants, so each XCD's
// L2 holds one octant's subtree; runs moved off them to even out a few per cent
// of time measured slower.)  One block of 256 threads.  Every run is at most
// `cap` groups and 8 cap >= ng, so a grid of 8 cap workgroups walks every
// group once.
constexpr double kWalkRebalance = 1.08;
// Waves that live less than this on average (s_memrealtime ticks, 100 MHz:
// 100 us) are bound by the rate at which workgroups are dispatched, which
// equal runs already share evenly.
constexpr unsigned long long kWalkBalanceMinTicks = 10000;
// The balance reads every 8th group's time: an eighth of the groups holds
// 256 samples or more from 2^17 targets on, and the pass stays a few loads
// per thread.
constexpr uint32_t kWalkBalanceSample = 8;

__device__ inline uint32_t walk_chunk_start(uint32_t c, uint32_t ng)
{
    return (uint32_t)(((uint64_t)c * ng + 255) >> 8);
}

// Bin of a group's time on a log scale, four bins per octave: bin 4e + m
// holds [(4 + m) 2^(e-2), (5 + m) 2^(e-2)) for e >= 2.
__device__ inline uint32_t time_bin(uint32_t v)
{
    if (v < 4) return v;
    const uint32_t e = 31u - (uint32_t)__builtin_clz(v);
    return 4 * e + ((v >> (e - 2)) & 3u);
}
__device__ inline uint32_t time_bin_floor(uint32_t b)
{
    if (b < 8) return b;
    return (4u + (b & 3u)) << ((b >> 2) - 2);
}

// Split groups: whether a walk's heaviest groups would end sooner as
// kWalkSplitParts waves each (the smallest time bin of which the samples put
// no more than walk_split_max groups at or above it must start more than
// kWalkSplitRatio times the mean time), and the list and flags of those groups.
constexpr double kWalkSplitRatio = 3.0;

__device__ void walk_bounds(uint32_t ng, uint32_t cap, bool hist, bool runs, bool split,
                            uint32_t *__restrict__ xb, int *__restrict__ want)
{
    const uint32_t *__restrict__ wdur = xb + kWalkBalanceHead;
    const uint32_t smax = walk_split_max(ng);
    uint32_t *__restrict__ slist = xb + kWalkBalanceHead + ng;
    uint32_t *__restrict__ sflag = slist + smax;
    __shared__ unsigned long long csum[256];
    __shared__ uint32_t tbin[128];
    __shared__ uint32_t ideal[8];
    __shared__ int balance;
    __shared__ uint32_t split_thr, split_n;
    const uint32_t t = threadIdx.x;
    csum[t] = 0;
    if (t < 128) tbin[t] = 0;
    if (t < 8) ideal[t] = 0;
    __syncthreads();
    if (hist) {
        // every kWalkBalanceSample-th group's time (sixteen loads in flight per
        // thread); a thread's groups only increase: add its run of times in
        // one chunk, then move on
        constexpr uint32_t S = kWalkBalanceSample;
        uint32_t c = 0, next = walk_chunk_start(1, ng);
        unsigned long long acc = 0;
        for (uint32_t g0 = S * t; g0 < ng; g0 += 16 * 256 * S) {
            uint32_t v[16];
#pragma unroll
            for (uint32_t j = 0; j < 16; ++j) {
                const uint32_t g = g0 + 256 * S * j;
                v[j] = g < ng ? wdur[g] : 0u;
            }
#pragma unroll
            for (uint32_t j = 0; j < 16; ++j) {
                const uint32_t g = g0 + 256 * S * j;
                if (g >= ng) continue;
                while (g >= next) {
                    if (acc) atomicAdd(&csum[c], acc);
                    acc = 0;
                    ++c;
                    next = walk_chunk_start(c + 1, ng);
                }
                acc += v[j];
                atomicAdd(&tbin[time_bin(v[j])], 1u);
            }
        }
        if (acc) atomicAdd(&csum[c], acc);
    }
    __syncthreads();
    if (t == 0) {
        // the split threshold: the smallest bin with at most smax groups (by
        // the samples) at or above it; if the heaviest bin alone holds more,
        // that bin (the list then takes the first smax of its groups)
        uint32_t above = 0, b = 128;
        while (b > 0 && (above + tbin[b - 1]) * kWalkBalanceSample <= smax) above += tbin[--b];
        if (above == 0 && b > 0) above = tbin[--b];
        unsigned long long total = 0;
        for (int k = 0; k < 256; ++k) total += csum[k];
        const unsigned long long samples = (ng + kWalkBalanceSample - 1) / kWalkBalanceSample;
        const bool heavy = hist && smax > 0 && b < 128 && above > 0 &&
                           (double)time_bin_floor(b) * (double)samples >
                               kWalkSplitRatio * (double)total;
        split_thr = heavy ? time_bin_floor(b) : 0xffffffffu;
        split_n = 0;
    }
    __syncthreads();
    // the split list: clear the flags of the groups listed before (all flags
    // for groups without a list yet), then list the groups at or above the
    // threshold when this walk can split them
    if (smax > 0) {
        if (!hist) {
            for (uint32_t g = t; g < ng; g += 256) sflag[g] = 0u;
        } else {
            const uint32_t old = min(xb[kWalkSplitCount], smax);
            for (uint32_t k = t; k < old; k += 256) sflag[slist[k]] = 0u;
        }
        __syncthreads();
        if (split && split_thr != 0xffffffffu) {
            for (uint32_t g = t; g < ng; g += 256) {
                if (wdur[g] >= split_thr) {
                    const uint32_t k = atomicAdd(&split_n, 1u);
                    if (k < smax) {
                        slist[k] = g;
                        sflag[g] = 1u;
                    }
                }
            }
        }
        __syncthreads();
        if (t == 0) xb[kWalkSplitCount] = min(split_n, smax);
    }
    if (t == 0) {
        unsigned long long total = 0, most = 0;
        for (int x = 0; x < 8; ++x) {
            unsigned long long e = 0;
            for (int k = 0; k < 32; ++k) e += csum[32 * x + k];
            total += e;
            most = max(most, e);
        }
        const unsigned long long samples = (ng + kWalkBalanceSample - 1) / kWalkBalanceSample;
        const int bal = hist && (double)most * 8.0 > kWalkRebalance * (double)total &&
                        total > samples * kWalkBalanceMinTicks;
        if (want) *want = bal | (split_thr != 0xffffffffu ? 2 : 0);
        balance = bal && runs;
    }
    __syncthreads();
    if (!balance) {
        if (t <= 8) xb[t] = t * (ng >> 3) + min(t, ng & 7u);
        return;
    }
    // inclusive scan of the chunk sums
    for (uint32_t o = 1; o < 256; o <<= 1) {
        const unsigned long long v = t >= o ? csum[t - o] : 0ull;
        __syncthreads();
        csum[t] += v;
        __syncthreads();
    }
    if (t >= 1 && t < 8) {
        // the chunk boundary nearest to where the times reach t/8 of the total
        const unsigned long long target = csum[255] * t / 8;
        uint32_t k = 0;
        while (k < 255 && csum[k] < target) ++k;
        const unsigned long long before = k ? csum[k - 1] : 0ull;
        const uint32_t kb = target - before <= csum[k] - target ? k : k + 1;
        ideal[t] = walk_chunk_start(kb, ng);
    }
    __syncthreads();
    if (t == 0) {
        // clamp: run x at most cap groups, and the runs after it able to hold
        // the rest
        uint32_t prev = 0;
        xb[0] = 0;
        for (uint32_t x = 1; x < 8; ++x) {
            const uint64_t tail = (uint64_t)(8 - x) * cap;
            const uint32_t lo = max(prev, (uint64_t)ng > tail ? (uint32_t)(ng - tail) : 0u);
            const uint32_t hi = min(prev + cap, ng);
            prev = min(max(ideal[x], lo), hi);
            xb[x] = prev;
        }
        xb[8] = ng;
    }
}

__global__ __launch_bounds__(256) void k_walk_nodes(const Node *__restrict__ nodes,
                                                    const DevParams *__restrict__ prm,
                                                    float theta, float eps2, uint32_t wn_cap,
                                                    Node *__restrict__ wnodes,
                                                    uint32_t ng, uint32_t cap, int eval,
                                                    int fresh, int runs,
                                                    uint32_t *__restrict__ balance,
                                                    int *__restrict__ want)
{
    // new runs from recent times, or the equal runs for groups without any;
    // otherwise the runs chosen last time stand
    if (balance && blockIdx.x == 0 && (eval || fresh))
        walk_bounds(ng, cap, eval != 0, (runs & 1) != 0, (runs & 2) != 0, balance, want);
    if (prm->status != 0) return;
    const uint32_t nn = prm->n_nodes;
    if (!(nn < kAsmMaxNodes && nn < wn_cap)) return;
    const double L = prm->L;
    const float T0 = (float)(L * L / ((double)theta * (double)theta));
    for (uint32_t X = blockIdx.x * blockDim.x + threadIdx.x; X <= nn; X += gridDim.x * blockDim.x) {
        const uint4 lo = reinterpret_cast<const uint4 *>(&nodes[X])[0];
        const uint4 hi = reinterpret_cast<const uint4 *>(&nodes[X])[1];
        const float T = ldexpf(T0, -2 * (int)node_level(hi.w)) + eps2;
        const uint32_t tb = (__float_as_uint(T) & 0x7fffffffu) | ((hi.w & kLeafBit) ? 0x80000000u : 0u);
        reinterpret_cast<uint4 *>(&wnodes[X])[0] = lo;
        reinterpret_cast<uint4 *>(&wnodes[X])[1] = make_uint4(hi.x, hi.y, hi.z << 5, tb);
    }
}

// inv[perm[k]] = k: the Morton rank of each caller index.
__global__ void k_invert(const uint32_t *__restrict__ perm, uint32_t n, uint32_t *__restrict__ inv)
{
    const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) inv[perm[k]] = k;
}

__global__ void k_fill_zero(float4 *out, uint32_t n)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <bool SOFT, bool SELF, bool COUNT, bool VOTE, bool UNSORTED>
void launch5(const WalkArgs &a, hipStream_t s)
{
    const uint32_t groups = walk_groups(a.n_targets);
    const uint32_t grid = a.balance_runs ? 8 * walk_xcd_cap(groups)
                          : a.balance_split ? groups + kWalkSplitParts * walk_split_max(groups)
                                            : groups;
    const int mode = a.balance_runs ? 1 : a.balance_split ? 2 : 0;
    hipLaunchKernelGGL((k_walk<SOFT, SELF, COUNT, VOTE, UNSORTED>), dim3(grid), dim3(kWalkThreads),
                       0, s, a.nodes, a.wnodes, a.wn_cap, a.src, a.tpos, a.tmap, a.prm, a.n_targets, a.theta, a.G,
                       a.eps * a.eps, a.out, a.count, a.balance, mode, a.balance_record);
}

template <bool SOFT, bool SELF, bool COUNT>
void launch3(const WalkArgs &a, hipStream_t s)
{
    if (a.vote) {
        if (a.unsorted) launch5<SOFT, SELF, COUNT, true, true>(a, s);
        else launch5<SOFT, SELF, COUNT, true, false>(a, s);
    } else {
        if (a.unsorted) launch5<SOFT, SELF, COUNT, false, true>(a, s);
        else launch5<SOFT, SELF, COUNT, false, false>(a, s);
    }
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

void launch_walk(const WalkArgs &args, hipStream_t s)
{
    if (args.n_targets == 0) return;
    // the balanced XCD runs are written by k_walk_nodes, which runs for the
    // per-target walks only; the caller-order and vote walks keep equal runs
    WalkArgs a = args;
    if (a.vote || a.unsorted || a.wn_cap == 0 || !a.balance) {
        a.balance = nullptr;
        a.balance_eval = a.balance_fresh = a.balance_runs = a.balance_split = 0;
        a.balance_record = 0;
        a.balance_want = nullptr;
    }
    if (!a.vote && a.wn_cap > 0) {
        const uint32_t blocks = (uint32_t)std::min<uint64_t>((a.wn_cap + 255) / 256, 2048);
        const uint32_t groups = walk_groups(a.n_targets);
        hipLaunchKernelGGL(k_walk_nodes, dim3(blocks), dim3(256), 0, s, a.nodes, a.prm, a.theta,
                           a.eps * a.eps, a.wn_cap, a.wnodes, groups, walk_xcd_cap(groups),
                           a.balance_eval, a.balance_fresh,
                           a.balance_runs ? 1 : a.balance_split ? 2 : 0, a.balance,
                           a.balance_want);
    }
    // Plummer softening with eps^2 > 0 never meets r^2 + eps^2 == 0
    if (a.eps * a.eps > 0.f) launch1<true>(a, s); else launch1<false>(a, s);
}

void launch_invert(const uint32_t *perm, uint32_t n, uint32_t *inv, hipStream_t s)
{
    if (n == 0) return;
    hipLaunchKernelGGL(k_invert, dim3((n + 255) / 256), dim3(256), 0, s, perm, n, inv);
}

void launch_fill_zero(float4 *out, uint32_t n, hipStream_t s)
{
    if (n == 0) return;
    hipLaunchKernelGGL(k_fill_zero, dim3((n + 255) / 256), dim3(256), 0, s, out, n);
}

}  // namespace bh
