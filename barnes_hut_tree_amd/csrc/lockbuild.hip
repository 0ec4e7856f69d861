// The lock-based dense octree build of [Tree] (构建树结构, 核心代码片段, 并发与
// 同步, and the embedded 基于稠密存储的并行树构建实现方案), kept to measure that
// design against the sorted-key build on the same device.
//
// Dense storage: a cell owns 8 child slots, child[cell * 8 + octant]; a slot
// holds kEmpty, kLocked, a particle index (0..n-1) or n + a cell id.  Cells
// are allocated downward from the top of the array by an atomic decrement,
// the root being the last cell.  Every thread inserts one particle: it walks
// down from the root following its octant at each cell, and at the first
// slot that is not a cell it takes the slot with a compare-and-swap to
// kLocked.  An empty slot receives the particle; a slot holding another
// particle is subdivided into fresh cells until the two fall into different
// octants; the new cells are written, a fence makes them visible, and the
// slot is released by storing the top new cell.  Nobody waits inside the
// critical section, so every wave makes progress.
//
// On this device a load can return an older value of a slot that a thread on
// another XCD has since changed (the pages' volatile loads and fences assume
// one coherent cache), so the loads only guide the walk: the compare-and-swap
// is the authority, and a failed one returns the slot's current value, from
// which the walk continues (descending if it has become a cell).  A slot seen
// locked is confirmed with a no-op compare-and-swap before the walk restarts
// from the root.  All slots are set empty before the insertion kernel, so a
// stale read can only return a state the slot has really held.
//
// Readings: octants come from the Morton key bits (the same quantisation as
// the rest of the library), so the tree is exactly the leaf-capacity-1 octree
// of the oracle; particles with identical keys are subdivided to the finest
// level and chained there through next[] (the pages do not treat them).  Each
// insertion gives up after kMaxRetries steps and sets a status bit, and
// allocation beyond the capacity restores the slot and sets the capacity bit,
// so every thread terminates.  Slots are read and written with device-scope
// atomics: the 8 XCDs do not share an L2.
#include <algorithm>

#include "bh_internal.h"

namespace bh {
namespace {

constexpr int kLockThreads = 256;
constexpr int32_t kEmpty = -1;
constexpr int32_t kLocked = -2;
constexpr uint32_t kMaxRetries = 4096;

__device__ inline int32_t ld_acquire(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_relaxed(int32_t *p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_release(int32_t *p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// octant of a key among the children of a level-l cell (children at level l + 1)
__device__ inline int32_t octant(uint64_t key, int bits, int l)
{
    return (int32_t)((key >> (3 * (bits - l - 1))) & 7u);
}

// Every slot empty (so that any value a read can return is a state the slot
// has actually held: empty, locked, a source, a cell), the root, the
// allocation counter, the chains.
__global__ void k_lock_init(int32_t *__restrict__ child, int32_t *__restrict__ level,
                            int32_t *__restrict__ next, uint32_t n, int32_t cap,
                            int32_t *__restrict__ counter)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t slots = (size_t)cap * 8;
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < slots; k += stride)
        child[k] = kEmpty;
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride)
        next[k] = kEmpty;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        level[cap - 1] = 0;
        *counter = cap - 1;   // cells cap-2, cap-3, ... are handed out next
    }
}

__global__ __launch_bounds__(kLockThreads) void k_lock_insert(
    const uint64_t *__restrict__ keys, uint32_t n, int bits, int32_t *__restrict__ child,
    int32_t *__restrict__ level, int32_t *__restrict__ next, int32_t cap,
    int32_t *__restrict__ counter, DevParams *__restrict__ prm)
{
    const uint32_t i = blockIdx.x * kLockThreads + threadIdx.x;
    if (i >= n) return;
    const uint64_t key = keys[i];
    const int32_t self = (int32_t)i, nn = (int32_t)n;
    // The walk down from the root; a cell reached from a slot of a level-l
    // cell is at level l + 1, so levels are counted, never read back.
    int32_t cell = cap - 1, lev = 0;
    size_t slot = (size_t)cell * 8 + octant(key, bits, 0);
    int32_t v = ld_acquire(&child[slot]);
    for (uint32_t step = 0;; ++step) {
        if (step == kMaxRetries) {
            atomicOr(&prm->status, kStatusLockRetry);
            return;
        }
        if (v >= nn) {   // a cell: go down
            if (v - nn >= cap) {   // cannot happen: every slot starts empty
                atomicOr(&prm->status, kStatusLockRetry);
                return;
            }
            cell = v - nn;
            ++lev;
            slot = (size_t)cell * 8 + octant(key, bits, lev);
            v = ld_acquire(&child[slot]);
            continue;
        }
        if (v == kLocked) {
            // confirm with a read-modify-write (a plain load may return an
            // older value on another XCD), then start again from the root
            const int32_t now = atomicCAS(&child[slot], kLocked, kLocked);
            if (now != kLocked) {
                v = now;
                continue;
            }
            cell = cap - 1;
            lev = 0;
            slot = (size_t)cell * 8 + octant(key, bits, 0);
            v = ld_acquire(&child[slot]);
            continue;
        }
        const int32_t old = atomicCAS(&child[slot], v, kLocked);
        if (old != v) {   // the slot had changed: the compare-and-swap returned its value
            v = old;
            continue;
        }
        if (v == kEmpty) {
            st_release(&child[slot], self);
            return;
        }
        // the slot held particle v (the head of a chain of identical keys)
        const uint64_t kv = keys[v];
        if (lev == bits - 1) {   // finest level: only identical keys share a slot
            next[i] = v;
            st_release(&child[slot], self);
            return;
        }
        int32_t top = -1;
        size_t link = 0;
        for (int l = lev + 1; l < bits; ++l) {
            const int32_t c = atomicSub(counter, 1) - 1;
            if (c < 0) {   // out of cells: give the slot back, report
                atomicOr(&prm->status, kStatusCapacity);
                st_release(&child[slot], v);
                return;
            }
            level[c] = l;
            for (int o = 0; o < 8; ++o) st_relaxed(&child[(size_t)c * 8 + o], kEmpty);
            if (top < 0) top = c; else st_relaxed(&child[link], nn + c);
            const int32_t oi = octant(key, bits, l), ov = octant(kv, bits, l);
            if (oi != ov) {
                st_relaxed(&child[(size_t)c * 8 + oi], self);
                st_relaxed(&child[(size_t)c * 8 + ov], v);
                break;
            }
            link = (size_t)c * 8 + oi;
            if (l == bits - 1) {   // identical keys: chain them at the finest level
                next[i] = v;
                st_relaxed(&child[link], self);
            }
        }
        __threadfence();
        st_release(&child[slot], nn + top);
        return;
    }
}

}  // namespace

void launch_lock_build(const uint64_t *keys, uint32_t n, int bits, int32_t *child,
                       int32_t *level, int32_t *next, int32_t cap, int32_t *counter,
                       DevParams *prm, hipStream_t s)
{
    const size_t slots = (size_t)cap * 8;
    const uint32_t blocks = (uint32_t)std::min<size_t>((slots + 255) / 256, 8192);
    hipLaunchKernelGGL(k_lock_init, dim3(blocks), dim3(256), 0, s, child, level, next, n, cap,
                       counter);
    if (n == 0) return;
    hipLaunchKernelGGL(k_lock_insert, dim3((n + kLockThreads - 1) / kLockThreads),
                       dim3(kLockThreads), 0, s, keys, n, bits, child, level, next, cap, counter,
                       prm);
}

}  // namespace bh
