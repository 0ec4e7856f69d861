// Stable LSD radix sort of (Morton key, index) pairs, 8-bit digits.
//
// The pages order particles by Morton key before the walk ([Tree] 实现步骤,
// 粒子空间排序) and keep the particle data in place behind a gather index
// ([GASPHiA] 排序算法: sort indices, not data).  Here the sort carries the
// index as payload and its last pass also gathers a sorted copy of the
// float4 rows, so the walk reads contiguous memory.
//
// Per pass three kernels: a per-tile digit histogram, a scan of each digit's
// row of tile counts (one workgroup per digit), and a scatter in which each
// workgroup ranks its tile stably in LDS (64-lane ballots give the rank among
// equal digits within a wave row), adds the digit bases (a scan of the 256
// digit totals) and writes the tile out digit-group by digit-group, so
// writes of one digit are contiguous.
#include "bh_internal.h"

namespace bh {
namespace {

constexpr int kWaves = kSortThreads / 64;

__device__ inline uint32_t lane_id() { return threadIdx.x & 63; }

__device__ inline uint32_t wave_incl_scan(uint32_t v)
{
    const uint32_t lane = lane_id();
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(v, o, 64);
        if (lane >= (uint32_t)o) v += t;
    }
    return v;
}

// Exclusive scan of v over a 256-thread workgroup; *total receives the sum.
__device__ inline uint32_t block_excl_scan_256(uint32_t v, uint32_t *tmp, uint32_t *total)
{
    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    uint32_t incl = wave_incl_scan(v);
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    uint32_t off = 0, sum = 0;
    for (int w = 0; w < kWaves; ++w) {
        uint32_t t = tmp[w];
        if ((uint32_t)w < wave) off += t;
        sum += t;
    }
    *total = sum;
    __syncthreads();
    return off + incl - v;
}

// Per-tile digit counts.  All ITEMS keys of a thread are loaded before the
// first LDS update, so a wave has its whole share of the tile in flight.
template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void k_hist(const uint64_t *__restrict__ keys, uint32_t n,
                                                       int shift, uint32_t *__restrict__ hist,
                                                       uint32_t n_tiles)
{
    __shared__ uint32_t h[kWaves][kRadix];
    const uint32_t wave = threadIdx.x >> 6;
    for (int d = threadIdx.x; d < kWaves * kRadix; d += kSortThreads) (&h[0][0])[d] = 0;
    const uint32_t tile = xcd_block(blockIdx.x, n_tiles);
    const uint32_t base = tile * (kSortThreads * ITEMS);
    uint32_t digit[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const uint32_t i = base + k * kSortThreads + threadIdx.x;
        digit[k] = i < n ? (uint32_t)(keys[i] >> shift) & 0xffu : kRadix;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
        if (digit[k] < kRadix) atomicAdd(&h[wave][digit[k]], 1u);
    __syncthreads();
    const uint32_t d = threadIdx.x;
    uint32_t c = 0;
    for (int w = 0; w < kWaves; ++w) c += h[w][d];
    hist[d * n_tiles + tile] = c;
}

template <bool GATHER, int ITEMS>
__global__ __launch_bounds__(kSortThreads) void k_scatter(
    const uint64_t *__restrict__ kin, const uint32_t *__restrict__ vin,
    uint64_t *__restrict__ kout, uint32_t *__restrict__ vout, uint32_t n, int shift,
    const uint32_t *__restrict__ row_pref, const uint32_t *__restrict__ row_tot,
    uint32_t n_tiles, const float4 *__restrict__ gsrc, float4 *__restrict__ gdst)
{
    constexpr uint32_t kTile = kSortThreads * ITEMS;
    __shared__ uint64_t skey[kTile];
    __shared__ uint32_t sval[kTile];
    // per wave and digit: the count, then the tile position of the wave's
    // first key of that digit; in the last phase, row 0 holds per digit the
    // output position minus the tile position
    __shared__ uint32_t wcnt[kWaves][kRadix];
    __shared__ uint32_t tmp[kWaves];

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int d = threadIdx.x; d < kWaves * kRadix; d += kSortThreads) (&wcnt[0][0])[d] = 0;
    __syncthreads();

    // Each wave owns ITEMS * 64 consecutive keys of the tile; row k holds
    // keys [k*64, k*64+64) of that range, so (wave, row, lane) is input order.
    const uint32_t tile = xcd_block(blockIdx.x, n_tiles);
    const uint32_t base = tile * kTile + wave * (ITEMS * 64);
    uint64_t key[ITEMS];
    uint32_t val[ITEMS];
    uint32_t rank[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const uint32_t i = base + k * 64 + lane;
        const bool valid = i < n;
        key[k] = valid ? kin[i] : 0;
        val[k] = valid ? vin[i] : 0;
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const uint32_t i = base + k * 64 + lane;
        const bool valid = i < n;
        const uint32_t digit = (uint32_t)(key[k] >> shift) & 0xffu;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (digit >> b) & 1u;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t before = wcnt[wave][digit];
        const uint32_t r = (uint32_t)__popcll(peers & lt_mask);
        if (valid && r == 0) wcnt[wave][digit] = before + (uint32_t)__popcll(peers);
        rank[k] = before + r;
    }
    __syncthreads();

    // Per digit: the tile-local start plus the exclusive prefix over waves,
    // and the shift from tile position to output position.
    uint32_t gshift;
    {
        const uint32_t d = threadIdx.x;
        uint32_t run = 0;
        for (int w = 0; w < kWaves; ++w) run += wcnt[w][d];
        uint32_t total;
        const uint32_t start = block_excl_scan_256(run, tmp, &total);
        run = start;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = wcnt[w][d];
            wcnt[w][d] = run;
            run += c;
        }
        // global start of digit d for this tile: all smaller digits, plus
        // digit d in earlier tiles
        const uint32_t digit_base = block_excl_scan_256(row_tot[d], tmp, &total);
        gshift = digit_base + row_pref[d * n_tiles + tile] - start;
    }
    __syncthreads();

#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const uint32_t i = base + k * 64 + lane;
        if (i < n) {
            const uint32_t digit = (uint32_t)(key[k] >> shift) & 0xffu;
            const uint32_t pos = wcnt[wave][digit] + rank[k];
            skey[pos] = key[k];
            sval[pos] = val[k];
        }
    }
    __syncthreads();
    wcnt[0][threadIdx.x] = gshift;
    __syncthreads();

    const uint32_t tile_base = tile * kTile;
    const uint32_t tile_n = min(kTile, n - tile_base);
    if (!GATHER) {
#pragma unroll 4
        for (int k = 0; k < ITEMS; ++k) {
            const uint32_t j = k * kSortThreads + threadIdx.x;
            if (j < tile_n) {
                const uint64_t kk = skey[j];
                const uint32_t vv = sval[j];
                const uint32_t digit = (uint32_t)(kk >> shift) & 0xffu;
                const uint32_t g = wcnt[0][digit] + j;
                kout[g] = kk;
                vout[g] = vv;
            }
        }
    } else {
        // the last pass also gathers the source rows: all of a thread's
        // random reads are issued before any of their stores
        uint32_t gi[ITEMS], vi[ITEMS];
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) {
            const uint32_t j = k * kSortThreads + threadIdx.x;
            gi[k] = 0xffffffffu;
            vi[k] = 0;
            if (j < tile_n) {
                const uint64_t kk = skey[j];
                const uint32_t vv = sval[j];
                const uint32_t digit = (uint32_t)(kk >> shift) & 0xffu;
                const uint32_t g = wcnt[0][digit] + j;
                kout[g] = kk;
                vout[g] = vv;
                gi[k] = g;
                vi[k] = vv;
            }
        }
        float4 row[ITEMS];
#pragma unroll
        for (int k = 0; k < ITEMS; ++k)
            row[k] = gi[k] != 0xffffffffu ? gsrc[vi[k]] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < ITEMS; ++k)
            if (gi[k] != 0xffffffffu) gdst[gi[k]] = row[k];
    }
}

// ---- runs of equal top bits ----------------------------------------------
//
// 63-bit keys are sorted by their top 40 bits in five passes; the keys that
// share those bits form runs (cells 2^-13.3 of the root cube wide: one to a few
// dozen sources in every workload measured), and each run is then put in
// order of its low 24 bits in one kernel, keeping the order of equal keys.
// A source whose run has at most kRunHalo members finds the run in LDS and
// its place by counting the run's members that precede it; longer runs are
// sorted by the workgroup that holds their first member: in LDS up to
// kRunLds members, else by three stable 8-bit counting passes over the run.
constexpr int kRunHalo = 64;
constexpr int kRunLds = 4096;
constexpr int kLowBits = 24;
// a tile that starts this many runs of more than kRunHalo members marks the
// keys as clustered: the workgroup sorts those runs one after another while
// the others wait for it
constexpr uint32_t kRunsClustered = 2;

__device__ inline uint32_t low_of(uint64_t k) { return (uint32_t)k & ((1u << kLowBits) - 1u); }

// One stable counting pass of the run [0, L) by the 8-bit digit at `shift` of
// the low bits: keys and values from (ki, vi) to (ko, vo), with the run held
// at offset s of every array.  Keys may also sit in packed float4 rows
// (PACKED_IN / PACKED_OUT: x, y = key halves, z = value).
template <bool PACKED_IN, bool PACKED_OUT>
__device__ void run_pass(const uint64_t *ki, const uint32_t *vi, const float4 *pi, uint64_t *ko,
                         uint32_t *vo, float4 *po, uint32_t s, uint32_t L, int shift,
                         uint32_t *hist, uint32_t (*wc)[kRadix], uint32_t *tmp)
{
    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    auto load = [&](uint32_t j, uint64_t &k, uint32_t &v) {
        if (PACKED_IN) {
            const uint4 r = reinterpret_cast<const uint4 *>(pi)[s + j];
            k = (uint64_t)r.x | ((uint64_t)r.y << 32);
            v = r.z;
        } else {
            k = ki[s + j];
            v = vi[s + j];
        }
    };
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (uint32_t j = threadIdx.x; j < L; j += kSortThreads) {
        uint64_t k;
        uint32_t v;
        load(j, k, v);
        atomicAdd(&hist[(low_of(k) >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    uint32_t total;
    const uint32_t base0 = block_excl_scan_256(hist[threadIdx.x], tmp, &total);
    __syncthreads();
    hist[threadIdx.x] = base0;   // running output start of each digit
    __syncthreads();
    for (uint32_t t0 = 0; t0 < L; t0 += kSortThreads) {
        const uint32_t j = t0 + threadIdx.x;
        const bool valid = j < L;
        uint64_t k = 0;
        uint32_t v = 0;
        if (valid) load(j, k, v);
        const uint32_t d = (low_of(k) >> shift) & 0xffu;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        for (int w = 0; w < kSortThreads / 64; ++w) wc[w][threadIdx.x] = 0;
        __syncthreads();
        if (valid && (peers & lt_mask) == 0) wc[wave][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t before = 0;
            for (uint32_t w = 0; w < wave; ++w) before += wc[w][d];
            const uint32_t pos = hist[d] + before + (uint32_t)__popcll(peers & lt_mask);
            if (PACKED_OUT) {
                reinterpret_cast<uint4 *>(po)[s + pos] =
                    make_uint4((uint32_t)k, (uint32_t)(k >> 32), v, 0u);
            } else {
                ko[s + pos] = k;
                vo[s + pos] = v;
            }
        }
        __syncthreads();
        {
            uint32_t c = 0;
            for (int w = 0; w < kSortThreads / 64; ++w) c += wc[w][threadIdx.x];
            hist[threadIdx.x] += c;
        }
        __syncthreads();
    }
}

// (kin, vin) sorted by the bits above kLowBits, stably; out: (kout, vout)
// sorted by the whole key, stably, and gdst[p] = gsrc[vout[p]].  clustered
// (host-mapped, may be null) is set to 1 when a tile starts kRunsClustered or
// more runs of more than kRunHalo members.
template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void k_runs(
    const uint64_t *__restrict__ kin, const uint32_t *__restrict__ vin,
    uint64_t *__restrict__ kout, uint32_t *__restrict__ vout, uint32_t n, uint32_t n_tiles,
    const float4 *__restrict__ gsrc, float4 *__restrict__ gdst,
    uint32_t *__restrict__ clustered)
{
    constexpr uint32_t kTile = kSortThreads * ITEMS;
    constexpr uint32_t kWin = kTile + 2 * kRunHalo;
    constexpr uint32_t kLds = kWin > (uint32_t)kRunLds ? kWin : (uint32_t)kRunLds;
    __shared__ uint64_t sk[kLds];                // the tile and its halo; then a run
    __shared__ uint32_t starts[kTile / (kRunHalo + 1) + 2];
    __shared__ uint32_t n_starts;
    __shared__ uint32_t hist[kRadix];
    __shared__ uint32_t wc[kSortThreads / 64][kRadix];
    __shared__ uint32_t tmp[kSortThreads / 64];
    __shared__ uint32_t found;

    const uint32_t tile = xcd_block(blockIdx.x, n_tiles);
    const int64_t t0 = (int64_t)tile * kTile;
    const int64_t w0 = t0 - kRunHalo;
    if (threadIdx.x == 0) n_starts = 0;
    for (uint32_t k = threadIdx.x; k < kWin; k += kSortThreads) {
        const int64_t a = w0 + k;
        sk[k] = (a >= 0 && a < (int64_t)n) ? kin[a] : 0ull;
    }
    __syncthreads();
    auto top = [](uint64_t k) { return k >> kLowBits; };
    for (int it = 0; it < ITEMS; ++it) {
        const int64_t i = t0 + it * kSortThreads + threadIdx.x;
        if (i >= (int64_t)n) break;
        const uint32_t li = (uint32_t)(i - w0);
        const uint64_t key = sk[li];
        const uint64_t h = top(key);
        // the run [s, e) around i, searched up to kRunHalo either side
        uint32_t ls = li, le = li + 1;
        int64_t s = i, e = i + 1;
        while (s > 0 && li - ls < (uint32_t)kRunHalo && top(sk[ls - 1]) == h) { --ls; --s; }
        while (e < (int64_t)n && le - li - 1 < (uint32_t)kRunHalo && top(sk[le]) == h) { ++le; ++e; }
        // a search that used all its steps stopped inside a run of more than
        // kRunHalo members; otherwise it stopped at the run's end
        const bool lo_cap = li - ls >= (uint32_t)kRunHalo;
        const bool hi_cap = le - li - 1 >= (uint32_t)kRunHalo;
        if (!lo_cap && !hi_cap && e - s <= kRunHalo) {
            uint32_t rank = 0;
            const uint32_t lo = low_of(key);
            for (uint32_t j = ls; j < le; ++j) {
                const uint32_t lj = low_of(sk[j]);
                rank += (lj < lo || (lj == lo && j < li)) ? 1u : 0u;
            }
            const int64_t p = s + rank;
            const uint32_t v = vin[i];
            kout[p] = key;
            vout[p] = v;
            gdst[p] = gsrc[v];
        } else if (ls == li) {
            starts[atomicAdd(&n_starts, 1u)] = (uint32_t)i;   // a long run starts here
        }
    }
    __syncthreads();
    const uint32_t ns = n_starts;
    if (clustered && threadIdx.x == 0 && ns >= kRunsClustered) *clustered = 1u;
    for (uint32_t r = 0; r < ns; ++r) {
        const uint32_t s = starts[r];
        const uint64_t h = top(kin[s]);
        // the run's end: the first position past s with other top bits
        uint32_t e = s + 1;
        for (;;) {
            if (threadIdx.x == 0) found = 0xffffffffu;
            __syncthreads();
            const uint32_t j = e + threadIdx.x;
            if (j < n && top(kin[j]) != h) atomicMin(&found, j);
            if (j >= n) atomicMin(&found, n);
            __syncthreads();
            const uint32_t f = found;
            __syncthreads();
            if (f != 0xffffffffu) {
                e = f;
                break;
            }
            e += kSortThreads;
        }
        const uint32_t L = e - s;
        if (L <= (uint32_t)kRunLds) {
            // bitonic sort of (low bits, place in the run) in LDS
            uint32_t P = 1;
            while (P < L) P <<= 1;
            for (uint32_t j = threadIdx.x; j < P; j += kSortThreads)
                sk[j] = j < L ? (((uint64_t)low_of(kin[s + j]) << 32) | j) : ~0ull;
            __syncthreads();
            for (uint32_t k = 2; k <= P; k <<= 1) {
                for (uint32_t m = k >> 1; m > 0; m >>= 1) {
                    for (uint32_t j = threadIdx.x; j < P; j += kSortThreads) {
                        const uint32_t q = j ^ m;
                        if (q > j) {
                            const uint64_t a = sk[j], b = sk[q];
                            const bool up = (j & k) == 0;
                            if ((a > b) == up) {
                                sk[j] = b;
                                sk[q] = a;
                            }
                        }
                    }
                    __syncthreads();
                }
            }
            for (uint32_t k = threadIdx.x; k < L; k += kSortThreads) {
                const uint32_t src = s + (uint32_t)(sk[k] & 0xffffffffull);
                const uint32_t v = vin[src];
                kout[s + k] = kin[src];
                vout[s + k] = v;
                gdst[s + k] = gsrc[v];
            }
            __syncthreads();
        } else {
            // three stable counting passes over the low bits: (kin, vin) ->
            // (kout, vout) -> rows of gdst -> (kout, vout), then the gather
            run_pass<false, false>(kin, vin, nullptr, kout, vout, nullptr, s, L, 0, hist, wc, tmp);
            run_pass<false, true>(kout, vout, nullptr, nullptr, nullptr, gdst, s, L, 8, hist, wc,
                                  tmp);
            run_pass<true, false>(nullptr, nullptr, gdst, kout, vout, nullptr, s, L, 16, hist, wc,
                                  tmp);
            for (uint32_t k = threadIdx.x; k < L; k += kSortThreads) gdst[s + k] = gsrc[vout[s + k]];
            __syncthreads();
        }
    }
}

constexpr int kScanThreads = 256;

// Exclusive scan of each row of a [rows][len] table, one workgroup per row:
// pref[r][t] = sum(in[r][0..t)), tot[r] = sum(in[r][0..len)).  Coalesced
// rounds of 256 entries carry the running sum.
__global__ __launch_bounds__(kScanThreads) void k_scan_rows(const uint32_t *__restrict__ in,
                                                            uint32_t *__restrict__ pref,
                                                            uint32_t *__restrict__ tot,
                                                            uint32_t len)
{
    __shared__ uint32_t tmp[kScanThreads / 64];
    const size_t row = (size_t)blockIdx.x * len;
    uint32_t carry = 0;
    for (uint32_t b = 0; b < len; b += kScanThreads) {
        const uint32_t t = b + threadIdx.x;
        const uint32_t v = t < len ? in[row + t] : 0u;
        uint32_t total;
        const uint32_t ex = block_excl_scan_256(v, tmp, &total);
        if (t < len) pref[row + t] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) tot[blockIdx.x] = carry;
}

}  // namespace

size_t sort_spine_entries(uint32_t n)
{
    size_t tiles = (n + kSortTile - 1) / kSortTile;
    if (tiles == 0) tiles = 1;
    return 2 * (size_t)kRadix * tiles + kRadix;
}

void launch_scan_rows(const uint32_t *in, uint32_t *pref, uint32_t *tot, uint32_t rows,
                      uint32_t len, hipStream_t s)
{
    hipLaunchKernelGGL(k_scan_rows, dim3(rows), dim3(kScanThreads), 0, s, in, pref, tot, len);
}

namespace {

template <int ITEMS>
void sort_passes(uint64_t *&ka, uint32_t *&va, uint64_t *&kb, uint32_t *&vb, uint32_t n,
                 int key_bits, int skip_bits, uint32_t *spine, const float4 *gather_src,
                 float4 *gather_dst, const SortRuns &sr, hipStream_t s)
{
    constexpr uint32_t tile = kSortThreads * ITEMS;
    const uint32_t tiles = (n + tile - 1) / tile;
    const uint32_t entries = kRadix * tiles;
    uint32_t *hist = spine, *pref = spine + entries, *tot = spine + 2 * entries;
    const int passes = (key_bits + 7) / 8;
    // long keys with a gather: passes over the bits above kLowBits, then runs
    // (unless the caller asks for every pass)
    const bool runs = gather_src && key_bits > 40 && !sr.all_passes;
    const int p0 = runs ? kLowBits / 8 : skip_bits / 8;
    for (int p = p0; p < passes; ++p) {
        const int shift = 8 * p;
        const bool last = !runs && (p == passes - 1);
        hipLaunchKernelGGL(k_hist<ITEMS>, dim3(tiles), dim3(kSortThreads), 0, s, ka, n, shift,
                           hist, tiles);
        launch_scan_rows(hist, pref, tot, kRadix, tiles, s);
        if (last && gather_src) {
            hipLaunchKernelGGL((k_scatter<true, ITEMS>), dim3(tiles), dim3(kSortThreads), 0, s, ka,
                               va, kb, vb, n, shift, pref, tot, tiles, gather_src, gather_dst);
        } else {
            hipLaunchKernelGGL((k_scatter<false, ITEMS>), dim3(tiles), dim3(kSortThreads), 0, s,
                               ka, va, kb, vb, n, shift, pref, tot, tiles,
                               (const float4 *)nullptr, (float4 *)nullptr);
        }
        uint64_t *tk = ka; ka = kb; kb = tk;
        uint32_t *tv = va; va = vb; vb = tv;
    }
    if (runs) {
        hipLaunchKernelGGL(k_runs<ITEMS>, dim3(tiles), dim3(kSortThreads), 0, s, ka, va, kb, vb,
                           n, tiles, gather_src, gather_dst, sr.clustered);
        uint64_t *tk = ka; ka = kb; kb = tk;
        uint32_t *tv = va; va = vb; vb = tv;
    }
}

}  // namespace

// Small inputs take 2048-key tiles (enough workgroups to fill the device);
// large ones 4096-key tiles, whose digit runs are twice as long, so more of
// the scattered writes fill whole cache lines.
void radix_sort(uint64_t *keys, uint32_t *vals, uint64_t *keys_alt, uint32_t *vals_alt,
                uint64_t **keys_out, uint32_t **vals_out, uint32_t n, int key_bits,
                int skip_bits, uint32_t *spine, const float4 *gather_src, float4 *gather_dst,
                const SortRuns &sr, hipStream_t s)
{
    uint64_t *ka = keys, *kb = keys_alt;
    uint32_t *va = vals, *vb = vals_alt;
    if (n > 0) {
        if (n >= kSortLargeN)
            sort_passes<kSortItemsLarge>(ka, va, kb, vb, n, key_bits, skip_bits, spine,
                                         gather_src, gather_dst, sr, s);
        else
            sort_passes<kSortItems>(ka, va, kb, vb, n, key_bits, skip_bits, spine, gather_src,
                                    gather_dst, sr, s);
    }
    *keys_out = ka;
    *vals_out = va;
}

}  // namespace bh
