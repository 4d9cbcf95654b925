// sort.hip -- stable counting sort of positions by bucket, per (b, h, round).
// "Reformer: The Efficient Transformer", §2: sorting by bucket (positions
// carried along) clusters same-bucket pairs; ties keep position order.
//
// Two launches over S = B*H*nh segments of L positions, in tiles of kTile
// positions (one workgroup per (segment, tile)):
//   sort_count    the tile's bucket counts, as 16-bit values -> cnt[S][T][nb]
//   sort_scatter  reads its segment's whole count matrix (a few tens of KB,
//                 from L2: all tiles of a segment run on one XCD) and forms
//                 from it both the bucket totals (their exclusive scan gives
//                 each bucket's first sorted index) and the counts of the
//                 earlier tiles; then ranks its positions stably and writes
//                 perm / inv / win_lo.
// No pass is serial over a segment, nothing needs zeroing between calls, and
// each segment's count matrix is re-read by its T tiles instead of being
// scanned once by a single workgroup.
#include <mutex>

#include "common.hpp"

namespace lsh {
namespace {

constexpr int kTile = 4096;                                 // positions per workgroup
constexpr int kMaxBuckets = 4096;
constexpr int kMaxTiles = 65536 / kTile;                    // L <= 65536
static_assert(kTile <= 65535, "tile counts are stored in 16 bits");
// Workgroups of W waves: 8 while the per-wave counters fit LDS beside the
// bucket starts (nb <= 2048), else 4.
constexpr int kWideBuckets = 2048;

// The tile's positions as the waves walk them: wave w owns the w-th part of
// kTile / W positions, group g of it the 64 positions from g * 64.
template <int W>
__device__ __forceinline__ int tile_pos(int tile, int wave, int g, int lane)
{
    return tile * kTile + wave * (kTile / W) + g * kWave + lane;
}

// A bucket id as both kernels use it: clamped into [0, nb), so that ids
// outside the range (undefined behaviour by the contract) still give in-range
// sorted indices, consistently in both kernels.
__device__ __forceinline__ int clamp_bucket(int32_t b, int nb) { return b < 0 ? 0 : (b >= nb ? nb - 1 : b); }

template <int W>
__global__ __launch_bounds__(W * kWave) void sort_count(int L, int nb, int ntiles, const int32_t *__restrict__ buckets,
                                                        uint32_t *__restrict__ cnt)
{
    constexpr int kThreads = W * kWave, kGroups = kTile / kThreads;
    extern __shared__ uint32_t h[];   // [nb]
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int tile = lb % ntiles, seg = lb / ntiles, tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int32_t *bk = buckets + (size_t)seg * L;
    int32_t x[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int t = tile_pos<W>(tile, wave, g, lane);
        x[g] = t < L ? clamp_bucket(bk[t], nb) : -1;
    }
    for (int b = tid; b < nb; b += kThreads)
        h[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
        if (x[g] >= 0)
            atomicAdd(&h[x[g]], 1u);
    __syncthreads();
    // two 16-bit counts per word (nb is even)
    uint32_t *out = cnt + ((size_t)seg * ntiles + tile) * (nb / 2);
    for (int p = tid; p < nb / 2; p += kThreads)
        out[p] = h[2 * p] | (h[2 * p + 1] << 16);
}

// Exclusive scan of v[0 .. n) in LDS (n <= kMaxBuckets) by a workgroup of W
// waves, in place; ends with a workgroup barrier.
template <int W>
__device__ void block_exclusive_scan(uint32_t *v, int n, uint32_t *wsum)
{
    constexpr int kThreads = W * kWave;
    constexpr int per = kMaxBuckets / kThreads;   // consecutive entries per thread
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    uint32_t loc[per];
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < per; ++k) {
        const int i = tid * per + k;
        loc[k] = i < n ? v[i] : 0u;
        sum += loc[k];
    }
    // inclusive scan of the thread sums within the wave, then across the waves
    uint32_t inc = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, kWave);
        if (lane >= o)
            inc += y;
    }
    if (lane == kWave - 1)
        wsum[wave] = inc;
    __syncthreads();
    uint32_t run = inc - sum;
    for (int w = 0; w < wave; ++w)
        run += wsum[w];
#pragma unroll
    for (int k = 0; k < per; ++k) {
        const int i = tid * per + k;
        if (i < n)
            v[i] = run;
        run += loc[k];
    }
    __syncthreads();
}

template <int W>
__global__ __launch_bounds__(W * kWave) void sort_scatter(int L, int nb, int nbits, int m, uint64_t mmagic, int ntiles,
                                                         const int32_t *__restrict__ buckets,
                                                         const uint32_t *__restrict__ cnt,
                                                         int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                         int32_t *__restrict__ win_lo)
{
    // LDS: bstart[nb] (bucket totals, then the first sorted index of each
    // bucket), pre[nb] (counts of the earlier tiles), wcnt[kWaves][nb]
    // (per-wave counts, then each wave's next sorted index per bucket)
    constexpr int kThreads = W * kWave, kWaves = W, kGroups = kTile / kThreads;
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t wsum[kWaves];
    uint32_t *bstart = lds, *pre = lds + nb, *wcnt = lds + 2 * nb;
    // all tiles of a segment on one XCD: their scattered 4-byte writes into
    // the segment's sorted order then meet in one L2, which merges them into
    // whole lines before they go to memory, and the segment's count matrix
    // is read from that L2 by all of them
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int tile = lb % ntiles, seg = lb / ntiles, tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int32_t *bk = buckets + (size_t)seg * L;
    int32_t x[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int t = tile_pos<W>(tile, wave, g, lane);
        x[g] = t < L ? clamp_bucket(bk[t], nb) : -1;
    }
    for (int k = tid; k < kWaves * nb; k += kThreads)
        wcnt[k] = 0u;
    // 1. the segment's bucket totals, and the counts of the tiles before this one
    const uint32_t *cs = cnt + (size_t)seg * ntiles * (nb / 2);
    for (int p = tid; p < nb / 2; p += kThreads) {
        uint32_t tot_lo = 0u, tot_hi = 0u, pre_lo = 0u, pre_hi = 0u;
        // every tile's word requested before any is added (at most kMaxTiles tiles)
        uint32_t cw[kMaxTiles];
#pragma unroll
        for (int t = 0; t < kMaxTiles; ++t)
            cw[t] = t < ntiles ? cs[(size_t)t * (nb / 2) + p] : 0u;
#pragma unroll
        for (int t = 0; t < kMaxTiles; ++t) {
            if (t == tile) {
                pre_lo = tot_lo;
                pre_hi = tot_hi;
            }
            tot_lo += cw[t] & 0xffffu;
            tot_hi += cw[t] >> 16;
        }
        bstart[2 * p] = tot_lo;
        bstart[2 * p + 1] = tot_hi;
        pre[2 * p] = pre_lo;
        pre[2 * p + 1] = pre_hi;
    }
    __syncthreads();
    // 2. each wave's counts of its quarter of the tile
    uint32_t *mine = wcnt + wave * nb;
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
        if (x[g] >= 0)
            atomicAdd(&mine[x[g]], 1u);
    // 3. first sorted index of each bucket (the barrier at its end also
    //    completes the counts above)
    block_exclusive_scan<W>(bstart, nb, wsum);
    // 4. first sorted index of each (wave, bucket) run of this tile
    for (int b = tid; b < nb; b += kThreads) {
        uint32_t run = bstart[b] + pre[b];
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = wcnt[w * nb + b];
            wcnt[w * nb + b] = run;
            run += c;
        }
    }
    __syncthreads();
    // 5. each wave walks its part in order, 64 positions at a time.  Lanes
    //    holding the same bucket are ranked by lane index (ballots over the
    //    bucket's bits); the group's lowest such lane takes the bucket's next
    //    sorted indices from the wave's counter with one fetch-and-add, whose
    //    result the others read from it.  A wave's LDS operations complete in
    //    program order, so earlier groups get lower indices, and no group waits
    //    for the one before it.
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t *pr = perm + (size_t)seg * L, *iv = inv + (size_t)seg * L, *wl = win_lo + (size_t)seg * L;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int t = tile_pos<W>(tile, wave, g, lane);
        const bool valid = x[g] >= 0;
        const int b = valid ? x[g] : 0;
        uint64_t peers = __ballot(valid);
        if (peers == 0ull)
            break;   // the rest of the wave's part is past L
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (b >> bit) & 1;
            const uint64_t set = __ballot(valid && on);
            peers &= on ? set : ~set;
        }
        const int rank = __popcll(peers & lt_mask);
        uint32_t base = 0u;
        if (valid && rank == 0)
            base = atomicAdd(&mine[b], (uint32_t)__popcll(peers));
        // the lowest peer (a lane without peers, past L, reads lane 63 and ignores it)
        base = (uint32_t)__shfl((int)base, (__ffsll((long long)peers) - 1) & (kWave - 1), kWave);
        if (valid) {
            const uint32_t s = base + (uint32_t)rank;
            pr[s] = t;
            iv[t] = (int32_t)s;
            // s / m as a multiply: floor(s * (floor(2^32 / m) + 1) / 2^32) is
            // exact for s < 2^16 and m <= 2^16
            const int lo_chunk = ((int)(((uint64_t)s * mmagic) >> 32) - 1) * m;
            const int lo_bucket = (int)bstart[b];
            wl[t] = lo_bucket > lo_chunk ? lo_bucket : lo_chunk;
        }
    }
}

int ntiles_of(const Dims &P) { return (P.L + kTile - 1) / kTile; }

}  // namespace

// Scratch of lsh_sort_noalloc: the count matrix in a static device array
// instead of a caller's workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` only names the
// symbol; its device address, per GPU, comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the GPU that `stream` belongs to (the
// current GPU for the null stream), looked up once per GPU with that GPU
// current, then kept.
hipError_t scratch_address(hipStream_t stream, void **out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess)
                e = r;
        }
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t sort_noalloc_max_bytes() { return kNoAllocScratchBytes; }

hipError_t launch_sort_noalloc(const Dims &P, const int32_t *buckets, int32_t *perm, int32_t *inv, int32_t *win_lo,
                               hipStream_t st)
{
    if (sort_ws_bytes(P) > kNoAllocScratchBytes)
        return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = scratch_address(st, &ws);
    if (e != hipSuccess)
        return e;
    return launch_sort(P, buckets, perm, inv, win_lo, ws, st);
}

size_t sort_ws_bytes(const Dims &P)
{
    const size_t S = (size_t)P.BH() * P.nh;
    return align_up(S * ntiles_of(P) * (P.nb / 2) * sizeof(uint32_t), 256);
}

hipError_t launch_sort(const Dims &P, const int32_t *buckets, int32_t *perm, int32_t *inv, int32_t *win_lo,
                       void *ws, hipStream_t st)
{
    if (P.nb > kMaxBuckets || (P.nb & 1) || P.L > 65536)
        return hipErrorInvalidValue;
    const int S = P.BH() * P.nh;
    const int nt = ntiles_of(P);
    uint32_t *cnt = (uint32_t *)ws;
    int nbits = 0;
    while ((1 << nbits) < P.nb)
        ++nbits;
    const unsigned grid = (unsigned)S * (unsigned)nt;
    const bool wide = P.nb <= kWideBuckets;
    {
        ProfScope prof(LSH_KERNEL_SORT_COUNT, st);
        if (wide)
            hipLaunchKernelGGL(sort_count<8>, dim3(grid), dim3(8 * kWave), (size_t)P.nb * sizeof(uint32_t), st, P.L,
                               P.nb, nt, buckets, cnt);
        else
            hipLaunchKernelGGL(sort_count<4>, dim3(grid), dim3(4 * kWave), (size_t)P.nb * sizeof(uint32_t), st, P.L,
                               P.nb, nt, buckets, cnt);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const uint64_t mmagic = (uint64_t)(0xffffffffull / (uint64_t)P.m) + 1u;
    ProfScope prof(LSH_KERNEL_SORT_SCATTER, st);
    if (wide)
        hipLaunchKernelGGL(sort_scatter<8>, dim3(grid), dim3(8 * kWave), (size_t)(2 + 8) * P.nb * sizeof(uint32_t), st,
                           P.L, P.nb, nbits, P.m, mmagic, nt, buckets, (const uint32_t *)cnt, perm, inv, win_lo);
    else
        hipLaunchKernelGGL(sort_scatter<4>, dim3(grid), dim3(4 * kWave), (size_t)(2 + 4) * P.nb * sizeof(uint32_t), st,
                           P.L, P.nb, nbits, P.m, mmagic, nt, buckets, (const uint32_t *)cnt, perm, inv, win_lo);
    return hipGetLastError();
}

}  // namespace lsh
