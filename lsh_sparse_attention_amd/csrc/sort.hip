// sort.hip -- stable counting sort of positions by bucket, per (b, h, round).
// "Reformer: The Efficient Transformer", §2: sorting by bucket (positions
// carried along) clusters same-bucket pairs; ties keep position order.
//
// Three launches over S = B*H*nh segments of L positions, tiles of kTile:
//   sort_hist    per (tile, segment): bucket counts of the tile   -> cnt[S][T][nb]
//   sort_scan    per segment: cnt becomes the first sorted index of each
//                (tile, bucket) run; bstart = first sorted index of each bucket
//   sort_scatter per (tile, segment): stable rank inside the tile, then
//                perm / inv / win_lo.
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kTile = 2048;
constexpr int kScatterThreads = 256;                      // 4 waves
constexpr int kWavePositions = kTile / (kScatterThreads / kWave);  // 512 per wave
constexpr int kScanThreads = 1024;
constexpr int kMaxBuckets = 4096;

__global__ __launch_bounds__(kScatterThreads) void sort_hist(int L, int nb, int ntiles,
                                                             const int32_t *__restrict__ buckets,
                                                             int32_t *__restrict__ cnt)
{
    extern __shared__ int32_t h[];
    const int tile = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x;
    for (int b = tid; b < nb; b += kScatterThreads)
        h[b] = 0;
    __syncthreads();
    const int32_t *bk = buckets + (size_t)seg * L;
    const int base = tile * kTile;
    for (int k = tid; k < kTile; k += kScatterThreads) {
        int t = base + k;
        if (t < L)
            atomicAdd(&h[bk[t]], 1);
    }
    __syncthreads();
    int32_t *out = cnt + ((size_t)seg * ntiles + tile) * nb;
    for (int b = tid; b < nb; b += kScatterThreads)
        out[b] = h[b];
}

// Exclusive scan of the nb bucket totals inside one block (nb <= 4 * 1024).
__device__ void block_exclusive_scan(int32_t *vals, int nb, int32_t *tmp)
{
    const int tid = threadIdx.x;
    constexpr int per = kMaxBuckets / kScanThreads;  // 4
    int32_t loc[per];
    int32_t sum = 0;
#pragma unroll
    for (int k = 0; k < per; ++k) {
        int b = tid * per + k;
        loc[k] = b < nb ? vals[b] : 0;
        sum += loc[k];
    }
    tmp[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int32_t add = tid >= off ? tmp[tid - off] : 0;
        __syncthreads();
        tmp[tid] += add;
        __syncthreads();
    }
    int32_t run = tmp[tid] - sum;  // exclusive prefix of this thread's group
#pragma unroll
    for (int k = 0; k < per; ++k) {
        int b = tid * per + k;
        if (b < nb)
            vals[b] = run;
        run += loc[k];
    }
    __syncthreads();
}

__global__ __launch_bounds__(kScanThreads) void sort_scan(int nb, int ntiles, int32_t *__restrict__ cnt,
                                                          int32_t *__restrict__ bstart)
{
    __shared__ int32_t tot[kMaxBuckets];
    __shared__ int32_t tmp[kScanThreads];
    const int seg = blockIdx.x, tid = threadIdx.x;
    int32_t *c = cnt + (size_t)seg * ntiles * nb;
    // per bucket: exclusive prefix over tiles, and the bucket total
    for (int b = tid; b < nb; b += kScanThreads) {
        int32_t run = 0;
        for (int t = 0; t < ntiles; ++t) {
            int32_t x = c[(size_t)t * nb + b];
            c[(size_t)t * nb + b] = run;
            run += x;
        }
        tot[b] = run;
    }
    __syncthreads();
    block_exclusive_scan(tot, nb, tmp);
    for (int b = tid; b < nb; b += kScanThreads) {
        int32_t s = tot[b];
        bstart[(size_t)seg * nb + b] = s;
        for (int t = 0; t < ntiles; ++t)
            c[(size_t)t * nb + b] += s;
    }
}

__global__ __launch_bounds__(kScatterThreads) void sort_scatter(int L, int nb, int nbits, int m, int ntiles,
                                                                const int32_t *__restrict__ buckets,
                                                                const int32_t *__restrict__ off,
                                                                const int32_t *__restrict__ bstart,
                                                                int32_t *__restrict__ perm,
                                                                int32_t *__restrict__ inv,
                                                                int32_t *__restrict__ win_lo)
{
    extern __shared__ int32_t wcnt[];  // [4][nb]
    // all tiles of a segment on one XCD: their scattered 4-byte writes into
    // the segment's sorted order then meet in one L2, which merges them into
    // whole lines before they go to memory
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int tile = lb % ntiles, seg = lb / ntiles, tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int nwaves = kScatterThreads / kWave;
    for (int k = tid; k < nwaves * nb; k += kScatterThreads)
        wcnt[k] = 0;
    __syncthreads();
    const int32_t *bk = buckets + (size_t)seg * L;
    const int wbase = tile * kTile + wave * kWavePositions;
    int32_t *mine = wcnt + wave * nb;
    // 1. counts of each wave's sub-range
    for (int g = 0; g < kWavePositions; g += kWave) {
        int t = wbase + g + lane;
        if (t < L)
            atomicAdd(&mine[bk[t]], 1);
    }
    __syncthreads();
    // 2. first sorted index of each (wave, bucket) run: tile offset plus the
    //    counts of the earlier waves of this tile
    const int32_t *toff = off + ((size_t)seg * ntiles + tile) * nb;
    for (int b = tid; b < nb; b += kScatterThreads) {
        int32_t run = toff[b];
        for (int w = 0; w < nwaves; ++w) {
            int32_t x = wcnt[w * nb + b];
            wcnt[w * nb + b] = run;
            run += x;
        }
    }
    __syncthreads();
    // 3. each wave walks its sub-range in order, 64 positions at a time;
    //    lanes holding the same bucket are ranked by lane index.
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t *bs = bstart + (size_t)seg * nb;
    int32_t *pr = perm + (size_t)seg * L, *iv = inv + (size_t)seg * L, *wl = win_lo + (size_t)seg * L;
    for (int g = 0; g < kWavePositions; g += kWave) {
        const int t = wbase + g + lane;
        const bool valid = t < L;
        const int b = valid ? bk[t] : 0;
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (b >> bit) & 1;
            const uint64_t set = __ballot(valid && on);
            peers &= on ? set : ~set;
        }
        const int rank = __popcll(peers & lt_mask);
        int32_t s = 0;
        if (valid)
            s = mine[b] + rank;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (valid && rank == 0)
            mine[b] = s + __popcll(peers);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (valid) {
            pr[s] = t;
            iv[t] = s;
            const int lo_chunk = (s / m - 1) * m;
            const int lo_bucket = bs[b];
            wl[t] = lo_bucket > lo_chunk ? lo_bucket : lo_chunk;
        }
    }
}

int ntiles_of(const Dims &P) { return (P.L + kTile - 1) / kTile; }

}  // namespace

size_t sort_ws_bytes(const Dims &P)
{
    size_t S = (size_t)P.BH() * P.nh;
    return align_up(S * ntiles_of(P) * P.nb * sizeof(int32_t), 256) + align_up(S * P.nb * sizeof(int32_t), 256);
}

hipError_t launch_sort(const Dims &P, const int32_t *buckets, int32_t *perm, int32_t *inv, int32_t *win_lo,
                       void *ws, hipStream_t st)
{
    if (P.nb > kMaxBuckets)
        return hipErrorInvalidValue;
    const int S = P.BH() * P.nh;
    const int nt = ntiles_of(P);
    int32_t *cnt = (int32_t *)ws;
    int32_t *bstart = (int32_t *)((char *)ws + align_up((size_t)S * nt * P.nb * sizeof(int32_t), 256));
    int nbits = 0;
    while ((1 << nbits) < P.nb)
        ++nbits;
    const size_t lds_hist = (size_t)P.nb * sizeof(int32_t);
    {
        ProfScope prof(LSH_KERNEL_SORT_HIST, st);
        hipLaunchKernelGGL(sort_hist, dim3(nt, S), dim3(kScatterThreads), lds_hist, st, P.L, P.nb, nt, buckets,
                           cnt);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    {
        ProfScope prof(LSH_KERNEL_SORT_SCAN, st);
        hipLaunchKernelGGL(sort_scan, dim3(S), dim3(kScanThreads), 0, st, P.nb, nt, cnt, bstart);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const size_t lds_scatter = (size_t)(kScatterThreads / kWave) * P.nb * sizeof(int32_t);
    ProfScope prof(LSH_KERNEL_SORT_SCATTER, st);
    hipLaunchKernelGGL(sort_scatter, dim3(nt * S), dim3(kScatterThreads), lds_scatter, st, P.L, P.nb, nbits, P.m,
                       nt, buckets, (const int32_t *)cnt, (const int32_t *)bstart, perm, inv, win_lo);
    return hipGetLastError();
}

}  // namespace lsh
