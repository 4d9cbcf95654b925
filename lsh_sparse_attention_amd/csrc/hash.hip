// hash.hip -- angular LSH by random rotation: bucket = argmax([qR_r ; -qR_r]).
// "Reformer: The Efficient Transformer", §2 (random projections).
// fp32 problems use a per-thread fp32 kernel; bf16 problems use the matrix
// cores (exact bf16 products, fp32 sums).
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kHashThreads = 256;
constexpr int kCols = 16;  // rotation columns accumulated per pass

// One thread per (row, round).  The query row sits in registers; the rotation
// column block is read with wave-uniform addresses (scalar loads).  Products
// are exact for bf16 inputs and summed in fp32 with fma.
template <typename T, int D>
__global__ __launch_bounds__(kHashThreads) void hash_generic(int L, int nh, int half, const T *__restrict__ q,
                                                             const T *__restrict__ rot,
                                                             int32_t *__restrict__ buckets)
{
    const int t = blockIdx.x * kHashThreads + threadIdx.x;
    const int r = blockIdx.y;
    const int bh = blockIdx.z;
    if (t >= L)
        return;
    const T *row = q + ((size_t)bh * L + t) * D;
    float qr[D];
#pragma unroll
    for (int k = 0; k < D; ++k)
        qr[k] = ld(row, k);
    const T *R = rot + (size_t)r * D * half;
    float best_pos = -INFINITY, best_neg = -INFINITY;
    int arg_pos = 0, arg_neg = 0;
    for (int j0 = 0; j0 < half; j0 += kCols) {
        float y[kCols];
#pragma unroll
        for (int c = 0; c < kCols; ++c)
            y[c] = 0.f;
        if (j0 + kCols <= half) {
#pragma unroll
            for (int k = 0; k < D; ++k) {
#pragma unroll
                for (int c = 0; c < kCols; ++c)
                    y[c] = fmaf(qr[k], ld(R, (size_t)k * half + j0 + c), y[c]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < D; ++k) {
#pragma unroll
                for (int c = 0; c < kCols; ++c)
                    if (j0 + c < half)
                        y[c] = fmaf(qr[k], ld(R, (size_t)k * half + j0 + c), y[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
            if (j0 + c < half) {
                if (y[c] > best_pos) {
                    best_pos = y[c];
                    arg_pos = j0 + c;
                }
                if (-y[c] > best_neg) {
                    best_neg = -y[c];
                    arg_neg = j0 + c;
                }
            }
        }
    }
    // first index of the maximum over the concatenation [+y ; -y]
    buckets[((size_t)bh * nh + r) * L + t] = (best_pos >= best_neg) ? arg_pos : half + arg_neg;
}

// bf16 path on the matrix cores.  A workgroup (4 waves) owns 256 rows of one
// (batch, head); a wave owns 64 rows as two 32-row MFMA column tiles.  For
// every round the rotation is walked in blocks of 64 columns, staged
// row-major in LDS (fetched one block ahead) and read transposed with
// ds_read_b64_tr_b16, so Y^T = R^T Q^T comes out with lane = row and 16
// columns per lane per 32-column tile.  The running argmax over [y ; -y]
// keeps, per row, the best entry's key and the scores of the tile that holds
// it (tile_track); the winning column is found in that tile when the round
// ends, and the two lane halves that share a row are merged last.  bf16
// products are exact in the fp32 accumulator.
constexpr int kHashRows = 256;
constexpr int kHashCols = 64;              // rotation columns per staged block

// Argmax over [y ; -y] with first-index ties, slot search deferred to the
// end of the round.  Per row (column tile ct) the round's
// best entry so far is kept as a key and the lane's 16 scores y' = -y of the
// tile that holds it; the slot inside that tile is searched for once, when
// the round ends.  Per tile the lane takes the largest +y entry (max of -y')
// and the largest -y entry (max of y') with three-input maxima; the larger
// one wins, +y on equal magnitude (it has the lower index).  Its key is
// (bits of the magnitude << 1) | (1 for +y): keys order entries like
// [y ; -y] does except for the index, and a strictly larger key replaces the
// tracked one, so an earlier tile (lower index) wins ties.  Every real key is
// at least 1 (a -y winner has nonzero magnitude), so the initial 0 is
// replaced by the first tile.
__device__ __forceinline__ void tile_track(const f32x16_t (&acc)[2], int j0, uint32_t (&bk)[2], int (&bj)[2],
                                           f32x16_t (&sv)[2])
{
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const f32x16_t &a = acc[ct];
        const float mp = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(-a[0], -a[1]), -a[2]), fmaxf(fmaxf(-a[3], -a[4]), -a[5])),
                                     fmaxf(fmaxf(fmaxf(-a[6], -a[7]), -a[8]), fmaxf(fmaxf(-a[9], -a[10]), -a[11]))),
                               fmaxf(fmaxf(fmaxf(-a[12], -a[13]), -a[14]), -a[15]));
        const float mn = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(a[0], a[1]), a[2]), fmaxf(fmaxf(a[3], a[4]), a[5])),
                                     fmaxf(fmaxf(fmaxf(a[6], a[7]), a[8]), fmaxf(fmaxf(a[9], a[10]), a[11]))),
                               fmaxf(fmaxf(fmaxf(a[12], a[13]), a[14]), a[15]));
        const bool plus = mp >= mn;
        const uint32_t key = (__float_as_uint(plus ? mp : mn) << 1) | (plus ? 1u : 0u);
        const bool better = key > bk[ct];
        bk[ct] = better ? key : bk[ct];
        bj[ct] = better ? j0 : bj[ct];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            sv[ct][e] = better ? a[e] : sv[ct][e];
    }
}

// End of a round under the deferred search: the first slot of the kept tile
// whose score is the tracked entry (y' = -magnitude for +y, +magnitude for
// -y; floating equality, so a zero matches either sign), then the merge with
// the other half of the row (larger key, else smaller column), the store and
// the reset.
__device__ __forceinline__ void round_store_tracked(uint32_t (&bk)[2], int (&bj)[2], const f32x16_t (&sv)[2], int h,
                                                    int c, int row0, int L, int half, int32_t *__restrict__ out)
{
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const uint32_t k0 = bk[ct];
        const float mag = __uint_as_float(k0 >> 1);
        const float want = (k0 & 1u) ? -mag : mag;
        int slot = 0;
#pragma unroll
        for (int e = 15; e >= 0; --e)
            slot = sv[ct][e] == want ? 8 * (e / 4) + (e % 4) : slot;
        int i0 = bj[ct] + slot + 4 * h;
        uint32_t kk = k0;
        const auto pk = __builtin_amdgcn_permlane32_swap(kk, kk, false, false);
        const auto pi = __builtin_amdgcn_permlane32_swap((uint32_t)i0, (uint32_t)i0, false, false);
        const uint32_t ok = h ? pk[0] : pk[1];
        const int oi = (int)(h ? pi[0] : pi[1]);
        if (ok > kk || (ok == kk && oi < i0)) {
            kk = ok;
            i0 = oi;
        }
        const int row = row0 + 32 * ct + c;
        if (h == 0 && row < L)
            out[row] = (kk & 1u) ? i0 : half + i0;
        bk[ct] = 0u;
        bj[ct] = 0;
    }
}

// A operand of tile jt of a staged block: lane (column 32 jt + c, half h)
// gets d = 16 ks + 8 h + 0..7, read transposed from the row-major block.
template <int D, int P>
__device__ __forceinline__ void read_rot(const uint16_t *Rs, int jt, int grp, int m, bf16x8_t (&aop)[D / 16])
{
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const int dr = 16 * ks + 8 * (grp / 2) + m / 4;
        const int col = 32 * jt + 16 * (grp % 2) + 4 * (m % 4);
        const uint2 x = lds_read_tr16(&Rs[dr * P + col]);
        const uint2 y = lds_read_tr16(&Rs[(dr + 4) * P + col]);
        aop[ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{x.x, x.y, y.x, y.y});
    }
}

template <int D>
__global__ __launch_bounds__(kHashThreads) void hash_mfma_kernel(int L, int nh, int half, const bf16 *__restrict__ q,
                                                                 const bf16 *__restrict__ rot,
                                                                 int32_t *__restrict__ buckets)
{
    constexpr int P = kHashCols + 8;   // LDS pitch (elements) of the row-major [d][64] block
    __shared__ __align__(16) uint16_t Rs[D * P];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int h = lane / 32, c = lane % 32, grp = lane / 16, m = lane % 16;
    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * kHashRows + wave * 64;

    bf16x8_t qop[2][D / 16];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int row = min(row0 + 32 * ct + c, L - 1);
        const bf16 *qrow = q + ((size_t)bh * L + row) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            // -q: the products then give y' = -y exactly (a sign flip is exact
            // in bf16 and round-to-nearest is symmetric)
            const u32x4_t u = ld16(qrow + 16 * ks + 8 * h) ^ 0x80008000u;
            qop[ct][ks] = as_bf16x8(u);
        }
    }
    const uint16_t *Rbits = reinterpret_cast<const uint16_t *>(rot);
    // staging: item i = (row d = i / 8, columns 8 (i % 8) .. +7 of the block)
    constexpr int kItems = D * (kHashCols / 8) / kHashThreads;   // 4 (D=128), 2 (D=64), 1 (D=32)
    const int nblk = (half + kHashCols - 1) / kHashCols;
    const bool vec = (half % 8) == 0;
    u32x4_t pre[kItems];
    auto fetch = [&](int blk) __attribute__((always_inline)) {
        const int r = blk / nblk, j0 = (blk % nblk) * kHashCols;
        const uint16_t *R = Rbits + (size_t)r * D * half;
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kHashThreads;
            const int d = i / 8, j = j0 + 8 * (i % 8);
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (vec && j + 8 <= half) {
                u = ld16(R + (size_t)d * half + j);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (j + e < half)
                        w[e / 2] |= (uint32_t)R[(size_t)d * half + j + e] << (16 * (e % 2));
                u = u32x4_t{w[0], w[1], w[2], w[3]};
            }
            pre[it] = u;
        }
    };

    uint32_t bk[2] = {0u, 0u};
    int bj[2] = {0, 0};
    f32x16_t sv[2] = {f32x16_t{}, f32x16_t{}};
    fetch(0);
    for (int blk = 0; blk < nh * nblk; ++blk) {
        const int r = blk / nblk, jb = (blk % nblk) * kHashCols;
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kHashThreads;
            st16(&Rs[(i / 8) * P + 8 * (i % 8)], pre[it]);
        }
        __syncthreads();
        if (blk + 1 < nh * nblk)
            fetch(blk + 1);
#pragma unroll
        for (int jt = 0; jt < kHashCols / 32; ++jt) {
            const int j0 = jb + 32 * jt;
            if (j0 >= half)
                break;
            bf16x8_t aop[D / 16];
            read_rot<D, P>(Rs, jt, grp, m, aop);
            f32x16_t acc[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                acc[ct] = f32x16_t{};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    acc[ct] = mfma32(aop[ks], qop[ct][ks], acc[ct]);
            }
            if (j0 + 32 > half) {
                // columns at or past half: a score of 0 wins only where every
                // real score of the row is 0 too, and then the search takes
                // the lowest column, a real one
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (j0 + 8 * (e / 4) + 4 * h + (e % 4) >= half)
                            acc[ct][e] = 0.f;
            }
            tile_track(acc, j0, bk, bj, sv);
        }
        if (jb + kHashCols >= half)   // last block of round r
            round_store_tracked(bk, bj, sv, h, c, row0, L, half, buckets + ((size_t)bh * nh + r) * L);
    }

}

// The same computation when every staged block holds 64 full columns
// (half % 64 == 0), software-pipelined within the wave: the matrix-core
// products of a tile and the argmax of the tile before it (its accumulators
// are a second register set) are independent code in one scheduling region,
// which the compiler interleaves so that vector work can issue while the
// matrix core is busy (explicit interleaving hints measured slower).  The argmax
// of a block's last tile runs under the next block's first tile; a round is
// stored once its last tile's argmax is done.  The staged blocks alternate
// between two LDS buffers, so one barrier per block suffices: block b + 1
// is written while block b is read.
template <int D>
__global__ __launch_bounds__(kHashThreads) void hash_mfma_pipe_kernel(int L, int nh, int half,
                                                                      const bf16 *__restrict__ q,
                                                                      const bf16 *__restrict__ rot,
                                                                      int32_t *__restrict__ buckets)
{
    // pitch 96 elements (48 banks): the four rows of a transposed read start
    // at banks 0, 48, 32, 16, so lane groups 0 and 1 (16 columns apart) read
    // disjoint banks in the same cycle
    constexpr int COLS = kHashCols, P = 96;
    constexpr int NT = COLS / 32;   // tiles per block (even: they alternate between two accumulator sets)
    __shared__ __align__(16) uint16_t Rs[2][D * P];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int h = lane / 32, c = lane % 32, grp = lane / 16, m = lane % 16;
    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * kHashRows + wave * 64;

    bf16x8_t qop[2][D / 16];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int row = min(row0 + 32 * ct + c, L - 1);
        const bf16 *qrow = q + ((size_t)bh * L + row) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qop[ct][ks] = as_bf16x8(ld16(qrow + 16 * ks + 8 * h) ^ 0x80008000u);   // -q, as above
    }
    const uint16_t *Rbits = reinterpret_cast<const uint16_t *>(rot);
    constexpr int CPR = COLS / 8;                          // 16-byte chunks per staged row
    constexpr int kItems = D * CPR / kHashThreads;
    const int nblk = half / COLS, total = nh * nblk;
    u32x4_t pre[kItems];
    auto fetch = [&](int blk) __attribute__((always_inline)) {
        const uint16_t *R = Rbits + (size_t)(blk / nblk) * D * half + (blk % nblk) * COLS;
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kHashThreads;
            pre[it] = ld16(R + (size_t)(i / CPR) * half + 8 * (i % CPR));
        }
    };
    auto stage = [&](uint16_t *buf) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kHashThreads;
            st16(&buf[(i / CPR) * P + 8 * (i % CPR)], pre[it]);
        }
    };
    auto products = [&](const uint16_t *buf, int jt, f32x16_t (&acc)[2]) __attribute__((always_inline)) {
        bf16x8_t aop[D / 16];
        read_rot<D, P>(buf, jt, grp, m, aop);
        acc[0] = acc[1] = f32x16_t{};
        // the two accumulator chains alternate
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                acc[ct] = mfma32(aop[ks], qop[ct][ks], acc[ct]);
    };

    uint32_t bk[2] = {0u, 0u};
    int bj[2] = {0, 0};
    f32x16_t sv[2] = {f32x16_t{}, f32x16_t{}};
    // accumulators of the previous block's last tile (none before the first
    // block: their tracking is skipped there)
    f32x16_t acc0[2], acc1[2] = {f32x16_t{}, f32x16_t{}};
    int prev_j = 0, prev_r = 0;   // first column and round of that tile
    bool prev_last = false;       // it ended its round
    fetch(0);
    stage(Rs[0]);
    if (total > 1)
        fetch(1);
    for (int blk = 0; blk < total; ++blk) {
        const int r = blk / nblk, jb = (blk % nblk) * COLS;
        const uint16_t *buf = Rs[blk % 2];
        // block blk is staged, and every wave is done with the other buffer
        __syncthreads();
        if (blk + 1 < total) {
            stage(Rs[(blk + 1) % 2]);
            if (blk + 2 < total)
                fetch(blk + 2);
        }
#pragma unroll
        for (int jt = 0; jt < NT; jt += 2) {
            products(buf, jt, acc0);
            if (jt > 0 || blk > 0)
                tile_track(acc1, jt == 0 ? prev_j : jb + 32 * (jt - 1), bk, bj, sv);
            if (jt == 0 && prev_last)
                round_store_tracked(bk, bj, sv, h, c, row0, L, half, buckets + ((size_t)bh * nh + prev_r) * L);
            products(buf, jt + 1, acc1);
            tile_track(acc0, jb + 32 * jt, bk, bj, sv);
        }
        prev_j = jb + COLS - 32;
        prev_r = r;
        prev_last = jb + COLS == half;
    }
    tile_track(acc1, prev_j, bk, bj, sv);
    round_store_tracked(bk, bj, sv, h, c, row0, L, half, buckets + ((size_t)bh * nh + prev_r) * L);
}

template <int D>
hipError_t go_mfma(const Dims &P, const void *q, const void *rot, int32_t *buckets, hipStream_t st)
{
    dim3 grid((P.L + kHashRows - 1) / kHashRows, P.BH());
    ProfScope prof(LSH_KERNEL_HASH, st);
    if ((P.nb / 2) % kHashCols == 0)
        hipLaunchKernelGGL((hash_mfma_pipe_kernel<D>), grid, dim3(kHashThreads), 0, st, P.L, P.nh, P.nb / 2,
                           (const bf16 *)q, (const bf16 *)rot, buckets);
    else
        hipLaunchKernelGGL((hash_mfma_kernel<D>), grid, dim3(kHashThreads), 0, st, P.L, P.nh, P.nb / 2,
                           (const bf16 *)q, (const bf16 *)rot, buckets);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t go(const Dims &P, const void *q, const void *rot, int32_t *buckets, hipStream_t st)
{
    dim3 grid((P.L + kHashThreads - 1) / kHashThreads, P.nh, P.BH());
    ProfScope prof(LSH_KERNEL_HASH, st);
    hipLaunchKernelGGL((hash_generic<T, D>), grid, dim3(kHashThreads), 0, st, P.L, P.nh, P.nb / 2,
                       (const T *)q, (const T *)rot, buckets);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hash(const Dims &P, int dtype, const void *q, const void *rot, int32_t *buckets,
                       hipStream_t st)
{
    if (dtype == LSH_BF16) {
        switch (P.d) {
        case 32: return go_mfma<32>(P, q, rot, buckets, st);
        case 64: return go_mfma<64>(P, q, rot, buckets, st);
        case 128: return go_mfma<128>(P, q, rot, buckets, st);
        }
    } else {
        switch (P.d) {
        case 32: return go<float, 32>(P, q, rot, buckets, st);
        case 64: return go<float, 64>(P, q, rot, buckets, st);
        case 128: return go<float, 128>(P, q, rot, buckets, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace lsh
