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
// every round, the rotation is walked in tiles of 32 columns, staged
// transposed in LDS; Y^T = R^T Q^T comes out with lane = row and 16 columns
// per lane, so the running argmax of +y and of -y stays in registers, in
// increasing column order (strict comparisons keep the first index).  The two
// lane halves that share a row are merged at the end.  bf16 products are exact
// in the fp32 accumulator.
constexpr int kHashRows = 256;

template <int D>
__global__ __launch_bounds__(kHashThreads) void hash_mfma_kernel(int L, int nh, int half, const bf16 *__restrict__ q,
                                                                 const bf16 *__restrict__ rot,
                                                                 int32_t *__restrict__ buckets)
{
    constexpr int P = D + 8;
    __shared__ __align__(16) uint16_t RT[32 * P];   // [column j][d]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int h = lane / 32, c = lane % 32;
    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * kHashRows + wave * 64;

    bf16x8_t qop[2][D / 16];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int row = min(row0 + 32 * ct + c, L - 1);
        const bf16 *qrow = q + ((size_t)bh * L + row) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qop[ct][ks] = as_bf16x8(ld16(qrow + 16 * ks + 8 * h));
    }
    const uint16_t *Rbits = reinterpret_cast<const uint16_t *>(rot);
    // Staging of one 32-column tile: item i = (row d = i / 4, columns
    // 8 (i % 4) .. +7), kItems per thread, fetched one tile ahead.
    constexpr int kItems = (D * 4 + kHashThreads - 1) / kHashThreads;
    const int ntile = (half + 31) / 32;
    const bool vec = (half % 8) == 0;
    u32x4_t pre[kItems];
    auto fetch = [&](int tile) __attribute__((always_inline)) {
        const int r = tile / ntile, j0 = (tile % ntile) * 32;
        const uint16_t *R = Rbits + (size_t)r * D * half;
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kHashThreads;
            const int d = i / 4, j = j0 + 8 * (i % 4);
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (i < D * 4) {
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
            }
            pre[it] = u;
        }
    };

    float bp[2] = {-INFINITY, -INFINITY}, bn[2] = {-INFINITY, -INFINITY};
    int ip[2] = {0, 0}, in[2] = {0, 0};
    fetch(0);
    for (int tile = 0; tile < nh * ntile; ++tile) {
        const int r = tile / ntile, j0 = (tile % ntile) * 32;
        __syncthreads();
        // RT[jj][d] = R[d][j0 + jj] (zero past the last column)
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kHashThreads;
            if (i < D * 4) {
                const int d = i / 4, jj = 8 * (i % 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    RT[(jj + e) * P + d] = (uint16_t)(pre[it][e / 2] >> (16 * (e % 2)));
            }
        }
        __syncthreads();
        if (tile + 1 < nh * ntile)
            fetch(tile + 1);
        const bool full = j0 + 32 <= half;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                acc = mfma32(as_bf16x8(ld16(&RT[c * P + 16 * ks + 8 * h])), qop[ct][ks], acc);
            // acc[4 g + t] = y[column j0 + 8 g + 4 h + t] of row c
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = j0 + 8 * (e / 4) + 4 * h + (e % 4);
                const float y = acc[e];
                if (full || j < half) {
                    if (y > bp[ct]) {
                        bp[ct] = y;
                        ip[ct] = j;
                    }
                    if (-y > bn[ct]) {
                        bn[ct] = -y;
                        in[ct] = j;
                    }
                }
            }
        }
        if (j0 + 32 >= half) {
            // last tile of round r
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                // merge with the other half of the row (first index on ties)
                const float obp = __shfl_xor(bp[ct], 32, kWave), obn = __shfl_xor(bn[ct], 32, kWave);
                const int oip = __shfl_xor(ip[ct], 32, kWave), oin = __shfl_xor(in[ct], 32, kWave);
                if (obp > bp[ct] || (obp == bp[ct] && oip < ip[ct])) {
                    bp[ct] = obp;
                    ip[ct] = oip;
                }
                if (obn > bn[ct] || (obn == bn[ct] && oin < in[ct])) {
                    bn[ct] = obn;
                    in[ct] = oin;
                }
                const int row = row0 + 32 * ct + c;
                if (h == 0 && row < L)
                    buckets[((size_t)bh * nh + r) * L + row] = (bp[ct] >= bn[ct]) ? ip[ct] : half + in[ct];
                bp[ct] = bn[ct] = -INFINITY;
                ip[ct] = in[ct] = 0;
            }
        }
    }
}

template <int D>
hipError_t go_mfma(const Dims &P, const void *q, const void *rot, int32_t *buckets, hipStream_t st)
{
    dim3 grid((P.L + kHashRows - 1) / kHashRows, P.BH());
    ProfScope prof(LSH_KERNEL_HASH, st);
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
