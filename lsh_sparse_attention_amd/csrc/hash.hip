// hash.hip -- angular LSH by random rotation: bucket = argmax([qR_r ; -qR_r]).
// "Reformer: The Efficient Transformer", §2 (random projections).
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
        case 32: return go<bf16, 32>(P, q, rot, buckets, st);
        case 64: return go<bf16, 64>(P, q, rot, buckets, st);
        case 128: return go<bf16, 128>(P, q, rot, buckets, st);
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
