// ff.hip -- the chunked feed-forward layer of the Reformer block, forward and
// backward, on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Method: "Reformer: The Efficient Transformer" §3 (Reversible Transformer):
// the feed-forward layer acts on each position independently, so its
// computation is split into c chunks of positions, and so are the
// recomputation and the backward pass; only one chunk's hidden activations
// (rows x d_ff) exist at a time.  The layer is the standard Transformer one,
// y = relu(x W1 + b1) W2 + b2.
//
// Every product is one kernel, C = A B^T with both operands stored K-major
// ([M][K] and [N][K]); operands that are not (W1 and W2 in the forward, the
// activations of a chunk for the weight gradients) are transposed into the
// workspace first.  A workgroup of 4 waves computes a 128 x 128 tile of C,
// each wave a 64 x 64 quarter as 2 x 2 MFMA tiles, with the K loop staged
// through double-buffered LDS in steps of 64; the next step's operands are
// fetched into registers while the current one is multiplied.  The epilogue
// adds the bias and applies the ReLU, or masks by ReLU' (the backward's
// dH = dY W2^T where the hidden value is positive), or accumulates fp32
// weight gradients over the chunks.
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;   // LDS row pitch in elements (16-byte aligned rows, shifted banks)
constexpr int kGemmThreads = 256;

enum Epi { kEpiBiasRelu = 0, kEpiBias = 1, kEpiMask = 2, kEpiPlain = 3, kEpiAccF32 = 4 };

// C[M][N] = epi(sum_k A[m][k] B[n][k]).  A, B bf16 with row pitches lda, ldb
// (multiples of 8); K a multiple of 8.  Epilogues: bias + ReLU or bias (bf16
// out, bias fp32 [N]); mask (bf16 out, zero where mask[m][n] is not positive);
// plain (bf16 out); fp32 accumulate (C += result, or C = result when
// accumulate is 0).
template <int EPI>
__global__ __launch_bounds__(kGemmThreads) void gemm_nt_kernel(int M, int N, int K, const bf16 *__restrict__ A,
                                                               int lda, const bf16 *__restrict__ B, int ldb,
                                                               const float *__restrict__ bias,
                                                               const bf16 *__restrict__ mask, int ldm,
                                                               void *__restrict__ C, int ldc, int accumulate)
{
    __shared__ __align__(16) uint16_t As[2][kBM * kPitch];
    __shared__ __align__(16) uint16_t Bs[2][kBN * kPitch];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
    const int h = lane / 32, c = lane % 32;

    // each thread moves 4 chunks of 8 elements of each operand per K step
    u32x4_t ra[4], rb[4];
    auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kGemmThreads * i, row = q / 8, k = k0 + 8 * (q % 8);
            const u32x4_t z = {0u, 0u, 0u, 0u};
            ra[i] = (m0 + row < M && k < K) ? ld16(A + (size_t)(m0 + row) * lda + k) : z;
            rb[i] = (n0 + row < N && k < K) ? ld16(B + (size_t)(n0 + row) * ldb + k) : z;
        }
    };
    auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kGemmThreads * i, row = q / 8, kc = q % 8;
            st16(&As[buf][row * kPitch + 8 * kc], ra[i]);
            st16(&Bs[buf][row * kPitch + 8 * kc], rb[i]);
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f32x16_t{};
    const int nk = (K + kBK - 1) / kBK;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            fetch((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            // lane (row c, half h) supplies k = 16 ks + 8 h .. +7 of its row
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = as_bf16x8(ld16(&As[buf][(wm * 64 + 32 * i + c) * kPitch + 16 * ks + 8 * h]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = as_bf16x8(ld16(&Bs[buf][(wn * 64 + 32 * j + c) * kPitch + 16 * ks + 8 * h]));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk)
            stash(buf ^ 1);
        __syncthreads();
    }

    // acc[i][j][4 g + t] is C[m0 + 64 wm + 32 i + 8 g + 4 h + t][n0 + 64 wn + 32 j + c]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + 32 * j + c;
        if (col >= N)
            continue;
        const float bj = (EPI == kEpiBiasRelu || EPI == kEpiBias) ? bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 64 + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
                if (row >= M)
                    continue;
                float v = acc[i][j][e] + bj;
                if constexpr (EPI == kEpiAccF32) {
                    float *p = reinterpret_cast<float *>(C) + (size_t)row * ldc + col;
                    *p = accumulate ? *p + v : v;
                } else {
                    if constexpr (EPI == kEpiBiasRelu)
                        v = fmaxf(v, 0.f);
                    if constexpr (EPI == kEpiMask) {
                        const uint16_t mb = mask[(size_t)row * ldm + col].bits;
                        if ((mb & 0x8000u) || mb == 0u)   // hidden value not positive: ReLU' = 0
                            v = 0.f;
                    }
                    reinterpret_cast<bf16 *>(C)[(size_t)row * ldc + col] = from_f<bf16>(v);
                }
            }
    }
}

// out[c][r] = in[r][c] for r < R (row pitch ldi), 0 for R <= r < Rp; out
// row pitch Rp.  64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(int R, int Ccols, int Rp, const bf16 *__restrict__ in, int ldi,
                                                        bf16 *__restrict__ out)
{
    __shared__ uint16_t t[64][66];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    for (int y = ty; y < 64; y += 4) {
        const int r = r0 + y, cc = c0 + tx;
        t[y][tx] = (r < R && cc < Ccols) ? in[(size_t)r * ldi + cc].bits : (uint16_t)0;
    }
    __syncthreads();
    for (int y = ty; y < 64; y += 4) {
        const int cc = c0 + y, r = r0 + tx;
        if (cc < Ccols && r < Rp)
            out[(size_t)cc * Rp + r].bits = t[tx][y];
    }
}

// out[row] (+)= sum of in[row][0 .. n): one wave per row (the sums of bias
// gradients, over a chunk's rows held transposed).
__global__ __launch_bounds__(256) void rowsum_kernel(int rows, int n, const bf16 *__restrict__ in, int ldi,
                                                     float *__restrict__ out, int accumulate)
{
    const int row = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (row >= rows)
        return;
    float s = 0.f;
    for (int k = lane; k < n; k += kWave)
        s += to_f(in[(size_t)row * ldi + k]);
    s = wave_sum(s);
    if (lane == 0)
        out[row] = accumulate ? out[row] + s : s;
}

template <int EPI>
hipError_t gemm(int M, int N, int K, const bf16 *A, int lda, const bf16 *B, int ldb, const float *bias,
                const bf16 *mask, int ldm, void *C, int ldc, int accumulate, hipStream_t st)
{
    if (M <= 0 || N <= 0)
        return hipSuccess;
    const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
    hipLaunchKernelGGL((gemm_nt_kernel<EPI>), grid, dim3(kGemmThreads), 0, st, M, N, K, A, lda, B, ldb, bias, mask,
                       ldm, C, ldc, accumulate);
    return hipGetLastError();
}

hipError_t transpose(int R, int Ccols, int Rp, const bf16 *in, int ldi, bf16 *out, hipStream_t st)
{
    const dim3 grid((Ccols + 63) / 64, (Rp + 63) / 64);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, R, Ccols, Rp, in, ldi, out);
    return hipGetLastError();
}

hipError_t rowsum(int rows, int n, const bf16 *in, int ldi, float *out, int accumulate, hipStream_t st)
{
    hipLaunchKernelGGL(rowsum_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, rows, n, in, ldi, out, accumulate);
    return hipGetLastError();
}

// Chunk geometry: rows [i cr, min(n, (i + 1) cr)) with cr = ceil(n / c);
// transposed copies of a chunk are padded to a multiple of 8 rows (zeros).
struct FF {
    int n, dm, dff, c, cr, crp;
};

FF ff_of(const lsh_ff_t *f)
{
    FF g{f->rows, f->d_model, f->d_ff, f->chunks, 0, 0};
    g.cr = (g.n + g.c - 1) / g.c;
    g.crp = (g.cr + 7) / 8 * 8;
    return g;
}

int ff_validate(const lsh_ff_t *f)
{
    if (!f || f->rows < 0 || f->d_model < 8 || f->d_ff < 8 || f->chunks < 1 || f->d_model % 8 || f->d_ff % 8)
        return LSH_ERR_INVALID;
    if (f->dtype != LSH_BF16)
        return LSH_ERR_UNSUPPORTED;
    if ((double)f->rows * f->d_model > 2147483647.0 || (double)f->d_model * f->d_ff > 2147483647.0 ||
        (double)((f->rows + f->chunks - 1) / f->chunks + 8) * f->d_ff > 2147483647.0)
        return LSH_ERR_UNSUPPORTED;
    return LSH_OK;
}

// Workspace: W1^T [dff][dm] and, forward, W2^T [dm][dff]; one chunk's hidden
// H [cr][dff]; backward also dH [cr][dff] and the transposed chunk copies
// H^T, dH^T [dff][crp], X^T, dY^T [dm][crp].
struct FfWs {
    bf16 *w1t, *w2t, *h, *dh, *ht, *dht, *xt, *dyt;
    size_t bytes;
};

FfWs ff_layout(const FF &g, bool backward, void *base)
{
    const uintptr_t b = (uintptr_t)base;
    FfWs w{};
    size_t o = 0;
    auto take = [&](size_t elems) {
        bf16 *p = (bf16 *)(b + o);
        o += align_up(elems * sizeof(bf16), 256);
        return p;
    };
    w.w1t = take((size_t)g.dff * g.dm);
    if (!backward)
        w.w2t = take((size_t)g.dm * g.dff);
    w.h = take((size_t)g.cr * g.dff);
    if (backward) {
        w.dh = take((size_t)g.cr * g.dff);
        w.ht = take((size_t)g.dff * g.crp);
        w.dht = take((size_t)g.dff * g.crp);
        w.xt = take((size_t)g.dm * g.crp);
        w.dyt = take((size_t)g.dm * g.crp);
    }
    w.bytes = o;
    return w;
}

bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? LSH_OK : LSH_ERR_HIP; }

}  // namespace
}  // namespace lsh

using namespace lsh;

extern "C" {

size_t lsh_ff_workspace_bytes(const lsh_ff_t *ff, int backward)
{
    if (ff_validate(ff) != LSH_OK || ff->rows == 0)
        return 0;
    return ff_layout(ff_of(ff), backward != 0, nullptr).bytes;
}

int lsh_ff_fwd(const lsh_ff_t *ff, const void *x, const void *w1, const float *b1, const void *w2, const float *b2,
               void *y, void *ws, size_t ws_bytes, void *stream)
{
    int st = ff_validate(ff);
    if (st != LSH_OK || ff->rows == 0)
        return st;
    if (!x || !w1 || !b1 || !w2 || !b2 || !y || !ws || !al16(x) || !al16(w1) || !al16(w2) || !al16(y) ||
        ((uintptr_t)ws & 255u))
        return LSH_ERR_INVALID;
    const FF g = ff_of(ff);
    const FfWs w = ff_layout(g, false, ws);
    if (ws_bytes < w.bytes)
        return LSH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    const bf16 *X = (const bf16 *)x;
    bf16 *Y = (bf16 *)y;
    hipError_t e = transpose(g.dm, g.dff, g.dm, (const bf16 *)w1, g.dff, w.w1t, s);
    if (e == hipSuccess)
        e = transpose(g.dff, g.dm, g.dff, (const bf16 *)w2, g.dm, w.w2t, s);
    for (int i = 0; i < g.c && e == hipSuccess; ++i) {
        const int r0 = i * g.cr, rows = g.n - r0 < g.cr ? g.n - r0 : g.cr;
        if (rows <= 0)
            break;
        // H = relu(X_c W1 + b1); Y_c = H W2 + b2
        e = gemm<kEpiBiasRelu>(rows, g.dff, g.dm, X + (size_t)r0 * g.dm, g.dm, w.w1t, g.dm, b1, nullptr, 0, w.h, g.dff,
                               0, s);
        if (e == hipSuccess)
            e = gemm<kEpiBias>(rows, g.dm, g.dff, w.h, g.dff, w.w2t, g.dff, b2, nullptr, 0, Y + (size_t)r0 * g.dm,
                               g.dm, 0, s);
    }
    return status_of(e);
}

int lsh_ff_bwd(const lsh_ff_t *ff, const void *x, const void *w1, const float *b1, const void *w2, const void *dy,
               void *dx, float *dw1, float *db1, float *dw2, float *db2, void *ws, size_t ws_bytes, void *stream)
{
    int st = ff_validate(ff);
    if (st != LSH_OK || ff->rows == 0)
        return st;
    if (!x || !w1 || !b1 || !w2 || !dy || !dx || !dw1 || !db1 || !dw2 || !db2 || !ws || !al16(x) || !al16(w1) ||
        !al16(w2) || !al16(dy) || !al16(dx) || ((uintptr_t)ws & 255u))
        return LSH_ERR_INVALID;
    const FF g = ff_of(ff);
    const FfWs w = ff_layout(g, true, ws);
    if (ws_bytes < w.bytes)
        return LSH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    const bf16 *X = (const bf16 *)x, *DY = (const bf16 *)dy, *W1 = (const bf16 *)w1, *W2 = (const bf16 *)w2;
    bf16 *DX = (bf16 *)dx;
    hipError_t e = transpose(g.dm, g.dff, g.dm, W1, g.dff, w.w1t, s);
    for (int i = 0; i < g.c && e == hipSuccess; ++i) {
        const int r0 = i * g.cr, rows = g.n - r0 < g.cr ? g.n - r0 : g.cr;
        if (rows <= 0)
            break;
        const int acc = i > 0 ? 1 : 0, kp = (rows + 7) / 8 * 8;
        const bf16 *Xc = X + (size_t)r0 * g.dm, *DYc = DY + (size_t)r0 * g.dm;
        // recompute H = relu(X_c W1 + b1)
        e = gemm<kEpiBiasRelu>(rows, g.dff, g.dm, Xc, g.dm, w.w1t, g.dm, b1, nullptr, 0, w.h, g.dff, 0, s);
        // dH = (dY_c W2^T) * relu'(H)   (W2 [dff][dm] is already K-major)
        if (e == hipSuccess)
            e = gemm<kEpiMask>(rows, g.dff, g.dm, DYc, g.dm, W2, g.dm, nullptr, w.h, g.dff, w.dh, g.dff, 0, s);
        // dX_c = dH W1^T   (W1 [dm][dff] is K-major)
        if (e == hipSuccess)
            e = gemm<kEpiPlain>(rows, g.dm, g.dff, w.dh, g.dff, W1, g.dff, nullptr, nullptr, 0,
                                DX + (size_t)r0 * g.dm, g.dm, 0, s);
        // weight gradients over the chunk's rows: dW2 += H^T dY_c, dW1 += X_c^T dH
        if (e == hipSuccess)
            e = transpose(rows, g.dff, kp, w.h, g.dff, w.ht, s);
        if (e == hipSuccess)
            e = transpose(rows, g.dm, kp, DYc, g.dm, w.dyt, s);
        if (e == hipSuccess)
            e = transpose(rows, g.dm, kp, Xc, g.dm, w.xt, s);
        if (e == hipSuccess)
            e = transpose(rows, g.dff, kp, w.dh, g.dff, w.dht, s);
        if (e == hipSuccess)
            e = gemm<kEpiAccF32>(g.dff, g.dm, kp, w.ht, kp, w.dyt, kp, nullptr, nullptr, 0, dw2, g.dm, acc, s);
        if (e == hipSuccess)
            e = gemm<kEpiAccF32>(g.dm, g.dff, kp, w.xt, kp, w.dht, kp, nullptr, nullptr, 0, dw1, g.dff, acc, s);
        if (e == hipSuccess)
            e = rowsum(g.dm, kp, w.dyt, kp, db2, acc, s);
        if (e == hipSuccess)
            e = rowsum(g.dff, kp, w.dht, kp, db1, acc, s);
    }
    return status_of(e);
}

}  // extern "C"
