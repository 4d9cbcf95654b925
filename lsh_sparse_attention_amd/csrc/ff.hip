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
// The row-wise products (x W1, h W2, dy W2^T, dh W1^T) are one kernel,
// C = A B^T with both operands stored K-major ([M][K] and [N][K]; W1 and W2
// are transposed once per call where needed).  A workgroup of 4 waves
// computes a 128 x 128 tile of C, each wave a 64 x 64 quarter as 2 x 2 MFMA
// tiles, with the K loop staged through one LDS stage in steps of 64; the
// next step's operands are fetched into registers while the current one is
// multiplied.  The epilogue adds the bias and applies the ReLU, or masks
// by ReLU' (the backward's dH = dY W2^T where the hidden value is positive).
// The weight gradients (x^T dh, h^T dy) sum over the chunk's rows, which are
// the leading dimension of both operands: a second kernel stages k-rows of
// both in LDS and reads the MFMA operands transposed (ds_read_b64_tr_b16),
// split over K into independent fp32 partial sums that accumulate over the
// chunks and are added up, in a fixed order, once at the end.  The bias
// gradients are column sums, by row blocks, finished the same way.
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;   // LDS row pitch in elements (16-byte aligned rows, shifted banks)
constexpr int kGemmThreads = 256;

enum Epi { kEpiBiasRelu = 0, kEpiBias = 1, kEpiMask = 2, kEpiPlain = 3 };

// C[M][N] = epi(sum_k A[m][k] B[n][k]), bf16 out.  A, B bf16 with row pitches
// lda, ldb (multiples of 8); K a multiple of 8.  Epilogues: bias + ReLU, or
// bias (bias fp32 [N]); mask (zero where mask[m][n] is not positive); plain.
template <int EPI>
__global__ __launch_bounds__(kGemmThreads) void gemm_nt_kernel(int M, int N, int K, const bf16 *__restrict__ A,
                                                               int lda, const bf16 *__restrict__ B, int ldb,
                                                               const float *__restrict__ bias,
                                                               const bf16 *__restrict__ mask, int ldm,
                                                               bf16 *__restrict__ C, int ldc)
{
    // one LDS stage (36 KB) with two barriers per K step: measured a little
    // faster than two alternating stages (occupancy is the same, two waves
    // per SIMD, set by the registers: 160 plus 64 for the accumulators)
    __shared__ __align__(16) uint16_t As[kBM * kPitch];
    __shared__ __align__(16) uint16_t Bs[kBN * kPitch];
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
    auto stash = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kGemmThreads * i, row = q / 8, kc = q % 8;
            st16(&As[row * kPitch + 8 * kc], ra[i]);
            st16(&Bs[row * kPitch + 8 * kc], rb[i]);
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
    stash();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        // the next K step's operands are loaded into registers while this one
        // is multiplied out of LDS
        if (kt + 1 < nk)
            fetch((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            // lane (row c, half h) supplies k = 16 ks + 8 h .. +7 of its row
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = as_bf16x8(ld16(&As[(wm * 64 + 32 * i + c) * kPitch + 16 * ks + 8 * h]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = as_bf16x8(ld16(&Bs[(wn * 64 + 32 * j + c) * kPitch + 16 * ks + 8 * h]));
            // B as the instruction's first operand: the tile comes out transposed,
            // so a lane holds 4 consecutive columns of one row of C
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32(b[j], a[i], acc[i][j]);
        }
        if (kt + 1 < nk) {
            __syncthreads();   // every wave is done reading the stage
            stash();
        }
        __syncthreads();
    }

    // acc[i][j][4 g + t] is C[m0 + 64 wm + 32 i + c][n0 + 64 wn + 32 j + 8 g + 4 h + t]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = m0 + wm * 64 + 32 * i + c;
        if (row >= M)
            continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * 64 + 32 * j + 8 * g + 4 * h;   // N is a multiple of 8
                if (col >= N)
                    continue;
                float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                if constexpr (EPI == kEpiBiasRelu || EPI == kEpiBias) {
                    const float4 b4 = *reinterpret_cast<const float4 *>(bias + col);
                    v[0] += b4.x;
                    v[1] += b4.y;
                    v[2] += b4.z;
                    v[3] += b4.w;
                }
                if constexpr (EPI == kEpiBiasRelu) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        v[t] = fmaxf(v[t], 0.f);
                }
                if constexpr (EPI == kEpiMask) {
                    const uint2 mb = *reinterpret_cast<const uint2 *>(mask + (size_t)row * ldm + col);
                    const uint32_t m4[4] = {mb.x & 0xffffu, mb.x >> 16, mb.y & 0xffffu, mb.y >> 16};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if ((m4[t] & 0x8000u) || m4[t] == 0u)   // hidden value not positive: ReLU' = 0
                            v[t] = 0.f;
                }
                *reinterpret_cast<uint2 *>(C + (size_t)row * ldc + col) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
    }
}

// C (+)= A^T B over a K range: A [K][M] (lda), B [K][N] (ldb), bf16, M and N
// multiples of 8, fp32 C [M][N] (ldc) of split blockIdx.z at C + z * split_stride.
// Tiles of 128 x 128 outputs; k-rows [k0, k0 + 32) of both operands are
// staged in LDS as stored (rows of M, resp. N, contiguous), and each MFMA
// operand is read transposed: lane (column c, half h) gets the 8 k-values
// 16 j + 4 h + {0..3} and 16 j + 8 + 4 h + {0..3} of its column (the same k
// order for both operands, so their products pair up).
// LDS pitch 144 elements (288 bytes, 72 banks): the 4 rows a group of 16
// lanes reads transposed start 8 banks apart and do not collide
constexpr int kTK = 32, kTPitch = 128 + 16;
__global__ __launch_bounds__(kGemmThreads) void gemm_tn_kernel(int M, int N, int K, int ksplit,
                                                               const bf16 *__restrict__ A, int lda,
                                                               const bf16 *__restrict__ B, int ldb,
                                                               float *__restrict__ C, int ldc, size_t split_stride,
                                                               int accumulate)
{
    __shared__ __align__(16) uint16_t As[2][kTK * kTPitch];
    __shared__ __align__(16) uint16_t Bs[2][kTK * kTPitch];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
    const int kb = blockIdx.z * ksplit, ke = min(K, kb + ksplit);
    const int h = lane / 32, c = lane % 32;
    float *Cz = C + (size_t)blockIdx.z * split_stride;

    // each thread moves 2 chunks of 8 elements of each operand per K step:
    // chunk q is k-row q / 16, columns 8 (q % 16) .. +7
    u32x4_t ra[2], rb[2];
    auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + kGemmThreads * i, kr = k0 + q / 16, col = 8 * (q % 16);
            const u32x4_t z = {0u, 0u, 0u, 0u};
            ra[i] = (kr < ke && m0 + col < M) ? ld16(A + (size_t)kr * lda + m0 + col) : z;
            rb[i] = (kr < ke && n0 + col < N) ? ld16(B + (size_t)kr * ldb + n0 + col) : z;
        }
    };
    auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + kGemmThreads * i, r = q / 16, col = 8 * (q % 16);
            st16(&As[buf][r * kTPitch + col], ra[i]);
            st16(&Bs[buf][r * kTPitch + col], rb[i]);
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f32x16_t{};
    const int nk = ke > kb ? (ke - kb + kTK - 1) / kTK : 0;
    if (nk > 0) {
        fetch(kb);
        stash(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            fetch(kb + (kt + 1) * kTK);
#pragma unroll
        for (int js = 0; js < kTK / 16; ++js) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = tile_t<kTPitch>(As[buf], js, wm * 64 + 32 * i, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = tile_t<kTPitch>(Bs[buf], js, wn * 64 + 32 * j, lane);
            // B first, as in gemm_nt_kernel: a lane holds 4 consecutive columns
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32(b[j], a[i], acc[i][j]);
        }
        if (kt + 1 < nk)
            stash(buf ^ 1);
        __syncthreads();
    }
    // acc[i][j][4 g + t] is C[m0 + 64 wm + 32 i + c][n0 + 64 wn + 32 j + 8 g + 4 h + t]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = m0 + wm * 64 + 32 * i + c;
        if (row >= M)
            continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * 64 + 32 * j + 8 * g + 4 * h;   // N is a multiple of 8
                if (col >= N)
                    continue;
                float4 *p = reinterpret_cast<float4 *>(Cz + (size_t)row * ldc + col);
                float4 v = make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                       acc[i][j][4 * g + 3]);
                if (accumulate) {
                    const float4 o = *p;
                    v.x += o.x;
                    v.y += o.y;
                    v.z += o.z;
                    v.w += o.w;
                }
                *p = v;
            }
    }
}

// out[i] = sum over s < S of part[s][i], s in order (the K splits).
__global__ __launch_bounds__(256) void split_sum_kernel(size_t n, int S, const float *__restrict__ part,
                                                        float *__restrict__ out)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    float s = 0.f;
    for (int z = 0; z < S; ++z)
        s += part[(size_t)z * n + i];
    out[i] = s;
}

// Column sums of in [rows][cols] (bf16) by row blocks of kColRows:
// part[blockIdx.y][c] (+)= sum of the block's rows; 8 columns per thread.
constexpr int kColRows = 32;
__global__ __launch_bounds__(256) void colsum_kernel(int rows, int cols, const bf16 *__restrict__ in, int ldi,
                                                     float *__restrict__ part, int accumulate)
{
    const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (c0 >= cols)
        return;
    const int r0 = blockIdx.y * kColRows, r1 = min(rows, r0 + kColRows);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = r0; r < r1; ++r) {
        float x[8];
        load8(in + (size_t)r * ldi + c0, x);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s[k] += x[k];
    }
    float *p = part + (size_t)blockIdx.y * cols + c0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        p[k] = accumulate ? p[k] + s[k] : s[k];
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

template <int EPI>
hipError_t gemm(int M, int N, int K, const bf16 *A, int lda, const bf16 *B, int ldb, const float *bias,
                const bf16 *mask, int ldm, bf16 *C, int ldc, hipStream_t st)
{
    if (M <= 0 || N <= 0)
        return hipSuccess;
    const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
    hipLaunchKernelGGL((gemm_nt_kernel<EPI>), grid, dim3(kGemmThreads), 0, st, M, N, K, A, lda, B, ldb, bias, mask,
                       ldm, C, ldc);
    return hipGetLastError();
}

hipError_t transpose(int R, int Ccols, int Rp, const bf16 *in, int ldi, bf16 *out, hipStream_t st)
{
    const dim3 grid((Ccols + 63) / 64, (Rp + 63) / 64);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, R, Ccols, Rp, in, ldi, out);
    return hipGetLastError();
}

hipError_t gemm_tn(int M, int N, int K, int S, const bf16 *A, int lda, const bf16 *B, int ldb, float *C, int ldc,
                   int accumulate, hipStream_t st)
{
    const int ksplit = (K + S - 1) / S;
    const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM, S);
    hipLaunchKernelGGL(gemm_tn_kernel, grid, dim3(kGemmThreads), 0, st, M, N, K, ksplit, A, lda, B, ldb, C, ldc,
                       (size_t)M * ldc, accumulate);
    return hipGetLastError();
}

hipError_t split_sum(size_t n, int S, const float *part, float *out, hipStream_t st)
{
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, S, part, out);
    return hipGetLastError();
}

hipError_t colsum(int rows, int cols, const bf16 *in, int ldi, float *part, int accumulate, hipStream_t st)
{
    const dim3 grid((cols / 8 + 255) / 256, (rows + kColRows - 1) / kColRows);
    hipLaunchKernelGGL(colsum_kernel, grid, dim3(256), 0, st, rows, cols, in, ldi, part, accumulate);
    return hipGetLastError();
}

// Chunk geometry: rows [i cr, min(n, (i + 1) cr)) with cr = ceil(n / c).
// The weight-gradient products split each chunk's rows S ways (S = 2 from
// 512 rows on); the column sums use rb row blocks per chunk.
struct FF {
    int n, dm, dff, c, cr, S, rb;
};

FF ff_of(const lsh_ff_t *f)
{
    FF g{f->rows, f->d_model, f->d_ff, f->chunks, 0, 1, 1};
    g.cr = (g.n + g.c - 1) / g.c;
    g.S = g.cr >= 512 ? 2 : 1;
    g.rb = (g.cr + kColRows - 1) / kColRows;
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
// H [cr][dff]; backward also dH [cr][dff], the fp32 partial weight gradients
// P1 [S][dm][dff], P2 [S][dff][dm] and the partial bias gradients
// Q1 [rb][dff], Q2 [rb][dm].
struct FfWs {
    bf16 *w1t, *w2t, *h, *dh;
    float *p1, *p2, *q1, *q2;
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
        w.p1 = (float *)take((size_t)2 * g.S * g.dm * g.dff);
        w.p2 = (float *)take((size_t)2 * g.S * g.dff * g.dm);
        w.q1 = (float *)take((size_t)2 * g.rb * g.dff);
        w.q2 = (float *)take((size_t)2 * g.rb * g.dm);
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
        e = gemm<kEpiBiasRelu>(rows, g.dff, g.dm, X + (size_t)r0 * g.dm, g.dm, w.w1t, g.dm, b1, nullptr, 0, w.h,
                               g.dff, s);
        if (e == hipSuccess)
            e = gemm<kEpiBias>(rows, g.dm, g.dff, w.h, g.dff, w.w2t, g.dff, b2, nullptr, 0, Y + (size_t)r0 * g.dm,
                               g.dm, s);
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
        const int acc = i > 0 ? 1 : 0;
        const bf16 *Xc = X + (size_t)r0 * g.dm, *DYc = DY + (size_t)r0 * g.dm;
        // recompute H = relu(X_c W1 + b1)
        e = gemm<kEpiBiasRelu>(rows, g.dff, g.dm, Xc, g.dm, w.w1t, g.dm, b1, nullptr, 0, w.h, g.dff, s);
        // dH = (dY_c W2^T) * relu'(H)   (W2 [dff][dm] is already K-major)
        if (e == hipSuccess)
            e = gemm<kEpiMask>(rows, g.dff, g.dm, DYc, g.dm, W2, g.dm, nullptr, w.h, g.dff, w.dh, g.dff, s);
        // dX_c = dH W1^T   (W1 [dm][dff] is K-major)
        if (e == hipSuccess)
            e = gemm<kEpiPlain>(rows, g.dm, g.dff, w.dh, g.dff, W1, g.dff, nullptr, nullptr, 0,
                                DX + (size_t)r0 * g.dm, g.dm, s);
        // weight gradients over the chunk's rows (the K of both products):
        // P2 += H^T dY_c, P1 += X_c^T dH, split S ways; bias gradients by row blocks
        if (e == hipSuccess)
            e = gemm_tn(g.dff, g.dm, rows, g.S, w.h, g.dff, DYc, g.dm, w.p2, g.dm, acc, s);
        if (e == hipSuccess)
            e = gemm_tn(g.dm, g.dff, rows, g.S, Xc, g.dm, w.dh, g.dff, w.p1, g.dff, acc, s);
        if (e == hipSuccess)
            e = colsum(rows, g.dm, DYc, g.dm, w.q2, acc, s);
        if (e == hipSuccess)
            e = colsum(rows, g.dff, w.dh, g.dff, w.q1, acc, s);
    }
    // the splits and row blocks added up in a fixed order
    if (e == hipSuccess)
        e = split_sum((size_t)g.dm * g.dff, g.S, w.p1, dw1, s);
    if (e == hipSuccess)
        e = split_sum((size_t)g.dff * g.dm, g.S, w.p2, dw2, s);
    if (e == hipSuccess)
        e = split_sum((size_t)g.dff, g.rb, w.q1, db1, s);
    if (e == hipSuccess)
        e = split_sum((size_t)g.dm, g.rb, w.q2, db2, s);
    return status_of(e);
}

}  // extern "C"
