// attn_generic.hip -- per-query (wave per sorted row) kernels of the chunked
// LSH attention, forward and backward, with fp32 arithmetic for both fp32 and
// bf16 storage.  These are the fp32 path, and the bf16 path for shapes the
// MFMA kernels do not take.
//
// Method: "Reformer: The Efficient Transformer" §2 (shared-QK attention over
// sorted chunks, causal mask through the permutation, self only as a
// fallback) and App. A (each query attends to the union of its round sets;
// duplicates are masked; per-round outputs combined by logsumexp weights).
//
// Round r of query i (sorted index s) attends to the sorted range
// [s - w, s - 1], w = s - win_lo; without causality (encoder attention) to
// [s - w, hi] minus s itself, hi being the last row of its bucket in its
// chunk (see window_kernel).  A member j is skipped in round r when it
// is also in the attended set of i in an earlier round r' < r, so that every
// member of the union is counted in exactly one round (the first that holds
// it).  Lanes of a wave take keys for the scores and head-dim components for
// the weighted sums.
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowsPerWave = 4;

// Read-once / write-once rows: the same as load8 / store8 with nontemporal
// accesses (prep's q, O and dO rows, the combine's per-round rows and its
// output: 10-12 % less time in either kernel at the long-text shape than
// plain accesses).
__device__ __forceinline__ void load8_nt(const bf16 *p, float out[8])
{
    const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(w[k] << 16);
        out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8_nt(const float *p, float out[8])
{
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p + 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[k] = a[k];
        out[4 + k] = b[k];
    }
}
__device__ __forceinline__ void store8_nt(bf16 *p, const float x[8])
{
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)from_f<bf16>(x[2 * k]).bits | ((uint32_t)from_f<bf16>(x[2 * k + 1]).bits << 16);
    __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4_t *>(p));
}
__device__ __forceinline__ void store8_nt(float *p, const float x[8])
{
    __builtin_nontemporal_store(f32x4_t{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4_t *>(p));
    __builtin_nontemporal_store(f32x4_t{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4_t *>(p + 4));
}

// ---------------------------------------------------------------------------
// prep: packed records, inverse norms, and (backward) D = dO . O.  The
// records' window start is win_lo, or with chunk_only (no bucket condition)
// the start of the chunk before the row's chunk.

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void prep_kernel(int L, int nh, int m, int chunk_only, const T *__restrict__ q,
                                                        const int32_t *__restrict__ inv,
                                                        const int32_t *__restrict__ win_lo,
                                                        uint32_t *__restrict__ meta, uint32_t *__restrict__ srec,
                                                        float *__restrict__ rnorm, const T *__restrict__ out,
                                                        const T *__restrict__ dout, float *__restrict__ Dvec)
{
    // D/8 lanes per token, each on 8 consecutive elements
    constexpr int CPT = D / 8, TPB = kThreads / CPT;
    const int grp = threadIdx.x / CPT, ch = threadIdx.x % CPT;
    // the blocks of one (b, h) on one XCD: the records written into its
    // rounds' sorted orders land at scattered places, and one L2 then
    // merges them into whole lines before they go to memory
    const int nbx = (L + TPB - 1) / TPB;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int t = (lb % nbx) * TPB + grp;
    const int bh = lb / nbx;
    const bool valid = t < L;
    const size_t tok = (size_t)bh * L + (valid ? t : 0);
    float x[8], y[8];
    if (meta) {
        float ss = 0.f;
        if (valid) {
            load8_nt(q + tok * D + ch * 8, x);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                ss = fmaf(x[k], x[k], ss);
        }
        ss = group_sum(ss, CPT);
        if (valid && ch == 0)
            rnorm[tok] = 1.0f / sqrtf(ss);
        if (valid) {
            for (int r = ch; r < nh; r += CPT) {
                const size_t idx = ((size_t)bh * nh + r) * L + t;
                const uint32_t s = (uint32_t)inv[idx];
                const int c = (int)s / m;
                const uint32_t w = s - (chunk_only ? (uint32_t)max(0, (c - 1) * m) : (uint32_t)win_lo[idx]);
                meta[tok * nh + r] = s | (w << 16);
                srec[((size_t)bh * nh + r) * L + s] = (uint32_t)t | (w << 16);
            }
        }
    }
    if (Dvec) {
        float acc = 0.f;
        if (valid) {
            load8_nt(out + tok * D + ch * 8, x);
            load8_nt(dout + tok * D + ch * 8, y);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                acc = fmaf(x[k], y[k], acc);
        }
        acc = group_sum(acc, CPT);
        if (valid && ch == 0)
            Dvec[tok] = acc;
    }
}

// Smallest position in each chunk of every (b, h, round): one wave per
// chunk, cmin[seg * (L / m) + c].
__global__ __launch_bounds__(kThreads) void chunk_min_kernel(int L, int m, size_t nchunks,
                                                             const uint32_t *__restrict__ srec,
                                                             uint32_t *__restrict__ cmin)
{
    const size_t ch = (size_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (ch >= nchunks)
        return;
    const size_t nc = L / m, seg = ch / nc;
    const uint32_t *sr = srec + seg * L + (ch % nc) * m;
    uint32_t mn = 0xffffffffu;
    for (int k = lane; k < m; k += kWave)
        mn = min(mn, rec_lo(sr[k]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
    if (lane == 0)
        cmin[ch] = mn;
}

// Window records of kRange / kRangePos problems: for every (b, h, round) and
// sorted row s, the candidates are the sorted range [s - w(s), hi(s)].  With
// the bucket condition (non-causal), hi(s) is the last row of s's bucket
// inside s's chunk: along the sorted order the window starts s' - w(s') do
// not decrease, and a later row s' of s's chunk starts its window at or
// before s exactly when it is in s's bucket (a later bucket starts after
// s), so hi(s) is found by bisection over [s, end of chunk).  Without it
// (chunk_only), hi(s) is the end of s's chunk.  Writes wmeta[tok nh + r] =
// hi | (hi - start) << 16.  With alone (causal, no bucket condition: the
// candidates not after the query are the members), alone[tok nh + r] = 1
// when no other position of the window comes before the row's: its
// position is the smallest of its chunk and below every position of the
// chunk before (cmin).
__global__ __launch_bounds__(kThreads) void window_kernel(int L, int nh, int m, int chunk_only, size_t total,
                                                          const uint32_t *__restrict__ srec,
                                                          uint32_t *__restrict__ wmeta,
                                                          const uint32_t *__restrict__ cmin,
                                                          uint8_t *__restrict__ alone)
{
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= total)
        return;
    const size_t seg = idx / L;   // bh * nh + r
    const int s = (int)(idx % L), r = (int)(seg % nh);
    const size_t bh = seg / nh;
    const uint32_t *sr = srec + seg * L;
    const uint32_t rec = sr[s];
    const int lo = s - (int)rec_hi(rec);
    const int c = s / m;
    int a = s, b = min((c + 1) * m, L) - 1;   // hi(s) in [a, b]
    if (chunk_only)
        a = b;
    while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if (mid - (int)rec_hi(sr[mid]) <= s)
            a = mid;
        else
            b = mid - 1;
    }
    const size_t tok = bh * L + rec_lo(rec);
    wmeta[tok * nh + r] = (uint32_t)a | ((uint32_t)(a - lo) << 16);
    if (alone) {
        const uint32_t pos = rec_lo(rec), *cm = cmin + seg * (size_t)(L / m);
        alone[tok * nh + r] = (uint8_t)(pos == cm[c] && (c == 0 || pos < cm[c - 1]));
    }
}

// Start of each row's bucket run, per (b, h, round): a row starts a run
// exactly when its window length w is 0 (its window start is then itself:
// the bucket begins there; a row inside a run has a window start before
// it), so the run start of sorted row s is the last s' <= s with w(s') = 0,
// a prefix maximum.  Two passes over tiles of 1024 sorted rows (one thread a
// row): the last run start of every tile (tmax), then each tile's prefix
// maximum seeded with the maximum of the tiles before it.  Writes
// bmeta[tok nh + r].
constexpr int kScanThreads = 1024;

__device__ __forceinline__ int block_max(int x, int *red)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x = max(x, __shfl_xor(x, o, kWave));
    if (lane == 0)
        red[wave] = x;
    __syncthreads();
    x = lane < kScanThreads / kWave ? red[lane] : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x = max(x, __shfl_xor(x, o, kWave));
    return x;
}

__global__ __launch_bounds__(kScanThreads) void run_tile_kernel(int L, const uint32_t *__restrict__ srec,
                                                                uint32_t *__restrict__ tmax)
{
    __shared__ int red[kScanThreads / kWave];
    const size_t seg = blockIdx.y;
    const int s = blockIdx.x * kScanThreads + threadIdx.x;
    const int v = (s < L && rec_hi(srec[seg * L + s]) == 0u) ? s : -1;
    const int m = block_max(v, red);
    if (threadIdx.x == 0)
        tmax[seg * gridDim.x + blockIdx.x] = (uint32_t)m;
}

__global__ __launch_bounds__(kScanThreads) void bucket_start_kernel(int L, int nh, const uint32_t *__restrict__ srec,
                                                                    const uint32_t *__restrict__ tmax,
                                                                    uint32_t *__restrict__ bmeta)
{
    __shared__ int red[kScanThreads / kWave];
    __shared__ int wave_max[kScanThreads / kWave];
    const size_t seg = blockIdx.y;
    const int r = (int)(seg % nh);
    const size_t bh = seg / nh;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    // the tiles before this one (at most 64 of them)
    int seed = -1;
    for (int t = threadIdx.x; t < (int)blockIdx.x; t += kScanThreads)
        seed = max(seed, (int)tmax[seg * gridDim.x + t]);
    seed = block_max(seed, red);
    const int s = blockIdx.x * kScanThreads + threadIdx.x;
    const uint32_t rec = s < L ? srec[seg * L + s] : 0u;
    int x = (s < L && rec_hi(rec) == 0u) ? s : -1;
    // inclusive prefix maximum over the block
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o)
            x = max(x, y);
    }
    if (lane == kWave - 1)
        wave_max[wave] = x;
    __syncthreads();
    for (int w = 0; w < wave; ++w)
        x = max(x, wave_max[w]);
    x = max(x, seed);
    if (s < L)
        bmeta[(bh * L + rec_lo(rec)) * nh + r] = (uint32_t)x;
}

// Dot of a per-lane row (global) with a wave-distributed vector whose
// component c sits in lane c % 64 of reg[c / 64].
template <typename T, int D>
__device__ __forceinline__ float dot_row_bcast(const T *row, const float (&reg)[(D + 63) / 64])
{
    float acc = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += 8) {
        float x[8];
        load8(row + c0, x);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            acc = fmaf(x[k], readlane(reg[(c0 + k) / 64], (c0 + k) % 64), acc);
    }
    return acc;
}

// Is key j masked in round r for query i because it belongs to i's
// attended set in an earlier round?  wm_i: i's non-causal window records, or
// null for causal problems.
__device__ __forceinline__ bool owned_earlier(const uint32_t *__restrict__ meta_i,
                                              const uint32_t *__restrict__ wm_i,
                                              const uint32_t *__restrict__ meta_j, int r)
{
    bool hit = false;
    if (wm_i) {
        for (int rr = 0; rr < r; ++rr)
            hit |= in_span(wm_i[rr], rec_lo(meta_j[rr]));
    } else {
        for (int rr = 0; rr < r; ++rr)
            hit |= in_window(meta_i[rr], rec_lo(meta_j[rr]));
    }
    return hit;
}

// Log of the duplicate divisor of a member under LSH_FLAG_DUP_BY_BUCKET: the
// number of rounds in which key j shares query i's bucket (from the
// bucket-run starts per round, bmeta); 0 without it (bmeta null).
__device__ __forceinline__ float dup_log(const uint32_t *__restrict__ bmeta, size_t tok_i, size_t tok_j, int nh)
{
    return bmeta ? logf((float)shared_buckets(bmeta + tok_i * nh, bmeta + tok_j * nh, nh)) : 0.f;
}

// Round-r key range of a sorted query row s: n candidates from sorted index
// lo on (causal: [s - w, s - 1]; non-causal: [s - w, hi], where s itself is
// skipped by the caller).
struct KeyRange {
    int lo, n;
};
__device__ __forceinline__ KeyRange key_range(int s, int w, const uint32_t *wm_i, int r)
{
    if (!wm_i)
        return KeyRange{s - w, w};
    const uint32_t x = wm_i[r];
    return KeyRange{(int)rec_lo(x) - (int)rec_hi(x), (int)rec_hi(x) + 1};
}

// ---------------------------------------------------------------------------
// forward: one wave per (round, sorted query row)

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(int L, int nh, float scale, const T *__restrict__ q,
                                                       const T *__restrict__ v, const uint32_t *__restrict__ meta,
                                                       const uint32_t *__restrict__ srec,
                                                       const uint32_t *__restrict__ wmeta, int pos_test,
                                                       const uint32_t *__restrict__ bmeta,
                                                       const float *__restrict__ rnorm, T *__restrict__ o_rounds,
                                                       float *__restrict__ lse_rounds)
{
    constexpr int NC = (D + 63) / 64;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r = blockIdx.y, bh = blockIdx.z;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int s = (blockIdx.x * kWaves + wave) * kRowsPerWave + k;
        if (s >= L)
            break;
        const uint32_t rec = sr[s];
        const int i = (int)rec_lo(rec), w = (int)rec_hi(rec);
        const uint32_t *mi = meta + (tok0 + i) * nh;
        const uint32_t *wi = wmeta ? wmeta + (tok0 + i) * nh : nullptr;
        const KeyRange kr0 = key_range(s, w, wi, r);
        float qreg[NC], acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            qreg[c] = e < D ? ld(q, (tok0 + i) * D + e) : 0.f;
            acc[c] = 0.f;
        }
        float M = -INFINITY, l = 0.f;
        for (int kb = 0; kb < kr0.n; kb += kWave) {
            const int idx = kb + lane;
            bool valid = idx < kr0.n && kr0.lo + idx != s;
            const uint32_t kr = valid ? sr[kr0.lo + idx] : rec;
            const int j = (int)rec_lo(kr);
            if (pos_test)
                valid = valid && j < i;   // not after the query (chunk window without buckets)
            // duplicates: the first-owner mask, or (bmeta) the log of the divisor
            if (valid && !bmeta)
                valid = !owned_earlier(mi, wi, meta + (tok0 + j) * nh, r);
            const float dlog = valid ? dup_log(bmeta, tok0 + i, tok0 + j, nh) : 0.f;
            const float dp = dot_row_bcast<T, D>(q + (tok0 + j) * D, qreg);
            const float logit = valid ? dp * scale * rnorm[tok0 + j] - dlog : -INFINITY;
            const float bm = wave_max(logit);
            if (bm == -INFINITY)
                continue;
            const float Mn = fmaxf(M, bm);
            const float corr = expf(M - Mn);
            const float p = valid ? expf(logit - Mn) : 0.f;
            l = l * corr + wave_sum(p);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[c] *= corr;
            M = Mn;
            const int nk = min(kWave, kr0.n - kb);
            for (int kk = 0; kk < nk; ++kk) {
                const float pk = readlane(p, kk);
                if (pk == 0.f)
                    continue;
                const int jk = readlane(j, kk);
                const T *vj = v + (tok0 + jk) * D;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int e = c * 64 + lane;
                    if (e < D)
                        acc[c] = fmaf(pk, ld(vj, e), acc[c]);
                }
            }
        }
        const size_t orow = ((size_t)bh * nh + r) * L + i;
        const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            if (e < D)
                o_rounds[orow * D + e] = from_f<T>(acc[c] * inv_l);
        }
        if (lane == 0)
            lse_rounds[orow] = l > 0.f ? M + logf(l) : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// combine: one wave per token


template <typename T, int D, int NH>
__global__ __launch_bounds__(kThreads) void combine_kernel(int L, int nh, int ntok, float scale,
                                                           const T *__restrict__ q, const T *__restrict__ v,
                                                           const T *__restrict__ o_rounds,
                                                           const float *__restrict__ lse_rounds,
                                                           T *__restrict__ out, float *__restrict__ lse)
{
    // D/8 lanes per token, each on 8 consecutive elements; the nh <= NH round
    // rows are all requested before any is used
    constexpr int CPT = D / 8, TPB = kThreads / CPT;
    const int grp = threadIdx.x / CPT, ch = threadIdx.x % CPT;
    const int tok = blockIdx.x * TPB + grp;
    const bool valid = tok < ntok;
    const int tk = valid ? tok : 0;
    const int bh = tk / L, t = tk % L;
    float ls[NH], x[NH][8];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        if (r < nh) {
            const size_t orow = ((size_t)bh * nh + r) * L + t;
            ls[r] = lse_rounds[orow];
            load8_nt(o_rounds + orow * D + ch * 8, x[r]);
        } else {
            ls[r] = -INFINITY;
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < NH; ++r)
        M = fmaxf(M, ls[r]);
    const bool alone = valid && M == -INFINITY;
    if (__ballot(alone) != 0ull) {
        // no member in any round: the token attends only to itself
        float y[8];
        float ss = 0.f;
        if (alone) {
            load8(q + (size_t)tk * D + ch * 8, y);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                ss = fmaf(y[k], y[k], ss);
        }
        ss = group_sum(ss, CPT);
        if (alone) {
            load8(v + (size_t)tk * D + ch * 8, y);
            store8(out + (size_t)tk * D + ch * 8, y);
            if (ch == 0)
                lse[tk] = scale * sqrtf(ss);
        }
    }
    if (!valid || alone)
        return;
    float den = 0.f;
#pragma unroll
    for (int r = 0; r < NH; ++r)
        den += expf(ls[r] - M);          // exp(-inf) = 0 for empty rounds and r >= nh
    const float total = M + logf(den);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        const float wgt = expf(ls[r] - total);
        if (r < nh) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                acc[k] = fmaf(wgt, x[r][k], acc[k]);
        }
    }
    store8_nt(out + (size_t)tk * D + ch * 8, acc);
    if (ch == 0)
        lse[tk] = total;
}

// ---------------------------------------------------------------------------
// backward, query side: dq_i of round r (wave per sorted query row)
//   p = exp(scale q_i.k_j - lse_i)  (global lse, so the rounds add up to the
//   union softmax),  g = p (dO_i.v_j - D_i),  dq_i += scale g k_j.

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(int L, int nh, float scale, const T *__restrict__ q,
                                                          const T *__restrict__ v, const T *__restrict__ dout,
                                                          const float *__restrict__ lse,
                                                          const float *__restrict__ Dvec,
                                                          const uint32_t *__restrict__ meta,
                                                          const uint32_t *__restrict__ srec,
                                                          const uint32_t *__restrict__ wmeta, int pos_test,
                                                          const uint32_t *__restrict__ bmeta,
                                                          const float *__restrict__ rnorm,
                                                          float *__restrict__ dq_part)
{
    constexpr int NC = (D + 63) / 64;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r = blockIdx.y, bh = blockIdx.z;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int s = (blockIdx.x * kWaves + wave) * kRowsPerWave + k;
        if (s >= L)
            break;
        const uint32_t rec = sr[s];
        const int i = (int)rec_lo(rec), w = (int)rec_hi(rec);
        const uint32_t *mi = meta + (tok0 + i) * nh;
        const uint32_t *wi = wmeta ? wmeta + (tok0 + i) * nh : nullptr;
        const KeyRange kr0 = key_range(s, w, wi, r);
        const float lse_i = lse[tok0 + i], D_i = Dvec[tok0 + i];
        float qreg[NC], goreg[NC], acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            qreg[c] = e < D ? ld(q, (tok0 + i) * D + e) : 0.f;
            goreg[c] = e < D ? ld(dout, (tok0 + i) * D + e) : 0.f;
            acc[c] = 0.f;
        }
        for (int kb = 0; kb < kr0.n; kb += kWave) {
            const int idx = kb + lane;
            bool valid = idx < kr0.n && kr0.lo + idx != s;
            const uint32_t kr = valid ? sr[kr0.lo + idx] : rec;
            const int j = (int)rec_lo(kr);
            if (pos_test)
                valid = valid && j < i;   // not after the query (chunk window without buckets)
            // duplicates: the first-owner mask, or (bmeta) the log of the divisor
            if (valid && !bmeta)
                valid = !owned_earlier(mi, wi, meta + (tok0 + j) * nh, r);
            const float dlog = valid ? dup_log(bmeta, tok0 + i, tok0 + j, nh) : 0.f;
            const float rn = rnorm[tok0 + j];
            const float dp = dot_row_bcast<T, D>(q + (tok0 + j) * D, qreg);
            const float dv = dot_row_bcast<T, D>(v + (tok0 + j) * D, goreg);
            const float p = valid ? expf(dp * scale * rn - lse_i - dlog) : 0.f;
            const float coef = scale * p * (dv - D_i) * rn;
            const int nk = min(kWave, kr0.n - kb);
            for (int kk = 0; kk < nk; ++kk) {
                const float ck = readlane(coef, kk);
                if (ck == 0.f)
                    continue;
                const int jk = readlane(j, kk);
                const T *qj = q + (tok0 + jk) * D;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int e = c * 64 + lane;
                    if (e < D)
                        acc[c] = fmaf(ck, ld(qj, e), acc[c]);
                }
            }
        }
        const size_t orow = ((size_t)bh * nh + r) * L + i;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            if (e < D)
                dq_part[orow * D + e] = acc[c];
        }
    }
}

// ---------------------------------------------------------------------------
// backward, key side: dk_j and dv_j of round r (wave per sorted key row).
// The queries whose round-r set holds key j (sorted index s) are the sorted
// rows s' > s with s' - w(s') <= s; win_lo is non-decreasing along the sorted
// order, so they form a prefix of s+1, s+2, ...  Without causality also the
// rows s' < s with hi(s') >= s (same bucket and chunk), all within
// [s - w(s), s - 1].

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(int L, int nh, float scale, const T *__restrict__ q,
                                                           const T *__restrict__ v, const T *__restrict__ dout,
                                                           const float *__restrict__ lse,
                                                           const float *__restrict__ Dvec,
                                                           const uint32_t *__restrict__ meta,
                                                           const uint32_t *__restrict__ srec,
                                                           const uint32_t *__restrict__ wmeta, int pos_test,
                                                           const uint32_t *__restrict__ bmeta,
                                                           const float *__restrict__ rnorm,
                                                           float *__restrict__ dk_part, float *__restrict__ dv_part)
{
    constexpr int NC = (D + 63) / 64;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r = blockIdx.y, bh = blockIdx.z;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int s = (blockIdx.x * kWaves + wave) * kRowsPerWave + k;
        if (s >= L)
            break;
        const uint32_t krec = sr[s];
        const int j = (int)rec_lo(krec);
        const uint32_t *mj = meta + (tok0 + j) * nh;
        const float rn = rnorm[tok0 + j];
        float kreg[NC], vreg[NC], dk[NC], dv[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            kreg[c] = e < D ? ld(q, (tok0 + j) * D + e) * rn : 0.f;
            vreg[c] = e < D ? ld(v, (tok0 + j) * D + e) : 0.f;
            dk[c] = dv[c] = 0.f;
        }
        // one batch of candidate queries (lane: query i, valid if it attends j)
        auto batch = [&](bool valid, int i, int nk) {
            if (pos_test)
                valid = valid && j < i;
            if (valid && !bmeta)
                valid = !owned_earlier(meta + (tok0 + i) * nh, wmeta ? wmeta + (tok0 + i) * nh : nullptr, mj, r);
            const float dlog = valid ? dup_log(bmeta, tok0 + i, tok0 + j, nh) : 0.f;
            const float dp = dot_row_bcast<T, D>(q + (tok0 + i) * D, kreg);
            const float dg = dot_row_bcast<T, D>(dout + (tok0 + i) * D, vreg);
            const float p = valid ? expf(dp * scale - lse[tok0 + i] - dlog) : 0.f;
            const float g = valid ? scale * p * (dg - Dvec[tok0 + i]) : 0.f;
            for (int kk = 0; kk < nk; ++kk) {
                const float pk = readlane(p, kk);
                if (pk == 0.f)
                    continue;
                const float gk = readlane(g, kk);
                const int ik = readlane(i, kk);
                const T *qi = q + (tok0 + ik) * D, *gi = dout + (tok0 + ik) * D;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int e = c * 64 + lane;
                    if (e < D) {
                        dv[c] = fmaf(pk, ld(gi, e), dv[c]);
                        dk[c] = fmaf(gk, ld(qi, e), dk[c]);
                    }
                }
            }
        };
        if (wmeta) {
            // earlier rows of j's bucket (or, without buckets, of j's window) in
        // j's chunk: kRange and kRangePos only
            for (int qb = s - (int)rec_hi(krec); qb < s; qb += kWave) {
                const int si = qb + lane;
                bool ok = false;
                int i = j;
                if (si < s) {
                    i = (int)rec_lo(sr[si]);
                    ok = (int)rec_lo(wmeta[(tok0 + i) * nh + r]) >= s;
                }
                batch(ok, i, min(kWave, s - qb));
            }
        }
        for (int qb = s + 1; qb < L; qb += kWave) {
            const int si = qb + lane;
            bool inwin = false;
            int i = j;
            if (si < L) {
                const uint32_t qrec = sr[si];
                i = (int)rec_lo(qrec);
                inwin = (si - (int)rec_hi(qrec)) <= s;
            }
            const bool more = __ballot(!inwin) == 0ull;  // whole batch in window: look further
            batch(inwin, i, min(kWave, L - qb));
            if (!more)
                break;
        }
        const size_t orow = ((size_t)bh * nh + r) * L + j;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            if (e < D) {
                dk_part[orow * D + e] = dk[c];
                dv_part[orow * D + e] = dv[c];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// backward reduce: sum the rounds, pass dk through k = q/|q|, add the
// self-only rows' dO to dv.  One wave per token.

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(int L, int nh, int ntok, const T *__restrict__ q,
                                                              const T *__restrict__ dout,
                                                              const uint32_t *__restrict__ meta,
                                                              const uint32_t *__restrict__ wmeta,
                                                              const uint8_t *__restrict__ aflag,
                                                              const float *__restrict__ rnorm,
                                                              const float *__restrict__ dq_part,
                                                              const float *__restrict__ dk_part,
                                                              const float *__restrict__ dv_part,
                                                              T *__restrict__ dq, T *__restrict__ dv)
{
    constexpr int NC = (D + 63) / 64;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int tok = blockIdx.x * kWaves + wave;
    if (tok >= ntok)
        return;
    const int bh = tok / L, t = tok % L;
    float aq[NC], ak[NC], av[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        aq[c] = ak[c] = av[c] = 0.f;
    bool alone = true;
    for (int r = 0; r < nh; ++r) {
        // no member but itself: w = 0 (kBand), span = 0 (kRange) or the lone flag (kRangePos)
        if (aflag)
            alone &= aflag[(size_t)tok * nh + r] != 0;
        else
            alone &= rec_hi((wmeta ? wmeta : meta)[(size_t)tok * nh + r]) == 0u;
        const size_t row = (((size_t)bh * nh + r) * L + t) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = c * 64 + lane;
            if (e < D) {
                aq[c] += dq_part[row + e];
                ak[c] += dk_part[row + e];
                av[c] += dv_part[row + e];
            }
        }
    }
    const float rn = rnorm[tok];
    float kreg[NC], kd = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int e = c * 64 + lane;
        kreg[c] = e < D ? ld(q, (size_t)tok * D + e) * rn : 0.f;
        kd = fmaf(kreg[c], ak[c], kd);
    }
    kd = wave_sum(kd);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int e = c * 64 + lane;
        if (e < D) {
            float gv = av[c];
            if (alone)
                gv += ld(dout, (size_t)tok * D + e);
            dq[(size_t)tok * D + e] = from_f<T>(aq[c] + (ak[c] - kreg[c] * kd) * rn);
            dv[(size_t)tok * D + e] = from_f<T>(gv);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers

template <typename T, int D>
hipError_t prep_go(const Dims &P, const void *q, const int32_t *inv, const int32_t *win_lo, uint32_t *meta,
                   uint32_t *srec, const Extra &x, float *rnorm, const void *out, const void *dout, float *Dv,
                   hipStream_t st)
{
    uint32_t *wmeta = x.wmeta, *cmin = x.cmin;
    uint8_t *alone = x.alone;
    constexpr int TPB = kThreads / (D / 8);
    dim3 grid((unsigned)(((P.L + TPB - 1) / TPB) * P.BH()));
    ProfScope prof(LSH_KERNEL_PREP, st);
    const int chunk_only = P.bucket_mask ? 0 : 1;
    hipLaunchKernelGGL((prep_kernel<T, D>), grid, dim3(kThreads), 0, st, P.L, P.nh, P.m, chunk_only, (const T *)q,
                       inv, win_lo, meta, srec, rnorm, (const T *)out, (const T *)dout, Dv);
    if (meta && wmeta) {
        if (alone) {
            const size_t nchunks = (size_t)P.BH() * P.nh * (P.L / P.m);
            hipLaunchKernelGGL(chunk_min_kernel, dim3((unsigned)((nchunks + kWaves - 1) / kWaves)), dim3(kThreads),
                               0, st, P.L, P.m, nchunks, srec, cmin);
        }
        const size_t total = (size_t)P.BH() * P.nh * P.L;
        hipLaunchKernelGGL(window_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           st, P.L, P.nh, P.m, chunk_only, total, srec, wmeta, cmin, alone);
    }
    if (meta && x.bmeta) {
        const dim3 grid((P.L + kScanThreads - 1) / kScanThreads, (unsigned)(P.BH() * P.nh));
        hipLaunchKernelGGL(run_tile_kernel, grid, dim3(kScanThreads), 0, st, P.L, srec, x.bscr);
        hipLaunchKernelGGL(bucket_start_kernel, grid, dim3(kScanThreads), 0, st, P.L, P.nh, srec, x.bscr, x.bmeta);
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t fwd_go(const Dims &P, const void *q, const void *v, const uint32_t *meta, const uint32_t *srec,
                  const Extra &x, const float *rnorm, void *o_rounds, float *lse_rounds, hipStream_t st)
{
    const int rows = kWaves * kRowsPerWave;
    dim3 grid((P.L + rows - 1) / rows, P.nh, P.BH());
    ProfScope prof(LSH_KERNEL_FWD, st);
    hipLaunchKernelGGL((fwd_kernel<T, D>), grid, dim3(kThreads), 0, st, P.L, P.nh, P.scale, (const T *)q,
                       (const T *)v, meta, srec, x.wmeta, P.kind() == kRangePos ? 1 : 0, x.bmeta, rnorm,
                       (T *)o_rounds, lse_rounds);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t combine_go(const Dims &P, const void *q, const void *v, const void *o_rounds, const float *lse_rounds,
                      void *out, float *lse, hipStream_t st)
{
    const int ntok = P.BH() * P.L;
    constexpr int TPB = kThreads / (D / 8);
    dim3 grid((ntok + TPB - 1) / TPB);
    ProfScope prof(LSH_KERNEL_COMBINE, st);
#define LSH_COMBINE(NH)                                                                                           \
    hipLaunchKernelGGL((combine_kernel<T, D, NH>), grid, dim3(kThreads), 0, st, P.L, P.nh, ntok, P.scale,        \
                       (const T *)q, (const T *)v, (const T *)o_rounds, lse_rounds, (T *)out, lse)
    if (P.nh <= 2)
        LSH_COMBINE(2);
    else if (P.nh <= 4)
        LSH_COMBINE(4);
    else if (P.nh <= 8)
        LSH_COMBINE(8);
    else
        LSH_COMBINE(16);
#undef LSH_COMBINE
    return hipGetLastError();
}

template <typename T, int D>
hipError_t reduce_go(const Dims &P, const void *q, const void *dout, const uint32_t *meta, const uint32_t *wmeta,
                     const uint8_t *alone, const float *rnorm, const float *dq_part, const float *dk_part,
                     const float *dv_part, void *dq, void *dv, hipStream_t st);

template <typename T, int D>
hipError_t bwd_go(const Dims &P, const void *q, const void *v, const void *dout, const float *lse,
                  const float *Dv, const uint32_t *meta, const uint32_t *srec, const Extra &x, const float *rnorm,
                  float *dq_part, float *dk_part, float *dv_part, void *dq, void *dv, hipStream_t st)
{
    const int rows = kWaves * kRowsPerWave;
    dim3 grid((P.L + rows - 1) / rows, P.nh, P.BH());
    const int pos_test = P.kind() == kRangePos ? 1 : 0;
    {
        ProfScope prof(LSH_KERNEL_BWD_DQ, st);
        hipLaunchKernelGGL((bwd_dq_kernel<T, D>), grid, dim3(kThreads), 0, st, P.L, P.nh, P.scale, (const T *)q,
                           (const T *)v, (const T *)dout, lse, Dv, meta, srec, x.wmeta, pos_test, x.bmeta, rnorm,
                           dq_part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    {
        ProfScope prof(LSH_KERNEL_BWD_DKV, st);
        hipLaunchKernelGGL((bwd_dkv_kernel<T, D>), grid, dim3(kThreads), 0, st, P.L, P.nh, P.scale, (const T *)q,
                           (const T *)v, (const T *)dout, lse, Dv, meta, srec, x.wmeta, pos_test, x.bmeta, rnorm,
                           dk_part, dv_part);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return reduce_go<T, D>(P, q, dout, meta, x.wmeta, x.alone, rnorm, dq_part, dk_part, dv_part, dq, dv, st);
}

template <typename T, int D>
hipError_t reduce_go(const Dims &P, const void *q, const void *dout, const uint32_t *meta, const uint32_t *wmeta,
                     const uint8_t *alone, const float *rnorm, const float *dq_part, const float *dk_part,
                     const float *dv_part, void *dq, void *dv, hipStream_t st)
{
    const int ntok = P.BH() * P.L;
    ProfScope prof(LSH_KERNEL_BWD_REDUCE, st);
    hipLaunchKernelGGL((bwd_reduce_kernel<T, D>), dim3((ntok + kWaves - 1) / kWaves), dim3(kThreads), 0, st,
                       P.L, P.nh, ntok, (const T *)q, (const T *)dout, meta, wmeta, alone, rnorm, dq_part, dk_part,
                       dv_part,
                       (T *)dq, (T *)dv);
    return hipGetLastError();
}

#define LSH_DISPATCH(dtype, d, CALL)                                                                          \
    do {                                                                                                      \
        if ((dtype) == LSH_BF16) {                                                                            \
            if ((d) == 32) { using T = bf16; constexpr int D = 32; return CALL; }                             \
            if ((d) == 64) { using T = bf16; constexpr int D = 64; return CALL; }                             \
            if ((d) == 128) { using T = bf16; constexpr int D = 128; return CALL; }                           \
        } else {                                                                                              \
            if ((d) == 32) { using T = float; constexpr int D = 32; return CALL; }                            \
            if ((d) == 64) { using T = float; constexpr int D = 64; return CALL; }                            \
            if ((d) == 128) { using T = float; constexpr int D = 128; return CALL; }                          \
        }                                                                                                     \
        return hipErrorInvalidValue;                                                                          \
    } while (0)

}  // namespace

hipError_t launch_prep(const Dims &P, int dtype, const void *q, const int32_t *perm, const int32_t *inv,
                       const int32_t *win_lo, uint32_t *meta, uint32_t *srec, const Extra &x, float *rnorm,
                       const void *out, const void *dout, float *Dv, hipStream_t st)
{
    (void)perm;
    LSH_DISPATCH(dtype, P.d, (prep_go<T, D>(P, q, inv, win_lo, meta, srec, x, rnorm, out, dout, Dv, st)));
}

hipError_t launch_attn_fwd(const Dims &P, int dtype, const void *q, const void *v, const uint32_t *meta,
                           const uint32_t *srec, const Extra &x, const float *rnorm, void *o_rounds,
                           float *lse_rounds, hipStream_t st)
{
    LSH_DISPATCH(dtype, P.d, (fwd_go<T, D>(P, q, v, meta, srec, x, rnorm, o_rounds, lse_rounds, st)));
}

hipError_t launch_combine(const Dims &P, int dtype, const void *q, const void *v, const void *o_rounds,
                          const float *lse_rounds, void *out, float *lse, hipStream_t st)
{
    LSH_DISPATCH(dtype, P.d, (combine_go<T, D>(P, q, v, o_rounds, lse_rounds, out, lse, st)));
}

hipError_t launch_attn_bwd(const Dims &P, int dtype, const void *q, const void *v, const void *dout,
                           const float *lse, const float *Dv, const uint32_t *meta, const uint32_t *srec,
                           const Extra &x, const float *rnorm, float *dq_part, float *dk_part, float *dv_part,
                           void *dq, void *dv, hipStream_t st)
{
    LSH_DISPATCH(dtype, P.d,
                 (bwd_go<T, D>(P, q, v, dout, lse, Dv, meta, srec, x, rnorm, dq_part, dk_part, dv_part, dq, dv, st)));
}

}  // namespace lsh
