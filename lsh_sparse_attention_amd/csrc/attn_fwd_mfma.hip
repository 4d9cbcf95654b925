// attn_fwd_mfma.hip -- per-round chunked LSH attention forward on bf16 MFMA.
//
// "Reformer: The Efficient Transformer" §2 (attention over chunks of the
// sorted order, causal mask through the permutation, self only as a
// fallback) and App. A (union over rounds, duplicates masked; per-round
// outputs combined later by logsumexp weights).
//
// Round r, query at sorted index s attends to the sorted keys [s - w, s - 1]
// (w = s - win_lo: same bucket, own chunk or the one before, not after the
// query), minus those that already belong to its set in an earlier round.
// The band needs no chunk arithmetic here: win_lo carries it.
//
// Work split: a workgroup (4 waves) owns 128 consecutive sorted query rows of
// one (batch, head, round); each wave owns 32 of them.  Keys stream through
// LDS in blocks of 32 sorted rows, from the block holding win_lo of the first
// row to the diagonal; the next block's rows are fetched into registers while
// the current one is used.  Per block each wave computes S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 (lane = query, 16 keys per lane), applies the
// band and duplicate masks, updates the online softmax in fp32 (exp2
// domain), and accumulates O^T += V^T P^T, with P^T taken straight from the
// accumulator registers.  The epilogue writes o and lse at the query's
// original position (the unsort).
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kQB = 128;      // query rows per workgroup
constexpr int kKB = 32;       // keys per block
constexpr int kThreads = 256;
constexpr int kMaxRounds = 16;

constexpr int kRecCache = 512;  // sorted records of a workgroup's key range kept in LDS
constexpr int kMetaPerThread = (kKB * (kMaxRounds - 1) + kThreads - 1) / kThreads;
// The running max of a query row is only raised when a block's max exceeds it
// by more than this many log2 units; exp2 arguments stay <= kLazy, so the
// accumulators need rescaling only on those (rare) raises.
constexpr float kLazy = 8.0f;

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(int L, int nh, float scale_log2,
                                                            const bf16 *__restrict__ q, const bf16 *__restrict__ v,
                                                            const uint32_t *__restrict__ meta,
                                                            const uint32_t *__restrict__ srec,
                                                            const float *__restrict__ rnorm,
                                                            bf16 *__restrict__ o_rounds,
                                                            float *__restrict__ lse_rounds)
{
    constexpr int P = D + 8;  // LDS row pitch (elements), keeps 16-byte rows off one bank set
    __shared__ __align__(16) uint16_t Ks[kKB * P];
    __shared__ __align__(16) uint16_t Vs[kKB * P];
    __shared__ __align__(16) float rnk[kKB];
    __shared__ __align__(16) uint16_t kmeta[kMaxRounds - 1][kKB];   // key sorted index in earlier rounds
    __shared__ uint32_t qmeta[kThreads / kWave][kMaxRounds - 1][32];  // query records of earlier rounds
    __shared__ uint32_t krec[kRecCache];                                 // sorted records of the key range

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int h = lane / 32, c = lane % 32;
    // 1-D grid in XCD-friendly order: row blocks fastest, then round, then (b, h)
    const int nblk = L / kQB;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int r = (lb / nblk) % nh, bh = lb / (nblk * nh);
    const int s0 = (lb % nblk) * kQB;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;

    // this lane's query (column c of the wave's 32)
    const int wq0 = s0 + wave * 32;
    const int sq = wq0 + c;
    const uint32_t qrec = sr[sq];
    const int qpos = (int)rec_lo(qrec), qw = (int)rec_hi(qrec);
    const int qlo = sq - qw;                      // window: sorted keys [qlo, sq)
    const int wlo = __builtin_amdgcn_readlane(qlo, 0);   // win_lo is non-decreasing: lane 0 is the wave minimum
    if (h == 0)
        for (int rr = 0; rr < r; ++rr)
            qmeta[wave][rr][c] = meta[(tok0 + qpos) * nh + rr];

    // B operand of S^T = K Q^T: lane holds Q[query c][16 ks + 8 h .. +7]
    bf16x8_t qop[D / 16];
    {
        const bf16 *qrow = q + (tok0 + qpos) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qop[ks] = as_bf16x8(ld16(qrow + 16 * ks + 8 * h));
    }

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        oacc[dt] = f32x16_t{};
    float mrun = -INFINITY, lrun = 0.f;

    const int wg_lo = s0 - (int)rec_hi(sr[s0]);
    const int kb_first = wg_lo & ~(kKB - 1);
    const int kb_end = s0 + kQB;

    constexpr int kChunks = kKB * (D / 8) / kThreads;  // 16-byte chunks per thread per tensor
    // the key range's sorted records, in LDS when they fit
    const bool cached = kb_end - kb_first <= kRecCache;
    if (cached)
        for (int i = tid; i < kb_end - kb_first; i += kThreads)
            krec[i] = sr[kb_first + i];
    __syncthreads();
    auto key_pos = [&](int s) __attribute__((always_inline)) {
        return rec_lo(cached ? krec[s - kb_first] : sr[s]);
    };
    u32x4_t pk[kChunks], pv[kChunks];
    float prn = 0.f;
    uint32_t pkm[kMetaPerThread];
    auto fetch = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int idx = tid + i * kThreads;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            const size_t pos = tok0 + key_pos(kb + row);
            pk[i] = ld16(q + pos * D + ch * 8);
            pv[i] = ld16(v + pos * D + ch * 8);
        }
        if (tid < kKB)
            prn = rnorm[tok0 + key_pos(kb + tid)] * scale_log2;
#pragma unroll
        for (int i = 0; i < kMetaPerThread; ++i) {
            const int idx = tid + i * kThreads;
            pkm[i] = 0u;
            if (idx < kKB * r)
                pkm[i] = rec_lo(meta[(tok0 + key_pos(kb + idx % kKB)) * nh + idx / kKB]);
        }
    };

    fetch(kb_first);
    for (int kb = kb_first; kb < kb_end; kb += kKB) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int idx = tid + i * kThreads;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            st16(&Ks[row * P + ch * 8], pk[i]);
            st16(&Vs[row * P + ch * 8], pv[i]);
        }
        if (tid < kKB)
            rnk[tid] = prn;
#pragma unroll
        for (int i = 0; i < kMetaPerThread; ++i) {
            const int idx = tid + i * kThreads;
            if (idx < kKB * r)
                kmeta[idx / kKB][idx % kKB] = pkm[i];
        }
        __syncthreads();
        // prefetch the next block (the last iteration re-reads its own block,
        // which keeps the staging registers free of control flow)
        fetch(kb + kKB < kb_end ? kb + kKB : kb);

        // keys [kb, kb+31] against this wave's windows: the last query of the
        // wave sees keys up to wq0 + 30, the first from wlo
        if (kb > wq0 || kb + kKB - 1 < wlo)
            continue;

        // S^T = K Q^T
        f32x16_t sacc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8_t a = as_bf16x8(ld16(&Ks[c * P + 16 * ks + 8 * h]));
            sacc = mfma32(a, qop[ks], sacc);
        }

        // band mask: key kb + 8 g + 4 h + t inside [qlo, sq)
        bool ok[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            ok[e] = (unsigned)(kb + 8 * (e / 4) + 4 * h + (e % 4) - qlo) < (unsigned)qw;
        // first-owner mask: drop keys that are in the query's set of an earlier
        // round (two keys per packed 16-bit test)
        if (r > 0) {
            uint32_t hit[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            for (int rr = 0; rr < r; ++rr) {
                const uint32_t qmr = qmeta[wave][rr][c];
                const uint32_t si1p = bcast16(rec_lo(qmr) - 1u), wp = bcast16(rec_hi(qmr));
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint2 kp = *reinterpret_cast<const uint2 *>(&kmeta[rr][8 * g + 4 * h]);
                    hit[2 * g] |= win_hits2(si1p, wp, kp.x);
                    hit[2 * g + 1] |= win_hits2(si1p, wp, kp.y);
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e)
                ok[e] = ok[e] && ((hit[e / 2] >> (16 * (e % 2))) & 0xffffu) == 0u;
        }
        // logits in log2 units
        float x[16];
        float bm = -INFINITY;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 rn4 = *reinterpret_cast<const float4 *>(&rnk[8 * g + 4 * h]);
            const float rn[4] = {rn4.x, rn4.y, rn4.z, rn4.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[4 * g + t] = ok[4 * g + t] ? sacc[4 * g + t] * rn[t] : -INFINITY;
                bm = fmaxf(bm, x[4 * g + t]);
            }
        }
        bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
        // lazy running max: raise it only when this block exceeds it by more
        // than kLazy (or it is still -inf); both halves of a query agree
        const bool raise = bm > mrun + kLazy;
        const float mnew = raise ? bm : mrun;
        // a query with nothing valid so far keeps m = -inf; reference 0 keeps
        // the arithmetic finite (its p come out 0)
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            x[e] = fast_exp2(x[e] - mref);
            ps += x[e];
        }
        ps += __shfl_xor(ps, 32, kWave);
        if (__ballot(raise) != 0ull) {
            const float corr = raise ? fast_exp2(mrun - mref) : 1.f;
            lrun *= corr;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                oacc[dt] *= corr;
        }
        lrun += ps;
        mrun = mnew;
        float *p = x;

        // O^T += V^T P^T; P^T slot s of MFMA j is p[8 j + s] (keys 16 j + 4 h + s,
        // then 16 j + 8 + 4 h + s - 4)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4_t pu;
            pu.x = pack_bf16x2(p[8 * j + 0], p[8 * j + 1]);
            pu.y = pack_bf16x2(p[8 * j + 2], p[8 * j + 3]);
            pu.z = pack_bf16x2(p[8 * j + 4], p[8 * j + 5]);
            pu.w = pack_bf16x2(p[8 * j + 6], p[8 * j + 7]);
            const bf16x8_t pb = as_bf16x8(pu);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                oacc[dt] = mfma32(tile_t<P>(Vs, j, 32 * dt, lane), pb, oacc[dt]);
        }
    }

    // epilogue: o^T lane c holds d = 32 dt + 8 g + 4 h + t of query c
    const size_t orow = ((size_t)bh * nh + r) * L + qpos;
    const float inv_l = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(oacc[dt][4 * g + 0] * inv_l, oacc[dt][4 * g + 1] * inv_l);
            w.y = pack_bf16x2(oacc[dt][4 * g + 2] * inv_l, oacc[dt][4 * g + 3] * inv_l);
            *reinterpret_cast<uint2 *>(o_rounds + orow * D + 32 * dt + 8 * g + 4 * h) = w;
        }
    }
    if (h == 0)
        lse_rounds[orow] = lrun > 0.f ? (mrun + __log2f(lrun)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

bool mfma_path_ok(const Dims &P, int dtype)
{
    return dtype == LSH_BF16 && (P.d == 64 || P.d == 128) && P.L % kQB == 0 && P.nh <= kMaxRounds;
}

hipError_t launch_attn_fwd_mfma(const Dims &P, const void *q, const void *v, const uint32_t *meta,
                                const uint32_t *srec, const float *rnorm, void *o_rounds, float *lse_rounds,
                                hipStream_t st)
{
    dim3 grid((P.L / kQB) * P.nh * P.BH());
    const float scale_log2 = P.scale * 1.4426950408889634f;
    ProfScope prof(LSH_KERNEL_FWD, st);
    if (P.d == 128)
        hipLaunchKernelGGL((fwd_mfma_kernel<128>), grid, dim3(kThreads), 0, st, P.L, P.nh, scale_log2,
                           (const bf16 *)q, (const bf16 *)v, meta, srec, rnorm, (bf16 *)o_rounds, lse_rounds);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<64>), grid, dim3(kThreads), 0, st, P.L, P.nh, scale_log2,
                           (const bf16 *)q, (const bf16 *)v, meta, srec, rnorm, (bf16 *)o_rounds, lse_rounds);
    return hipGetLastError();
}

}  // namespace lsh
