// attn_bwd_mfma.hip -- backward of the per-round chunked LSH attention on
// bf16 MFMA, with the bucket assignment and sort order held fixed (no
// gradient through hashing or sorting, as the Reformer authors state in
// Hacker News thread 22095523).
//
// With the global lse of each query (from the combine), the per-round
// probabilities p = exp(scale q_i.k_j - lse_i) over the round's unmasked
// members are already that round's share of the union softmax, so every
// round's gradient is computed independently:
//   g_ij = p_ij (dO_i . v_j - D_i),  D_i = dO_i . o_i,
//   dq_i += scale g_ij k_j,  dk_j += scale g_ij q_i,  dv_j += p_ij dO_i.
// The masks are those of the forward: band [win_lo, s) in sorted order, and
// keys that are in the query's set of an earlier round are dropped.
//
// Two kernels per call, each over all rounds, each writing complete per-round
// results as bf16 (no atomics, deterministic), then a reduction over rounds:
//   bwd_dq_mfma   a workgroup owns 128 sorted query rows (wave: 32); keys
//                 stream in blocks of 32 (lane = query, as in the forward);
//                 dQ^T += K^T (G^T scaled per key) on the MFMA.
//   bwd_dkv_mfma  a workgroup owns 128 sorted key rows (wave: 32); queries
//                 stream in blocks of 32 (lane = key): S = Q K^T,
//                 dP = dO V^T, dV^T += dO^T P, dK^T += Q^T G.
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kRows = 128;     // rows owned by a workgroup
constexpr int kBlk = 32;       // streamed rows per block
constexpr int kThreads = 256;
constexpr int kMaxRounds = 16;
constexpr int kRecCache = 512;  // sorted records of a workgroup's streamed range kept in LDS
constexpr int kMetaPerThread = (kBlk * (kMaxRounds - 1) + kThreads - 1) / kThreads;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8_t pack8(const float *x)
{
    u32x4_t u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]);
    u.w = pack_bf16x2(x[6], x[7]);
    return as_bf16x8(u);
}

// ---------------------------------------------------------------------------
// query side

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_mfma_kernel(int L, int nh, float scale,
                                                               const bf16 *__restrict__ q, const bf16 *__restrict__ v,
                                                               const bf16 *__restrict__ dout,
                                                               const float *__restrict__ lse,
                                                               const float *__restrict__ Dvec,
                                                               const uint32_t *__restrict__ meta,
                                                               const uint32_t *__restrict__ srec,
                                                               const float *__restrict__ rnorm,
                                                               bf16 *__restrict__ dq_part)
{
    constexpr int P = D + 8;
    __shared__ __align__(16) uint16_t Ks[kBlk * P];
    __shared__ __align__(16) uint16_t Vs[kBlk * P];
    __shared__ __align__(16) float rnk[kBlk];
    __shared__ __align__(16) uint16_t kmeta[kMaxRounds - 1][kBlk];
    __shared__ uint32_t qmeta[kThreads / kWave][kMaxRounds - 1][32];
    __shared__ uint32_t krec[kRecCache];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int h = lane / 32, c = lane % 32;
    const int nblk = L / kRows;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int r = (lb / nblk) % nh, bh = lb / (nblk * nh);
    const int s0 = (lb % nblk) * kRows;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;
    const float scale_log2 = scale * kLog2e;

    const int wq0 = s0 + wave * 32;
    const int sq = wq0 + c;
    const uint32_t qrec = sr[sq];
    const int qpos = (int)rec_lo(qrec), qw = (int)rec_hi(qrec);
    const int qlo = sq - qw;
    const int wlo = __builtin_amdgcn_readlane(qlo, 0);
    if (h == 0)
        for (int rr = 0; rr < r; ++rr)
            qmeta[wave][rr][c] = meta[(tok0 + qpos) * nh + rr];
    const float lse2 = lse[tok0 + qpos] * kLog2e;
    const float Di = Dvec[tok0 + qpos];

    bf16x8_t qop[D / 16], gop[D / 16];
    {
        const bf16 *qrow = q + (tok0 + qpos) * D, *grow = dout + (tok0 + qpos) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            qop[ks] = as_bf16x8(ld16(qrow + 16 * ks + 8 * h));
            gop[ks] = as_bf16x8(ld16(grow + 16 * ks + 8 * h));
        }
    }
    f32x16_t acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = f32x16_t{};

    const int wg_lo = s0 - (int)rec_hi(sr[s0]);
    const int kb_first = wg_lo & ~(kBlk - 1);
    const int kb_end = s0 + kRows;

    constexpr int kChunks = kBlk * (D / 8) / kThreads;
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
        if (tid < kBlk)
            prn = rnorm[tok0 + key_pos(kb + tid)];
#pragma unroll
        for (int i = 0; i < kMetaPerThread; ++i) {
            const int idx = tid + i * kThreads;
            pkm[i] = 0u;
            if (idx < kBlk * r)
                pkm[i] = rec_lo(meta[(tok0 + key_pos(kb + idx % kBlk)) * nh + idx / kBlk]);
        }
    };

    fetch(kb_first);
    for (int kb = kb_first; kb < kb_end; kb += kBlk) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int idx = tid + i * kThreads;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            st16(&Ks[row * P + ch * 8], pk[i]);
            st16(&Vs[row * P + ch * 8], pv[i]);
        }
        if (tid < kBlk)
            rnk[tid] = prn;
#pragma unroll
        for (int i = 0; i < kMetaPerThread; ++i) {
            const int idx = tid + i * kThreads;
            if (idx < kBlk * r)
                kmeta[idx / kBlk][idx % kBlk] = pkm[i];
        }
        __syncthreads();
        fetch(kb + kBlk < kb_end ? kb + kBlk : kb);
        if (kb > wq0 || kb + kBlk - 1 < wlo)
            continue;

        // S^T = K Q^T and dP^T = V dO^T (lane = query c, keys 8 g + 4 h + t)
        f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            sacc = mfma32(as_bf16x8(ld16(&Ks[c * P + 16 * ks + 8 * h])), qop[ks], sacc);
            pacc = mfma32(as_bf16x8(ld16(&Vs[c * P + 16 * ks + 8 * h])), gop[ks], pacc);
        }
        bool ok[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            ok[e] = (unsigned)(kb + 8 * (e / 4) + 4 * h + (e % 4) - qlo) < (unsigned)qw;
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
        // g^T scaled by scale * rnorm_k (the key is q_j rnorm_j)
        float gs[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 rn4 = *reinterpret_cast<const float4 *>(&rnk[8 * g + 4 * h]);
            const float rn[4] = {rn4.x, rn4.y, rn4.z, rn4.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = 4 * g + t;
                const float pr = ok[e] ? fast_exp2(sacc[e] * rn[t] * scale_log2 - lse2) : 0.f;
                gs[e] = pr * (pacc[e] - Di) * (scale * rn[t]);
            }
        }
        // dQ^T += K^T Gs^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8_t gb = pack8(gs + 8 * j);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = mfma32(tile_t<P>(Ks, j, 32 * dt, lane), gb, acc[dt]);
        }
    }

    // dq lane c: d = 32 dt + 8 g + 4 h + t; stored as bf16
    bf16 *out = dq_part + (((size_t)bh * nh + r) * L + qpos) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(acc[dt][4 * g + 0], acc[dt][4 * g + 1]);
            w.y = pack_bf16x2(acc[dt][4 * g + 2], acc[dt][4 * g + 3]);
            *reinterpret_cast<uint2 *>(out + 32 * dt + 8 * g + 4 * h) = w;
        }
}

// ---------------------------------------------------------------------------
// key side

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkv_mfma_kernel(int L, int nh, float scale,
                                                                const bf16 *__restrict__ q,
                                                                const bf16 *__restrict__ v,
                                                                const bf16 *__restrict__ dout,
                                                                const float *__restrict__ lse,
                                                                const float *__restrict__ Dvec,
                                                                const uint32_t *__restrict__ meta,
                                                                const uint32_t *__restrict__ srec,
                                                                const float *__restrict__ rnorm,
                                                                bf16 *__restrict__ dqk_part,
                                                                bf16 *__restrict__ dv_part)
{
    constexpr int P = D + 8;
    __shared__ __align__(16) uint16_t Qs[kBlk * P];
    __shared__ __align__(16) uint16_t Gs[kBlk * P];   // dO rows
    __shared__ __align__(16) float qlse2[kBlk];
    __shared__ __align__(16) float qD[kBlk];
    __shared__ __align__(16) int qlo_s[kBlk];
    __shared__ __align__(16) int qw_s[kBlk];
    __shared__ __align__(16) uint16_t qsi1[kMaxRounds - 1][kBlk];    // query sorted index - 1, earlier rounds
    __shared__ __align__(16) uint16_t qw16[kMaxRounds - 1][kBlk];    // query window length, earlier rounds
    __shared__ uint32_t kmeta[kThreads / kWave][kMaxRounds - 1][32];  // key sorted index in earlier rounds
    __shared__ uint32_t qrec_s[kRecCache];                             // sorted records from k0 on

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int h = lane / 32, c = lane % 32;
    const int nblk = L / kRows;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int r = (lb / nblk) % nh, bh = lb / (nblk * nh);
    const int k0 = (lb % nblk) * kRows;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;

    const int wk0 = k0 + wave * 32;
    const int sk = wk0 + c;                       // this lane's key (sorted)
    const int kpos = (int)rec_lo(sr[sk]);
    const float krn2 = rnorm[tok0 + kpos] * scale * kLog2e;
    if (h == 0)
        for (int rr = 0; rr < r; ++rr)
            kmeta[wave][rr][c] = rec_lo(meta[(tok0 + kpos) * nh + rr]);

    bf16x8_t kop[D / 16], vop[D / 16];
    {
        const bf16 *krow = q + (tok0 + kpos) * D, *vrow = v + (tok0 + kpos) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            kop[ks] = as_bf16x8(ld16(krow + 16 * ks + 8 * h));
            vop[ks] = as_bf16x8(ld16(vrow + 16 * ks + 8 * h));
        }
    }
    f32x16_t dka[D / 32], dva[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        dka[dt] = dva[dt] = f32x16_t{};

    // queries: sorted rows after the first key whose window reaches the last key
    const int qb_first = k0;
    const int k_last = k0 + kRows - 1;

    constexpr int kChunks = kBlk * (D / 8) / kThreads;
    const int cache_end = min(L, k0 + kRecCache);
    for (int i = tid; i < cache_end - k0; i += kThreads)
        qrec_s[i] = sr[k0 + i];
    __syncthreads();
    auto qrec_of = [&](int s) __attribute__((always_inline)) { return s < cache_end ? qrec_s[s - k0] : sr[s]; };
    u32x4_t pq[kChunks], pg[kChunks];
    float plse = 0.f, pD = 0.f;
    int plo = 0, pw = 0;
    uint32_t pqm[kMetaPerThread];
    auto fetch = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int idx = tid + i * kThreads;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            const size_t pos = tok0 + rec_lo(qrec_of(qb + row));
            pq[i] = ld16(q + pos * D + ch * 8);
            pg[i] = ld16(dout + pos * D + ch * 8);
        }
        if (tid < kBlk) {
            const uint32_t rec = qrec_of(qb + tid);
            const size_t pos = tok0 + rec_lo(rec);
            plse = lse[pos] * kLog2e;
            pD = Dvec[pos];
            pw = (int)rec_hi(rec);
            plo = qb + tid - pw;
        }
#pragma unroll
        for (int i = 0; i < kMetaPerThread; ++i) {
            const int idx = tid + i * kThreads;
            pqm[i] = 0u;
            if (idx < kBlk * r)
                pqm[i] = meta[(tok0 + rec_lo(qrec_of(qb + idx % kBlk))) * nh + idx / kBlk];
        }
    };

    fetch(qb_first);
    for (int qb = qb_first; qb < L; qb += kBlk) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int idx = tid + i * kThreads;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            st16(&Qs[row * P + ch * 8], pq[i]);
            st16(&Gs[row * P + ch * 8], pg[i]);
        }
        if (tid < kBlk) {
            qlse2[tid] = plse;
            qD[tid] = pD;
            qlo_s[tid] = plo;
            qw_s[tid] = pw;
        }
#pragma unroll
        for (int i = 0; i < kMetaPerThread; ++i) {
            const int idx = tid + i * kThreads;
            if (idx < kBlk * r) {
                qsi1[idx / kBlk][idx % kBlk] = (uint16_t)(rec_lo(pqm[i]) - 1u);
                qw16[idx / kBlk][idx % kBlk] = (uint16_t)rec_hi(pqm[i]);
            }
        }
        __syncthreads();
        // win_lo is non-decreasing, so the block's first row has its smallest
        // window start: once that is past the last key, no later query sees
        // any key of this workgroup
        const int blk_lo = qlo_s[0];
        if (blk_lo > k_last)
            break;
        fetch(qb + kBlk < L ? qb + kBlk : qb);
        // this wave's keys [wk0, wk0+31]: queries must come after a key and
        // start their window at or before it
        if (qb + kBlk - 1 <= wk0 || blk_lo > wk0 + 31)
            continue;

        // S = Q K^T, dP = dO V^T (lane = key c, queries 8 g + 4 h + t)
        f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            sacc = mfma32(as_bf16x8(ld16(&Qs[c * P + 16 * ks + 8 * h])), kop[ks], sacc);
            pacc = mfma32(as_bf16x8(ld16(&Gs[c * P + 16 * ks + 8 * h])), vop[ks], pacc);
        }
        bool ok[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int4 lo4 = *reinterpret_cast<const int4 *>(&qlo_s[8 * g + 4 * h]);
            const int4 w4 = *reinterpret_cast<const int4 *>(&qw_s[8 * g + 4 * h]);
            ok[4 * g + 0] = (unsigned)(sk - lo4.x) < (unsigned)w4.x;
            ok[4 * g + 1] = (unsigned)(sk - lo4.y) < (unsigned)w4.y;
            ok[4 * g + 2] = (unsigned)(sk - lo4.z) < (unsigned)w4.z;
            ok[4 * g + 3] = (unsigned)(sk - lo4.w) < (unsigned)w4.w;
        }
        if (r > 0) {
            uint32_t hit[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            for (int rr = 0; rr < r; ++rr) {
                const uint32_t skp = bcast16(kmeta[wave][rr][c]);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint2 s1 = *reinterpret_cast<const uint2 *>(&qsi1[rr][8 * g + 4 * h]);
                    const uint2 ww = *reinterpret_cast<const uint2 *>(&qw16[rr][8 * g + 4 * h]);
                    hit[2 * g] |= win_hits2(s1.x, ww.x, skp);
                    hit[2 * g + 1] |= win_hits2(s1.y, ww.y, skp);
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e)
                ok[e] = ok[e] && ((hit[e / 2] >> (16 * (e % 2))) & 0xffffu) == 0u;
        }
        float pr[16], gr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 l4 = *reinterpret_cast<const float4 *>(&qlse2[8 * g + 4 * h]);
            const float4 d4 = *reinterpret_cast<const float4 *>(&qD[8 * g + 4 * h]);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = 4 * g + t;
                pr[e] = ok[e] ? fast_exp2(sacc[e] * krn2 - lv[t]) : 0.f;
                gr[e] = pr[e] * (pacc[e] - dv[t]) * scale;
            }
        }
        // dV^T += dO^T P, dK^T += Q^T G (scale folded into G)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8_t pb = pack8(pr + 8 * j), gb = pack8(gr + 8 * j);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                dva[dt] = mfma32(tile_t<P>(Gs, j, 32 * dt, lane), pb, dva[dt]);
                dka[dt] = mfma32(tile_t<P>(Qs, j, 32 * dt, lane), gb, dka[dt]);
            }
        }
    }

    // Through the key normalisation k = q rn: the query-side gradient of dk is
    // (dk - k (k . dk)) rn = (dk - q rn^2 (q . dk)) rn, formed here in fp32
    // while dk is complete for this round; lane c holds d = 32 dt + 8 g + 4 h + t.
    const float rn = rnorm[tok0 + kpos];
    const bf16 *krow = q + (tok0 + kpos) * D;
    float qv[D / 32][16];
    float qd = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint2 u = *reinterpret_cast<const uint2 *>(krow + 32 * dt + 8 * g + 4 * h);
            qv[dt][4 * g + 0] = __uint_as_float(u.x << 16);
            qv[dt][4 * g + 1] = __uint_as_float(u.x & 0xffff0000u);
            qv[dt][4 * g + 2] = __uint_as_float(u.y << 16);
            qv[dt][4 * g + 3] = __uint_as_float(u.y & 0xffff0000u);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                qd = fmaf(qv[dt][4 * g + t], dka[dt][4 * g + t], qd);
        }
    qd += __shfl_xor(qd, 32, kWave);
    const float proj = rn * rn * qd;
    const size_t row = (((size_t)bh * nh + r) * L + kpos) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * dt + 8 * g + 4 * h;
            float e[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                e[t] = (dka[dt][4 * g + t] - qv[dt][4 * g + t] * proj) * rn;
            uint2 w;
            w.x = pack_bf16x2(e[0], e[1]);
            w.y = pack_bf16x2(e[2], e[3]);
            *reinterpret_cast<uint2 *>(dqk_part + row + d0) = w;
            w.x = pack_bf16x2(dva[dt][4 * g + 0], dva[dt][4 * g + 1]);
            w.y = pack_bf16x2(dva[dt][4 * g + 2], dva[dt][4 * g + 3]);
            *reinterpret_cast<uint2 *>(dv_part + row + d0) = w;
        }
}

// Sum of the per-round partials: dQ = sum_r (dq_r + dqk_r), dV = sum_r dv_r,
// plus dO for tokens that attend only to themselves (o = v).  D/8 lanes per
// token, 8 elements each.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_reduce_mfma_kernel(int L, int nh, int ntok,
                                                                   const bf16 *__restrict__ dout,
                                                                   const uint32_t *__restrict__ meta,
                                                                   const bf16 *__restrict__ dq_part,
                                                                   const bf16 *__restrict__ dqk_part,
                                                                   const bf16 *__restrict__ dv_part,
                                                                   bf16 *__restrict__ dq, bf16 *__restrict__ dv)
{
    constexpr int CPT = D / 8, TPB = kThreads / CPT;
    const int grp = threadIdx.x / CPT, ch = threadIdx.x % CPT;
    const int tok = blockIdx.x * TPB + grp;
    if (tok >= ntok)
        return;
    const int bh = tok / L, t = tok % L;
    float aq[8] = {}, av[8] = {};
    bool alone = true;
    for (int r = 0; r < nh; ++r) {
        alone = alone && rec_hi(meta[(size_t)tok * nh + r]) == 0u;
        const size_t off = (((size_t)bh * nh + r) * L + t) * D + ch * 8;
        float x[8], y[8], z[8];
        load8(dq_part + off, x);
        load8(dqk_part + off, y);
        load8(dv_part + off, z);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            aq[k] += x[k] + y[k];
            av[k] += z[k];
        }
    }
    if (alone) {
        float x[8];
        load8(dout + (size_t)tok * D + ch * 8, x);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            av[k] += x[k];
    }
    store8(dq + (size_t)tok * D + ch * 8, aq);
    store8(dv + (size_t)tok * D + ch * 8, av);
}

template <int D>
hipError_t go(const Dims &P, const void *q, const void *v, const void *dout, const float *lse, const float *Dv,
              const uint32_t *meta, const uint32_t *srec, const float *rnorm, void *part, void *dq, void *dv,
              hipStream_t st)
{
    const size_t n = (size_t)P.BH() * P.nh * P.L * D;
    bf16 *dq_part = (bf16 *)part, *dqk_part = dq_part + n, *dv_part = dqk_part + n;
    dim3 grid((P.L / kRows) * P.nh * P.BH());
    {
        ProfScope prof(LSH_KERNEL_BWD_DQ, st);
        hipLaunchKernelGGL((bwd_dq_mfma_kernel<D>), grid, dim3(kThreads), 0, st, P.L, P.nh, P.scale,
                           (const bf16 *)q, (const bf16 *)v, (const bf16 *)dout, lse, Dv, meta, srec, rnorm,
                           dq_part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    {
        ProfScope prof(LSH_KERNEL_BWD_DKV, st);
        hipLaunchKernelGGL((bwd_dkv_mfma_kernel<D>), grid, dim3(kThreads), 0, st, P.L, P.nh, P.scale,
                           (const bf16 *)q, (const bf16 *)v, (const bf16 *)dout, lse, Dv, meta, srec, rnorm,
                           dqk_part, dv_part);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int ntok = P.BH() * P.L;
    constexpr int TPB = kThreads / (D / 8);
    ProfScope prof(LSH_KERNEL_BWD_REDUCE, st);
    hipLaunchKernelGGL((bwd_reduce_mfma_kernel<D>), dim3((ntok + TPB - 1) / TPB), dim3(kThreads), 0, st, P.L, P.nh,
                       ntok, (const bf16 *)dout, meta, dq_part, dqk_part, dv_part, (bf16 *)dq, (bf16 *)dv);
    return hipGetLastError();
}

}  // namespace

size_t bwd_mfma_part_bytes(const Dims &P) { return 3 * (size_t)P.BH() * P.nh * P.L * P.d * sizeof(uint16_t); }

hipError_t launch_attn_bwd_mfma(const Dims &P, const void *q, const void *v, const void *dout, const float *lse,
                                const float *Dv, const uint32_t *meta, const uint32_t *srec, const float *rnorm,
                                void *part, void *dq, void *dv, hipStream_t st)
{
    if (P.d == 128)
        return go<128>(P, q, v, dout, lse, Dv, meta, srec, rnorm, part, dq, dv, st);
    return go<64>(P, q, v, dout, lse, Dv, meta, srec, rnorm, part, dq, dv, st);
}

}  // namespace lsh
