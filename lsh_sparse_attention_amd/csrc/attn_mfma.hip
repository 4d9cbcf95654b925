// attn_mfma.hip -- per-round chunked LSH attention, forward and backward, on
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) with direct global-to-LDS loads.
//
// Method: "Reformer: The Efficient Transformer" §2 (attention over chunks of
// the sorted order: each query sees the keys of its own bucket in its own
// chunk and the one before, not after itself; self only as a fallback) and
// App. A (a query attends to the union of its round sets; duplicates are
// masked so each member counts once; per-round outputs are combined by
// logsumexp weights).  Backward with bucket assignment and sort order held
// fixed (no gradient through hashing or sorting, as the Reformer authors
// state in Hacker News thread 22095523).
//
// Round r, query at sorted index s attends to the sorted keys [s - w, s - 1]
// (w = s - win_lo), minus those that belong to its set in an earlier round
// r' < r (the first round that holds a member counts it).  The band needs
// no chunk arithmetic: win_lo carries it.
//
// Dataflow: a workgroup owns 128 consecutive sorted rows of one (batch, head,
// round); the other operand streams through LDS in blocks of 32 sorted rows.
// Rows are fetched by position straight into LDS with global_load_lds_dwordx4
// (no staging registers) into a ring of LDS stages, several blocks ahead of
// the block in use, so that enough bytes are in flight per CU to cover the
// loaded memory latency; each wave waits on its own outstanding loads with
// s_waitcnt vmcnt, and a workgroup barrier (the per-tile kernels) or an LDS
// counter of the waves whose loads have landed (the persistent ones)
// publishes the block.  Two kernel families: for chunk lengths that divide
// 128 (every workload), persistent 8-wave workgroups (one per CU) walk runs
// of consecutive 128-row tiles with an 8-stage ring shared between
// neighbouring tiles (q_stream_kernel, dkv_stream_kernel, below); for other
// chunk lengths, one 4-wave workgroup per
// tile (fwd_kernel, dq_kernel with a 4-stage ring and two workgroups per CU;
// dkv_kernel).  Tiles are stored unpadded with the
// 16-byte chunks of row r XOR-swizzled by r, so that both the row reads
// (ds_read_b128) and the transposed reads (ds_read_b64_tr_b16) spread over
// the LDS banks.  Per-block metadata (inverse key norms, the keys' sorted
// indices in earlier rounds; for the key side also lse, D and the queries'
// windows) comes from tiles that the prep kernel lays out per 32 sorted rows,
// so it arrives with the same kind of contiguous load.
#include "common.hpp"

namespace lsh {
namespace {

constexpr int kRows = 128;     // rows owned by a workgroup
constexpr int kBlk = 32;       // streamed rows per block
constexpr int kThreads = 256;
constexpr int kQStages = 4;     // ring depth of the query-owned kernels (two workgroups per CU)
constexpr int kKvStages = 8;    // blocks resident at once in the key-owned kernel (one workgroup per CU)
constexpr int kRecCache = 1024;           // sorted records of a workgroup's streamed range
constexpr int kMaxEarlier = 13;           // earlier rounds a tile holds (n_hashes <= 14)
constexpr int kKTile = 1024;              // key tile: rn * scale * log2(e) [32] f32, sk[13][32] u16
constexpr int kQTile = 2048;              // query tile: lse2[32], D[32] f32, w[32] u16, (si1, w)[13][32] u16
// In global memory a tile stores only the fields of the nh - 1 earlier rounds
// it can have, rounded up to 256 bytes; in LDS it keeps the full layout
// above, and copies move only that prefix (16 bytes per lane).
__host__ __device__ constexpr int ktile_stride(int nh) { return (128 + 64 * (nh - 1) + 255) & ~255; }
__host__ __device__ constexpr int qtile_stride(int nh) { return (320 + 128 * (nh - 1) + 255) & ~255; }
static_assert(ktile_stride(kMaxEarlier + 1) <= kKTile && qtile_stride(kMaxEarlier + 1) <= kQTile, "tile sizes");
// Per-round bf16 gradient partials, token-major: for token tok (= bh L + pos)
// and round r, the dq, dk rn and dv rows follow one another, so the reduce
// streams one contiguous run of 3 nh rows per token.  Element offset of the
// (tok, r) dq row; dk rn and dv are D and 2 D further on.
__host__ __device__ constexpr size_t part_row(size_t tok, int nh, int r, int D)
{
    return ((tok * (size_t)nh + (size_t)r) * 3) * (size_t)D;
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLazy = 8.0f;             // lazy running-max threshold (log2 units)

#define LDS_AS __attribute__((address_space(3)))

// 16-byte global -> LDS copy (global_load_lds_dwordx4); lane l lands at
// lds_wave_base + 16 l (the base is wave-uniform and goes through M0).  The
// instruction has no register result.  It is issued from inline assembly so
// that the compiler neither orders it against unrelated LDS reads nor drains
// it with its own waits: completion is waited for explicitly with wait_vm,
// followed by a workgroup barrier, before the LDS data is read.
__device__ __forceinline__ void dma16(const void *g, void *lds_wave_base)
{
    const uint32_t lds = (uint32_t)(uintptr_t)((LDS_AS void *)lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// Workgroup barrier that orders memory operations for the compiler only; the
// hardware waits are the explicit wait_vm before it (LDS reads of the previous
// block have been consumed by the time a wave reaches the barrier).
__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's own LDS stores (ds_write) must be
// visible to the other waves; vector-memory loads are not waited for.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait for the oldest block of the ring: n younger blocks (OPS loads each)
// may stay in flight.  n is wave-uniform and at most MAXN.
template <int OPS, int MAXN>
__device__ __forceinline__ void wait_ring(int n)
{
    if constexpr (MAXN == 0) {
        wait_vm<0>();
    } else {
        if (n >= MAXN)
            wait_vm<MAXN * OPS>();
        else
            wait_ring<OPS, MAXN - 1>(n);
    }
}

// element offset of (row, col) in an unpadded D-wide bf16 tile whose 16-byte
// chunks are XOR-swizzled by row
template <int D>
__device__ __forceinline__ int swz(int row, int col)
{
    constexpr int CPR = D / 8;
    return row * D + ((((col >> 3) ^ (row & (CPR - 1)))) << 3) + (col & 7);
}

// A operand (row = tile row c, 8 consecutive columns starting at k0) of a swizzled tile
template <int D>
__device__ __forceinline__ bf16x8_t tile_row(const uint16_t *T, int row, int k0)
{
    return as_bf16x8(ld16(T + swz<D>(row, k0)));
}

// A operand read transposed from a swizzled tile (see tile_t in common.hpp):
// lane (column col0 + l % 32, half h) gets rows 16 j + 4 h + {0..3}, 16 j + 8 + 4 h + {0..3}
template <int D>
__device__ __forceinline__ bf16x8_t tile_tr(const uint16_t *T, int j, int col0, int lane)
{
    const int g = lane / 16, m = lane % 16;
    const int row = 16 * j + 4 * (g / 2) + m / 4;
    const int col = col0 + 16 * (g % 2) + 4 * (m % 4);
    const uint2 a = lds_read_tr16(T + swz<D>(row, col));
    const uint2 b = lds_read_tr16(T + swz<D>(row + 8, col));
    const u32x4_t u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ bf16x8_t pack8(const float *x)
{
    u32x4_t u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]);
    u.w = pack_bf16x2(x[6], x[7]);
    return as_bf16x8(u);
}

// Issue this thread's part of one block: rows [kb, kb + 32) of tensors a and
// b (positions from the record cache) into stage buffers A and B.
template <int D>
__device__ __forceinline__ void dma_rows(const bf16 *__restrict__ a, const bf16 *__restrict__ b, uint16_t *A,
                                         uint16_t *B, const uint32_t *rec, int kb, size_t tok0, int tid, int wave)
// rec[kb + row] is the sorted record of streamed row kb + row (kb relative to the cache start)
{
    constexpr int CPR = D / 8, KPT = D / 64;
    // every record first: the copies are asm statements that LDS reads cannot move past
    size_t off[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int qc = i * kThreads + tid;            // linear 16-byte chunk of the tile
        const int row = qc / CPR, p = qc % CPR;
        const int lc = p ^ (row & (CPR - 1));         // logical chunk stored at physical p
        off[i] = (tok0 + rec_lo(rec[kb + row])) * D + lc * 8;
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int base = (i * kThreads + wave * kWave) * 8;   // elements
        dma16(a + off[i], A + base);
        dma16(b + off[i], B + base);
    }
}

// 1 in each 16-bit half where a and b differ, else 0 (the halves of a sum of
// such values count differing rounds without carrying into each other)
__device__ __forceinline__ uint32_t ne16(uint32_t a, uint32_t b)
{
    const u16x2_t x = __builtin_bit_cast(u16x2_t, a ^ b);
    const u16x2_t one = {1, 1};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(x, one));
}

// packed earlier-round test over 16 scores; ok[e] cleared where the key is in
// the query's set of round rr.  qrec: (si1, w) pairs (query side) and
// skp: key sorted-index pairs, arranged by the caller.
__device__ __forceinline__ void clear_hits(bool (&ok)[16], const uint32_t (&hit)[8])
{
#pragma unroll
    for (int e = 0; e < 16; ++e)
        ok[e] = ok[e] && ((hit[e / 2] >> (16 * (e % 2))) & 0xffffu) == 0u;
}

// ---------------------------------------------------------------------------
// metadata tiles, per 32 sorted rows of each (b, h, round)

// One wave per tile of 32 sorted rows: lanes 0..31 fill the key tile (unless
// ktile is null), lanes 32..63 the query tile (unless qtile is null); every
// field is written as one contiguous run.  Query windows: causal problems
// store w for the tile's round and (s - 1, w) for the earlier ones (the set
// without the query is [s - w, s - 1]); non-causal problems (wmeta not null)
// store w | (hi - s) << 8 for the tile's round (w < 256 and hi - s < 128 as
// chunks are at most 128 rows) and (hi, span + 1) for the earlier ones (the
// set with the query is [hi - span, hi]).
// With bmeta (duplicates counted over buckets) the nh - 1 entries of both
// tiles hold the bucket-run starts of the other rounds (round rr < r, then
// rr + 1), in the key tile's index field and the query tile's first field.
__global__ __launch_bounds__(kThreads) void tile_prep_kernel(int L, int nh, int ntiles, float scale_log2,
                                                             const uint32_t *__restrict__ srec,
                                                             const uint32_t *__restrict__ meta,
                                                             const uint32_t *__restrict__ wmeta,
                                                             const uint32_t *__restrict__ bmeta,
                                                             const float *__restrict__ rnorm,
                                                             const float *__restrict__ lse,
                                                             const float *__restrict__ Dvec,
                                                             uint8_t *__restrict__ ktile, uint8_t *__restrict__ qtile)
{
    const int lane = threadIdx.x % kWave;
    // the tiles of one (b, h) on one XCD: their gathers of that head's
    // records, norms, lse and D then share one L2
    const int tile = xcd_block(blockIdx.x, gridDim.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (tile >= ntiles)
        return;
    const int per = L / kBlk;
    const int blk = tile % per, r = (tile / per) % nh, bh = tile / (per * nh);
    const int k = lane % kBlk;
    const uint32_t rec = srec[((size_t)bh * nh + r) * L + blk * kBlk + k];
    const size_t tok = (size_t)bh * L + rec_lo(rec);
    const int nr = bmeta ? nh - 1 : (r < kMaxEarlier ? r : kMaxEarlier);
    // a token's nh records of one kind, 16 bytes at a time when nh is a
    // multiple of 4 (then they start 16-byte aligned): a gather of 4 records
    // costs one line request instead of four
    auto recs_of = [&](const uint32_t *base, uint32_t (&v)[kMaxEarlier + 3]) __attribute__((always_inline)) {
        const uint32_t *p = base + tok * nh;
        if ((nh & 3) == 0) {
#pragma unroll
            for (int i = 0; i < (kMaxEarlier + 3) / 4; ++i)
                if (4 * i < nh) {
                    const u32x4_t u = ld16(p + 4 * i);
                    v[4 * i] = u.x;
                    v[4 * i + 1] = u.y;
                    v[4 * i + 2] = u.z;
                    v[4 * i + 3] = u.w;
                }
        } else {
#pragma unroll
            for (int i = 0; i < kMaxEarlier + 3; ++i)
                if (i < nh)
                    v[i] = p[i];
        }
    };
    // record of round rr (< r) or, with bmeta, of the other rounds in turn
    auto other = [&](int rr) __attribute__((always_inline)) { return rr < r ? rr : rr + 1; };
    uint32_t mv[kMaxEarlier + 3];
    if (lane < kBlk) {
        if (!ktile)
            return;
        recs_of(bmeta ? bmeta : meta, mv);
        uint8_t *kt = ktile + (size_t)tile * ktile_stride(nh);
        reinterpret_cast<float *>(kt)[k] = rnorm[tok] * scale_log2;
#pragma unroll
        for (int rr = 0; rr < kMaxEarlier; ++rr)
            if (rr < nr)
                reinterpret_cast<uint16_t *>(kt + 128 + 64 * rr)[k] =
                    (uint16_t)(bmeta ? mv[other(rr)] : rec_lo(mv[rr]));
    } else if (qtile) {
        uint8_t *qt = qtile + (size_t)tile * qtile_stride(nh);
        reinterpret_cast<float *>(qt)[k] = lse[tok] * kLog2e;
        reinterpret_cast<float *>(qt + 128)[k] = Dvec[tok];
        if (bmeta) {
            recs_of(bmeta, mv);
            if (wmeta) {
                const uint32_t u = rec_lo(wmeta[tok * nh + r]) - (uint32_t)(blk * kBlk + k);
                reinterpret_cast<uint16_t *>(qt + 256)[k] = (uint16_t)(rec_hi(rec) | (u << 8));
            } else {
                reinterpret_cast<uint16_t *>(qt + 256)[k] = (uint16_t)rec_hi(rec);
            }
#pragma unroll
            for (int rr = 0; rr < kMaxEarlier; ++rr)
                if (rr < nr) {
                    reinterpret_cast<uint16_t *>(qt + 320 + 128 * rr)[k] = (uint16_t)mv[other(rr)];
                    reinterpret_cast<uint16_t *>(qt + 320 + 128 * rr + 64)[k] = 0;
                }
        } else if (wmeta) {
            recs_of(wmeta, mv);
            const uint32_t u = rec_lo(mv[r]) - (uint32_t)(blk * kBlk + k);
            reinterpret_cast<uint16_t *>(qt + 256)[k] = (uint16_t)(rec_hi(rec) | (u << 8));
#pragma unroll
            for (int rr = 0; rr < kMaxEarlier; ++rr)
                if (rr < nr) {
                    const uint32_t x = mv[rr];
                    reinterpret_cast<uint16_t *>(qt + 320 + 128 * rr)[k] = (uint16_t)rec_lo(x);
                    reinterpret_cast<uint16_t *>(qt + 320 + 128 * rr + 64)[k] = (uint16_t)(rec_hi(x) + 1u);
                }
        } else {
            recs_of(meta, mv);
            reinterpret_cast<uint16_t *>(qt + 256)[k] = (uint16_t)rec_hi(rec);
#pragma unroll
            for (int rr = 0; rr < kMaxEarlier; ++rr)
                if (rr < nr) {
                    const uint32_t mr = mv[rr];
                    reinterpret_cast<uint16_t *>(qt + 320 + 128 * rr)[k] = (uint16_t)(rec_lo(mr) - 1u);
                    reinterpret_cast<uint16_t *>(qt + 320 + 128 * rr + 64)[k] = (uint16_t)rec_hi(mr);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// common workgroup prologue: which (b, h, round, row block), and the sorted
// records of the streamed range in LDS

struct Where {
    int r, bh, s0;
};

__device__ __forceinline__ Where where_of(int L, int nh)
{
    const int nblk = L / kRows;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    return Where{(lb / nblk) % nh, lb / (nblk * nh), (lb % nblk) * kRows};
}

// ---------------------------------------------------------------------------
// forward (query-owned)

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(int L, int nh, int maxw, float scale_log2, const bf16 *__restrict__ q,
                                                       const bf16 *__restrict__ v, const uint32_t *__restrict__ meta,
                                                       const uint32_t *__restrict__ srec,
                                                       const uint8_t *__restrict__ ktile,
                                                       bf16 *__restrict__ o_rounds, float *__restrict__ lse_rounds)
{
    constexpr int KPT = D / 64;
    __shared__ __align__(16) uint16_t Ks[kQStages][kBlk * D];
    __shared__ __align__(16) uint16_t Vs[kQStages][kBlk * D];
    __shared__ __align__(16) uint8_t Ts[kQStages][kKTile];
    __shared__ uint32_t krec[kRecCache];
    __shared__ uint32_t qmeta[kThreads / kWave][kMaxEarlier][32];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int h = lane / 32, c = lane % 32;
    const Where W = where_of(L, nh);
    const int r = W.r, bh = W.bh, s0 = W.s0;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;

    // Prologue, two dependent memory round trips: (1) the sorted records of
    // every row the workgroup can touch, [s0 - maxw, s0 + 128) (maxw bounds
    // a window); (2) the first key blocks (straight into LDS) together with
    // this lane's query row and its earlier-round records.
    const int c0 = s0 - min(s0, maxw);
    const int cache_n = s0 + kRows - c0;
    for (int i = tid; i < cache_n; i += kThreads)
        krec[i] = sr[c0 + i];
    wait_vm<0>();
    lds_barrier();
    const int wq0 = s0 + wave * 32;
    const int sq = wq0 + c;
    const uint32_t qrec = krec[sq - c0];
    const int qpos = (int)rec_lo(qrec), qw = (int)rec_hi(qrec);
    const int qlo = sq - qw;
    const int wlo = __builtin_amdgcn_readlane(qlo, 0);
    const int kb_first = (s0 - (int)rec_hi(krec[s0 - c0])) & ~(kBlk - 1);
    const int nblocks = (s0 + kRows - kb_first) / kBlk;
    const uint32_t *kr = krec + (kb_first - c0);
    const int kts = ktile_stride(nh);
    const uint8_t *ktb = ktile + ((size_t)bh * nh + r) * (L / kBlk) * kts;

    auto issue = [&](int b) __attribute__((always_inline)) {
        const int kb = kb_first + b * kBlk, st = b % kQStages;
        dma_rows<D>(q, v, Ks[st], Vs[st], kr, b * kBlk, tok0, tid, wave);
        if (wave == 0 && 16 * lane < kts)
            dma16(ktb + (size_t)(kb / kBlk) * kts + 16 * lane, Ts[st]);
    };
    constexpr int AHEAD = kQStages - 1;
    for (int b = 0; b < AHEAD && b < nblocks; ++b)
        issue(b);

    if (h == 0)
        for (int rr = 0; rr < r; ++rr)
            qmeta[wave][rr][c] = meta[(tok0 + qpos) * nh + rr];
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

    // the register operands and the first blocks are complete before the
    // ring turns, so no wait inside the loop has to cover a register load
    wait_vm<0>();
    for (int b = 0; b < nblocks; ++b) {
        const int younger = min(AHEAD - 1, nblocks - 1 - b);
        if (wave == 0)
            wait_ring<2 * KPT + 1, AHEAD - 1>(younger);
        else
            wait_ring<2 * KPT, AHEAD - 1>(younger);
        block_barrier();
        if (b + AHEAD < nblocks)
            issue(b + AHEAD);
        const int kb = kb_first + b * kBlk, st = b % kQStages;
        // keys [kb, kb+31] against this wave's windows
        if (kb > wq0 || kb + kBlk - 1 < wlo)
            continue;
        const uint16_t *K = Ks[st], *V = Vs[st];
        const float *rnk = reinterpret_cast<const float *>(Ts[st]);
        const uint16_t *skm = reinterpret_cast<const uint16_t *>(Ts[st] + 128);

        // S^T = K Q^T (lane = query c; keys 8 g + 4 h + t)
        f32x16_t sacc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            sacc = mfma32(tile_row<D>(K, c, 16 * ks + 8 * h), qop[ks], sacc);

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
                    const uint2 kp = *reinterpret_cast<const uint2 *>(skm + 32 * rr + 8 * g + 4 * h);
                    hit[2 * g] |= win_hits2(si1p, wp, kp.x);
                    hit[2 * g + 1] |= win_hits2(si1p, wp, kp.y);
                }
            }
            clear_hits(ok, hit);
        }
        float x[16];
        float bm = -INFINITY;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 rn4 = *reinterpret_cast<const float4 *>(rnk + 8 * g + 4 * h);
            const float rn[4] = {rn4.x, rn4.y, rn4.z, rn4.w};   // already times scale log2(e)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[4 * g + t] = ok[4 * g + t] ? sacc[4 * g + t] * rn[t] : -INFINITY;
                bm = fmaxf(bm, x[4 * g + t]);
            }
        }
        bm = max_xor32(bm);
        const bool raise = bm > mrun + kLazy;
        const float mnew = raise ? bm : mrun;
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            x[e] = fast_exp2(x[e] - mref);
            ps += x[e];
        }
        ps = sum_xor32(ps);
        if (__ballot(raise) != 0ull) {
            const float corr = raise ? fast_exp2(mrun - mref) : 1.f;
            lrun *= corr;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                oacc[dt] *= corr;
        }
        lrun += ps;
        mrun = mnew;
        // O^T += V^T P^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8_t pb = pack8(x + 8 * j);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                oacc[dt] = mfma32(tile_tr<D>(V, j, 32 * dt, lane), pb, oacc[dt]);
        }
    }

    const size_t orow = ((size_t)bh * nh + r) * L + qpos;
    const float inv_l = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(oacc[dt][4 * g + 0] * inv_l, oacc[dt][4 * g + 1] * inv_l);
            w.y = pack_bf16x2(oacc[dt][4 * g + 2] * inv_l, oacc[dt][4 * g + 3] * inv_l);
            *reinterpret_cast<uint2 *>(o_rounds + orow * D + 32 * dt + 8 * g + 4 * h) = w;
        }
    if (h == 0)
        lse_rounds[orow] = lrun > 0.f ? (mrun + __log2f(lrun)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
// backward, query side: dq of each round (query-owned, as the forward)
//   p = exp(scale q_i.k_j - lse_i) with the global lse, g = p (dO_i.v_j - D_i),
//   dq_i += scale g k_j = scale g rn_j q_j

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(int L, int nh, int maxw, float scale, const bf16 *__restrict__ q,
                                                      const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                                                      const float *__restrict__ lse, const float *__restrict__ Dvec,
                                                      const uint32_t *__restrict__ meta,
                                                      const uint32_t *__restrict__ srec,
                                                      const uint8_t *__restrict__ ktile, bf16 *__restrict__ dq_part)
{
    constexpr int KPT = D / 64;
    __shared__ __align__(16) uint16_t Ks[kQStages][kBlk * D];
    __shared__ __align__(16) uint16_t Vs[kQStages][kBlk * D];
    __shared__ __align__(16) uint8_t Ts[kQStages][kKTile];
    __shared__ uint32_t krec[kRecCache];
    __shared__ uint32_t qmeta[kThreads / kWave][kMaxEarlier][32];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int h = lane / 32, c = lane % 32;
    const Where W = where_of(L, nh);
    const int r = W.r, bh = W.bh, s0 = W.s0;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;

    // Prologue in two dependent memory round trips, as in the forward.
    const int c0 = s0 - min(s0, maxw);
    const int cache_n = s0 + kRows - c0;
    for (int i = tid; i < cache_n; i += kThreads)
        krec[i] = sr[c0 + i];
    wait_vm<0>();
    lds_barrier();
    const int wq0 = s0 + wave * 32;
    const int sq = wq0 + c;
    const uint32_t qrec = krec[sq - c0];
    const int qpos = (int)rec_lo(qrec), qw = (int)rec_hi(qrec);
    const int qlo = sq - qw;
    const int wlo = __builtin_amdgcn_readlane(qlo, 0);
    const int kb_first = (s0 - (int)rec_hi(krec[s0 - c0])) & ~(kBlk - 1);
    const int nblocks = (s0 + kRows - kb_first) / kBlk;
    const uint32_t *kr = krec + (kb_first - c0);
    const int kts = ktile_stride(nh);
    const uint8_t *ktb = ktile + ((size_t)bh * nh + r) * (L / kBlk) * kts;

    auto issue = [&](int b) __attribute__((always_inline)) {
        const int kb = kb_first + b * kBlk, st = b % kQStages;
        dma_rows<D>(q, v, Ks[st], Vs[st], kr, b * kBlk, tok0, tid, wave);
        if (wave == 0 && 16 * lane < kts)
            dma16(ktb + (size_t)(kb / kBlk) * kts + 16 * lane, Ts[st]);
    };
    constexpr int AHEAD = kQStages - 1;
    for (int b = 0; b < AHEAD && b < nblocks; ++b)
        issue(b);

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

    // the register operands and the first blocks are complete before the
    // ring turns, so no wait inside the loop has to cover a register load
    wait_vm<0>();
    for (int b = 0; b < nblocks; ++b) {
        const int younger = min(AHEAD - 1, nblocks - 1 - b);
        if (wave == 0)
            wait_ring<2 * KPT + 1, AHEAD - 1>(younger);
        else
            wait_ring<2 * KPT, AHEAD - 1>(younger);
        block_barrier();
        if (b + AHEAD < nblocks)
            issue(b + AHEAD);
        const int kb = kb_first + b * kBlk, st = b % kQStages;
        if (kb > wq0 || kb + kBlk - 1 < wlo)
            continue;
        const uint16_t *K = Ks[st], *V = Vs[st];
        const float *rnk = reinterpret_cast<const float *>(Ts[st]);
        const uint16_t *skm = reinterpret_cast<const uint16_t *>(Ts[st] + 128);

        // S^T = K Q^T and dP^T = V dO^T (lane = query c, keys 8 g + 4 h + t)
        f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            sacc = mfma32(tile_row<D>(K, c, 16 * ks + 8 * h), qop[ks], sacc);
            pacc = mfma32(tile_row<D>(V, c, 16 * ks + 8 * h), gop[ks], pacc);
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
                    const uint2 kp = *reinterpret_cast<const uint2 *>(skm + 32 * rr + 8 * g + 4 * h);
                    hit[2 * g] |= win_hits2(si1p, wp, kp.x);
                    hit[2 * g + 1] |= win_hits2(si1p, wp, kp.y);
                }
            }
            clear_hits(ok, hit);
        }
        float gs[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 rn4 = *reinterpret_cast<const float4 *>(rnk + 8 * g + 4 * h);
            const float rn[4] = {rn4.x, rn4.y, rn4.z, rn4.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = 4 * g + t;
                const float pr = ok[e] ? fast_exp2(fmaf(sacc[e], rn[t], -lse2)) : 0.f;
                gs[e] = pr * (pacc[e] - Di) * (rn[t] * kLn2);
            }
        }
        // dQ^T += K^T Gs^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8_t gb = pack8(gs + 8 * j);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = mfma32(tile_tr<D>(K, j, 32 * dt, lane), gb, acc[dt]);
        }
    }

    bf16 *out = dq_part + part_row(bh * L + qpos, nh, r, D);
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
// backward, key side: dk and dv of each round (key-owned; queries stream)
//   dv_j += p dO_i,  dk_j += scale g q_i,  S = Q K^T and dP = dO V^T with lane = key.
// Runs on v_mfma_f32_16x16x32_bf16 with 16 keys per wave and 8 waves per
// workgroup (128 keys), which halves the per-lane dK^T / dV^T accumulators
// of a 32-key wave so that two waves fit on a SIMD.
// 16x16x32 operands: lane l supplies A[l%16][8(l/16) .. +7] and B[8(l/16) .. +7][l%16];
// it receives C[4(l/16) + t][l%16] in acc[t].

constexpr int kKvThreads = 512;

// A operand (16 rows d = col0 + l%16, 8 queries) read transposed from a
// swizzled tile: lane group g gets rows 4 g .. 4 g + 3 and 16 + 4 g .. + 3,
// matching a B operand made of accumulator values (half 0: t = 0..3, half 1: t = 0..3).
template <int D>
__device__ __forceinline__ bf16x8_t tile_tr16x(const uint16_t *T, int col0, int lane)
{
    const int g = lane / 16, m = lane % 16;
    const int row = 4 * g + m / 4;
    const int col = col0 + 4 * (m % 4);
    const uint2 a = lds_read_tr16(T + swz<D>(row, col));
    const uint2 b = lds_read_tr16(T + swz<D>(row + 16, col));
    const u32x4_t u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8_t, u);
}

// This thread's part of one query block for 512 threads: rows [qb, qb + 32)
// of a (chunks 0 .. 4D-1) then of b (4D .. 8D-1); a wave's 64 chunks stay
// within one tensor.
template <int D>
__device__ __forceinline__ void dma_rows512(const bf16 *__restrict__ a, const bf16 *__restrict__ b, uint16_t *A,
                                            uint16_t *B, const uint32_t *rec, int qb, size_t tok0, int tid, int wave)
{
    constexpr int CPR = D / 8, PER = 8 * D / kKvThreads, TCH = 4 * D;
    size_t off[PER];   // records first (see dma_rows)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int cc = (i * kKvThreads + tid) % TCH;
        const int row = cc / CPR, p = cc % CPR;
        const int lc = p ^ (row & (CPR - 1));
        off[i] = (tok0 + rec_lo(rec[qb + row])) * D + lc * 8;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int qc = i * kKvThreads + tid;
        const int base = ((i * kKvThreads + wave * kWave) % TCH) * 8;
        if (qc / TCH == 0)
            dma16(a + off[i], A + base);
        else
            dma16(b + off[i], B + base);
    }
}

// One wave loads one tensor of a block: rows [0, 32) of a (positions from
// rec) into the swizzled tile A, D/16 instructions.
template <int D, int G = kBlk * D / 8 / kWave>
__device__ __forceinline__ void dma_tensor_wave(const bf16 *__restrict__ a, uint16_t *A, const uint32_t *rec,
                                                size_t tok0, int lane)
{
    constexpr int CPR = D / 8, N = kBlk * CPR / kWave;
    const bf16 *base = a + tok0 * D;   // the (b, h) slice: offsets within it fit 32 bits
    // records first (see dma_rows), G rows' worth at a time
#pragma unroll
    for (int i0 = 0; i0 < N; i0 += G) {
        uint32_t off[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int qc = (i0 + i) * kWave + lane;
            const int row = qc / CPR, p = qc % CPR;
            const int lc = p ^ (row & (CPR - 1));
            off[i] = rec_lo(rec[row]) * (uint32_t)D + lc * 8;
        }
#pragma unroll
        for (int i = 0; i < G; ++i)
            dma16(base + off[i], A + (i0 + i) * kWave * 8);
    }
}

template <int D>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkv_kernel(
    int L, int nh, float scale, const bf16 *__restrict__ q, const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
    const uint32_t *__restrict__ srec, const uint8_t *__restrict__ ktile, const uint8_t *__restrict__ qtile,
    bf16 *__restrict__ dkr_part, bf16 *__restrict__ dv_part)
{
    __shared__ __align__(16) uint16_t Qs[kKvStages][kBlk * D];
    __shared__ __align__(16) uint16_t Gs[kKvStages][kBlk * D];   // dO rows
    __shared__ __align__(16) uint8_t Ts[kKvStages][kQTile];
    __shared__ __align__(16) uint8_t Kt[kRows / kBlk][kKTile];    // key tiles of the owned keys
    __shared__ uint32_t qrecs[kRecCache];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int g = lane / 16, c = lane % 16;
    const Where W = where_of(L, nh);
    const int r = W.r, bh = W.bh, k0 = W.s0;
    const uint32_t *sr = srec + ((size_t)bh * nh + r) * L;
    const size_t tok0 = (size_t)bh * L;
    const int kts = ktile_stride(nh), qts = qtile_stride(nh);
    const uint8_t *qtb = qtile + ((size_t)bh * nh + r) * (L / kBlk) * qts;

    // Prologue, two dependent memory round trips: (1) the sorted records of
    // the streamed range and the key tiles of the owned keys; (2) the query
    // blocks (straight into LDS) together with this lane's key and value rows.
    if (wave < kRows / kBlk && 16 * lane < kts)
        dma16(ktile + (((size_t)bh * nh + r) * (L / kBlk) + k0 / kBlk + wave) * kts + 16 * lane, Kt[wave]);
    const int cache_n = min(L - k0, kRecCache);
    for (int i = tid; i < cache_n; i += kKvThreads)
        qrecs[i] = sr[k0 + i];
    wait_vm<0>();
    lds_barrier();

    const int wk0 = k0 + wave * 16;
    const int sk = wk0 + c;                       // this lane's key (sorted)
    const int kpos = (int)rec_lo(qrecs[sk - k0]);
    const uint8_t *kt = Kt[wave / 2];             // this wave's 16 keys are entries 16 (wave % 2) + c
    const int ke = 16 * (wave % 2) + c;
    const float krn2 = reinterpret_cast<const float *>(kt)[ke];   // rn * scale * log2(e)
    const float rn = krn2 / (scale * kLog2e);
    // query blocks [k0 + 32 b, +32) whose first query's window reaches the owned keys
    // (window starts do not decrease along the sorted order)
    const int k_last = k0 + kRows - 1;
    const int nblocks = __builtin_popcountll(__ballot(kBlk * lane < cache_n &&
                                                      k0 + kBlk * lane - (int)rec_hi(qrecs[min(kBlk * lane, cache_n - 1)]) <= k_last));

    auto issue = [&](int b, int st) __attribute__((always_inline)) {
        const int qb = k0 + b * kBlk;
        dma_rows512<D>(q, dout, Qs[st], Gs[st], qrecs, b * kBlk, tok0, tid, wave);
        if (wave < 2 && 1024 * wave + 16 * lane < qts)
            dma16(qtb + (size_t)(qb / kBlk) * qts + 1024 * wave + 16 * lane, Ts[st] + 1024 * wave);
    };
    for (int i = 0; i < kKvStages && i < nblocks; ++i)
        issue(i, i);

    bf16x8_t kop[D / 32], vop[D / 32];
    {
        const bf16 *krow = q + (tok0 + kpos) * D, *vrow = v + (tok0 + kpos) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            kop[ks] = as_bf16x8(ld16(krow + 32 * ks + 8 * g));
            vop[ks] = as_bf16x8(ld16(vrow + 32 * ks + 8 * g));
        }
    }

    f32x4_t dka[D / 16], dva[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        dka[dt] = dva[dt] = f32x4_t{};

    // Blocks are loaded kKvStages at a time (every block of the window at
    // once when 128 + 2 m <= 32 kKvStages); a wave then works through the
    // blocks that reach its keys without waiting for the other waves.
    for (int base = 0; base < nblocks; base += kKvStages) {
        const int nb = min(kKvStages, nblocks - base);
        if (base > 0) {
            block_barrier();                      // the previous group's stages are no longer read
            for (int i = 0; i < nb; ++i)
                issue(base + i, i);
        }
        wait_vm<0>();
        block_barrier();
        for (int i = 0; i < nb; ++i) {
            const int b = base + i, qb = k0 + b * kBlk;
            const uint16_t *Qt = Qs[i], *Gt = Gs[i];
            const float *qlse2 = reinterpret_cast<const float *>(Ts[i]);
            const float *qD = reinterpret_cast<const float *>(Ts[i] + 128);
            const uint16_t *qwv = reinterpret_cast<const uint16_t *>(Ts[i] + 256);
            // this wave's keys [wk0, wk0+15]: queries after a key whose window reaches it
            const int blk_lo = qb - (int)rec_hi(qrecs[b * kBlk]);
            if (qb + kBlk - 1 <= wk0 || blk_lo > wk0 + 15)
                continue;

            // S = Q K^T, dP = dO V^T for the two 16-query halves (lane = key c;
            // value t of half u is query 16 u + 4 g + t).  All operand reads
            // are issued before the first product so their latencies overlap.
            bf16x8_t qa[2][D / 32], ga[2][D / 32];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    qa[u][ks] = tile_row<D>(Qt, 16 * u + c, 32 * ks + 8 * g);
                    ga[u][ks] = tile_row<D>(Gt, 16 * u + c, 32 * ks + 8 * g);
                }
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t sacc[2], pacc[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                sacc[u] = pacc[u] = f32x4_t{};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    sacc[u] = mfma16(qa[u][ks], kop[ks], sacc[u]);
                    pacc[u] = mfma16(ga[u][ks], vop[ks], pacc[u]);
                }
            }
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint2 w4 = *reinterpret_cast<const uint2 *>(qwv + 16 * u + 4 * g);
                const int wv[4] = {(int)(w4.x & 0xffffu), (int)(w4.x >> 16), (int)(w4.y & 0xffffu), (int)(w4.y >> 16)};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int sq = qb + 16 * u + 4 * g + t;   // key in [sq - w, sq)
                    ok[4 * u + t] = (unsigned)(sk - sq + wv[t]) < (unsigned)wv[t];
                }
            }
            if (r > 0) {
                uint32_t hit[4] = {0u, 0u, 0u, 0u};
                for (int rr = 0; rr < r; ++rr) {
                    const uint32_t skp = bcast16(reinterpret_cast<const uint16_t *>(kt + 128 + 64 * rr)[ke]);
                    const uint16_t *s1 = reinterpret_cast<const uint16_t *>(Ts[i] + 320 + 128 * rr);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const uint2 a = *reinterpret_cast<const uint2 *>(s1 + 16 * u + 4 * g);
                        const uint2 ww = *reinterpret_cast<const uint2 *>(s1 + 32 + 16 * u + 4 * g);
                        hit[2 * u] |= win_hits2(a.x, ww.x, skp);
                        hit[2 * u + 1] |= win_hits2(a.y, ww.y, skp);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ok[e] = ok[e] && ((hit[e / 2] >> (16 * (e % 2))) & 0xffffu) == 0u;
            }
            float pr[8], gr[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float4 l4 = *reinterpret_cast<const float4 *>(qlse2 + 16 * u + 4 * g);
                const float4 d4 = *reinterpret_cast<const float4 *>(qD + 16 * u + 4 * g);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int e = 4 * u + t;
                    pr[e] = ok[e] ? fast_exp2(sacc[u][t] * krn2 - lv[t]) : 0.f;
                    gr[e] = pr[e] * (pacc[u][t] - dv[t]) * scale;
                }
            }
            // dV^T += dO^T P, dK^T += Q^T G: B slot s is value s of pr / gr
            const bf16x8_t pb = pack8(pr), gb = pack8(gr);
            bf16x8_t gt[D / 16], qt[D / 16];
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                gt[dt] = tile_tr16x<D>(Gt, 16 * dt, lane);
                qt[dt] = tile_tr16x<D>(Qt, 16 * dt, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                dva[dt] = mfma16(gt[dt], pb, dva[dt]);
                dka[dt] = mfma16(qt[dt], gb, dka[dt]);
            }
        }
    }

    // dk of this round times the key's inverse norm; the projection through
    // the normalisation k = q rn is linear, so it is applied once to the sum
    // over rounds (reduce_kernel).  Lane (key c, group g) holds d = 16 dt + 4 g + t.
    const size_t row = part_row(bh * L + kpos, nh, r, D);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const int d0 = 16 * dt + 4 * g;
        uint2 w;
        w.x = pack_bf16x2(dka[dt][0] * rn, dka[dt][1] * rn);
        w.y = pack_bf16x2(dka[dt][2] * rn, dka[dt][3] * rn);
        *reinterpret_cast<uint2 *>(dkr_part + row + d0) = w;
        w.x = pack_bf16x2(dva[dt][0], dva[dt][1]);
        w.y = pack_bf16x2(dva[dt][2], dva[dt][3]);
        *reinterpret_cast<uint2 *>(dv_part + row + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// backward, key side, persistent form for chunk lengths that divide 128.
//
// A key tile [k0, k0 + 128) is then reached only by queries in [k0, k0 + 256)
// (a key is seen from its own chunk and the next one), i.e. by query blocks
// k0/32 + 0..7, and the next tile needs this tile's blocks 4..7 plus four new
// ones.  A workgroup walks a run of consecutive tiles of one (b, h, round)
// with those eight blocks resident in LDS stages indexed by absolute block
// mod 8.  Once the waves are through blocks 0..3 of a tile, the freed stages
// receive the next tile's new blocks while blocks 4..7 are worked on, so the
// loads of tile j+1 overlap the work of tile j.  The owned keys' rows come
// from the resident query blocks (shared QK); their value rows are loaded
// one tile ahead into registers; per-32-row key tiles and the sorted
// records arrive by the same direct-to-LDS loads.
//
// The waves do not meet at a workgroup barrier.  Two LDS counters per tile
// parity: waves through blocks 0..3, and waves whose share of the loads
// issued in the tile has landed.  The wave that completes the first count
// issues its share at once, the others at the tile's end (checking after
// each of blocks 4..7 as well costs the d = 128 kernel spills inside the
// loop); a wave waits for the second count of the previous tile before its
// blocks 4..7.

constexpr int kStreamStages = 8;
constexpr int kRecRing = 512;                 // records of sorted rows x at x mod 512

// Whether the key's sorted indices in the NR earlier rounds stay in
// registers for a tile (else they are read from the key tile per block).
template <int D, int NR>
constexpr bool kv_sk_in_regs() { return D < 128 || NR <= 3; }
// the same under the bucket duplicate count, whose divisor arithmetic needs
// more registers at d = 128
template <int D, int NR, bool DUPB>
constexpr bool kv_sk_regs() { return DUPB ? D < 128 : kv_sk_in_regs<D, NR>(); }

// One query block against this wave's 16 keys.  The queries' windows, lse
// and D are read with the operand rows, before any arithmetic.  skp[rr]:
// this lane's key's sorted index in round rr (NR >= r), both halves of a
// pair, or (see kv_sk_regs) entry ke of the key tile kt.  MODE: the kind
// of set (SetKind; kRange and kRangePos use the range layout of the query
// tile, kRangePos also compares positions: qrec are the block's 32 sorted
// records, kpos the lane's key position).
// DUPB: duplicates weighed by the shared-bucket count (the nh - 1 tile
// entries are bucket-run starts of the other rounds) instead of the
// first-owner mask.
template <int D, int NR, int MODE, bool DUPB>
__device__ __forceinline__ void dkv_block(const uint16_t *Qt, const uint16_t *Gt, const uint8_t *T, const uint8_t *kt,
                                          const uint32_t *qrec, int kpos, int ke, int r, int nh, int qb, int sk, int g,
                                          int c, int lane, float krn2,
                                          float scale, const uint32_t (&skp)[NR], const bf16x8_t (&kop)[D / 32],
                                          const bf16x8_t (&vop)[D / 32], f32x4_t (&dka)[D / 16],
                                          f32x4_t (&dva)[D / 16])
{
    const float *qlse2 = reinterpret_cast<const float *>(T);
    const float *qD = reinterpret_cast<const float *>(T + 128);
    const uint16_t *qwv = reinterpret_cast<const uint16_t *>(T + 256);
    bf16x8_t qa[2][D / 32], ga[2][D / 32];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            qa[u][ks] = tile_row<D>(Qt, 16 * u + c, 32 * ks + 8 * g);
            ga[u][ks] = tile_row<D>(Gt, 16 * u + c, 32 * ks + 8 * g);
        }
    constexpr bool NC = MODE != kBand;
    uint2 w4[2];
    float4 l4[2], d4[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        w4[u] = *reinterpret_cast<const uint2 *>(qwv + 16 * u + 4 * g);
        l4[u] = *reinterpret_cast<const float4 *>(qlse2 + 16 * u + 4 * g);
        d4[u] = *reinterpret_cast<const float4 *>(qD + 16 * u + 4 * g);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t sacc[2], pacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        sacc[u] = pacc[u] = f32x4_t{};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            sacc[u] = mfma16(qa[u][ks], kop[ks], sacc[u]);
            pacc[u] = mfma16(ga[u][ks], vop[ks], pacc[u]);
        }
    }
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int wv[4] = {(int)(w4[u].x & 0xffffu), (int)(w4[u].x >> 16), (int)(w4[u].y & 0xffffu),
                           (int)(w4[u].y >> 16)};
        uint4 p4{};   // the queries' records (positions), kRangePos only: read after the products
        if constexpr (MODE == kRangePos)
            p4 = *reinterpret_cast<const uint4 *>(qrec + 16 * u + 4 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int sq = qb + 16 * u + 4 * g + t;
            if constexpr (NC) {
                // key in [sq - w, sq + hi - sq], not the query itself (and,
                // kRangePos, not after it)
                const int w = wv[t] & 0xff, n = w + (wv[t] >> 8) + 1;
                ok[4 * u + t] = (unsigned)(sk - sq + w) < (unsigned)n && sk != sq;
                if constexpr (MODE == kRangePos) {
                    const uint32_t pr4[4] = {p4.x, p4.y, p4.z, p4.w};
                    ok[4 * u + t] = ok[4 * u + t] && (uint32_t)kpos < rec_lo(pr4[t]);
                }
            } else {
                // key in [sq - w, sq)
                ok[4 * u + t] = (unsigned)(sk - sq + wv[t]) < (unsigned)wv[t];
            }
        }
    }
    // DUPB: rounds in which a query's bucket differs from the key's, per
    // 16-bit half (score e in half e % 2 of dif[e / 2])
    uint32_t dif[4] = {0u, 0u, 0u, 0u};
    if (DUPB ? nh > 1 : r > 0) {
        uint32_t hit[4] = {0u, 0u, 0u, 0u};
        const int nrec = DUPB ? nh - 1 : r;
        if constexpr (kv_sk_regs<D, NR, DUPB>()) {
            // the queries' (start - 1, length) pairs of every round rr < NR,
            // read without a branch so that they go out together (pairs of
            // rounds rr >= r lie within the LDS tile and are not used)
            uint2 qa1[NR][2], qww[NR][2];
#pragma unroll
            for (int rr = 0; rr < NR; ++rr)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint16_t *s1 = reinterpret_cast<const uint16_t *>(T + 320 + 128 * rr);
                    qa1[rr][u] = *reinterpret_cast<const uint2 *>(s1 + 16 * u + 4 * g);
                    if constexpr (!DUPB)   // DUPB uses the first field only
                        qww[rr][u] = *reinterpret_cast<const uint2 *>(s1 + 32 + 16 * u + 4 * g);
                }
#pragma unroll
            for (int rr = 0; rr < NR; ++rr)
                if (rr < nrec) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        if constexpr (DUPB) {
                            hit[2 * u] += ne16(qa1[rr][u].x, skp[rr]);
                            hit[2 * u + 1] += ne16(qa1[rr][u].y, skp[rr]);
                        } else {
                            hit[2 * u] |= win_hits2(qa1[rr][u].x, qww[rr][u].x, skp[rr]);
                            hit[2 * u + 1] |= win_hits2(qa1[rr][u].y, qww[rr][u].y, skp[rr]);
                        }
                    }
                }
        } else {
#pragma unroll
            for (int rr = 0; rr < NR; ++rr)
                if (rr < nrec) {
                    const uint32_t kp = bcast16(reinterpret_cast<const uint16_t *>(kt + 128 + 64 * rr)[ke]);
                    // the queries' (start - 1, length) pairs in round rr
                    const uint16_t *s1 = reinterpret_cast<const uint16_t *>(T + 320 + 128 * rr);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const uint2 a = *reinterpret_cast<const uint2 *>(s1 + 16 * u + 4 * g);
                        if constexpr (DUPB) {
                            hit[2 * u] += ne16(a.x, kp);
                            hit[2 * u + 1] += ne16(a.y, kp);
                        } else {
                            const uint2 ww = *reinterpret_cast<const uint2 *>(s1 + 32 + 16 * u + 4 * g);
                            hit[2 * u] |= win_hits2(a.x, ww.x, kp);
                            hit[2 * u + 1] |= win_hits2(a.y, ww.y, kp);
                        }
                    }
                }
        }
        if constexpr (DUPB) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dif[k] = hit[k];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ok[e] = ok[e] && ((hit[e / 2] >> (16 * (e % 2))) & 0xffffu) == 0u;
        }
    }
    float pr[8], gr[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float lv[4] = {l4[u].x, l4[u].y, l4[u].z, l4[u].w}, dv[4] = {d4[u].x, d4[u].y, d4[u].z, d4[u].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int e = 4 * u + t;
            // log2 of the duplicate divisor: the rounds sharing the bucket
            const float lg = DUPB ? __log2f((float)(nh - (int)((dif[e / 2] >> (16 * (e % 2))) & 0xffffu))) : 0.f;
            pr[e] = ok[e] ? fast_exp2(sacc[u][t] * krn2 - lv[t] - lg) : 0.f;
            gr[e] = pr[e] * (pacc[u][t] - dv[t]) * scale;
        }
    }
    const bf16x8_t pb = pack8(pr), gb = pack8(gr);
    bf16x8_t gt[D / 16], qt[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        gt[dt] = tile_tr16x<D>(Gt, 16 * dt, lane);
        qt[dt] = tile_tr16x<D>(Qt, 16 * dt, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        dva[dt] = mfma16(gt[dt], pb, dva[dt]);
        dka[dt] = mfma16(qt[dt], gb, dka[dt]);
    }
}

// Stores one row of 16x16-MFMA accumulators times sc in bf16: lane (row c,
// group g) holds d = 16 dt + 4 g + t.  Lanes g and g ^ 1 trade half of a pair
// of d-groups (v_permlane16_swap: the odd row of the first operand with the
// even row of the second), so each lane writes 8 consecutive d with one
// 16-byte store and a row gets 64 contiguous bytes per instruction: g even
// keeps group 2 dp and takes its partner's half of it, g odd takes the
// partner's half of group 2 dp + 1.
template <int D>
__device__ __forceinline__ void store_row16(bf16 *row, int g, float sc, const f32x4_t (&acc)[D / 16])
{
    const bool odd = g & 1;
#pragma unroll
    for (int dp = 0; dp < D / 32; ++dp) {
        const uint32_t u0 = pack_bf16x2(acc[2 * dp][0] * sc, acc[2 * dp][1] * sc);
        const uint32_t u1 = pack_bf16x2(acc[2 * dp][2] * sc, acc[2 * dp][3] * sc);
        const uint32_t u2 = pack_bf16x2(acc[2 * dp + 1][0] * sc, acc[2 * dp + 1][1] * sc);
        const uint32_t u3 = pack_bf16x2(acc[2 * dp + 1][2] * sc, acc[2 * dp + 1][3] * sc);
        const auto p = __builtin_amdgcn_permlane16_swap(u0, u2, false, false);
        const auto q = __builtin_amdgcn_permlane16_swap(u1, u3, false, false);
        const u32x4_t w = odd ? u32x4_t{p[0], q[0], u2, u3} : u32x4_t{u0, u1, p[1], q[1]};
        st16(row + 32 * dp + 16 * (g & 1) + 8 * (g >> 1), w);
    }
}

// stores dk rn and dv of one key (lane: key c, d = 16 dt + 4 g + t)
template <int D>
__device__ __forceinline__ void dkv_store(bf16 *dkr_part, bf16 *dv_part, size_t row, int g, float rn,
                                          const f32x4_t (&dka)[D / 16], const f32x4_t (&dva)[D / 16])
{
    store_row16<D>(dkr_part + row, g, rn, dka);
    store_row16<D>(dv_part + row, g, 1.f, dva);
}

template <int D, int NR, int MODE, bool DUPB>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkv_stream_kernel(
    int L, int nh, int T, int m, float scale, const bf16 *__restrict__ q, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const uint32_t *__restrict__ srec, const uint8_t *__restrict__ ktile,
    const uint8_t *__restrict__ qtile, bf16 *__restrict__ dkr_part, bf16 *__restrict__ dv_part)
{
    __shared__ __align__(16) uint16_t Qs[kStreamStages][kBlk * D];
    __shared__ __align__(16) uint16_t Gs[kStreamStages][kBlk * D];   // dO rows
    __shared__ __align__(16) uint8_t Ts[kStreamStages][kQTile];
    __shared__ __align__(16) uint8_t Kt[3][kRows / kBlk][kKTile];     // key tiles, two tiles ahead
    __shared__ __align__(16) uint32_t recs[kRecRing];
    // per tile parity, monotonic, 8 per tile: waves through blocks 0..3 of
    // their tile, and waves whose share of the loads issued in that tile
    // has landed
    __shared__ uint32_t through[2], loaded[2];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int g = lane / 16, c = lane % 16;
    // 16-key group of this wave: waves w and w + 4 share a SIMD, and the
    // early key groups (reached by more query blocks) pair with late ones
    const int kg = wave < 4 ? wave : 11 - wave;
    const int nt = L / kRows, nblk = L / kBlk;
    const int rps = (nt + T - 1) / T;                      // runs per (b, h, round)
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    // rounds in descending order within a (b, h): see stream_run_tiles
    const int run = lb % rps, r = nh - 1 - (lb / rps) % nh, bh = (lb / rps) / nh;
    const int seg = bh * nh + r;
    const int t_begin = run * T, t_end = min(nt, t_begin + T);
    const uint32_t *sr = srec + (size_t)seg * L;
    const size_t tok0 = (size_t)bh * L;
    const int kts = ktile_stride(nh), qts = qtile_stride(nh);
    const uint8_t *qtb = qtile + (size_t)seg * nblk * qts;
    const uint8_t *ktb = ktile + (size_t)seg * nblk * kts;
    const float inv_sl2 = 1.f / (scale * kLog2e);

    // absolute query block a: its rows of q and dO, and its query tile
    auto issue_block = [&](int a) __attribute__((always_inline)) {
        const int st = a % kStreamStages;
        dma_rows512<D>(q, dout, Qs[st], Gs[st], recs + (a * kBlk) % kRecRing, 0, tok0, tid, wave);
        if (wave < 2 && 1024 * wave + 16 * lane < qts)
            dma16(qtb + (size_t)a * qts + 1024 * wave + 16 * lane, Ts[st] + 1024 * wave);
    };
    // key tiles of tile t into buffer buf (waves 2..5, one 32-row tile each)
    auto issue_ktiles = [&](int t, int buf) __attribute__((always_inline)) {
        if (wave >= 2 && wave < 6 && 16 * lane < kts)
            dma16(ktb + ((size_t)t * (kRows / kBlk) + (wave - 2)) * kts + 16 * lane, Kt[buf][wave - 2]);
    };
    // records of rows [row0, row0 + 128) (row0 a multiple of 128), by wave wv
    auto issue_recs = [&](int row0, int wv) __attribute__((always_inline)) {
        if (wave == wv && lane < kRows / 4)
            dma16(sr + row0 + 4 * lane, recs + row0 % kRecRing);
    };

    // prologue: records of the first tile's window and the one after, the
    // key tiles of the first two tiles; then the first tile's eight query
    // blocks and the value rows of its keys
    if (tid < 2) {
        through[tid] = 0u;
        loaded[tid] = 0u;
    }
    {
        const int k0 = t_begin * kRows;
        issue_recs(k0, 6);
        if (k0 + kRows < L)
            issue_recs(k0 + kRows, 7);
        if (k0 + 2 * kRows < L)
            issue_recs(k0 + 2 * kRows, 6);
        issue_ktiles(t_begin, 0);
        if (t_begin + 1 < t_end)
            issue_ktiles(t_begin + 1, 1);
        wait_vm<0>();
        block_barrier();
        for (int i = 0; i < kStreamStages; ++i)
            if (k0 / kBlk + i < nblk)
                issue_block(k0 / kBlk + i);
    }
    bf16x8_t vop[D / 32];
    {
        const int kpos = (int)rec_lo(recs[(t_begin * kRows + kg * 16 + c) % kRecRing]);
        const bf16 *vrow = v + (tok0 + kpos) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            vop[ks] = as_bf16x8(ld16(vrow + 32 * ks + 8 * g));
    }
    wait_vm<0>();
    block_barrier();

    f32x4_t dka[D / 16], dva[D / 16];
    int kpos_prev = 0;
    float rn_prev = 0.f;
    // this wave's last share, not yet counted as landed: it is (after a
    // wait for the wave's loads) kSettle blocks after its issue, or at the
    // latest before the wave waits for the others' shares or issues another
    bool due = false;
    int due_slot = 0, since = 0;
    constexpr int kSettle = 2;
    auto settle = [&](bool now) __attribute__((always_inline)) {
        if (due && (now || ++since >= kSettle)) {
            wait_vm<0>();
            if (lane == 0)
                atomicAdd(&loaded[due_slot], 1u);
            due = false;
        }
    };
    for (int t = t_begin; t < t_end; ++t) {
        const int k0 = t * kRows, a0 = k0 / kBlk, j = t - t_begin;
        if (t > t_begin)
            dkv_store<D>(dkr_part, dv_part, part_row(tok0 + kpos_prev, nh, r, D), g, rn_prev, dka, dva);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            dka[dt] = dva[dt] = f32x4_t{};

        const int sk = k0 + kg * 16 + c;                      // this lane's key (sorted)
        const int kpos = (int)rec_lo(recs[sk % kRecRing]);
        const uint8_t *kt = Kt[j % 3][kg / 2];                // entries 16 (kg % 2) + c
        const int ke = 16 * (kg % 2) + c;
        const float krn2 = reinterpret_cast<const float *>(kt)[ke];   // rn * scale * log2(e)
        const float rn = krn2 * inv_sl2;
        uint32_t skp[NR];   // the key's sorted index in the earlier rounds
        if constexpr (kv_sk_regs<D, NR, DUPB>()) {
            // read for every rr < NR without a branch, so the reads go out
            // together (entries rr >= r are within the LDS tile and unused)
#pragma unroll
            for (int rr = 0; rr < NR; ++rr)
                skp[rr] = bcast16(reinterpret_cast<const uint16_t *>(kt + 128 + 64 * rr)[ke]);
        }
        bf16x8_t kop[D / 32];
        {
            const uint16_t *Kq = Qs[(a0 + kg / 2) % kStreamStages];
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                kop[ks] = tile_row<D>(Kq, ke, 32 * ks + 8 * g);
        }
        // query blocks whose first query's window reaches the tile (window
        // starts do not decrease along the sorted order)
        const int x = k0 + kBlk * lane;
        const int nb = __builtin_popcountll(__ballot(lane < kStreamStages && x < L &&
                                                     x - (int)rec_hi(recs[min(x, L - 1) % kRecRing]) <= k0 + kRows - 1));
        const int wk0 = k0 + kg * 16;
        auto work = [&](int b) __attribute__((always_inline)) {
            const int qb = k0 + b * kBlk, st = (a0 + b) % kStreamStages;
            const int blk_lo = qb - (int)rec_hi(recs[qb % kRecRing]);
            // causal: a block entirely at or before the keys sees none of
            // them; non-causal: one entirely before the chunk of the first key
            // (m is a power of two)
            const bool before = MODE != kBand ? qb + kBlk - 1 < (wk0 & -m) : qb + kBlk - 1 <= wk0;
            if (before || blk_lo > wk0 + 15)
                return;
            dkv_block<D, NR, MODE, DUPB>(Qs[st], Gs[st], Ts[st], kt, recs + qb % kRecRing, kpos, ke, r, nh, qb, sk, g,
                                         c, lane, krn2, scale, skp, kop, vop, dka, dva);
        };
        // raised wave priority while the blocks that gate the next loads are
        // worked on (see q_stream_kernel)
        __builtin_amdgcn_s_setprio(2);
        for (int b = 0; b < 4 && b < nb; ++b) {
            work(b);
            settle(false);
        }
        __builtin_amdgcn_s_setprio(0);
        // Once every wave is through blocks 0..3 (and so through the
        // previous tile), their stages, the key-tile buffer of the previous
        // tile and its records take this tile's loads for the next two
        // tiles, each wave issuing its share: one tensor of one block.
        const uint32_t goal = 8u * (uint32_t)(j / 2 + 1);
        bool pending = t + 1 < t_end;
        auto issue_share = [&]() __attribute__((always_inline)) {
            settle(true);   // the previous share (a tile without blocks 4..7 never waits for it)
            const int a = a0 + 8 + wave / 2, st = a % kStreamStages, h = wave % 2;
            if (a < nblk) {
                dma_tensor_wave<D, 2>(h ? dout : q, h ? Gs[st] : Qs[st], recs + (a * kBlk) % kRecRing, tok0, lane);
                if (1024 * h + 16 * lane < qts)
                    dma16(qtb + (size_t)a * qts + 1024 * h + 16 * lane, Ts[st] + 1024 * h);
            }
            if (t + 2 < t_end)
                issue_ktiles(t + 2, (j + 2) % 3);
            if (k0 + 3 * kRows < L)
                issue_recs(k0 + 3 * kRows, 6);
            pending = false;
            due = true;
            due_slot = (j + 1) % 2;
            since = 0;
        };
        auto check = [&]() __attribute__((always_inline)) {
            if (pending && *(volatile LDS_AS uint32_t *)(LDS_AS uint32_t *)&through[j % 2] >= goal)
                issue_share();
        };
        {
            uint32_t old = 0u;
            if (lane == 0)
                old = atomicAdd(&through[j % 2], 1u);
            old = __builtin_amdgcn_readfirstlane(old);
            if (pending && old + 1u == goal)
                issue_share();
        }
        bf16x8_t vnext[D / 32];
        if (t + 1 < t_end) {
            // value rows of the next tile's keys (records loaded two tiles ago)
            const int kn = (int)rec_lo(recs[(k0 + kRows + kg * 16 + c) % kRecRing]);
            const bf16 *vrow = v + (tok0 + kn) * D;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                vnext[ks] = as_bf16x8(ld16(vrow + 32 * ks + 8 * g));
        }
        // blocks 4..7 were loaded during the previous tile: wait for every
        // wave's share of them (the prologue loaded the first tile's)
        if (j > 0 && nb > 4) {
            settle(true);
            const uint32_t want = 8u * (uint32_t)((j + 1) / 2);
            for (int spin = 0; spin < (1 << 22); ++spin) {
                if (*(volatile LDS_AS uint32_t *)(LDS_AS uint32_t *)&loaded[j % 2] >= want)
                    break;
                __builtin_amdgcn_s_sleep(1);
            }
            asm volatile("" ::: "memory");
        }
        for (int b = 4; b < nb; ++b) {
            work(b);
            settle(false);
        }
        // every wave reaches the count above without waiting, so this ends
        for (int spin = 0; pending && spin < (1 << 22); ++spin) {
            __builtin_amdgcn_s_sleep(1);
            check();
        }
        kpos_prev = kpos;
        rn_prev = rn;
        if (t + 1 < t_end) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                vop[ks] = vnext[ks];
        }
    }
    dkv_store<D>(dkr_part, dv_part, part_row(tok0 + kpos_prev, nh, r, D), g, rn_prev, dka, dva);
}

// ---------------------------------------------------------------------------
// query-owned kernels (forward, and dq of the backward), persistent form for
// chunk lengths that divide 128.
//
// A query tile [s0, s0 + 128) then reaches keys in [s0 - 128, s0 + 128) (a
// window lies in the query's chunk and the one before), i.e. key blocks
// s0/32 - 4 .. s0/32 + 3, and the next tile needs this tile's last four
// blocks plus four new ones.  Eight waves own 16 queries each
// (v_mfma_f32_16x16x32_bf16).  Stages hold the key (= query) rows, value rows
// and key tiles of a block, indexed by absolute block mod 8.  Per tile: the
// four earlier blocks first; then their stages take the next tile's new
// blocks (and the next tile's query rows are loaded into registers) while
// the tile's own four blocks are worked on.
//
// No workgroup barrier between tiles: a wave starts the next tile as soon as
// all eight shares of its new blocks have landed (an LDS counter per tile
// parity).  A share is issued only once every wave is through the four
// earlier blocks it overwrites (a second counter), so waves drift apart by
// less than a tile, and the record ring (rows x at x mod 512, written two
// tiles ahead) never overwrites rows a slower wave still reads.

template <int D, bool BWD, int NR, int MODE, bool DUPB>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void q_stream_kernel(
    int L, int nh, int T, float scale, const bf16 *__restrict__ q, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ Dvec,
    const uint32_t *__restrict__ meta, const uint32_t *__restrict__ srec, const uint32_t *__restrict__ wmeta,
    const uint32_t *__restrict__ bmeta, const uint8_t *__restrict__ ktile, bf16 *__restrict__ out,
    float *__restrict__ lse_rounds)
{
    // the kind of set: kRange and kRangePos take the query's window from
    // wmeta; kRangePos also compares positions.  DUPB: duplicates weighed by
    // the shared-bucket count instead of the first-owner mask; the records
    // of the other nh - 1 rounds (round rr < r, then rr + 1) are then
    // bucket-run starts (bmeta), and so are the key tiles' entries.
    constexpr bool NC = MODE != kBand;
    __shared__ __align__(16) uint16_t Ks[kStreamStages][kBlk * D];
    __shared__ __align__(16) uint16_t Vs[kStreamStages][kBlk * D];
    __shared__ __align__(16) uint8_t Kts[kStreamStages][kKTile];
    __shared__ __align__(16) uint32_t recs[kRecRing];
    // per tile slot (tile index mod 2), monotonic: waves through the earlier
    // blocks of their tile (8 per tile), and waves whose share of the next
    // tile's blocks has landed in LDS (8 per tile)
    __shared__ uint32_t through[2], loaded[2];
    // with more than seven earlier rounds the queries' records of those
    // rounds wait in LDS during a tile rather than in registers
    constexpr bool kKeepWin = NR <= 7;
    __shared__ uint32_t qmL[kKeepWin ? 1 : kKvThreads / kWave][kKeepWin ? 1 : NR][16];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int g = lane / 16, c = lane % 16;
    // 16-query group of this wave: waves w and w + 4 share a SIMD, and the
    // late query groups (which see more of the tile's own keys) pair with
    // early ones
    const int qg = wave < 4 ? wave : 11 - wave;
    const int nt = L / kRows, nblk = L / kBlk;
    const int rps = (nt + T - 1) / T;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    // rounds in descending order within a (b, h): see stream_run_tiles
    const int run = lb % rps, r = nh - 1 - (lb / rps) % nh, bh = (lb / rps) / nh;
    const int seg = bh * nh + r;
    const int nrec = DUPB ? nh - 1 : r;   // other-round records in use
    const int t_begin = run * T, t_end = min(nt, t_begin + T);
    const uint32_t *sr = srec + (size_t)seg * L;
    const size_t tok0 = (size_t)bh * L;
    const size_t part0 = (size_t)seg * L;
    const int kts = ktile_stride(nh);
    const uint8_t *ktb = ktile + (size_t)seg * nblk * kts;

    auto issue_block = [&](int a) __attribute__((always_inline)) {
        const int st = a % kStreamStages;
        dma_rows512<D>(q, v, Ks[st], Vs[st], recs + (a * kBlk) % kRecRing, 0, tok0, tid, wave);
        if (wave == 0 && 16 * lane < kts)
            dma16(ktb + (size_t)a * kts + 16 * lane, Kts[st]);
    };
    auto issue_recs = [&](int row0, int wv) __attribute__((always_inline)) {
        if (wave == wv && lane < kRows / 4)
            dma16(sr + row0 + 4 * lane, recs + row0 % kRecRing);
    };

    // this lane's query of tile t (16 per wave) in registers; its q row is
    // not among them: the tile's own key blocks hold the query rows (shared
    // QK), so the operand is read from LDS once the tile's blocks are in.
    // Windows: causal, the keys [s - qw, s - 1] of the round and the records
    // (s, w) of the earlier rounds; non-causal (NC), the keys [qhi - qw + 1,
    // qhi] of the round (the query itself skipped) and the window records
    // (hi, span) of the earlier rounds.
    struct QRegs {
        bf16x8_t gop[D / 32];
        uint32_t qm[NR];   // the query's records in the earlier rounds (NR >= r)
        int qpos, qw, qhi;
        float lse2, Di;
    };
    auto load_q = [&](int t, QRegs &R) __attribute__((always_inline)) {
        const int sq = t * kRows + qg * 16 + c;
        const uint32_t rec = recs[sq % kRecRing];
        R.qpos = (int)rec_lo(rec);
        R.qw = (int)rec_hi(rec);
        const size_t tok = tok0 + R.qpos;
        if constexpr (NC) {
            const uint32_t x = wmeta[tok * nh + r];
            R.qhi = (int)rec_lo(x);
            R.qw = (int)rec_hi(x) + 1;
        }
        if constexpr (BWD) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                R.gop[ks] = as_bf16x8(ld16(dout + tok * D + 32 * ks + 8 * g));
            R.lse2 = lse[tok] * kLog2e;
            R.Di = Dvec[tok];
        }
#pragma unroll
        for (int rr = 0; rr < NR; ++rr)
            if (rr < nrec)
                R.qm[rr] = DUPB ? bmeta[tok * nh + (rr < r ? rr : rr + 1)] : (NC ? wmeta : meta)[tok * nh + rr];
    };
    // the earlier-round test of a query record: key sorted index sk hits
    // when (x - sk) mod 2^16 < n, as pairs of 16-bit halves (DUPB: x is the
    // bucket-run start, compared for equality)
    auto win_x = [](uint32_t qm) { return bcast16(DUPB || NC ? rec_lo(qm) : rec_lo(qm) - 1u); };
    auto win_n = [](uint32_t qm) { return bcast16(NC ? rec_hi(qm) + 1u : rec_hi(qm)); };

    // prologue: records [s0 - 128, s0 + 256), then the first tile's eight blocks and query rows
    if (tid < 2) {
        through[tid] = 0u;
        loaded[tid] = 0u;
    }
    {
        const int s0 = t_begin * kRows;
        if (s0 >= kRows)
            issue_recs(s0 - kRows, 5);
        issue_recs(s0, 6);
        if (s0 + kRows < L)
            issue_recs(s0 + kRows, 7);
        wait_vm<0>();
        lds_barrier();   // also publishes the zeroed release counters
        for (int a = s0 / kBlk - 4; a < s0 / kBlk + 4; ++a)
            if (a >= 0 && a < nblk)
                issue_block(a);
    }
    QRegs cur;
    load_q(t_begin, cur);

    constexpr int NA = BWD ? D / 16 : D / 16;
    f32x4_t acc[NA];
    float mrun = -INFINITY, lrun = 0.f;
    int qpos_prev = 0;
    auto finish = [&](int qpos) __attribute__((always_inline)) {
        // forward: o_rounds [b][h][r][L][D]; dq: the partial's row (see part_row)
        const size_t row = BWD ? part_row(tok0 + qpos, nh, r, D) : (part0 + qpos) * D;
        float sc = 1.f;
        if constexpr (!BWD)
            sc = lrun > 0.f ? 1.f / lrun : 0.f;
        store_row16<D>(out + row, g, sc, acc);
        if constexpr (!BWD)
            if (g == 0)
                lse_rounds[part0 + qpos] = lrun > 0.f ? (mrun + __log2f(lrun)) * 0.69314718055994531f : -INFINITY;
    };

    QRegs nxt;
    for (int t = t_begin; t < t_end; ++t) {
        const int s0 = t * kRows, a0 = s0 / kBlk;
        // everything issued during the previous tile has landed
        wait_vm<0>();
        if (t > t_begin) {
            finish(qpos_prev);
            cur = nxt;
        }
        if constexpr (!kKeepWin) {
            if (g == 0) {
#pragma unroll
                for (int rr = 0; rr < NR; ++rr)
                    if (rr < nrec)
                        qmL[wave][rr][c] = cur.qm[rr];
            }
        }
        const int jt = t - t_begin;
        if (jt == 0) {
            block_barrier();   // the prologue's blocks, loaded by every wave
        } else {
            // every wave's share of this tile's four new blocks has landed
            const uint32_t want = 8u * (uint32_t)((jt + 1) / 2);
            for (int spin = 0; spin < (1 << 22); ++spin) {
                if (*(volatile LDS_AS uint32_t *)(LDS_AS uint32_t *)&loaded[jt % 2] >= want)
                    break;
                __builtin_amdgcn_s_sleep(1);
            }
            asm volatile("" ::: "memory");
        }
        // query operand: rows 16 (qg % 2) + c of own block a0 + qg / 2
        bf16x8_t qop[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            qop[ks] = tile_row<D>(Ks[(a0 + qg / 2) % kStreamStages], 16 * (qg % 2) + c, 32 * ks + 8 * g);
#pragma unroll
        for (int dt = 0; dt < NA; ++dt)
            acc[dt] = f32x4_t{};
        mrun = -INFINITY;
        lrun = 0.f;

        const int wq0 = s0 + qg * 16;
        const int sq = wq0 + c;
        const int qlo = NC ? cur.qhi - cur.qw + 1 : sq - cur.qw;
        // window starts and ends do not decrease along the sorted order: the
        // wave's keys lie in [wlo, whi]
        const int wlo = __builtin_amdgcn_readlane(qlo, 0);
        const int whi = NC ? __builtin_amdgcn_readlane(cur.qhi, 15) : wq0 + 14;

        // earlier-round window tests: (end, length) of the query's set in
        // round rr (see win_x), both halves of a packed pair (kept for up to
        // seven rounds, formed per block from LDS beyond that)
        uint32_t si1p[kKeepWin ? NR : 1], wp[kKeepWin ? NR : 1];
        if constexpr (kKeepWin) {
#pragma unroll
            for (int rr = 0; rr < NR; ++rr) {
                si1p[rr] = win_x(cur.qm[rr]);
                wp[rr] = win_n(cur.qm[rr]);
            }
        }

        auto work = [&](int a) __attribute__((always_inline)) {
            const int kb = a * kBlk, st = a % kStreamStages;
            if (kb > whi || kb + kBlk - 1 < wlo)
                return;
            const uint16_t *K = Ks[st], *V = Vs[st];
            const float *rnk = reinterpret_cast<const float *>(Kts[st]);
            const uint16_t *skm = reinterpret_cast<const uint16_t *>(Kts[st] + 128);
            // The LDS reads of the block are issued here, before any of the
            // arithmetic, so the block waits for LDS once (register space
            // permitting: the dq kernel reads K^T after the softmax, and with
            // more than seven earlier rounds their key indices are read in the
            // mask loop).
            constexpr bool kEarlyTr = !BWD, kEarlySk = NR <= (BWD ? 3 : 7);
            // S^T = K Q^T (and dP^T = V dO^T): lane (query c, group g) gets keys 16 kk + 4 g + t
            bf16x8_t ka[2][D / 32], va[2][D / 32];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    ka[kk][ks] = tile_row<D>(K, 16 * kk + c, 32 * ks + 8 * g);
                    if constexpr (BWD)
                        va[kk][ks] = tile_row<D>(V, 16 * kk + c, 32 * ks + 8 * g);
                }
            float4 rn4[2];   // rn * scale * log2(e) of the lane's keys
            auto read_rn = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    rn4[kk] = *reinterpret_cast<const float4 *>(rnk + 16 * kk + 4 * g);
            };
            if constexpr (kEarlySk)
                read_rn();
            // the keys' sorted indices in the earlier rounds
            auto read_sk = [&](int rr, int kk) __attribute__((always_inline)) {
                return *reinterpret_cast<const uint2 *>(skm + 32 * rr + 16 * kk + 4 * g);
            };
            uint2 kp[kEarlySk ? NR : 1][2];
            if constexpr (kEarlySk) {
#pragma unroll
                for (int rr = 0; rr < NR; ++rr)
                    if (rr < nrec) {
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk)
                            kp[rr][kk] = read_sk(rr, kk);
                    }
            }
            // the operand of the second product: V^T (forward) or K^T (dq)
            bf16x8_t tr[D / 16];
            auto read_tr = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    tr[dt] = tile_tr16x<D>(BWD ? K : V, 16 * dt, lane);
            };
            if constexpr (kEarlyTr)
                read_tr();
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t sacc[2], pacc[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                sacc[kk] = f32x4_t{};
                pacc[kk] = f32x4_t{};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    sacc[kk] = mfma16(ka[kk][ks], qop[ks], sacc[kk]);
                    if constexpr (BWD)
                        pacc[kk] = mfma16(va[kk][ks], cur.gop[ks], pacc[kk]);
                }
            }
            bool ok[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = kb + 16 * (e / 4) + 4 * g + (e % 4);
                ok[e] = (unsigned)(key - qlo) < (unsigned)cur.qw && (!NC || key != sq);
            }
            if constexpr (MODE == kRangePos) {
                // keys not after the query (positions from the record ring)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const uint4 p = *reinterpret_cast<const uint4 *>(recs + (kb + 16 * kk + 4 * g) % kRecRing);
                    const uint32_t pk[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        ok[4 * kk + t] = ok[4 * kk + t] && rec_lo(pk[t]) < (uint32_t)cur.qpos;
                }
            }
            float lg[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // log2 of the duplicate divisor (DUPB)
            if (nrec > 0) {
                uint32_t hit[4] = {0u, 0u, 0u, 0u};   // DUPB: rounds with a different bucket, per 16-bit half
#pragma unroll
                for (int rr = 0; rr < NR; ++rr)
                    if (rr < nrec) {
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) {
                            const uint2 k2 = kEarlySk ? kp[kEarlySk ? rr : 0][kk] : read_sk(rr, kk);
                            const uint32_t qmr = kKeepWin ? 0u : qmL[kKeepWin ? 0 : wave][kKeepWin ? 0 : rr][c];
                            const uint32_t s1 = kKeepWin ? si1p[kKeepWin ? rr : 0] : win_x(qmr);
                            if constexpr (DUPB) {
                                hit[2 * kk] += ne16(s1, k2.x);
                                hit[2 * kk + 1] += ne16(s1, k2.y);
                            } else {
                                const uint32_t w1 = kKeepWin ? wp[kKeepWin ? rr : 0] : win_n(qmr);
                                hit[2 * kk] |= win_hits2(s1, w1, k2.x);
                                hit[2 * kk + 1] |= win_hits2(s1, w1, k2.y);
                            }
                        }
                    }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t h = (hit[e / 2] >> (16 * (e % 2))) & 0xffffu;
                    if constexpr (DUPB)
                        lg[e] = __log2f((float)(nh - (int)h));
                    else
                        ok[e] = ok[e] && h == 0u;
                }
            }
            if constexpr (!kEarlySk)
                read_rn();
            float x[8];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float rn[4] = {rn4[kk].x, rn4[kk].y, rn4[kk].z, rn4[kk].w};
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int e = 4 * kk + tt;
                    if constexpr (BWD) {
                        const float pr = ok[e] ? fast_exp2(fmaf(sacc[kk][tt], rn[tt], -cur.lse2) - lg[e]) : 0.f;
                        x[e] = pr * (pacc[kk][tt] - cur.Di) * (rn[tt] * kLn2);
                    } else {
                        x[e] = ok[e] ? sacc[kk][tt] * rn[tt] - lg[e] : -INFINITY;
                    }
                }
            }
            if constexpr (!BWD) {
                float bm = x[0];
#pragma unroll
                for (int e = 1; e < 8; ++e)
                    bm = fmaxf(bm, x[e]);
                bm = max_xor32(max_xor16(bm));
                const bool raise = bm > mrun + kLazy;
                const float mnew = raise ? bm : mrun;
                const float mref = (mnew == -INFINITY) ? 0.f : mnew;
                float ps = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x[e] = fast_exp2(x[e] - mref);
                    ps += x[e];
                }
                ps = sum_xor32(sum_xor16(ps));
                if (__ballot(raise) != 0ull) {
                    const float corr = raise ? fast_exp2(mrun - mref) : 1.f;
                    lrun *= corr;
#pragma unroll
                    for (int dt = 0; dt < NA; ++dt)
                        acc[dt] *= corr;
                }
                lrun += ps;
                mrun = mnew;
            }
            // O^T += V^T P^T, or dQ^T += K^T G^T: B slot s is value s of x
            const bf16x8_t xb = pack8(x);
            if constexpr (!kEarlyTr) {
                read_tr();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                acc[dt] = mfma16(tr[dt], xb, acc[dt]);
        };

        // The earlier blocks first.  Once every wave is through them, their
        // stages take the next tile's four new blocks (its own rows), each
        // wave loading one tensor of one block: the wave that completes the
        // count at once, the others at their next check (after each of their
        // own blocks, and at the latest before the tile's end), so the loads
        // start early and no wave carries all of them.
        // raised wave priority while the blocks that gate the next loads are
        // worked on (the SIMD's other wave yields to a wave still in them)
        __builtin_amdgcn_s_setprio(2);
        for (int a = a0 - 4; a < a0; ++a)
            if (a >= 0)
                work(a);
        __builtin_amdgcn_s_setprio(0);
        const uint32_t goal = 8u * (uint32_t)(jt / 2 + 1);
        bool pending = t + 1 < t_end;
        bool signaled = !pending;
        auto issue_share = [&]() __attribute__((always_inline)) {
            const int a = a0 + 4 + wave / 2, st = a % kStreamStages;
            if (a < nblk) {
                dma_tensor_wave<D>(wave % 2 ? v : q, wave % 2 ? Vs[st] : Ks[st], recs + (a * kBlk) % kRecRing, tok0,
                                   lane);
                if (wave % 2 == 0 && 16 * lane < kts)
                    dma16(ktb + (size_t)a * kts + 16 * lane, Kts[st]);
            }
            pending = false;
        };
        auto check = [&]() __attribute__((always_inline)) {
            if (pending && *(volatile LDS_AS uint32_t *)(LDS_AS uint32_t *)&through[jt % 2] >= goal)
                issue_share();
        };
        {
            uint32_t old = 0u;
            if (lane == 0)
                old = atomicAdd(&through[jt % 2], 1u);
            old = __builtin_amdgcn_readfirstlane(old);
            if (pending && old + 1u == goal)
                issue_share();
        }
        if (t + 1 < t_end) {
            load_q(t + 1, nxt);
            if (s0 + 2 * kRows < L)
                issue_recs(s0 + 2 * kRows, 6);
        }
        // once this wave's share has landed, tell the others: they wait for
        // all eight shares at the next tile's start.  The wait for the share
        // comes after kSettle of the wave's own blocks (the forward at d = 128
        // has the least work per block to hide the loads behind).
        constexpr int kSettle = BWD || D <= 64 ? 1 : 3;
        auto settle = [&]() __attribute__((always_inline)) {
            if (!pending && !signaled) {
                wait_vm<0>();
                if (lane == 0)
                    atomicAdd(&loaded[(jt + 1) % 2], 1u);
                signaled = true;
            }
        };
        for (int a = a0; a < a0 + 4; ++a) {
            work(a);
            if (a - a0 + 1 >= kSettle)
                settle();
            check();
        }
        // every wave reaches the count above without waiting, so this ends
        for (int spin = 0; pending && spin < (1 << 22); ++spin) {
            __builtin_amdgcn_s_sleep(1);
            check();
        }
        settle();
        qpos_prev = cur.qpos;
    }
    finish(qpos_prev);
}

// Sum of the per-round partials and the key-normalisation backward:
//   a = sum_r dq_r,  b = sum_r dk_r rn  (rn = 1/|q|),  k = q rn,
//   dQ = a + b - k (k . b),  dV = sum_r dv_r,
// plus dO for tokens that attend only to themselves (o = v).  D/8 lanes per
// token, 8 elements each.  The partials are read once and the results written
// once, so both bypass the caches' normal retention (nontemporal accesses:
// 13 % less time at the long-text shape than plain ones).
template <int D, int NH>
__global__ __launch_bounds__(kThreads) void reduce_kernel(int L, int nh, int ntok, const bf16 *__restrict__ q,
                                                          const float *__restrict__ rnorm,
                                                          const bf16 *__restrict__ dout,
                                                          const uint32_t *__restrict__ meta,
                                                          const uint32_t *__restrict__ wmeta,
                                                          const uint8_t *__restrict__ aflag,
                                                          const bf16 *__restrict__ dq_part,
                                                          const bf16 *__restrict__ dkr_part,
                                                          const bf16 *__restrict__ dv_part, bf16 *__restrict__ dq,
                                                          bf16 *__restrict__ dv)
{
    constexpr int CPT = D / 8, TPB = kThreads / CPT;
    const int grp = threadIdx.x / CPT, ch = threadIdx.x % CPT;
    const int tok = blockIdx.x * TPB + grp;
    if (tok >= ntok)
        return;
    float aq[8] = {}, ak[8] = {}, av[8] = {};
    bool alone = true;
    // every round's rows requested before any is summed (nh <= NH)
    u32x4_t xq[NH], xk[NH], xv[NH];
#pragma unroll
    for (int r = 0; r < NH; ++r)
        if (r < nh) {
            const size_t off = part_row(tok, nh, r, D) + ch * 8;   // the round's three rows are adjacent
            xq[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(dq_part + off));
            xk[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(dkr_part + off));
            xv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(dv_part + off));
            // no member but itself: w = 0 (kBand), span = 0 (kRange) or the lone flag (kRangePos)
            alone = alone && (aflag ? aflag[(size_t)tok * nh + r] != 0
                                    : rec_hi((wmeta ? wmeta : meta)[(size_t)tok * nh + r]) == 0u);
        }
    float qv[8];
    load8(q + (size_t)tok * D + ch * 8, qv);
#pragma unroll
    for (int r = 0; r < NH; ++r)
        if (r < nh) {
            const uint32_t wq[4] = {xq[r].x, xq[r].y, xq[r].z, xq[r].w};
            const uint32_t wk[4] = {xk[r].x, xk[r].y, xk[r].z, xk[r].w};
            const uint32_t wv[4] = {xv[r].x, xv[r].y, xv[r].z, xv[r].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                aq[2 * k] += __uint_as_float(wq[k] << 16);
                aq[2 * k + 1] += __uint_as_float(wq[k] & 0xffff0000u);
                ak[2 * k] += __uint_as_float(wk[k] << 16);
                ak[2 * k + 1] += __uint_as_float(wk[k] & 0xffff0000u);
                av[2 * k] += __uint_as_float(wv[k] << 16);
                av[2 * k + 1] += __uint_as_float(wv[k] & 0xffff0000u);
            }
        }
    float qb = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        qb = fmaf(qv[k], ak[k], qb);
    qb = group_sum(qb, CPT);
    const float rn = rnorm[tok];
    const float proj = rn * rn * qb;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        aq[k] += ak[k] - qv[k] * proj;
    if (alone) {
        float x[8];
        load8(dout + (size_t)tok * D + ch * 8, x);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            av[k] += x[k];
    }
    auto st8 = [](bf16 *p, const float *x) {
        u32x4_t u;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)from_f<bf16>(x[2 * k]).bits | ((uint32_t)from_f<bf16>(x[2 * k + 1]).bits << 16);
        u.x = w[0]; u.y = w[1]; u.z = w[2]; u.w = w[3];
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t *>(p));
    };
    st8(dq + (size_t)tok * D + ch * 8, aq);
    st8(dv + (size_t)tok * D + ch * 8, av);
}

// Tiles per run of the persistent kernels: one run per CU in total (a
// workgroup of these kernels fills a CU), or two when one per CU gives runs
// of kMinSplitTiles to kMaxSplitTiles tiles (2x the minimum to the maximum);
// runs within one (b, h, round), at most kMaxRunTiles tiles.  A round's tiles cost more the more earlier rounds its
// membership tests cover (the last of eight rounds about 1.5x the first), so
// with one run per segment the CUs holding round 0 idle for a third of the
// launch.  Runs dealt out as CUs free up, with the rounds of a (b, h) taken
// last to first so that the cheap runs come last, even that out; each run
// costs a prologue whose loads nothing overlaps, hence the bounds.
constexpr int kMaxRunTiles = 128;
constexpr int kMinSplitTiles = 12, kMaxSplitTiles = 32;
int stream_run_tiles(int nt, int segs)
{
    constexpr int kCUs = 256;
    const long total = (long)nt * segs;
    int T = (int)((total + kCUs - 1) / kCUs);
    const int half = (int)((total + 2 * kCUs - 1) / (2 * kCUs));
    if (T <= kMaxSplitTiles && half >= kMinSplitTiles)
        T = half;
    T = T > kMaxRunTiles ? kMaxRunTiles : T;
    return T < 1 ? 1 : (T > nt ? nt : T);
}

// Rows before a workgroup's first row that its first row's window can reach:
// a window lies in the query's chunk and the one before, so it is shorter
// than 2 m; rounded up to whole blocks.
int max_window(const Dims &P) { return (2 * P.m + kBlk - 1) / kBlk * kBlk; }

// The query-side stream kernel for the bound NR on the earlier rounds
// (n_hashes - 1 rounded up to 1, 3, 7 or 13) and the kind of set.
template <int D, bool BWD, int MODE, bool DUPB>
void q_stream_nc(const Dims &P, const void *q, const void *v, const void *dout, const float *lse, const float *Dv,
                 const uint32_t *meta, const uint32_t *srec, const uint32_t *wmeta, const uint32_t *bmeta,
                 const uint8_t *ktile, void *out, float *lse_rounds, hipStream_t st)
{
    const int nt = P.L / kRows, segs = P.BH() * P.nh;
    const int T = stream_run_tiles(nt, segs);
    const dim3 grid(segs * ((nt + T - 1) / T));
#define LSH_QSTREAM(NR)                                                                                            \
    hipLaunchKernelGGL((q_stream_kernel<D, BWD, NR, MODE, DUPB>), grid, dim3(kKvThreads), 0, st, P.L, P.nh, T,      \
                       P.scale, (const bf16 *)q, (const bf16 *)v, (const bf16 *)dout, lse, Dv, meta, srec, wmeta,   \
                       bmeta, ktile, (bf16 *)out, lse_rounds)
    if (P.nh <= 2)
        LSH_QSTREAM(1);
    else if (P.nh <= 4)
        LSH_QSTREAM(3);
    else if (P.nh <= 8)
        LSH_QSTREAM(7);
    else
        LSH_QSTREAM(13);
#undef LSH_QSTREAM
}

template <int D, bool BWD>
void q_stream_go(const Dims &P, const void *q, const void *v, const void *dout, const float *lse, const float *Dv,
                 const uint32_t *meta, const uint32_t *srec, const Extra &x, const uint8_t *ktile, void *out,
                 float *lse_rounds, hipStream_t st)
{
    const uint32_t *wm = x.wmeta, *bm = x.bmeta;
    if (P.dup_bucket) {
        if (P.kind() == kBand)
            q_stream_nc<D, BWD, kBand, true>(P, q, v, dout, lse, Dv, meta, srec, nullptr, bm, ktile, out, lse_rounds,
                                             st);
        else
            q_stream_nc<D, BWD, kRange, true>(P, q, v, dout, lse, Dv, meta, srec, wm, bm, ktile, out, lse_rounds, st);
    } else if (P.kind() == kBand) {
        q_stream_nc<D, BWD, kBand, false>(P, q, v, dout, lse, Dv, meta, srec, nullptr, nullptr, ktile, out,
                                          lse_rounds, st);
    } else if (P.kind() == kRange) {
        q_stream_nc<D, BWD, kRange, false>(P, q, v, dout, lse, Dv, meta, srec, wm, nullptr, ktile, out, lse_rounds,
                                           st);
    } else {
        q_stream_nc<D, BWD, kRangePos, false>(P, q, v, dout, lse, Dv, meta, srec, wm, nullptr, ktile, out,
                                              lse_rounds, st);
    }
}

// (non-causal problems take the stream kernels only: mfma_path_ok)
template <int D>
hipError_t fwd_go(const Dims &P, const void *q, const void *v, const uint32_t *meta, const uint32_t *srec,
                  const Extra &x, const uint8_t *ktile, void *o_rounds, float *lse_rounds, hipStream_t st)
{
    ProfScope prof(LSH_KERNEL_FWD, st);
    if (kRows % P.m == 0) {
        q_stream_go<D, false>(P, q, v, nullptr, nullptr, nullptr, meta, srec, x, ktile, o_rounds, lse_rounds, st);
    } else {
        hipLaunchKernelGGL((fwd_kernel<D>), dim3((P.L / kRows) * P.nh * P.BH()), dim3(kThreads), 0, st, P.L, P.nh,
                           max_window(P), P.scale * kLog2e, (const bf16 *)q, (const bf16 *)v, meta, srec, ktile,
                           (bf16 *)o_rounds, lse_rounds);
    }
    return hipGetLastError();
}

template <int D>
hipError_t bwd_go(const Dims &P, const void *q, const void *v, const void *dout, const float *lse, const float *Dv,
                  const uint32_t *meta, const uint32_t *srec, const Extra &x, const float *rnorm,
                  const uint8_t *ktile, const uint8_t *qtile, void *part, void *dq, void *dv, hipStream_t st)
{
    // rows of one (token, round) are dq, dk rn, dv in turn (part_row)
    bf16 *dq_part = (bf16 *)part, *dkr_part = dq_part + D, *dv_part = dq_part + 2 * D;
    const dim3 grid((P.L / kRows) * P.nh * P.BH());
    {
        ProfScope prof(LSH_KERNEL_BWD_DQ, st);
        if (kRows % P.m == 0) {
            q_stream_go<D, true>(P, q, v, dout, lse, Dv, meta, srec, x, ktile, dq_part, nullptr, st);
        } else {
            hipLaunchKernelGGL((dq_kernel<D>), grid, dim3(kThreads), 0, st, P.L, P.nh, max_window(P), P.scale,
                               (const bf16 *)q, (const bf16 *)v, (const bf16 *)dout, lse, Dv, meta, srec, ktile,
                               dq_part);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    {
        ProfScope prof(LSH_KERNEL_BWD_DKV, st);
        if (kRows % P.m == 0) {
            const int nt = P.L / kRows, segs = P.BH() * P.nh;
            const int T = stream_run_tiles(nt, segs);
            const int runs = segs * ((nt + T - 1) / T);
#define LSH_DKV(NR, MODE, DUPB)                                                                                \
    hipLaunchKernelGGL((dkv_stream_kernel<D, NR, MODE, DUPB>), dim3(runs), dim3(kKvThreads), 0, st, P.L, P.nh, T,  \
                       P.m, P.scale, (const bf16 *)q, (const bf16 *)v, (const bf16 *)dout, srec, ktile, qtile,       \
                       dkr_part, dv_part)
#define LSH_DKV_NR(MODE, DUPB)      \
    if (P.nh <= 2)                  \
        LSH_DKV(1, MODE, DUPB);     \
    else if (P.nh <= 4)             \
        LSH_DKV(3, MODE, DUPB);     \
    else if (P.nh <= 8)             \
        LSH_DKV(7, MODE, DUPB);     \
    else                            \
        LSH_DKV(13, MODE, DUPB)
            if (P.dup_bucket) {
                if (P.kind() == kBand) {
                    LSH_DKV_NR(kBand, true);
                } else {
                    LSH_DKV_NR(kRange, true);
                }
            } else if (P.kind() == kBand) {
                LSH_DKV_NR(kBand, false);
            } else if (P.kind() == kRange) {
                LSH_DKV_NR(kRange, false);
            } else {
                LSH_DKV_NR(kRangePos, false);
            }
#undef LSH_DKV_NR
#undef LSH_DKV
        } else {
            hipLaunchKernelGGL((dkv_kernel<D>), grid, dim3(kKvThreads), 0, st, P.L, P.nh, P.scale, (const bf16 *)q,
                               (const bf16 *)v, (const bf16 *)dout, srec, ktile, qtile, dkr_part, dv_part);
        }
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int ntok = P.BH() * P.L;
    constexpr int TPB = kThreads / (D / 8);
    ProfScope prof(LSH_KERNEL_BWD_REDUCE, st);
#define LSH_REDUCE(NH)                                                                                            \
    hipLaunchKernelGGL((reduce_kernel<D, NH>), dim3((ntok + TPB - 1) / TPB), dim3(kThreads), 0, st, P.L, P.nh, ntok, \
                       (const bf16 *)q, rnorm, (const bf16 *)dout, meta, x.wmeta, x.alone, dq_part, dkr_part,       \
                       dv_part, (bf16 *)dq, (bf16 *)dv)
    if (P.nh <= 2)
        LSH_REDUCE(2);
    else if (P.nh <= 4)
        LSH_REDUCE(4);
    else if (P.nh <= 8)
        LSH_REDUCE(8);
    else
        LSH_REDUCE(16);
#undef LSH_REDUCE
    return hipGetLastError();
}

hipError_t tiles_go(const Dims &P, const uint32_t *srec, const uint32_t *meta, const uint32_t *wmeta,
                    const uint32_t *bmeta, const float *rnorm, const float *lse, const float *Dv, uint8_t *ktile,
                    uint8_t *qtile, hipStream_t st)
{
    const int ntiles = P.BH() * P.nh * (P.L / kBlk);
    const int per_block = kThreads / kWave;
    ProfScope prof(LSH_KERNEL_TILES, st);
    hipLaunchKernelGGL(tile_prep_kernel, dim3((ntiles + per_block - 1) / per_block), dim3(kThreads), 0, st, P.L, P.nh,
                       ntiles, P.scale * kLog2e, srec, meta, wmeta, bmeta, rnorm, lse, Dv, ktile, qtile);
    return hipGetLastError();
}

}  // namespace

bool mfma_path_ok(const Dims &P, int dtype)
{
    // the streamed range of a workgroup (at most 128 + 2 m + 31 sorted rows)
    // must fit the LDS record cache, and the metadata tiles hold 13 earlier
    // rounds; sets other than the causal band run on the stream kernels only
    // (chunk lengths that divide 128)
    return dtype == LSH_BF16 && (P.d == 64 || P.d == 128) && P.L % kRows == 0 && P.nh <= kMaxEarlier + 1 &&
           kRows + 2 * P.m + kBlk <= kRecCache && ((P.kind() == kBand && !P.dup_bucket) || kRows % P.m == 0);
}

size_t mfma_ktile_bytes(const Dims &P) { return (size_t)P.BH() * P.nh * (P.L / kBlk) * ktile_stride(P.nh); }
size_t mfma_qtile_bytes(const Dims &P) { return (size_t)P.BH() * P.nh * (P.L / kBlk) * qtile_stride(P.nh); }
size_t bwd_mfma_part_bytes(const Dims &P) { return 3 * (size_t)P.BH() * P.nh * P.L * P.d * sizeof(uint16_t); }

hipError_t launch_attn_fwd_mfma(const Dims &P, const void *q, const void *v, const uint32_t *meta,
                                const uint32_t *srec, const Extra &x, const float *rnorm, uint8_t *ktile,
                                void *o_rounds, float *lse_rounds, hipStream_t st)
{
    hipError_t e = tiles_go(P, srec, meta, x.wmeta, x.bmeta, rnorm, nullptr, nullptr, ktile, nullptr, st);
    if (e != hipSuccess)
        return e;
    if (P.d == 128)
        return fwd_go<128>(P, q, v, meta, srec, x, ktile, o_rounds, lse_rounds, st);
    return fwd_go<64>(P, q, v, meta, srec, x, ktile, o_rounds, lse_rounds, st);
}

hipError_t launch_attn_bwd_mfma(const Dims &P, const void *q, const void *v, const void *dout, const float *lse,
                                const float *Dv, const uint32_t *meta, const uint32_t *srec, const Extra &x,
                                const float *rnorm, uint8_t *ktile, bool make_ktile, uint8_t *qtile, void *part,
                                void *dq, void *dv, hipStream_t st)
{
    hipError_t e =
        tiles_go(P, srec, meta, x.wmeta, x.bmeta, rnorm, lse, Dv, make_ktile ? ktile : nullptr, qtile, st);
    if (e != hipSuccess)
        return e;
    if (P.d == 128)
        return bwd_go<128>(P, q, v, dout, lse, Dv, meta, srec, x, rnorm, ktile, qtile, part, dq, dv, st);
    return bwd_go<64>(P, q, v, dout, lse, Dv, meta, srec, x, rnorm, ktile, qtile, part, dq, dv, st);
}

}  // namespace lsh
