// lsh_api.cpp -- the C ABI of liblsh: argument validation, workspace layout
// and launches.  Declarations and contracts are in include/lsh.h.
#include <math.h>

#include "common.hpp"

using namespace lsh;

namespace {

hipEvent_t g_prof_start[LSH_KERNEL_COUNT];
hipEvent_t g_prof_stop[LSH_KERNEL_COUNT];

const char *const kKernelNames[LSH_KERNEL_COUNT] = {
    "hash", "sort_count", "sort_scatter", "prep", "attn_fwd", "combine", "bwd_dq", "bwd_dkv", "bwd_reduce",
    "tiles"};

}  // namespace

namespace lsh {

void prof_begin(int k, hipStream_t st)
{
    if (g_prof_start[k])
        (void)hipEventRecord(g_prof_start[k], st);
}

void prof_end(int k, hipStream_t st)
{
    if (g_prof_stop[k])
        (void)hipEventRecord(g_prof_stop[k], st);
}

}  // namespace lsh

namespace {

constexpr int kMaxHashes = 16;
constexpr int kMaxLen = 65536;   // sorted indices and positions are packed in 16 bits
constexpr int kMaxBucketsAbi = 4096;

int validate(const lsh_problem_t *p)
{
    if (!p)
        return LSH_ERR_INVALID;
    if (p->batch < 0 || p->heads < 0 || p->seq_len < 0 || p->head_dim < 1 || p->n_hashes < 1 ||
        p->n_buckets < 2 || (p->n_buckets & 1) || p->chunk_len < 1 || p->seq_len % p->chunk_len ||
        !isfinite(p->scale) || (p->dtype != LSH_F32 && p->dtype != LSH_BF16) || (p->causal != 0 && p->causal != 1) ||
        (p->flags & ~(int32_t)(LSH_FLAG_NO_BUCKET_MASK | LSH_FLAG_DUP_BY_BUCKET)) ||
        ((p->flags & LSH_FLAG_NO_BUCKET_MASK) && (p->flags & LSH_FLAG_DUP_BY_BUCKET)))
        return LSH_ERR_INVALID;
    if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128)
        return LSH_ERR_UNSUPPORTED;
    if (p->seq_len > kMaxLen || p->n_hashes > kMaxHashes || p->n_buckets > kMaxBucketsAbi)
        return LSH_ERR_UNSUPPORTED;
    // every element index must fit in size_t arithmetic and every segment count in int;
    // the (b, h, round) segments index a grid dimension of at most 65535
    const double tok_rounds = (double)p->batch * p->heads * p->n_hashes * p->seq_len;
    if (tok_rounds > 2147483647.0 || (double)p->batch * p->heads * p->n_hashes > 65535.0)
        return LSH_ERR_UNSUPPORTED;
    return LSH_OK;
}

// B, H or L of zero: nothing to compute; every call returns LSH_OK without
// reading its pointers or touching the device.
bool empty(const lsh_problem_t *p) { return p->batch == 0 || p->heads == 0 || p->seq_len == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? LSH_OK : LSH_ERR_HIP; }

// The extra records (see Extra) exist only where the problem uses them.
struct FwdWs {
    uint32_t *meta, *srec;
    Extra x;
    float *rnorm;
    uint8_t *ktile;
    size_t bytes;
};

struct BwdWs {
    uint32_t *meta, *srec;
    Extra x;
    float *rnorm, *D, *dq_part, *dk_part, *dv_part;
    uint8_t *ktile, *qtile;
    size_t bytes;
};

// The forward's part, shared by both layouts (a backward takes it over
// from lsh_attn_fwd in lsh_attn_bwd_saved).
template <typename W>
size_t fwd_part(const Dims &P, uintptr_t b, W &w)
{
    const size_t tok = (size_t)P.BH() * P.L, rnd = tok * P.nh;
    size_t o = 0;
    w.meta = (uint32_t *)(b + o); o += align_up(rnd * 4, 256);
    w.srec = (uint32_t *)(b + o); o += align_up(rnd * 4, 256);
    w.rnorm = (float *)(b + o); o += align_up(tok * 4, 256);
    w.ktile = (uint8_t *)(b + o); o += align_up(mfma_ktile_bytes(P), 256);
    if (P.kind() != kBand) {
        w.x.wmeta = (uint32_t *)(b + o); o += align_up(rnd * 4, 256);
    }
    if (P.kind() == kRangePos) {
        w.x.alone = (uint8_t *)(b + o); o += align_up(rnd, 256);
        w.x.cmin = (uint32_t *)(b + o); o += align_up((size_t)P.BH() * P.nh * (P.L / P.m) * 4, 256);
    }
    if (P.dup_bucket) {
        w.x.bmeta = (uint32_t *)(b + o); o += align_up(rnd * 4, 256);
        w.x.bscr = (uint32_t *)(b + o); o += align_up((size_t)P.BH() * P.nh * ((P.L + 1023) / 1024) * 4, 256);
    }
    return o;
}

FwdWs fwd_layout(const Dims &P, void *base)
{
    FwdWs w{};
    w.bytes = fwd_part(P, (uintptr_t)base, w);
    return w;
}

BwdWs bwd_layout(const Dims &P, int dtype, void *base)
{
    const size_t tok = (size_t)P.BH() * P.L, rnd = tok * P.nh, part = rnd * P.d * sizeof(float);
    const uintptr_t b = (uintptr_t)base;
    BwdWs w{};
    size_t o = fwd_part(P, b, w);
    // up to here the same offsets as the forward's workspace, so that a
    // backward can take over the forward's records
    w.D = (float *)(b + o); o += align_up(tok * 4, 256);
    w.dq_part = (float *)(b + o);
    if (mfma_path_ok(P, dtype)) {
        // bf16 partials, the three rows of a (token, round) side by side, and the query tiles
        o += align_up(bwd_mfma_part_bytes(P), 256);
        w.qtile = (uint8_t *)(b + o); o += align_up(mfma_qtile_bytes(P), 256);
    } else {
        // fp32 partials of the per-query kernels
        o += align_up(part, 256);
        w.dk_part = (float *)(b + o); o += align_up(part, 256);
        w.dv_part = (float *)(b + o); o += align_up(part, 256);
    }
    w.bytes = o;
    return w;
}

// lsh_attn_bwd_rehash's workspace: the backward's own, then the buckets,
// sorted order and window starts it recomputes, then the sort's scratch.
struct RehashWs {
    void *bwd;
    size_t bwd_bytes;
    int32_t *buckets, *perm, *inv, *win_lo;
    void *sort;
    size_t sort_bytes;
    size_t bytes;
};

RehashWs rehash_layout(const Dims &P, int dtype, void *base)
{
    const size_t rnd = (size_t)P.BH() * P.nh * P.L;
    const uintptr_t b = (uintptr_t)base;
    RehashWs w{};
    size_t o = 0;
    w.bwd = (void *)(b + o);
    w.bwd_bytes = bwd_layout(P, dtype, nullptr).bytes;
    o += align_up(w.bwd_bytes, 256);
    w.buckets = (int32_t *)(b + o); o += align_up(rnd * 4, 256);
    w.perm = (int32_t *)(b + o); o += align_up(rnd * 4, 256);
    w.inv = (int32_t *)(b + o); o += align_up(rnd * 4, 256);
    w.win_lo = (int32_t *)(b + o); o += align_up(rnd * 4, 256);
    w.sort = (void *)(b + o);
    w.sort_bytes = sort_ws_bytes(P);
    o += align_up(w.sort_bytes, 256);
    w.bytes = o;
    return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Tensor arguments of a backward: present, and 16-byte aligned where rows are read in 16-byte pieces.
bool bwd_args_ok(const void *q, const void *v, const void *out, const void *dout, const float *lse, const void *dq,
                 const void *dv)
{
    return q && v && out && dout && lse && dq && dv && aligned16(q) && aligned16(v) && aligned16(out) &&
           aligned16(dout) && aligned16(dq) && aligned16(dv);
}

// The backward behind the three entry points.  With perm null the packed
// records, norms and key tiles are taken as lsh_attn_fwd left them in ws
// (same offsets); otherwise they are derived from perm, inv, win_lo first.
int attn_bwd(const lsh_problem_t *prob, const void *q, const void *v, const void *out, const void *dout,
             const float *lse, const int32_t *perm, const int32_t *inv, const int32_t *win_lo, void *dq, void *dv,
             void *ws, size_t ws_bytes, void *stream)
{
    const Dims P = dims_of(prob);
    if (!bwd_args_ok(q, v, out, dout, lse, dq, dv) || !ws || ((uintptr_t)ws & 255u))
        return LSH_ERR_INVALID;
    const BwdWs w = bwd_layout(P, prob->dtype, ws);
    if (ws_bytes < w.bytes)
        return LSH_ERR_INVALID;
    const bool derive = perm != nullptr;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_prep(P, prob->dtype, q, perm, inv, win_lo, derive ? w.meta : nullptr, w.srec, w.x,
                               w.rnorm, out, dout, w.D, s);
    if (e == hipSuccess) {
        if (mfma_path_ok(P, prob->dtype)) {
            e = launch_attn_bwd_mfma(P, q, v, dout, lse, w.D, w.meta, w.srec, w.x, w.rnorm, w.ktile, derive, w.qtile,
                                     w.dq_part, dq, dv, s);
        } else {
            e = launch_attn_bwd(P, prob->dtype, q, v, dout, lse, w.D, w.meta, w.srec, w.x, w.rnorm, w.dq_part,
                                w.dk_part, w.dv_part, dq, dv, s);
        }
    }
    return hip_status(e);
}

}  // namespace

extern "C" {

const char *lsh_status_string(int status)
{
    switch (status) {
    case LSH_OK: return "ok";
    case LSH_ERR_INVALID: return "invalid argument";
    case LSH_ERR_UNSUPPORTED: return "unsupported problem";
    case LSH_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int lsh_version(void) { return 600; }

const char *lsh_kernel_name(int kernel)
{
    return (kernel >= 0 && kernel < LSH_KERNEL_COUNT) ? kKernelNames[kernel] : nullptr;
}

int lsh_profile_kernel(int kernel, void *start_event, void *stop_event)
{
    if (kernel < 0 || kernel >= LSH_KERNEL_COUNT)
        return LSH_ERR_INVALID;
    if (!start_event || !stop_event) {
        g_prof_start[kernel] = g_prof_stop[kernel] = nullptr;
    } else {
        g_prof_start[kernel] = (hipEvent_t)start_event;
        g_prof_stop[kernel] = (hipEvent_t)stop_event;
    }
    return LSH_OK;
}

size_t lsh_workspace_bytes(const lsh_problem_t *prob, int kind)
{
    if (validate(prob) != LSH_OK || empty(prob))
        return 0;
    const Dims P = dims_of(prob);
    switch (kind) {
    case LSH_WS_SORT: return sort_ws_bytes(P);
    case LSH_WS_FWD: return fwd_layout(P, nullptr).bytes;
    case LSH_WS_BWD:
    case LSH_WS_TRAIN: return bwd_layout(P, prob->dtype, nullptr).bytes;
    case LSH_WS_REHASH: return rehash_layout(P, prob->dtype, nullptr).bytes;
    default: return 0;
    }
}

int lsh_hash(const lsh_problem_t *prob, const void *q, const void *rot, int32_t *buckets, void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    if (!q || !rot || !buckets || !aligned16(q) || !aligned16(rot) || !aligned16(buckets))
        return LSH_ERR_INVALID;
    return hip_status(launch_hash(dims_of(prob), prob->dtype, q, rot, buckets, (hipStream_t)stream));
}

int lsh_sort(const lsh_problem_t *prob, const int32_t *buckets, int32_t *perm, int32_t *inv, int32_t *win_lo,
             void *ws, size_t ws_bytes, void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    const Dims P = dims_of(prob);
    if (!buckets || !perm || !inv || !win_lo || !ws || ws_bytes < sort_ws_bytes(P) || ((uintptr_t)ws & 255u))
        return LSH_ERR_INVALID;
    return hip_status(launch_sort(P, buckets, perm, inv, win_lo, ws, (hipStream_t)stream));
}

int lsh_sort_noalloc(const lsh_problem_t *prob, const int32_t *buckets, int32_t *perm, int32_t *inv, int32_t *win_lo,
                     void *stream)
{
    static_assert(LSH_SORT_NOALLOC_MAX_BYTES == (size_t)16 << 20, "header and library agree on the scratch size");
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    const Dims P = dims_of(prob);
    if (!buckets || !perm || !inv || !win_lo)
        return LSH_ERR_INVALID;
    if (sort_ws_bytes(P) > sort_noalloc_max_bytes())
        return LSH_ERR_UNSUPPORTED;
    return hip_status(launch_sort_noalloc(P, buckets, perm, inv, win_lo, (hipStream_t)stream));
}

int lsh_attn_fwd(const lsh_problem_t *prob, const void *q, const void *v, const int32_t *perm, const int32_t *inv,
                 const int32_t *win_lo, void *o_rounds, float *lse_rounds, void *ws, size_t ws_bytes, void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    const Dims P = dims_of(prob);
    if (!q || !v || !perm || !inv || !win_lo || !o_rounds || !lse_rounds || !ws || ((uintptr_t)ws & 255u) ||
        !aligned16(q) || !aligned16(v) || !aligned16(o_rounds))
        return LSH_ERR_INVALID;
    const FwdWs w = fwd_layout(P, ws);
    if (ws_bytes < w.bytes)
        return LSH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_prep(P, prob->dtype, q, perm, inv, win_lo, w.meta, w.srec, w.x, w.rnorm, nullptr, nullptr,
                               nullptr, s);
    if (e == hipSuccess) {
        if (mfma_path_ok(P, prob->dtype))
            e = launch_attn_fwd_mfma(P, q, v, w.meta, w.srec, w.x, w.rnorm, w.ktile, o_rounds, lse_rounds, s);
        else
            e = launch_attn_fwd(P, prob->dtype, q, v, w.meta, w.srec, w.x, w.rnorm, o_rounds, lse_rounds, s);
    }
    return hip_status(e);
}

int lsh_combine(const lsh_problem_t *prob, const void *q, const void *v, const void *o_rounds,
                const float *lse_rounds, void *out, float *lse, void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    if (!q || !v || !o_rounds || !lse_rounds || !out || !lse || !aligned16(q) || !aligned16(v) ||
        !aligned16(o_rounds) || !aligned16(out))
        return LSH_ERR_INVALID;
    return hip_status(
        launch_combine(dims_of(prob), prob->dtype, q, v, o_rounds, lse_rounds, out, lse, (hipStream_t)stream));
}

int lsh_attn_bwd(const lsh_problem_t *prob, const void *q, const void *v, const void *out, const void *dout,
                 const float *lse, const int32_t *perm, const int32_t *inv, const int32_t *win_lo, void *dq, void *dv,
                 void *ws, size_t ws_bytes, void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    if (!perm || !inv || !win_lo)
        return LSH_ERR_INVALID;
    return attn_bwd(prob, q, v, out, dout, lse, perm, inv, win_lo, dq, dv, ws, ws_bytes, stream);
}

int lsh_attn_bwd_rehash(const lsh_problem_t *prob, const void *q, const void *v, const void *rot, const void *out,
                        const void *dout, const float *lse, void *dq, void *dv, void *ws, size_t ws_bytes,
                        void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    const Dims P = dims_of(prob);
    // every argument is checked before the hash and sort are launched
    if (!rot || !aligned16(rot) || !bwd_args_ok(q, v, out, dout, lse, dq, dv) || !ws || ((uintptr_t)ws & 255u))
        return LSH_ERR_INVALID;
    const RehashWs w = rehash_layout(P, prob->dtype, ws);
    if (ws_bytes < w.bytes)
        return LSH_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_hash(P, prob->dtype, q, rot, w.buckets, s);
    if (e == hipSuccess)
        e = launch_sort(P, w.buckets, w.perm, w.inv, w.win_lo, w.sort, s);
    if (e != hipSuccess)
        return hip_status(e);
    return attn_bwd(prob, q, v, out, dout, lse, w.perm, w.inv, w.win_lo, dq, dv, w.bwd, w.bwd_bytes, stream);
}

int lsh_attn_bwd_saved(const lsh_problem_t *prob, const void *q, const void *v, const void *out, const void *dout,
                       const float *lse, void *dq, void *dv, void *ws, size_t ws_bytes, void *stream)
{
    int st = validate(prob);
    if (st != LSH_OK || empty(prob))
        return st;
    return attn_bwd(prob, q, v, out, dout, lse, nullptr, nullptr, nullptr, dq, dv, ws, ws_bytes, stream);
}

}  // extern "C"
