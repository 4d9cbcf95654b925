// common.hpp -- internal helpers shared by the gfx950 kernels of liblsh.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsh.h"

namespace lsh {

constexpr int kWave = 64;

// bf16 stored as raw bits.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return __uint_as_float(uint32_t(x.bits) << 16); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x)
{
    // round to nearest even; NaN stays NaN
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return bf16{uint16_t((u >> 16) | 0x40u)};
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16{uint16_t(u >> 16)};
}

template <typename T> __device__ __forceinline__ float ld(const T *p, size_t i) { return to_f(p[i]); }

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += __shfl_xor(x, o, kWave);
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}

// Packed per-(position, round) record: low 16 bits = sorted index of the
// position in that round, high 16 bits = w = sorted index - win_lo, the number
// of members of the round's attended set other than the position itself.
// Sorted-order record: low 16 bits = position, high 16 bits = w.
__device__ __forceinline__ uint32_t rec_lo(uint32_t r) { return r & 0xffffu; }
__device__ __forceinline__ uint32_t rec_hi(uint32_t r) { return r >> 16; }

// Is key j (sorted index sj in round r') a member other than i of the
// round-r' attended set of query i, given i's record (si, wi) for r'?
// The set without i is the sorted range [si - wi, si - 1].
__device__ __forceinline__ bool in_window(uint32_t qrec, uint32_t sj)
{
    uint32_t si = rec_lo(qrec), wi = rec_hi(qrec);
    return (si - 1u - sj) < wi;   // unsigned: 0 <= si-1-sj < wi
}

// Non-causal window record, per (position, round): low 16 bits = hi, the
// last sorted index of the round's attended set (the last row of the
// position's bucket inside its chunk), high 16 bits = span = hi - win_lo.
// The set, self included, is the sorted range [hi - span, hi].
__device__ __forceinline__ bool in_span(uint32_t wrec, uint32_t sj)
{
    return (rec_lo(wrec) - sj) <= rec_hi(wrec);   // unsigned: 0 <= hi-sj <= span
}

// Kinds of attended set (see include/lsh.h): the causal band of a bucket
// run (kBand), a sorted range [win_lo, hi] per query (kRange: non-causal
// problems, with or without the bucket condition), or, causal without the
// bucket condition, the chunk window filtered by position (kRangePos).
enum SetKind { kBand = 0, kRange = 1, kRangePos = 2 };

// dup_bucket: duplicates counted over bucket membership (LSH_FLAG_DUP_BY_BUCKET)
// instead of the first-owner rule.
struct Dims {
    int B, H, L, d, nh, nb, m;
    float scale;
    bool causal, bucket_mask, dup_bucket;
    int BH() const { return B * H; }
    int kind() const { return causal ? (bucket_mask ? kBand : kRangePos) : kRange; }
};

inline Dims dims_of(const lsh_problem_t *p)
{
    return Dims{p->batch, p->heads, p->seq_len, p->head_dim, p->n_hashes, p->n_buckets, p->chunk_len,
                p->scale, p->causal != 0, (p->flags & LSH_FLAG_NO_BUCKET_MASK) == 0,
                (p->flags & LSH_FLAG_DUP_BY_BUCKET) != 0};
}

// Number of rounds in which two rows share a bucket, given each one's
// per-round bucket-run starts (the sorted index where its bucket begins).
__device__ __forceinline__ int shared_buckets(const uint32_t *__restrict__ bi, const uint32_t *__restrict__ bj,
                                              int nh)
{
    int n = 0;
    for (int r = 0; r < nh; ++r)
        n += bi[r] == bj[r];
    return n;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Instrumentation brackets around kernel launches (see lsh_profile_kernel).
void prof_begin(int kernel, hipStream_t st);
void prof_end(int kernel, hipStream_t st);

struct ProfScope {
    int k;
    hipStream_t s;
    ProfScope(int kernel, hipStream_t st) : k(kernel), s(st) { prof_begin(k, s); }
    ~ProfScope() { prof_end(k, s); }
};

// Launch helpers implemented per kernel file; all return hipError_t.
hipError_t launch_hash(const Dims &, int dtype, const void *q, const void *rot, int32_t *buckets,
                       hipStream_t);
hipError_t launch_sort(const Dims &, const int32_t *buckets, int32_t *perm, int32_t *inv,
                       int32_t *win_lo, void *ws, hipStream_t);
size_t sort_ws_bytes(const Dims &);
// lsh_sort with its count matrix in the library's static device array (no
// workspace argument): fails with hipErrorInvalidValue if sort_ws_bytes
// exceeds sort_noalloc_max_bytes().
hipError_t launch_sort_noalloc(const Dims &, const int32_t *buckets, int32_t *perm, int32_t *inv, int32_t *win_lo,
                               hipStream_t);
size_t sort_noalloc_max_bytes();
// Window-related records beyond meta and srec, each null where the problem
// has no use for it: wmeta (kRange / kRangePos window ends), alone and cmin
// (kRangePos lone flags and their per-chunk scratch), bmeta and bscr
// (dup_bucket: the start of each row's bucket run per round, [B*H*L][nh],
// and its scratch of one word per 1024 sorted rows).
struct Extra {
    uint32_t *wmeta;
    uint8_t *alone;
    uint32_t *cmin, *bmeta, *bscr;
};

// Packed records, inverse norms, the extra records and (with out, dout)
// D = dO . O; with meta null only D is written (the records are already in
// place).
hipError_t launch_prep(const Dims &, int dtype, const void *q, const int32_t *perm, const int32_t *inv,
                       const int32_t *win_lo, uint32_t *meta, uint32_t *srec, const Extra &x, float *rnorm,
                       const void *out, const void *dout, float *D, hipStream_t);
hipError_t launch_attn_fwd(const Dims &, int dtype, const void *q, const void *v, const uint32_t *meta,
                           const uint32_t *srec, const Extra &x, const float *rnorm, void *o_rounds,
                           float *lse_rounds, hipStream_t);
hipError_t launch_combine(const Dims &, int dtype, const void *q, const void *v, const void *o_rounds,
                          const float *lse_rounds, void *out, float *lse, hipStream_t);
hipError_t launch_attn_bwd(const Dims &, int dtype, const void *q, const void *v, const void *dout,
                           const float *lse, const float *D, const uint32_t *meta, const uint32_t *srec,
                           const Extra &x, const float *rnorm, float *dq_part, float *dk_part, float *dv_part,
                           void *dq, void *dv, hipStream_t);

}  // namespace lsh

namespace lsh {

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void load8(const bf16 *p, float out[8])
{
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(w[k] << 16);
        out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load8(const float *p, float out[8])
{
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Store 8 consecutive elements.
__device__ __forceinline__ void store8(bf16 *p, const float x[8])
{
    uint4 u;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)from_f<bf16>(x[2 * k]).bits | ((uint32_t)from_f<bf16>(x[2 * k + 1]).bits << 16);
    u.x = w[0]; u.y = w[1]; u.z = w[2]; u.w = w[3];
    *reinterpret_cast<uint4 *>(p) = u;
}

__device__ __forceinline__ void store8(float *p, const float x[8])
{
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Sum over aligned groups of n lanes (n a power of two dividing 64).
__device__ __forceinline__ float group_sum(float x, int n)
{
    for (int o = n / 2; o > 0; o >>= 1)
        x += __shfl_xor(x, o, kWave);
    return x;
}

__device__ __forceinline__ float readlane(float x, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ int readlane(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// Order LDS traffic of the lanes of one wave.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace lsh

namespace lsh {

// MFMA operand types (gfx950 bf16 matrix instructions).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// plain 16-byte vector (HIP's uint4 is a struct that defeats register promotion of arrays)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16: lane l supplies A[l%32][8(l/32) .. +7] and
// B[8(l/32) .. +7][l%32]; it receives C[8g + 4(l/32) + t][l%32] in acc[4g+t].
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8(l/16) .. +7] and
// B[8(l/16) .. +7][l%16]; it receives C[4(l/16) + t][l%16] in acc[t].
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ u32x4_t ld16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4_t v) { *reinterpret_cast<u32x4_t *>(p) = v; }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives in slot
// k element i % 4 of the 4-element chunk addressed by lane 4 k + i / 4.  If
// lane m of the group addresses row R0 + m / 4, columns C0 + 4 (m % 4) .. +3 of
// a row-major bf16 tile, lane i receives rows R0 .. R0 + 3 of column C0 + i:
// a transposed read.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p)
{
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)((__attribute__((address_space(3))) uint16_t *)p));
    return __builtin_bit_cast(uint2, v);
}

// A operand of v_mfma_f32_32x32x16_bf16 read transposed from a row-major LDS
// tile T[row][col] (pitch P elements): lane l (column col0 + l % 32, half
// h = l / 32) receives rows 16 j + 4 h + {0..3} in slots 0..3 and
// 16 j + 8 + 4 h + {0..3} in slots 4..7.  This matches a B operand whose slot s
// holds accumulator value 8 j + s of a 32x32 tile (rows 8 g + 4 h + t).
template <int P>
__device__ __forceinline__ bf16x8_t tile_t(const uint16_t *T, int j, int col0, int lane)
{
    const int g = lane / 16, m = lane % 16;
    const int row = 16 * j + 4 * (g / 2) + m / 4;
    const int col = col0 + 16 * (g % 2) + 4 * (m % 4);
    const uint2 a = lds_read_tr16(T + row * P + col);
    const uint2 b = lds_read_tr16(T + (row + 8) * P + col);
    const u32x4_t u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8_t, u);
}

// exp2 on the transcendental unit (v_exp_f32, denormal results flushed)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Packed 16-bit window test for two keys at once.  With si1 = s_i - 1 and
// w_i of query i in some round (both broadcast to the two halves), and the two
// keys' sorted indices sk in that round, a half of the result is nonzero iff
// that key lies in the sorted window [s_i - w_i, s_i - 1] (wrapping 16-bit
// subtraction, then saturating: w - (si1 - sk) > 0  <=>  si1 - sk < w).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t win_hits2(uint32_t si1p, uint32_t wp, uint32_t skp)
{
    const u16x2_t x = __builtin_bit_cast(u16x2_t, si1p) - __builtin_bit_cast(u16x2_t, skp);
    const u16x2_t z = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, wp), x);
    return __builtin_bit_cast(uint32_t, z);
}
// Exchange across lanes l and l ^ 16 (l ^ 32) with v_permlane16_swap_b32
// (v_permlane32_swap_b32): swapping a value with itself leaves the row pair's
// two values in the two results, in the same order on both lanes.
__device__ __forceinline__ float max_xor16(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ uint32_t bcast16(uint32_t x) { return (x & 0xffffu) * 0x10001u; }

// Workgroup index remapped so that consecutive logical blocks run on the same
// XCD (the hardware deals workgroups round-robin over the 8 XCDs, each with
// its own L2): logical = (i % 8) * (n / 8) + i / 8 when 8 divides n.
__device__ __forceinline__ int xcd_block(int i, int n)
{
    return (n % 8 == 0) ? (i % 8) * (n / 8) + i / 8 : i;
}

// MFMA path (bf16, d in {64, 128}); see attn_mfma.hip
bool mfma_path_ok(const Dims &, int dtype);
size_t mfma_ktile_bytes(const Dims &);
size_t mfma_qtile_bytes(const Dims &);
// bf16 per-round partials dq (query side), dk rn (key side, before the key
// normalisation) and dv, [B*H*L][nh][3][d] (token-major), in one buffer of this size
size_t bwd_mfma_part_bytes(const Dims &);
hipError_t launch_attn_fwd_mfma(const Dims &, const void *q, const void *v, const uint32_t *meta,
                                const uint32_t *srec, const Extra &x, const float *rnorm, uint8_t *ktile,
                                void *o_rounds, float *lse_rounds, hipStream_t);
hipError_t launch_attn_bwd_mfma(const Dims &, const void *q, const void *v, const void *dout, const float *lse,
                                const float *D, const uint32_t *meta, const uint32_t *srec, const Extra &x,
                                const float *rnorm, uint8_t *ktile, bool make_ktile, uint8_t *qtile, void *part,
                                void *dq, void *dv, hipStream_t);

}  // namespace lsh
