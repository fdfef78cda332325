// Wave64 and workgroup primitives for gfx950 (CDNA4).
//
// Cross-lane moves use DPP (data-parallel primitives of the GFX9 family):
// row_shr:1/2/4/8 scan inside each row of 16 lanes, row_bcast:15 and
// row_bcast:31 carry row totals across the four rows, wave_shr:1 turns an
// inclusive scan into an exclusive one.  A lane whose DPP source does not
// exist keeps the `old` operand, which is always the operation's identity
// here.  Integer sums are order-free; the pair composition of the exact sum
// is associative but not commutative, and every scan below composes the
// lower lanes' value first.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "exseq_rules.h"

namespace exseq {

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// DPP controls (GFX9 encoding).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, Ctrl, RowMask, 0xF, false);
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ int64_t dpp_i64(int64_t v, int64_t old)
{
    const uint32_t lo = dpp_u32<Ctrl, RowMask>((uint32_t)v, (uint32_t)old);
    const uint32_t hi = dpp_u32<Ctrl, RowMask>((uint32_t)((uint64_t)v >> 32),
                                               (uint32_t)((uint64_t)old >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ double dpp_f64(double v, double old)
{
    return bitsd((uint64_t)dpp_i64<Ctrl, RowMask>((int64_t)dbits(v), (int64_t)dbits(old)));
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ Pair dpp_pair(Pair v)
{
    return Pair{dpp_i64<Ctrl, RowMask>(v.r0, 0), dpp_i64<Ctrl, RowMask>(v.r1, 0)};
}

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    return bitsd((uint64_t)readlane_i64((int64_t)dbits(v), lane));
}
__device__ __forceinline__ Pair readlane_pair(Pair v, int lane)
{
    return Pair{readlane_i64(v.r0, lane), readlane_i64(v.r1, lane)};
}

// Inclusive prefix sum over the wave (int64).
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v)
{
    v += dpp_i64<kDppRowShr1>(v, 0);
    v += dpp_i64<kDppRowShr2>(v, 0);
    v += dpp_i64<kDppRowShr4>(v, 0);
    v += dpp_i64<kDppRowShr8>(v, 0);
    v += dpp_i64<kDppRowBcast15, 0xA>(v, 0);
    v += dpp_i64<kDppRowBcast31, 0xC>(v, 0);
    return v;
}

// Inclusive ordered scan of pairs over the wave: lane i gets lanes 0..i
// composed in order.
__device__ __forceinline__ Pair wave_incl_scan_pair(Pair v)
{
    v = compose(dpp_pair<kDppRowShr1>(v), v);
    v = compose(dpp_pair<kDppRowShr2>(v), v);
    v = compose(dpp_pair<kDppRowShr4>(v), v);
    v = compose(dpp_pair<kDppRowShr8>(v), v);
    v = compose(dpp_pair<kDppRowBcast15, 0xA>(v), v);
    v = compose(dpp_pair<kDppRowBcast31, 0xC>(v), v);
    return v;
}

// The previous lane's value (identity in lane 0).
__device__ __forceinline__ Pair wave_shift_pair(Pair v) { return dpp_pair<kDppWaveShr1>(v); }

// Sum over the wave in a fixed order (a row scan then the row totals); the
// same bits in every lane.
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v)
{
    return readlane_i64(wave_incl_scan_i64(v), 63);
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<kDppRowShr1>(v, 0.0);
    v += dpp_f64<kDppRowShr2>(v, 0.0);
    v += dpp_f64<kDppRowShr4>(v, 0.0);
    v += dpp_f64<kDppRowShr8>(v, 0.0);
    v += dpp_f64<kDppRowBcast15, 0xA>(v, 0.0);
    v += dpp_f64<kDppRowBcast31, 0xC>(v, 0.0);
    return readlane_f64(v, 63);
}

// N independent wave sums, each step taken for all N before the next so
// that the N dependency chains overlap.  Each sum has the same fixed order
// as the single-value version.
template <int N>
__device__ __forceinline__ void wave_sum_i64_n(int64_t *v)
{
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_i64<kDppRowShr1>(v[k], 0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_i64<kDppRowShr2>(v[k], 0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_i64<kDppRowShr4>(v[k], 0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_i64<kDppRowShr8>(v[k], 0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_i64<kDppRowBcast15, 0xA>(v[k], 0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_i64<kDppRowBcast31, 0xC>(v[k], 0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] = readlane_i64(v[k], 63);
}

template <int N>
__device__ __forceinline__ void wave_sum_f64_n(double *v)
{
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_f64<kDppRowShr1>(v[k], 0.0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_f64<kDppRowShr2>(v[k], 0.0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_f64<kDppRowShr4>(v[k], 0.0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_f64<kDppRowShr8>(v[k], 0.0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_f64<kDppRowBcast15, 0xA>(v[k], 0.0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] += dpp_f64<kDppRowBcast31, 0xC>(v[k], 0.0);
#pragma unroll
    for (int k = 0; k < N; k++)
        v[k] = readlane_f64(v[k], 63);
}

// Minimum and maximum over the wave, in every lane.
__device__ __forceinline__ int64_t wave_min_i64(int64_t v)
{
    int64_t o;
    o = dpp_i64<kDppRowShr1>(v, v);
    v = o < v ? o : v;
    o = dpp_i64<kDppRowShr2>(v, v);
    v = o < v ? o : v;
    o = dpp_i64<kDppRowShr4>(v, v);
    v = o < v ? o : v;
    o = dpp_i64<kDppRowShr8>(v, v);
    v = o < v ? o : v;
    o = dpp_i64<kDppRowBcast15, 0xA>(v, v);
    v = o < v ? o : v;
    o = dpp_i64<kDppRowBcast31, 0xC>(v, v);
    v = o < v ? o : v;
    return readlane_i64(v, 63);
}
__device__ __forceinline__ int64_t wave_max_i64(int64_t v)
{
    int64_t o;
    o = dpp_i64<kDppRowShr1>(v, v);
    v = o > v ? o : v;
    o = dpp_i64<kDppRowShr2>(v, v);
    v = o > v ? o : v;
    o = dpp_i64<kDppRowShr4>(v, v);
    v = o > v ? o : v;
    o = dpp_i64<kDppRowShr8>(v, v);
    v = o > v ? o : v;
    o = dpp_i64<kDppRowBcast15, 0xA>(v, v);
    v = o > v ? o : v;
    o = dpp_i64<kDppRowBcast31, 0xC>(v, v);
    v = o > v ? o : v;
    return readlane_i64(v, 63);
}

// Ordered composition of the wave's pairs (lane 0 first), in every lane.
__device__ __forceinline__ Pair wave_reduce_pair(Pair v)
{
    return readlane_pair(wave_incl_scan_pair(v), 63);
}

// Cross-workgroup status words.  Each word is self-contained (epoch, flag
// and value in one 64-bit atomic access), so no other memory has to be
// ordered with it: relaxed atomics at agent scope (coherent across the 8
// XCDs, whose L2s are separate) are enough, and they avoid the L2
// write-back/invalidate that release/acquire ordering costs on this chip.
__device__ __forceinline__ uint64_t load_relaxed_u64(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed_u64(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace exseq
