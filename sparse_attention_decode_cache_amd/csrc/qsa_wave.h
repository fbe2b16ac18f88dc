// qsa_wave.h -- wave64 reductions and scans on DPP lane moves (gfx9 DPP:
// quad_perm, row_shr, row_mirror, row_bcast:15/31), which execute as VALU
// operand modifiers instead of LDS-crossbar permutes, plus readlane for the
// four 16-lane rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {
namespace wave {

// DPP control codes (gfx9)
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowMirror = 0x140;    // lane i <- 15 - i within a row
constexpr int kRowHalfMirror = 0x141; // lane i <- 7 - i within a half row
constexpr int kRowBcast15 = 0x142;   // lane 15 of row r -> row r+1
constexpr int kRowBcast31 = 0x143;   // lane 31 -> rows 2 and 3

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline uint32_t dpp(uint32_t x)
{
    // lanes without a source (or in masked rows) read 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}

template <int CTRL>
__device__ inline uint64_t dpp64(uint64_t x)
{
    const uint32_t lo = dpp<CTRL>((uint32_t)x), hi = dpp<CTRL>((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint32_t readlane(uint32_t x, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Inclusive prefix sum over the 64 lanes.
__device__ inline uint32_t incl_scan_add(uint32_t x)
{
    x += dpp<kRowShr1>(x);
    x += dpp<kRowShr2>(x);
    x += dpp<kRowShr4>(x);
    x += dpp<kRowShr8>(x);
    x += dpp<kRowBcast15, 0xA>(x);
    x += dpp<kRowBcast31, 0xC>(x);
    return x;
}

// Reduce within each 16-lane row with an associative, commutative op; every
// lane of a row ends with the row's result.
template <class Op>
__device__ inline uint32_t row_reduce(uint32_t x, Op op)
{
    x = op(x, dpp<kQuadXor1>(x));
    x = op(x, dpp<kQuadXor2>(x));
    x = op(x, dpp<kRowHalfMirror>(x));
    x = op(x, dpp<kRowMirror>(x));
    return x;
}

template <class Op>
__device__ inline uint64_t row_reduce64(uint64_t x, Op op)
{
    x = op(x, dpp64<kQuadXor1>(x));
    x = op(x, dpp64<kQuadXor2>(x));
    x = op(x, dpp64<kRowHalfMirror>(x));
    x = op(x, dpp64<kRowMirror>(x));
    return x;
}

// Float reductions inside each 16-lane row (every lane of a row gets its row's
// result; fixed combination order).
__device__ inline float row_max_f(float v)
{
    return __uint_as_float(row_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}

__device__ inline float row_sum_f(float v)
{
    return __uint_as_float(row_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

// Whole-wave reductions; the result is wave-uniform.
__device__ inline uint32_t reduce_add(uint32_t x)
{
    x = row_reduce(x, [](uint32_t a, uint32_t b) { return a + b; });
    return readlane(x, 0) + readlane(x, 16) + readlane(x, 32) + readlane(x, 48);
}

__device__ inline float reduce_add_f(float v)
{
    uint32_t x = __float_as_uint(v);
    x = row_reduce(x, [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    });
    // fixed combination order: (r0 + r1) + (r2 + r3)
    return (__uint_as_float(readlane(x, 0)) + __uint_as_float(readlane(x, 16))) +
           (__uint_as_float(readlane(x, 32)) + __uint_as_float(readlane(x, 48)));
}

__device__ inline float reduce_max_f(float v)
{
    uint32_t x = __float_as_uint(v);
    x = row_reduce(x, [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    });
    return fmaxf(fmaxf(__uint_as_float(readlane(x, 0)), __uint_as_float(readlane(x, 16))),
                 fmaxf(__uint_as_float(readlane(x, 32)), __uint_as_float(readlane(x, 48))));
}

__device__ inline float reduce_min_f(float v)
{
    uint32_t x = __float_as_uint(v);
    x = row_reduce(x, [](uint32_t a, uint32_t b) {
        return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
    });
    return fminf(fminf(__uint_as_float(readlane(x, 0)), __uint_as_float(readlane(x, 16))),
                 fminf(__uint_as_float(readlane(x, 32)), __uint_as_float(readlane(x, 48))));
}

__device__ inline uint32_t reduce_min_u32(uint32_t x)
{
    auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
    x = row_reduce(x, mn);
    return mn(mn(readlane(x, 0), readlane(x, 16)), mn(readlane(x, 32), readlane(x, 48)));
}

__device__ inline uint32_t reduce_max_u32(uint32_t x)
{
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    x = row_reduce(x, mx);
    return mx(mx(readlane(x, 0), readlane(x, 16)), mx(readlane(x, 32), readlane(x, 48)));
}

__device__ inline uint64_t readlane64(uint64_t x, int lane)
{
    return ((uint64_t)readlane((uint32_t)(x >> 32), lane) << 32) | readlane((uint32_t)x, lane);
}

__device__ inline uint64_t reduce_min_u64(uint64_t x)
{
    auto mn = [](uint64_t a, uint64_t b) { return a < b ? a : b; };
    x = row_reduce64(x, mn);
    return mn(mn(readlane64(x, 0), readlane64(x, 16)), mn(readlane64(x, 32), readlane64(x, 48)));
}

__device__ inline uint64_t reduce_max_u64(uint64_t x)
{
    auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
    x = row_reduce64(x, mx);
    return mx(mx(readlane64(x, 0), readlane64(x, 16)), mx(readlane64(x, 32), readlane64(x, 48)));
}

}  // namespace wave
}  // namespace qsa
