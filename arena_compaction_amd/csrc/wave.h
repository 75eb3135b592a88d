// wave.h -- scans and reductions across the 64 lanes of one wave through DPP
// (an operand of a VALU instruction read from another lane of the same
// wave), in place of LDS permutes: no LDS round trip and no lane-index
// arithmetic per step, which is most of a small table's scan latency.
//
// DPP controls used (CDNA/GFX9 encoding):
//   row_shr:d       lane i reads lane i - d of its row of 16; a lane with
//                   i % 16 < d has no source and reads 0
//   row_bcast:15    each lane of rows 1 and 3 reads lane 15 of the row before
//   row_bcast:31    each lane of rows 2 and 3 reads lane 31
//   wave_shr:1      lane i reads lane i - 1; lane 0 reads 0
//   quad_perm, row_half_mirror, row_mirror: permutations inside a row
// A row outside an instruction's row mask is not written and reads 0 too.
// Values wider than 32 bits move one 32-bit word at a time.
#ifndef ARENA_COMPACTION_WAVE_H
#define ARENA_COMPACTION_WAVE_H
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ac {
namespace {

constexpr int kDppRowShr = 0x110;  // | d, for d in 1..15
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2, 3, 0, 1]

// x as read from the lane the control names (0 where there is none).
template <int CTRL, int ROW_MASK = 0xf, typename T>
__device__ inline T dpp_move(const T &x) {
    static_assert(sizeof(T) % 4 == 0, "whole 32-bit words");
    constexpr int W = sizeof(T) / 4;
    int w[W];
    __builtin_memcpy(w, &x, sizeof(T));
#pragma unroll
    for (int k = 0; k < W; ++k) w[k] = __builtin_amdgcn_update_dpp(0, w[k], CTRL, ROW_MASK, 0xf, true);
    T y;
    __builtin_memcpy(&y, w, sizeof(T));
    return y;
}

// x of lane L, in every lane (a wave-uniform value).
template <int L, typename T>
__device__ inline T read_lane(const T &x) {
    static_assert(sizeof(T) % 4 == 0, "whole 32-bit words");
    constexpr int W = sizeof(T) / 4;
    int w[W];
    __builtin_memcpy(w, &x, sizeof(T));
#pragma unroll
    for (int k = 0; k < W; ++k) w[k] = __builtin_amdgcn_readlane(w[k], L);
    T y;
    __builtin_memcpy(&y, w, sizeof(T));
    return y;
}

// x, the same in every active lane of the wave (a value read from LDS that
// every lane read at one address, say), in scalar registers: the compiler
// cannot see that it is uniform, and would keep one copy a lane.
template <typename T>
__device__ inline T wave_uniform(const T &x) {
    static_assert(sizeof(T) % 4 == 0, "whole 32-bit words");
    constexpr int W = sizeof(T) / 4;
    int w[W];
    __builtin_memcpy(w, &x, sizeof(T));
#pragma unroll
    for (int k = 0; k < W; ++k) w[k] = __builtin_amdgcn_readfirstlane(w[k]);
    T y;
    __builtin_memcpy(&y, w, sizeof(T));
    return y;
}

// Inclusive scan in lane order: lane i gets op(x_0, ..., x_i).  op(a, b)
// combines a before b, is associative, and has the all-zero value as its
// identity.  SPAN: lanes that hold values (64, or at most 16; lanes past it
// hold the identity, and the result is defined for the first SPAN lanes).
template <int SPAN = 64, typename T, typename Op>
__device__ inline T wave_incl_scan(T x, Op op) {
    static_assert(SPAN == 64 || (SPAN >= 1 && SPAN <= 16), "a whole wave or one row");
    if constexpr (SPAN > 1) x = op(dpp_move<kDppRowShr | 1>(x), x);
    if constexpr (SPAN > 2) x = op(dpp_move<kDppRowShr | 2>(x), x);
    if constexpr (SPAN > 4) x = op(dpp_move<kDppRowShr | 4>(x), x);
    if constexpr (SPAN > 8) x = op(dpp_move<kDppRowShr | 8>(x), x);
    if constexpr (SPAN > 16) {
        x = op(dpp_move<kDppRowBcast15, 0xa>(x), x);  // rows 1, 3 after rows 0, 2
        x = op(dpp_move<kDppRowBcast31, 0xc>(x), x);  // rows 2, 3 after rows 0-1
    }
    return x;
}

// The inclusive result of the lane before (the identity in lane 0): with
// wave_incl_scan, the exclusive scan.
template <typename T>
__device__ inline T wave_shift_up(const T &x) {
    return dpp_move<kDppWaveShr1>(x);
}

// op over the first SPAN lanes (64, or a power of two up to 16), in every
// lane.  op is associative and commutative; no identity is needed.
template <int SPAN = 64, typename T, typename Op>
__device__ inline T wave_reduce(T x, Op op) {
    static_assert(SPAN == 64 || (SPAN >= 1 && SPAN <= 16 && (SPAN & (SPAN - 1)) == 0),
                  "a whole wave or a power of two inside one row");
    if constexpr (SPAN > 1) x = op(x, dpp_move<kDppQuadSwap1>(x));
    if constexpr (SPAN > 2) x = op(x, dpp_move<kDppQuadSwap2>(x));
    if constexpr (SPAN > 4) x = op(x, dpp_move<kDppRowHalfMirror>(x));
    if constexpr (SPAN > 8) x = op(x, dpp_move<kDppRowMirror>(x));  // each row's total
    if constexpr (SPAN > 16) {
        // rows 1 and 3 take rows 0 and 2; row 3 then takes rows 0-1: lane 63
        // holds the total (rows 0 and 2 end with partial values)
        x = op(x, dpp_move<kDppRowBcast15, 0xa>(x));
        x = op(x, dpp_move<kDppRowBcast31, 0xc>(x));
        return read_lane<63>(x);
    } else {
        return read_lane<0>(x);
    }
}

}  // namespace
}  // namespace ac

#endif
