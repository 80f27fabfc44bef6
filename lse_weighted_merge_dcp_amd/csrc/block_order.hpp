// block_order.hpp -- XCD-aware orders of a one-dimensional grid's workgroups.
//
// An MI355X dispatches workgroup b of a grid to XCD b mod 8 (round robin);
// each XCD has its own L2.  A kernel that wants a different order maps its
// dispatch index b to a logical block index with one of these functions.
// Both are bijections of [0, n) (unit-tested on the host for many n).
// Plain C++: the same code runs on the host and on the GPU.
#pragma once
#include <stdint.h>

#include "fastdiv.hpp"   // DCP_HD

namespace dcp {

// Each XCD walks one contiguous range of the logical blocks: XCD x takes
// [x q + min(x, r), ...) of n = 8 q + r blocks, in dispatch order.
DCP_HD uint32_t xcd_contiguous_order(uint32_t b, uint32_t n) {
    const uint32_t x = b & 7u, k = b >> 3;
    const uint32_t q = n >> 3, rem = n & 7u;
    return x * q + (x < rem ? x : rem) + k;
}

// The XCDs take turns on chunks of C consecutive logical blocks: XCD x's
// k-th workgroup is block k mod C of chunk (k / C) * 8 + x, so at any time
// the eight XCDs work on eight neighbouring chunks.  Blocks past the last
// whole round of 8 C fall back to the contiguous order among themselves;
// a grid of at most 8 C blocks is exactly xcd_contiguous_order.
template <uint32_t C>
DCP_HD uint32_t xcd_chunked_order(uint32_t b, uint32_t n) {
    const uint32_t full = n / (8u * C) * (8u * C);
    if (b < full) {
        const uint32_t x = b & 7u, k = b >> 3;
        return ((k / C) * 8u + x) * C + (k % C);
    }
    return full + xcd_contiguous_order(b - full, n - full);
}

// The same order computed without a branch on the grid size (both sides
// evaluated, then selected), so that a kernel can issue all its argument
// loads before its first wait.
template <uint32_t C>
DCP_HD uint32_t xcd_chunked_order_sel(uint32_t b, uint32_t n) {
    const uint32_t full = n / (8u * C) * (8u * C);
    const uint32_t x = b & 7u, k = b >> 3;
    const uint32_t in_round = ((k / C) * 8u + x) * C + (k % C);
    const uint32_t tail = full + xcd_contiguous_order(b >= full ? b - full : 0u, n - full);
    return b < full ? in_round : tail;
}

}  // namespace dcp
