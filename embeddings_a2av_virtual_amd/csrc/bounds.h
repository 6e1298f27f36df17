// bounds.h — the last-line bounds check of the payload kernels, written so
// that no sum can wrap.
//
// A copy of n rows starting at row r0 stays inside a buffer of cap rows when
// r0 + n <= cap. Written as that sum, the check passes corrupt values whose
// sum wraps past 2^64 (or, as signed int64, past 2^63) back into range: a
// negative n, or an r0 near 2^64, would be let through. Compared as below,
// with every value read as an unsigned 64-bit integer, it passes exactly the
// pairs with 0 <= r0, 0 <= n and r0 + n <= cap in exact integer arithmetic,
// for any cap in [0, 2^63) (a negative int64 r0 or n reads as 2^63 or more
// and fails the first or the second comparison).
//
// Plain C++ with no HIP dependency, so the host tests compile and exercise
// the very same function.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define A2AV_HD __host__ __device__
#else
#define A2AV_HD
#endif

namespace a2av {

// Rows [r0, r0 + n) lie inside [0, cap): r0 <= cap and n <= cap - r0, with
// no sum formed. cap is a row count the host has checked to be in [0, 2^63).
A2AV_HD inline bool span_fits(uint64_t r0, uint64_t n, uint64_t cap) {
    return r0 <= cap && n <= cap - r0;
}

}  // namespace a2av
