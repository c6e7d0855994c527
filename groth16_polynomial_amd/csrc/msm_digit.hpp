// The MSM's signed window digits and their 16-bit codes (host and device).
#pragma once

#include <stdint.h>

#include "fr.hpp"  // G16_HD

namespace g16 {

// Bits [pos, pos + len) of a 256-bit scalar k (eight little-endian words), len <= 31;
// bits past 255 read as zero.
G16_HD uint32_t msm_bits(const uint32_t k[8], uint32_t pos, uint32_t len) {
    const uint32_t i = pos >> 5, s = pos & 31u;
    const uint64_t lo = i < 8 ? k[i] : 0u;
    const uint64_t hi = i + 1 < 8 ? k[i + 1] : 0u;
    return (uint32_t)((lo | (hi << 32)) >> s) & ((1u << len) - 1u);
}

// The signed digits of a scalar k < 2^254 in windows of c bits (1 <= c <= 30), least
// significant first, passed to emit(w, d): d_w = raw_w + carry_w, where raw_w is bits
// [wc, wc + c), and a digit above 2^(c-1) becomes d_w - 2^c with a carry of one into the
// next window.  So every d_w lies in [1 - 2^(c-1), 2^(c-1)] (2^c values: the magnitudes
// 1 .. 2^(c-1) name the window's buckets) and sum_w d_w 2^(wc) = k.  The last of the
// ceil(255/c) windows never carries out: it holds bits below 254 only, fewer than c, so
// its raw value is below 2^(c-1).
template <class Emit>
G16_HD void msm_recode(const uint32_t k[8], uint32_t c, Emit&& emit) {
    const uint32_t windows = (255u + c - 1u) / c;
    const uint32_t half = 1u << (c - 1u);
    uint32_t carry = 0;
    for (uint32_t w = 0; w < windows; ++w) {
        const uint32_t v = msm_bits(k, w * c, c) + carry;
        carry = v > half ? 1u : 0u;
        emit(w, (int32_t)v - (int32_t)(carry << c));
    }
}

// A digit as a 16-bit code (c <= 16): d + 2^(c-1) - 1, in [0, 2^c).  The zero digit is
// 2^(c-1) - 1.
G16_HD uint32_t msm_code(int32_t d, uint32_t c) {
    return (uint32_t)(d + (int32_t)(1u << (c - 1u)) - 1);
}

// The bucket row |d| - 1 and the sign of a code's digit; false for the zero digit.
G16_HD bool msm_decode(uint32_t code, uint32_t c, uint32_t& row, uint32_t& neg) {
    const int32_t e = (int32_t)code - (int32_t)(1u << (c - 1u));  // d - 1
    neg = e < -1 ? 1u : 0u;
    row = (uint32_t)(e >= 0 ? e : -e - 2);
    return e != -1;
}

}  // namespace g16
