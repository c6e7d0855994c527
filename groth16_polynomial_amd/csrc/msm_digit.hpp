// The MSM's signed window digits (host and device).
#pragma once

#include <stdint.h>

#include "fr.hpp"  // G16_HD

namespace g16 {

// Signed digit of window w of a 256-bit scalar k (eight little-endian words):
// d = raw + b(wc - 1) - 2^c b(wc + c - 1), where raw is bits [wc, wc + c) and b(j) bit j.
// Summed over the windows the correction terms telescope, so sum_w d_w 2^(wc) = k when
// the last window's top bit is zero (k < 2^(c ceil(255/c) - 1), true for k < 2^254);
// |d| <= 2^(c-1).  c <= 31.
G16_HD int32_t msm_digit(const uint32_t k[8], uint32_t w, uint32_t c) {
    auto bits = [&](uint32_t pos, uint32_t len) -> uint32_t {
        const uint32_t i = pos >> 5, s = pos & 31u;
        const uint64_t lo = i < 8 ? k[i] : 0u;
        const uint64_t hi = i + 1 < 8 ? k[i + 1] : 0u;
        return (uint32_t)((lo | (hi << 32)) >> s) & ((1u << len) - 1u);
    };
    const uint32_t start = w * c;
    const uint32_t raw = bits(start, c);
    const uint32_t below = start ? bits(start - 1, 1) : 0u;
    const uint32_t top = raw >> (c - 1);
    return (int32_t)raw + (int32_t)below - (int32_t)(top << c);
}

}  // namespace g16
