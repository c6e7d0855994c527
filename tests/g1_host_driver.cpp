// Host build of the library's base-field and G1 layers (fp.hpp, g1.hpp) and of the MSM's
// digit recoding (msm_digit.hpp), driven by tests/test_g1_host.py.
//
// Input lines "op arg..." with hexadecimal arguments; field ops act on Montgomery
// representatives as stored, point ops take and print affine STANDARD coordinates
// (0 0 = infinity).  Output: one line of hexadecimal values per input line (digits:
// signed decimal).
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "g1.hpp"
#include "msm_digit.hpp"

using g16::Fp;
using g16::G1Aff;
using g16::G1Xyzz;

static Fp parse(const std::string& h) {
    Fp x = g16::fp_zero();
    int nib = 0;
    for (int i = (int)h.size() - 1; i >= 0 && nib < 64; --i, ++nib) {
        char c = h[i];
        uint32_t v = (c >= '0' && c <= '9') ? c - '0' : (c >= 'a' && c <= 'f') ? c - 'a' + 10 : c - 'A' + 10;
        x.w[nib / 8] |= v << (4 * (nib % 8));
    }
    return x;
}

static void put(const Fp& x) {
    for (int i = 7; i >= 0; --i) std::printf("%08x", x.w[i]);
}

static G1Aff aff_in(const std::string& x, const std::string& y) {
    G1Aff a;
    Fp xs = parse(x), ys = parse(y);
    if (g16::fp_is_zero(xs) && g16::fp_is_zero(ys)) {
        a.x = xs;
        a.y = ys;
        return a;
    }
    a.x = g16::fp_to_mont(xs);
    a.y = g16::fp_to_mont(ys);
    return a;
}

static void aff_out(const G1Xyzz& p) {
    const G1Aff a = g16::xyzz_to_aff(p);
    put(g16::fp_from_mont(a.x));
    std::printf(" ");
    put(g16::fp_from_mont(a.y));
    std::printf("\n");
}

int main() {
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string op;
        in >> op;
        std::vector<std::string> a;
        for (std::string t; in >> t;) a.push_back(t);
        if (op == "fpmul" || op == "fpadd" || op == "fpsub") {
            Fp x = parse(a[0]), y = parse(a[1]);
            put(op == "fpmul" ? g16::fp_mul(x, y) : op == "fpadd" ? g16::fp_add(x, y) : g16::fp_sub(x, y));
            std::printf("\n");
        } else if (op == "fpinv" || op == "tomont" || op == "frommont" || op == "fpneg") {
            Fp x = parse(a[0]);
            put(op == "fpinv" ? g16::fp_inv(x) : op == "tomont" ? g16::fp_to_mont(x)
                : op == "frommont" ? g16::fp_from_mont(x) : g16::fp_neg(x));
            std::printf("\n");
        } else if (op == "f29mul" || op == "f29add" || op == "f29sub" || op == "f29canon") {
            // through the 29-bit digit form: in and out canonical 2^256 Montgomery form
            g16::Fp29 x = g16::fp29_from_fp(parse(a[0])), y = g16::fp29_from_fp(parse(a[1]));
            g16::Fp29 z = op == "f29mul" ? g16::fp29_mul(x, y) : op == "f29add" ? g16::fp29_add(x, y)
                        : op == "f29sub" ? g16::fp29_sub(x, y) : x;
            put(g16::fp29_to_fp(z));
            std::printf("\n");
        } else if (op == "f29sqr") {
            put(g16::fp29_to_fp(g16::fp29_sqr(g16::fp29_from_fp(parse(a[0])))));
            std::printf("\n");
        } else if (op == "f29mulsub") {  // a b - c d with one reduction
            g16::Fp29 v[4];
            for (int i = 0; i < 4; ++i) v[i] = g16::fp29_from_fp(parse(a[i]));
            put(g16::fp29_to_fp(g16::fp29_mul_sub(v[0], v[1], v[2], v[3])));
            std::printf("\n");
        } else if (op == "f29zero") {    // zero tests of a + b and a - b (lazy, below 64p)
            g16::Fp29 x = g16::fp29_from_fp(parse(a[0])), y = g16::fp29_from_fp(parse(a[1]));
            std::printf("%d %d\n", (int)g16::fp29_is_zero(g16::fp29_add(x, y)),
                        (int)g16::fp29_is_zero(g16::fp29_sub(x, y)));
        } else if (op == "f29lazy") {    // (x - 7y)(x - 7y) - 5 (x y): lazy inputs far from canonical
            g16::Fp29 x = g16::fp29_from_fp(parse(a[0])), y = g16::fp29_from_fp(parse(a[1]));
            g16::Fp29 y7 = g16::fp29_zero();
            for (int i = 0; i < 7; ++i) y7 = g16::fp29_add(y7, y);
            g16::Fp29 d = g16::fp29_sub(x, y7);
            g16::Fp29 xy = g16::fp29_mul(x, y), t = xy;
            for (int i = 0; i < 4; ++i) t = g16::fp29_add(t, xy);
            put(g16::fp29_to_fp(g16::fp29_sub(g16::fp29_mul(d, d), t)));
            std::printf("\n");
        } else if (op == "madd29") {     // (2 P) + Q in digits
            auto p = g16::xyzz_dbl(g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[0], a[1]))));
            aff_out(g16::xyzz_from29(g16::xyzz_madd(p, g16::aff_to29(aff_in(a[2], a[3])))));
        } else if (op == "madd129") {    // P + Q in digits, P straight from affine
            auto p = g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[0], a[1])));
            aff_out(g16::xyzz_from29(g16::xyzz_madd(p, g16::aff_to29(aff_in(a[2], a[3])))));
        } else if (op == "add29") {      // (2 P) + (2 Q) in digits
            auto p = g16::xyzz_dbl(g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[0], a[1]))));
            auto q = g16::xyzz_dbl(g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[2], a[3]))));
            aff_out(g16::xyzz_from29(g16::xyzz_add(p, q)));
        } else if (op == "add129") {
            auto p = g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[0], a[1])));
            auto q = g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[2], a[3])));
            aff_out(g16::xyzz_from29(g16::xyzz_add(p, q)));
        } else if (op == "mulsmall29") {
            uint32_t k = (uint32_t)std::stoul(a[0], nullptr, 16);
            auto p = g16::xyzz_to29(g16::xyzz_from_aff(aff_in(a[1], a[2])));
            aff_out(g16::xyzz_from29(g16::xyzz_mul_small(p, k)));
        } else if (op == "madd") {        // (2 P) + Q, the accumulator with ZZ != 1
            G1Xyzz p = g16::xyzz_dbl(g16::xyzz_from_aff(aff_in(a[0], a[1])));
            aff_out(g16::xyzz_madd(p, aff_in(a[2], a[3])));
        } else if (op == "madd1") {       // P + Q with P straight from affine
            aff_out(g16::xyzz_madd(g16::xyzz_from_aff(aff_in(a[0], a[1])), aff_in(a[2], a[3])));
        } else if (op == "add") {         // (2 P) + (2 Q)
            G1Xyzz p = g16::xyzz_dbl(g16::xyzz_from_aff(aff_in(a[0], a[1])));
            G1Xyzz q = g16::xyzz_dbl(g16::xyzz_from_aff(aff_in(a[2], a[3])));
            aff_out(g16::xyzz_add(p, q));
        } else if (op == "add1") {        // P + Q, both straight from affine
            aff_out(g16::xyzz_add(g16::xyzz_from_aff(aff_in(a[0], a[1])),
                                  g16::xyzz_from_aff(aff_in(a[2], a[3]))));
        } else if (op == "dbl") {         // 2 (2 P)
            aff_out(g16::xyzz_dbl(g16::xyzz_dbl(g16::xyzz_from_aff(aff_in(a[0], a[1])))));
        } else if (op == "dblaff") {      // 2 P from affine
            aff_out(g16::xyzz_dbl_aff(aff_in(a[0], a[1])));
        } else if (op == "mulsmall") {    // k P
            uint32_t k = (uint32_t)std::stoul(a[0], nullptr, 16);
            aff_out(g16::xyzz_mul_small(g16::xyzz_from_aff(aff_in(a[1], a[2])), k));
        } else if (op == "digits") {      // c k: every window's signed digit
            uint32_t c = (uint32_t)std::stoul(a[0], nullptr, 16);
            Fp k = parse(a[1]);
            g16::msm_recode(k.w, c, [](uint32_t, int32_t d) { std::printf("%d ", d); });
            std::printf("\n");
        } else if (op == "code") {        // c d (d as a 32-bit two's complement word): code, decoded
            uint32_t c = (uint32_t)std::stoul(a[0], nullptr, 16);
            const int32_t d = (int32_t)(uint32_t)std::stoul(a[1], nullptr, 16);
            const uint32_t code = g16::msm_code(d, c);
            uint32_t row = 0, neg = 0;
            const bool nz = g16::msm_decode(code, c, row, neg);
            std::printf("%u %d %u %u\n", code, (int)nz, row, neg);
        } else {
            return 2;
        }
    }
    return 0;
}
