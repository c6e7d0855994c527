// Host build of the library's 29-bit limb layer (fr29.hpp), driven by
// tests/test_fr29_host.py.  Each input line is an operation name followed by hex
// numbers; each output line is hex numbers.
// Digits are printed and read as signed decimal numbers, 256-bit values as hex.
//   entry  wm                 -> w[0..8] wp[0..8]      (table entry of Montgomery-form wm)
//   shoup  x[0..8] wm         -> y[0..8]               (product by the entry of wm)
//   shoup2 x[0..8] y[0..8] wm vm -> two products computed together
//   canon  x[0..8]            -> canonical 256-bit value
//   norm   x[0..8]            -> digits after fr29_normalize
//   sub    a[0..8] b[0..8]    -> digits of a - b
//   split  x                  -> digits of a canonical 256-bit value
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include "fr29.hpp"

using namespace g16;

static Fr parse_fr(const std::string& h) {
    Fr x = fr_zero();
    int nib = 0;
    for (int i = (int)h.size() - 1; i >= 0 && nib < 64; --i, ++nib) {
        char c = h[i];
        uint32_t v = (c >= '0' && c <= '9') ? c - '0' : (c >= 'a' && c <= 'f') ? c - 'a' + 10 : c - 'A' + 10;
        x.w[nib / 8] |= v << (4 * (nib % 8));
    }
    return x;
}

static void print_fr(const Fr& x) {
    for (int i = 7; i >= 0; --i) std::printf("%08x", x.w[i]);
}

static V29 read_v(std::istream& in) {
    V29 v;
    for (int k = 0; k < 9; ++k) {
        long long d;
        in >> d;
        v.l[k] = (int32_t)d;
    }
    return v;
}

static void print_v(const int32_t* l) {
    for (int k = 0; k < 9; ++k) std::printf("%s%d", k ? " " : "", l[k]);
}

int main() {
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string op;
        if (!(in >> op)) continue;
        if (op == "entry") {
            std::string h;
            in >> h;
            Tw29 t = tw29_entry(parse_fr(h));
            print_v(t.w);
            std::printf(" ");
            print_v(t.wp);
        } else if (op == "shoup") {
            V29 x = read_v(in);
            std::string h;
            in >> h;
            Tw29 t = tw29_entry(parse_fr(h));
            V29 y = shoup_mul(x, t);
            print_v(y.l);
        } else if (op == "canon") {
            print_fr(fr29_canon(read_v(in)));
        } else if (op == "norm") {
            print_v(fr29_normalize(read_v(in)).l);
        } else if (op == "shoup2") {
            V29 x[2] = {read_v(in), read_v(in)};
            std::string h0, h1;
            in >> h0 >> h1;
            Tw29 t[2] = {tw29_entry(parse_fr(h0)), tw29_entry(parse_fr(h1))};
            V29 y[2];
            shoup_mul_n<2>(x, t, y);
            print_v(y[0].l);
            std::printf(" ");
            print_v(y[1].l);
        } else if (op == "sub") {
            V29 a = read_v(in);
            V29 b = read_v(in);
            print_v(fr29_sub(a, b).l);
        } else if (op == "split") {
            std::string h;
            in >> h;
            print_v(fr29_from_fr(parse_fr(h)).l);
        } else {
            return 2;
        }
        std::printf("\n");
    }
    return 0;
}
