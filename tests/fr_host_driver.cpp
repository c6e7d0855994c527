// Host build of the library's Fr layer (fr.hpp), driven by tests/test_fr_host.py.
// Reads lines "op a b" (hex, op in mul/add/sub/tomont/frommont/pow/inv) and prints
// the result in hex.
#include <cstdio>
#include <cstring>
#include <string>
#include <iostream>
#include "fr.hpp"

using g16::Fr;

static Fr parse(const std::string& h) {
    Fr x = g16::fr_zero();
    int nib = 0;
    for (int i = (int)h.size() - 1; i >= 0 && nib < 64; --i, ++nib) {
        char c = h[i];
        uint32_t v = (c >= '0' && c <= '9') ? c - '0' : (c >= 'a' && c <= 'f') ? c - 'a' + 10 : c - 'A' + 10;
        x.w[nib / 8] |= v << (4 * (nib % 8));
    }
    return x;
}

static void print(const Fr& x) {
    for (int i = 7; i >= 0; --i) std::printf("%08x", x.w[i]);
    std::printf("\n");
}

int main() {
    std::string op, a, b;
    while (std::cin >> op >> a >> b) {
        Fr x = parse(a), y = parse(b), z;
        if (op == "mul") z = g16::fr_mul(x, y);
        else if (op == "add") z = g16::fr_add(x, y);
        else if (op == "sub") z = g16::fr_sub(x, y);
        else if (op == "c261") z = g16::fr_c261();
        else if (op == "tomont") z = g16::fr_to_mont(x);
        else if (op == "frommont") z = g16::fr_from_mont(x);
        else if (op == "pow") z = g16::fr_pow_u64(x, ((uint64_t)y.w[1] << 32) | y.w[0]);
        else if (op == "inv") z = g16::fr_inv(x);
        else return 2;
        print(z);
    }
    return 0;
}
