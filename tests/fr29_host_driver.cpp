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
//   shl5   x                  -> digits of x 2^5 for a canonical x
//   mmul   x[0..8] y[0..8]    -> digits of the radix-2^29 REDC product x y 2^-261
//   redc1  x[0..8]            -> digits of x 2^-261
//   mul29  a b                -> fr_mul29(a, b), canonical 256-bit value
//   fm29   a                  -> fr_from_mont29(a), canonical 256-bit value
//   join   a b x[0..8]        -> h = canon(REDC(a 2^5, b) - normalize(x)) and REDC(h 2^5):
//                                the join epilogue's arithmetic on a transform's lazy x
//   batch  K inv triv seed x_0 .. x_{2^K-1}
//                             -> "ok M" or "bad i": one slice of 2^K canonical values run
//                                through K passes in the transform kernels' schedule (see
//                                run_batch), checked against the 8 x 32-bit layer; M is
//                                the largest digit magnitude met
#include <cstdint>
#include <cstdio>
#include <vector>
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

// SplitMix64 (Steele, Lea, Flood 2014): the batch op's random table values.
static uint64_t splitmix(uint64_t& s) {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static Fr random_canonical(uint64_t& s) {
    for (;;) {
        Fr x;
        for (int i = 0; i < 4; ++i) {
            uint64_t v = splitmix(s);
            x.w[2 * i] = (uint32_t)v;
            x.w[2 * i + 1] = (uint32_t)(v >> 32);
        }
        x.w[7] &= 0x3fffffffu;
        Fr d;
        uint32_t borrow = 0;
        for (int i = 0; i < 8; ++i) d.w[i] = subb(x.w[i], r_limb(i), borrow);
        if (borrow) return x;  // x < r
    }
}

// Digit-wise a + b or a - b with a check that no digit leaves the int32 range; tracks the
// largest magnitude met.
static bool addsub_checked(const V29& a, const V29& b, bool sub, V29& out, int64_t& maxabs) {
    for (int k = 0; k < 9; ++k) {
        const int64_t v = sub ? (int64_t)a.l[k] - b.l[k] : (int64_t)a.l[k] + b.l[k];
        if (v > INT32_MAX || v < INT32_MIN) return false;
        out.l[k] = (int32_t)v;
        if ((v < 0 ? -v : v) > maxabs) maxabs = v < 0 ? -v : v;
    }
    return true;
}

// One slice through K passes as the transform kernels run them: register groups of two
// passes (one for an odd K's last group), forward order (bits 0 up) or inverse order (bits
// K-1 down, groups from the top); before every group but the first, the elements that are
// "lo" in the group's first pass are normalized; each butterfly is (lo + t, lo - t) with
// t = w hi a product by a table entry, or t = hi where the kernels skip twiddle 1 (triv:
// the first group of a contiguous forward batch: its first pass, and the second pass's
// pairs with m = 0; the top group of an inverse top batch: its first pass, and the second
// pass's pair with q >> 1 = 0).  Table values are random (the bounds do not depend on
// them).  The 8 x 32-bit layer runs the same butterflies as the reference.
static void run_batch(int K, bool inv, bool triv, uint64_t seed, std::vector<Fr> in) {
    const int n = 1 << K;
    std::vector<V29> x(n);
    std::vector<Fr> ref = in;
    int64_t maxabs = 0;
    for (int i = 0; i < n; ++i) x[i] = fr29_from_fr(in[i]);
    // groups: forward [0,1], [2,3], ...; inverse [K-2,K-1] from the top (lower bit B0)
    std::vector<int> b0s;
    for (int b0 = 0; b0 < K; b0 += 2) b0s.push_back(b0);
    if (inv) std::vector<int>(b0s.rbegin(), b0s.rend()).swap(b0s);
    bool first_group = true;
    for (int b0 : b0s) {
        const int R = (K - b0) < 2 ? (K - b0) : 2;
        // passes of the group in execution order, as bit numbers
        std::vector<int> bits;
        for (int u = 0; u < R; ++u) bits.push_back(b0 + u);
        if (inv) std::vector<int>(bits.rbegin(), bits.rend()).swap(bits);
        if (!first_group) {  // normalize the lo elements of the group's first pass
            for (int i = 0; i < n; ++i)
                if (!((i >> bits[0]) & 1)) x[i] = fr29_normalize(x[i]);
        }
        for (int s = 0; s < R; ++s) {
            const int b = bits[s];
            for (int i = 0; i < n; ++i) {
                if ((i >> b) & 1) continue;
                const int j = i | (1 << b);
                // trivial twiddles as in the kernels (only in the group that starts the batch)
                bool one = false;
                if (triv && first_group) {
                    if (!inv) {
                        const int m = (i >> b0) & ((1 << s) - 1);  // pair index bits below the pass
                        one = (s == 0) || (R == 2 && s == 1 && m == 0 && b0 == 0);
                    } else {
                        const int a = i >> (b + 1);  // pair index bits above the pass
                        one = (s == 0 && b == K - 1) || (R == 2 && s == 1 && a == 0);
                    }
                }
                V29 t;
                Fr tref;
                if (one) {
                    t = x[j];
                    tref = ref[j];
                } else {
                    const Fr wm = random_canonical(seed);
                    for (int k = 0; k < 9; ++k) {
                        const int64_t v = x[j].l[k] < 0 ? -(int64_t)x[j].l[k] : x[j].l[k];
                        if (v > maxabs) maxabs = v;
                    }
                    t = shoup_mul(x[j], tw29_entry(wm));
                    tref = fr_mul(ref[j], wm);
                }
                V29 lo = x[i], hi;
                if (!addsub_checked(lo, t, false, x[i], maxabs) ||
                    !addsub_checked(lo, t, true, hi, maxabs)) {
                    std::printf("bad %d", i);
                    return;
                }
                x[j] = hi;
                const Fr rl = ref[i];
                ref[i] = fr_add(rl, tref);
                ref[j] = fr_sub(rl, tref);
            }
        }
        first_group = false;
    }
    for (int i = 0; i < n; ++i) {
        if (!fr_is_equal(fr29_canon(x[i]), ref[i])) {
            std::printf("bad %d", i);
            return;
        }
    }
    std::printf("ok %lld", (long long)maxabs);
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
        } else if (op == "shl5") {
            std::string h;
            in >> h;
            print_v(fr29_from_fr_shl5(parse_fr(h)).l);
        } else if (op == "mmul") {
            V29 x = read_v(in);
            V29 y = read_v(in);
            print_v(fr29_mont_mul(x, y).l);
        } else if (op == "redc1") {
            print_v(fr29_redc1(read_v(in)).l);
        } else if (op == "mul29") {
            std::string ha, hb;
            in >> ha >> hb;
            print_fr(fr_mul29(parse_fr(ha), parse_fr(hb)));
        } else if (op == "fm29") {
            std::string h;
            in >> h;
            print_fr(fr_from_mont29(parse_fr(h)));
        } else if (op == "join") {
            std::string ha, hb;
            in >> ha >> hb;
            V29 x = read_v(in);
            const V29 ab = fr29_mont_mul(fr29_from_fr_shl5(parse_fr(ha)), fr29_from_fr(parse_fr(hb)));
            const Fr h = fr29_canon(fr29_sub(ab, fr29_normalize(x)));
            print_fr(h);
            std::printf(" ");
            print_fr(fr_from_mont29(h));
        } else if (op == "split") {
            std::string h;
            in >> h;
            print_v(fr29_from_fr(parse_fr(h)).l);
        } else if (op == "batch") {
            int K, inv, triv;
            unsigned long long seed;
            in >> K >> inv >> triv >> seed;
            std::vector<Fr> xs((size_t)1 << K);
            for (auto& v : xs) {
                std::string h;
                in >> h;
                v = parse_fr(h);
            }
            run_batch(K, inv != 0, triv != 0, seed, xs);
        } else {
            return 2;
        }
        std::printf("\n");
    }
    return 0;
}
