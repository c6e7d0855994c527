// BN254 G1 (y^2 = x^3 + 3 over Fp) points for the multi-scalar multiplication.
//
// The MSM_CU page accumulates buckets in extended Jacobian "XYZZ" coordinates with affine
// bases (section 3 of its header, "POINTS ACCUMULATE IN XYZZ, BASES STAY AFFINE"): a
// point (X, Y, ZZ, ZZZ) stands for (X/ZZ, Y/ZZZ) with ZZ^3 = ZZZ^2, and ZZ = 0 is the
// point at infinity.  The formulas are those of the Explicit-Formulas Database for
// short Weierstrass curves in xyzz coordinates with a = 0 (Sutherland 2008):
// madd-2008-s (mixed addition), add-2008-s, dbl-2008-s-1 and mdbl-2008-s-1.  The
// database's formulas assume distinct, finite inputs; the special cases (an input at
// infinity, equal points, opposite points) are tested here first.
//
// Affine points are (x, y) in Montgomery form; (0, 0), which is not on the curve, stands
// for the point at infinity.
#pragma once

#include "fp.hpp"

namespace g16 {

struct G1Aff {
    Fp x, y;
};

struct G1Xyzz {
    Fp x, y, zz, zzz;
};

G16_HD G1Xyzz xyzz_zero() {
    G1Xyzz p;
    p.x = fp_zero();
    p.y = fp_zero();
    p.zz = fp_zero();
    p.zzz = fp_zero();
    return p;
}

G16_HD bool aff_is_inf(const G1Aff& a) { return fp_is_zero(a.x) && fp_is_zero(a.y); }
G16_HD bool xyzz_is_inf(const G1Xyzz& p) { return fp_is_zero(p.zz); }

G16_HD G1Xyzz xyzz_from_aff(const G1Aff& a) {
    if (aff_is_inf(a)) return xyzz_zero();
    G1Xyzz p;
    p.x = a.x;
    p.y = a.y;
    p.zz = fp_one();
    p.zzz = fp_one();
    return p;
}

G16_HD G1Xyzz xyzz_neg(const G1Xyzz& p) {
    G1Xyzz r = p;
    r.y = fp_neg(p.y);
    return r;
}

// 3 x^2 (the tangent slope's numerator for a = 0)
G16_HD Fp fp_three_sq(const Fp& x) {
    const Fp xx = fp_sqr(x);
    return fp_add(fp_dbl(xx), xx);
}

// 2 Q for an affine Q (mdbl-2008-s-1): U = 2y, V = U^2, W = U V, S = x V, M = 3 x^2,
// X3 = M^2 - 2 S, Y3 = M (S - X3) - W y, ZZ3 = V, ZZZ3 = W.
G16_HD G1Xyzz xyzz_dbl_aff(const G1Aff& q) {
    const Fp u = fp_dbl(q.y);
    const Fp v = fp_sqr(u);
    const Fp w = fp_mul(u, v);
    const Fp s = fp_mul(q.x, v);
    const Fp m = fp_three_sq(q.x);
    G1Xyzz r;
    r.x = fp_sub(fp_sqr(m), fp_dbl(s));
    r.y = fp_sub(fp_mul(m, fp_sub(s, r.x)), fp_mul(w, q.y));
    r.zz = v;
    r.zzz = w;
    return r;
}

// 2 P (dbl-2008-s-1); the point at infinity (ZZ = 0) maps to ZZ3 = V ZZ = 0 by itself.
G16_HD G1Xyzz xyzz_dbl(const G1Xyzz& p) {
    const Fp u = fp_dbl(p.y);
    const Fp v = fp_sqr(u);
    const Fp w = fp_mul(u, v);
    const Fp s = fp_mul(p.x, v);
    const Fp m = fp_three_sq(p.x);
    G1Xyzz r;
    r.x = fp_sub(fp_sqr(m), fp_dbl(s));
    r.y = fp_sub(fp_mul(m, fp_sub(s, r.x)), fp_mul(w, p.y));
    r.zz = fp_mul(v, p.zz);
    r.zzz = fp_mul(w, p.zzz);
    return r;
}

// P + Q for an affine Q (madd-2008-s): U2 = X2 ZZ1, S2 = Y2 ZZZ1, P = U2 - X1,
// R = S2 - Y1, PP = P^2, PPP = P PP, Q = X1 PP, X3 = R^2 - PPP - 2 Q,
// Y3 = R (Q - X3) - Y1 PPP, ZZ3 = ZZ1 PP, ZZZ3 = ZZZ1 PPP.
G16_HD G1Xyzz xyzz_madd(const G1Xyzz& p, const G1Aff& q) {
    if (aff_is_inf(q)) return p;
    if (xyzz_is_inf(p)) return xyzz_from_aff(q);
    const Fp u2 = fp_mul(q.x, p.zz);
    const Fp s2 = fp_mul(q.y, p.zzz);
    const Fp pd = fp_sub(u2, p.x);
    const Fp rd = fp_sub(s2, p.y);
    if (fp_is_zero(pd)) return fp_is_zero(rd) ? xyzz_dbl_aff(q) : xyzz_zero();
    const Fp pp = fp_sqr(pd);
    const Fp ppp = fp_mul(pd, pp);
    const Fp qv = fp_mul(p.x, pp);
    G1Xyzz r;
    r.x = fp_sub(fp_sub(fp_sqr(rd), ppp), fp_dbl(qv));
    r.y = fp_sub(fp_mul(rd, fp_sub(qv, r.x)), fp_mul(p.y, ppp));
    r.zz = fp_mul(p.zz, pp);
    r.zzz = fp_mul(p.zzz, ppp);
    return r;
}

// P + Q (add-2008-s): U1 = X1 ZZ2, U2 = X2 ZZ1, S1 = Y1 ZZZ2, S2 = Y2 ZZZ1, P = U2 - U1,
// R = S2 - S1, PP = P^2, PPP = P PP, Q = U1 PP, X3 = R^2 - PPP - 2 Q,
// Y3 = R (Q - X3) - S1 PPP, ZZ3 = ZZ1 ZZ2 PP, ZZZ3 = ZZZ1 ZZZ2 PPP.
G16_HD G1Xyzz xyzz_add(const G1Xyzz& p, const G1Xyzz& q) {
    if (xyzz_is_inf(p)) return q;
    if (xyzz_is_inf(q)) return p;
    const Fp u1 = fp_mul(p.x, q.zz);
    const Fp u2 = fp_mul(q.x, p.zz);
    const Fp s1 = fp_mul(p.y, q.zzz);
    const Fp s2 = fp_mul(q.y, p.zzz);
    const Fp pd = fp_sub(u2, u1);
    const Fp rd = fp_sub(s2, s1);
    if (fp_is_zero(pd)) return fp_is_zero(rd) ? xyzz_dbl(p) : xyzz_zero();
    const Fp pp = fp_sqr(pd);
    const Fp ppp = fp_mul(pd, pp);
    const Fp qv = fp_mul(u1, pp);
    G1Xyzz r;
    r.x = fp_sub(fp_sub(fp_sqr(rd), ppp), fp_dbl(qv));
    r.y = fp_sub(fp_mul(rd, fp_sub(qv, r.x)), fp_mul(s1, ppp));
    r.zz = fp_mul(fp_mul(p.zz, q.zz), pp);
    r.zzz = fp_mul(fp_mul(p.zzz, q.zzz), ppp);
    return r;
}

// k P for a small k (left to right, from k's highest set bit).
G16_HD G1Xyzz xyzz_mul_small(const G1Xyzz& p, uint32_t k) {
    G1Xyzz acc = xyzz_zero();
    for (int i = 31; i >= 0; --i) {
        if (!xyzz_is_inf(acc)) acc = xyzz_dbl(acc);
        if ((k >> i) & 1u) acc = xyzz_add(acc, p);
    }
    return acc;
}

// (X/ZZ, Y/ZZZ) with one inversion: t = (ZZ ZZZ)^-1, 1/ZZ = t ZZZ, 1/ZZZ = t ZZ.
G16_HD G1Aff xyzz_to_aff(const G1Xyzz& p) {
    G1Aff a;
    if (xyzz_is_inf(p)) {
        a.x = fp_zero();
        a.y = fp_zero();
        return a;
    }
    const Fp t = fp_inv(fp_mul(p.zz, p.zzz));
    a.x = fp_mul(p.x, fp_mul(t, p.zzz));
    a.y = fp_mul(p.y, fp_mul(t, p.zz));
    return a;
}

// The generator (1, 2), Montgomery form.
G16_HD G1Aff g1_generator() {
    Fp one = fp_zero(), two = fp_zero();
    one.w[0] = 1u;
    two.w[0] = 2u;
    G1Aff g;
    g.x = fp_to_mont(one);
    g.y = fp_to_mont(two);
    return g;
}

}  // namespace g16
