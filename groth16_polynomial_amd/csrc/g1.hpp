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
#include "fp29.hpp"

namespace g16 {

// The formulas below are written once over the field representation: Fp (8 x 32-bit
// limbs, canonical; host code and storage) or Fp29 (nine 29-bit digits, lazy; the
// device's hot loops).  f_inf tests a coordinate for the exact zero that stands for
// infinity: every infinity is built as all-zero limbs or digits and stays so, because
// a product with an exact zero factor is exactly zero and no other value is zero mod p
// (points of the group have odd order, so Y and Z are never zero).  f_is_zero is the
// test mod p (the equal- and opposite-point cases).
G16_HD Fp f_add(const Fp& a, const Fp& b) { return fp_add(a, b); }
G16_HD Fp f_sub(const Fp& a, const Fp& b) { return fp_sub(a, b); }
G16_HD Fp f_dbl(const Fp& a) { return fp_dbl(a); }
G16_HD Fp f_neg(const Fp& a) { return fp_neg(a); }
G16_HD Fp f_mul(const Fp& a, const Fp& b) { return fp_mul(a, b); }
G16_HD Fp f_sqr(const Fp& a) { return fp_sqr(a); }
G16_HD Fp f_mul_sub(const Fp& a, const Fp& b, const Fp& c, const Fp& d) {
    return fp_sub(fp_mul(a, b), fp_mul(c, d));
}
G16_HD bool f_is_zero(const Fp& a) { return fp_is_zero(a); }
G16_HD bool f_inf(const Fp& a) { return fp_is_zero(a); }
G16_HD Fp29 f_add(const Fp29& a, const Fp29& b) { return fp29_add(a, b); }
G16_HD Fp29 f_sub(const Fp29& a, const Fp29& b) { return fp29_sub(a, b); }
G16_HD Fp29 f_dbl(const Fp29& a) { return fp29_dbl(a); }
G16_HD Fp29 f_neg(const Fp29& a) { return fp29_neg(a); }
G16_HD Fp29 f_mul(const Fp29& a, const Fp29& b) { return fp29_mul(a, b); }
G16_HD Fp29 f_sqr(const Fp29& a) { return fp29_sqr(a); }
G16_HD Fp29 f_mul_sub(const Fp29& a, const Fp29& b, const Fp29& c, const Fp29& d) {
    return fp29_mul_sub(a, b, c, d);
}
G16_HD bool f_is_zero(const Fp29& a) { return fp29_is_zero(a); }
G16_HD bool f_inf(const Fp29& a) { return fp29_digits_zero(a); }

template <class F> G16_HD F f_zero();
template <> G16_HD Fp f_zero<Fp>() { return fp_zero(); }
template <> G16_HD Fp29 f_zero<Fp29>() { return fp29_zero(); }
template <class F> G16_HD F f_one();
template <> G16_HD Fp f_one<Fp>() { return fp_one(); }
template <> G16_HD Fp29 f_one<Fp29>() { return fp29_from_fp(fp_one()); }

template <class F>
struct AffT {
    F x, y;
};

template <class F>
struct XyzzT {
    F x, y, zz, zzz;
};

using G1Aff = AffT<Fp>;
using G1Xyzz = XyzzT<Fp>;

template <class F = Fp>
G16_HD XyzzT<F> xyzz_zero() {
    XyzzT<F> p;
    p.x = f_zero<F>();
    p.y = f_zero<F>();
    p.zz = f_zero<F>();
    p.zzz = f_zero<F>();
    return p;
}

template <class F>
G16_HD bool aff_is_inf(const AffT<F>& a) { return f_inf(a.x) && f_inf(a.y); }
template <class F>
G16_HD bool xyzz_is_inf(const XyzzT<F>& p) { return f_inf(p.zz); }

template <class F>
G16_HD XyzzT<F> xyzz_from_aff(const AffT<F>& a) {
    if (aff_is_inf(a)) return xyzz_zero<F>();
    XyzzT<F> p;
    p.x = a.x;
    p.y = a.y;
    p.zz = f_one<F>();
    p.zzz = f_one<F>();
    return p;
}

template <class F>
G16_HD XyzzT<F> xyzz_neg(const XyzzT<F>& p) {
    XyzzT<F> r = p;
    r.y = f_neg(p.y);
    return r;
}

// 3 x^2 (the tangent slope's numerator for a = 0)
template <class F>
G16_HD F f_three_sq(const F& x) {
    const F xx = f_sqr(x);
    return f_add(f_dbl(xx), xx);
}

// 2 Q for an affine Q (mdbl-2008-s-1): U = 2y, V = U^2, W = U V, S = x V, M = 3 x^2,
// X3 = M^2 - 2 S, Y3 = M (S - X3) - W y, ZZ3 = V, ZZZ3 = W.
template <class F>
G16_HD XyzzT<F> xyzz_dbl_aff(const AffT<F>& q) {
    const F u = f_dbl(q.y);
    const F v = f_sqr(u);
    const F w = f_mul(u, v);
    const F s = f_mul(q.x, v);
    const F m = f_three_sq(q.x);
    XyzzT<F> r;
    r.x = f_sub(f_sqr(m), f_dbl(s));
    r.y = f_mul_sub(m, f_sub(s, r.x), w, q.y);
    r.zz = v;
    r.zzz = w;
    return r;
}

// 2 P (dbl-2008-s-1); the point at infinity (ZZ = 0) maps to ZZ3 = V ZZ = 0 by itself.
template <class F>
G16_HD XyzzT<F> xyzz_dbl(const XyzzT<F>& p) {
    const F u = f_dbl(p.y);
    const F v = f_sqr(u);
    const F w = f_mul(u, v);
    const F s = f_mul(p.x, v);
    const F m = f_three_sq(p.x);
    XyzzT<F> r;
    r.x = f_sub(f_sqr(m), f_dbl(s));
    r.y = f_mul_sub(m, f_sub(s, r.x), w, p.y);
    r.zz = f_mul(v, p.zz);
    r.zzz = f_mul(w, p.zzz);
    return r;
}

// P + Q for an affine Q (madd-2008-s): U2 = X2 ZZ1, S2 = Y2 ZZZ1, P = U2 - X1,
// R = S2 - Y1, PP = P^2, PPP = P PP, Q = X1 PP, X3 = R^2 - PPP - 2 Q,
// Y3 = R (Q - X3) - Y1 PPP, ZZ3 = ZZ1 PP, ZZZ3 = ZZZ1 PPP.
template <class F>
G16_HD XyzzT<F> xyzz_madd(const XyzzT<F>& p, const AffT<F>& q) {
    if (aff_is_inf(q)) return p;
    if (xyzz_is_inf(p)) return xyzz_from_aff(q);
    const F u2 = f_mul(q.x, p.zz);
    const F s2 = f_mul(q.y, p.zzz);
    const F pd = f_sub(u2, p.x);
    const F rd = f_sub(s2, p.y);
    if (f_is_zero(pd)) return f_is_zero(rd) ? xyzz_dbl_aff(q) : xyzz_zero<F>();
    const F pp = f_sqr(pd);
    const F ppp = f_mul(pd, pp);
    const F qv = f_mul(p.x, pp);
    XyzzT<F> r;
    r.x = f_sub(f_sub(f_sqr(rd), ppp), f_dbl(qv));
    r.y = f_mul_sub(rd, f_sub(qv, r.x), p.y, ppp);
    r.zz = f_mul(p.zz, pp);
    r.zzz = f_mul(p.zzz, ppp);
    return r;
}

// P + Q (add-2008-s): U1 = X1 ZZ2, U2 = X2 ZZ1, S1 = Y1 ZZZ2, S2 = Y2 ZZZ1, P = U2 - U1,
// R = S2 - S1, PP = P^2, PPP = P PP, Q = U1 PP, X3 = R^2 - PPP - 2 Q,
// Y3 = R (Q - X3) - S1 PPP, ZZ3 = ZZ1 ZZ2 PP, ZZZ3 = ZZZ1 ZZZ2 PPP.
template <class F>
G16_HD XyzzT<F> xyzz_add(const XyzzT<F>& p, const XyzzT<F>& q) {
    if (xyzz_is_inf(p)) return q;
    if (xyzz_is_inf(q)) return p;
    const F u1 = f_mul(p.x, q.zz);
    const F u2 = f_mul(q.x, p.zz);
    const F s1 = f_mul(p.y, q.zzz);
    const F s2 = f_mul(q.y, p.zzz);
    const F pd = f_sub(u2, u1);
    const F rd = f_sub(s2, s1);
    if (f_is_zero(pd)) return f_is_zero(rd) ? xyzz_dbl(p) : xyzz_zero<F>();
    const F pp = f_sqr(pd);
    const F ppp = f_mul(pd, pp);
    const F qv = f_mul(u1, pp);
    XyzzT<F> r;
    r.x = f_sub(f_sub(f_sqr(rd), ppp), f_dbl(qv));
    r.y = f_mul_sub(rd, f_sub(qv, r.x), s1, ppp);
    r.zz = f_mul(f_mul(p.zz, q.zz), pp);
    r.zzz = f_mul(f_mul(p.zzz, q.zzz), ppp);
    return r;
}

// k P for a small k (left to right, from k's highest set bit).
template <class F>
G16_HD XyzzT<F> xyzz_mul_small(const XyzzT<F>& p, uint32_t k) {
    XyzzT<F> acc = xyzz_zero<F>();
    for (int i = 31; i >= 0; --i) {
        if (!xyzz_is_inf(acc)) acc = xyzz_dbl(acc);
        if ((k >> i) & 1u) acc = xyzz_add(acc, p);
    }
    return acc;
}

// Between the stored form (Fp, canonical) and the digit form of the hot loops.
G16_HD AffT<Fp29> aff_to29(const G1Aff& a) {
    AffT<Fp29> r;
    r.x = fp29_from_fp(a.x);
    r.y = fp29_from_fp(a.y);
    return r;
}
G16_HD XyzzT<Fp29> xyzz_to29(const G1Xyzz& a) {
    XyzzT<Fp29> r;
    r.x = fp29_from_fp(a.x);
    r.y = fp29_from_fp(a.y);
    r.zz = fp29_from_fp(a.zz);
    r.zzz = fp29_from_fp(a.zzz);
    return r;
}
// Infinity stays all zero (ZZ's exact zero is kept rather than reduced).
G16_HD G1Xyzz xyzz_from29(const XyzzT<Fp29>& a) {
    if (xyzz_is_inf(a)) return xyzz_zero<Fp>();
    G1Xyzz r;
    r.x = fp29_to_fp(a.x);
    r.y = fp29_to_fp(a.y);
    r.zz = fp29_to_fp(a.zz);
    r.zzz = fp29_to_fp(a.zzz);
    return r;
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

// The same from the digit form: one inversion in digits, then canonical coordinates.
G16_HD G1Aff xyzz_to_aff(const XyzzT<Fp29>& p) {
    G1Aff a;
    if (xyzz_is_inf(p)) {
        a.x = fp_zero();
        a.y = fp_zero();
        return a;
    }
    const Fp29 t = fp29_inv(fp29_mul(p.zz, p.zzz));
    a.x = fp29_to_fp(fp29_mul(p.x, fp29_mul(t, p.zzz)));
    a.y = fp29_to_fp(fp29_mul(p.y, fp29_mul(t, p.zz)));
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
