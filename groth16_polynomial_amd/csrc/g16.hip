// libg16.so: host side of the C ABI declared in include/g16.h.
//
// Argument checks run on the host before anything is enqueued; every call then only
// enqueues kernels on the caller's stream (the NTT_CU page: one stream, launches
// queued asynchronously, one synchronisation by the caller at the end).
#include "g16.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "host_util.hpp"
#include "kernels.hpp"
#include "pointwise_kernels.hpp"
#include "group_launch.hpp"

using g16::Fr;

namespace {

constexpr uint32_t kMagic = 0x47313643u;  // "G16C"
constexpr uint32_t kDead = 0xdeadc0deu;
constexpr size_t kAlign = 256;
constexpr uint32_t kThreads = 256;
constexpr uint32_t kMaxBatches = 27;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

struct g16_ctx {
    uint32_t magic;
    uint32_t log_n;
    int device;
    g16::TwTab tw_fwd;    // powers of omega by level (n - 1 entries)
    g16::TwTab tw_inv;    // powers of omega^-1 by level, bit-reversed within each level
    g16::TwTab tw_coset;  // tw_fwd with the coset shift folded into the levels of bits >= 2
                          // (each in five planes of n 16-byte parts)
    g16::TwTab kappa;     // the rest of the shift and 1/n, by position mod 4 (four entries)
    Fr* scratch;  // three n-element vectors
    const uint8_t* ws_begin;
    size_t ws_bytes;
    Fr omega, omega_inv, shift, size_inv;  // Montgomery form
    g16::Tw29 size_inv_entry;              // n^-1 as a table entry (inverse transform)
    bool radix2;  // G16_RADIX2 set at prepare time: every batch on the radix-2 kernel
    int narrow;   // G16_NARROW at prepare time: 0 never, 1 always, -1 by launch size
    uint32_t n_batches;
    uint32_t batch_k[kMaxBatches];  // lowest bits first
};

namespace {

// Largest number of passes one workgroup batches in LDS (2^k elements of 32 bytes), from
// the environment (G16_MAX_K), or 0: the default plan.
uint32_t env_max_k() {
    const char* env = std::getenv("G16_MAX_K");
    if (env) {
        int v = std::atoi(env);
        if (v >= 1 && v <= 12) return (uint32_t)v;
    }
    return 0u;
}

// Split log_n passes into ceil(log_n / kmax) batches of near-equal size, the larger
// ones at the low end (the NTT_CU page, "SHARED MEMORY BUDGET" section: 18 = 9 + 9
// rather than 10 + 8, so no batch degenerates into a tiny tail).
uint32_t plan_batches(uint32_t log_n, uint32_t kmax, uint32_t* ks) {
    uint32_t nb = (log_n + kmax - 1) / kmax;
    uint32_t q = log_n / nb, rem = log_n % nb;
    for (uint32_t i = 0; i < nb; ++i) ks[i] = q + (i < rem ? 1u : 0u);
    return nb;
}

// The default plan: the near-equal split under a cap of 10 passes, except on the domains
// where a plan of mostly even batches measured faster (2^21 -2.5%, 2^22 -3.0%, 2^23 -1%,
// 2^25 -2.2%, 2^26 -2.4%; the same three batches, every batch 6..10 passes, so still no
// tiny tail).  In the radix-4 geometry a batch of an odd number of passes ends in a one-pass
// register group, which loads, exchanges and stores its elements for half the products of
// a two-pass group.  Lowest bits first.
uint32_t default_plan(uint32_t log_n, uint32_t* ks) {
    static constexpr uint8_t kMeasured[][4] = {
        {21, 6, 7, 8}, {22, 8, 6, 8}, {23, 8, 7, 8}, {25, 10, 8, 7}, {26, 10, 8, 8}};
    for (const auto& m : kMeasured)
        if (m[0] == log_n) {
            for (int i = 0; i < 3; ++i) ks[i] = m[1 + i];
            return 3u;
        }
    return plan_batches(log_n, 10u, ks);
}

// kmax = 0: G16_MAX_K if set, else the default plan.
uint32_t plan_for(uint32_t log_n, uint32_t kmax, uint32_t* ks) {
    if (kmax == 0) kmax = env_max_k();
    return kmax ? plan_batches(log_n, kmax, ks) : default_plan(log_n, ks);
}

// Contexts handed out and not yet released.  Every entry point looks its context up
// here before touching it, so a released (freed) or foreign pointer is refused without
// being read.
std::mutex g_live_mu;
std::unordered_set<const g16_ctx*> g_live;

bool ctx_ok(const g16_ctx* c) {
    if (!c) return false;
    std::lock_guard<std::mutex> lock(g_live_mu);
    return g_live.count(c) != 0;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

using g16::device_range;

int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? G16_OK : G16_EHIP;
}

// Host-side domain roots (Montgomery form): g = 5, w28 = g^((r-1)/2^28),
// s = w28^(2^(27-L)), omega = s^2.
void domain_roots(uint32_t log_n, Fr* omega, Fr* shift, Fr* size_inv) {
    Fr five = g16::fr_zero();
    five.w[0] = 5u;
    five = g16::fr_to_mont(five);
    uint32_t e[8];
    // (r - 1) >> 28, limb by limb
    uint32_t rl[8];
    for (int i = 0; i < 8; ++i) rl[i] = g16::r_limb(i);
    rl[0] -= 1u;
    for (int i = 0; i < 8; ++i) e[i] = (rl[i] >> 28) | (i < 7 ? (rl[i + 1] << 4) : 0u);
    Fr s = g16::fr_pow(five, e);
    for (uint32_t i = 0; i < 27 - log_n; ++i) s = g16::fr_mul(s, s);
    *shift = s;
    *omega = g16::fr_mul(s, s);
    Fr n = g16::fr_zero();
    if (log_n < 32) n.w[0] = 1u << log_n;
    *size_inv = g16::fr_inv(g16::fr_to_mont(n));
}

// Launches of at most this many elements (vectors x 2^log_n) take the narrow geometry of
// the register-group kernel unless G16_NARROW says otherwise.  Below it the radix-4
// groups leave CUs idle or thinly occupied and each thread's chain of products sets the
// time; the narrow geometry halves the chain and doubles the threads.  Above it the
// radix-4 groups' fewer LDS exchanges and table loads win.  Measured on MI355X, the two
// geometries alternating (H pipeline, three vectors): 2^12 55 / 26 us, 2^16 77 / 56,
// 2^18 141 / 138, 2^19 262 / 269, 2^20 527 / 600 (radix-4 / narrow); proof batches of
// 64 x 2^12 125 / 121 us and 16 x 2^16 524 / 599; one forward transform of 2^19 54 / 54.
constexpr uint64_t kNarrowMaxElems = uint64_t(3) << 18;

bool use_narrow(const g16_ctx* c, uint64_t n_vec) {
    if (c->narrow >= 0) return c->narrow != 0;
    return (n_vec << c->log_n) <= kNarrowMaxElems;
}

// The register-group kernel takes batches of 6..10 passes with at least one full workgroup
// of slices; the radix-2 kernel takes the rest (small domains, other batch sizes).
template <g16::Mode M, bool J>
bool try_groups(const g16::BatchParams& p, uint32_t n_vec, bool narrow, hipStream_t stream,
                int* rc) {
    const uint32_t k = p.k, L = p.log_n;
    auto fits = [&](uint32_t spw) { return (1ull << (L - k)) >= spw; };
    hipError_t e;
    switch (k) {
#define G16_GROUP_CASE(KK)                                                              \
        case KK:                                                                       \
            if (!fits(narrow ? g16::NarrowGeomFor<KK, M>::kSpw                         \
                             : g16::GroupGeomFor<KK, g16::kGroupPasses, M>::kSpw))    \
                return false;                                                          \
            e = g16::launch_groups<KK, M, J>(p, n_vec, narrow, stream);                \
            *rc = e == hipSuccess ? G16_OK : G16_EHIP;                                 \
            return true;
        G16_GROUP_CASE(6)
        G16_GROUP_CASE(7)
        G16_GROUP_CASE(8)
        G16_GROUP_CASE(9)
        G16_GROUP_CASE(10)
#undef G16_GROUP_CASE
        default:
            return false;
    }
}

// Whether the pipeline's last launch (M = FwdStrided or Fused) of batch size k can take
// the three kinds of a proof in one narrow workgroup (ntt_group_kernel with NK = 3).
template <g16::Mode M>
bool join3_fits(uint32_t k, uint32_t L) {
    switch (k) {
#define G16_J3_CASE(KK)                                                               \
        case KK:                                                                      \
            return g16::narrow_join3_fits<KK, M>() &&                                 \
                   (1ull << (L - KK)) >= (uint64_t)g16::NarrowGeomFor<KK, M>::kSpw;
        G16_J3_CASE(6)
        G16_J3_CASE(7)
        G16_J3_CASE(8)
        G16_J3_CASE(9)
        G16_J3_CASE(10)
#undef G16_J3_CASE
        default:
            return false;
    }
}

template <g16::Mode M>
int launch_join3(const g16::BatchParams& p, uint32_t n_proof, hipStream_t stream) {
    hipError_t e;
    switch (p.k) {
        case 6: e = g16::launch_groups_join3<6, M>(p, n_proof, stream); break;
        case 7: e = g16::launch_groups_join3<7, M>(p, n_proof, stream); break;
        case 8: e = g16::launch_groups_join3<8, M>(p, n_proof, stream); break;
        case 9: e = g16::launch_groups_join3<9, M>(p, n_proof, stream); break;
        case 10: e = g16::launch_groups_join3<10, M>(p, n_proof, stream); break;
        default: return G16_EINVAL;
    }
    return e == hipSuccess ? G16_OK : G16_EHIP;
}

template <g16::Mode M, bool J>
int launch_batch(const g16::BatchParams& p, uint32_t n_vec, bool radix2, bool narrow,
                 hipStream_t stream) {
    int rc = G16_OK;
    if (!radix2 && try_groups<M, J>(p, n_vec, narrow, stream, &rc)) return rc;
    // radix-2 batch kernel: small batches and small domains
    const uint32_t k = p.k, L = p.log_n;
    g16::BatchParams q = p;
    uint32_t log_spw = 0;
    if (k < 9) log_spw = (9 - k) < (L - k) ? (9 - k) : (L - k);
    q.log_spw = log_spw;
    uint64_t groups = (1ull << (L - k)) >> log_spw;
    size_t lds = (size_t(1) << (k + log_spw)) * sizeof(Fr);
    // batches of 12 passes (G16_MAX_K = 12) need 128 KiB
    if (g16::allow_lds((const void*)g16::ntt_batch_kernel<M, J>, lds) != hipSuccess)
        return G16_EHIP;
    dim3 grid((uint32_t)groups, n_vec, 1);
    hipLaunchKernelGGL((g16::ntt_batch_kernel<M, J>), grid, dim3(kThreads), lds, stream, q);
    return launch_status();
}

g16::BatchParams base_params(const g16_ctx* c) {
    g16::BatchParams p;
    std::memset(&p, 0, sizeof p);
    p.log_n = c->log_n;
    p.n_kind = 1;
    return p;
}

uint32_t batch_s0(const g16_ctx* c, uint32_t idx) {
    uint32_t s = 0;
    for (uint32_t i = 0; i < idx; ++i) s += c->batch_k[i];
    return s;
}

size_t vec_bytes(const g16_ctx* c) { return (size_t(1) << c->log_n) * sizeof(Fr); }

// Forward (inverse = false) or inverse transform, natural order in and out.
int run_ntt(g16_ctx* c, const void* in, void* out, void* stream, bool inverse) {
    if (!ctx_ok(c)) return c ? G16_ESTATE : G16_EINVAL;
    if (!in || !out) return G16_EINVAL;
    const size_t nbytes = vec_bytes(c);
    if (in != out && overlaps(in, nbytes, out, nbytes)) return G16_EALIAS;
    if (overlaps(in, nbytes, c->ws_begin, c->ws_bytes) ||
        overlaps(out, nbytes, c->ws_begin, c->ws_bytes))
        return G16_EALIAS;
    if (!device_range(in, nbytes) || !device_range(out, nbytes)) return G16_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    Fr* scr = c->scratch;
    g16::BatchParams p = base_params(c);
    // both directions run the forward passes (the inverse on x[-k mod n], see head_index)
    p.tw = c->tw_fwd;
    p.head_inverse = inverse ? 1u : 0u;
    p.kscale = c->size_inv_entry;
    p.s0 = 0;
    p.k = c->batch_k[0];
    p.src[0] = (const Fr*)in;
    const bool single = c->n_batches == 1;
    p.dst[0] = (single && in != out) ? (Fr*)out : scr;
    p.lazy_out = single ? 0u : 1u;  // only the last batch's output must be canonical
    const bool narrow = use_narrow(c, 1);
    int rc = launch_batch<g16::Mode::HeadBitrev, false>(p, 1, c->radix2, narrow, s);
    if (rc) return rc;
    if (single) {
        if (in == out) {
            if (hipMemcpyAsync(out, scr, nbytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
                return G16_EHIP;
        }
        return G16_OK;
    }
    for (uint32_t b = 1; b < c->n_batches; ++b) {
        g16::BatchParams t = base_params(c);
        t.tw = p.tw;
        t.s0 = batch_s0(c, b);
        t.k = c->batch_k[b];
        t.src[0] = scr;
        t.dst[0] = (b + 1 == c->n_batches) ? (Fr*)out : scr;
        t.lazy_out = (b + 1 == c->n_batches) ? 0u : 1u;
        rc = launch_batch<g16::Mode::FwdStrided, false>(t, 1, c->radix2, narrow, s);
        if (rc) return rc;
    }
    return G16_OK;
}

// One kernel launch of a pipeline: which kernel, its parameters and vector count.
struct Launch {
    g16::Mode mode;
    bool join;
    bool join3;  // the three kinds of each proof in one workgroup (n_vec counts proofs)
    bool radix2;
    bool narrow;
    g16::BatchParams p;
    uint32_t n_vec;
};

constexpr uint32_t kMaxLaunches = 2 * kMaxBatches + 2;

int exec_launch(const Launch& l, hipStream_t s) {
    using g16::Mode;
    const bool r2 = l.radix2, nw = l.narrow;
    if (l.join3)
        return l.mode == Mode::Fused ? launch_join3<Mode::Fused>(l.p, l.n_vec, s)
                                     : launch_join3<Mode::FwdStrided>(l.p, l.n_vec, s);
    switch (l.mode) {
        case Mode::Fused:
            return l.join ? launch_batch<Mode::Fused, true>(l.p, l.n_vec, r2, nw, s)
                          : launch_batch<Mode::Fused, false>(l.p, l.n_vec, r2, nw, s);
        case Mode::FwdStrided:
            return l.join ? launch_batch<Mode::FwdStrided, true>(l.p, l.n_vec, r2, nw, s)
                          : launch_batch<Mode::FwdStrided, false>(l.p, l.n_vec, r2, nw, s);
        case Mode::InvStrided:
            return launch_batch<Mode::InvStrided, false>(l.p, l.n_vec, r2, nw, s);
        default:
            return launch_batch<Mode::HeadBitrev, false>(l.p, l.n_vec, r2, nw, s);
    }
}

// The launches of stages 1-3 for n_kind vectors srcs[v] -> coset evaluations in dsts[v]
// of each of n_proof proofs, proof q's vectors vstride elements after proof q - 1's
// (dsts may equal srcs only when the context has a single batch).  With join, the last
// kind's final batch writes H = dsts[0] * dsts[1] - x into h_mont / h_std instead, in a
// launch of its own after the other vectors are finished; or, for launches small enough
// for the narrow geometry, the final batch of all three kinds is one launch whose
// workgroups join A', B' and C' in LDS (dsts[0], dsts[1] are then not written by it).
uint32_t plan_coset(const g16_ctx* c, const Fr* const* srcs, Fr* const* dsts, uint32_t n_kind,
                    uint32_t n_proof, uint64_t vstride, bool join, Fr* h_mont, Fr* h_std,
                    Launch* out) {
    const uint32_t nb = c->n_batches;
    const uint32_t plain_kind = join ? n_kind - 1 : n_kind;
    uint32_t count = 0;
    auto add = [&](g16::Mode m, bool j, g16::BatchParams p, uint32_t kinds) {
        p.n_kind = kinds;
        p.vstride = vstride;
        out[count].mode = m;
        out[count].join = j;
        out[count].join3 = false;
        out[count].radix2 = c->radix2;
        out[count].narrow = use_narrow(c, (uint64_t)kinds * n_proof);
        out[count].p = p;
        out[count].n_vec = kinds * n_proof;
        ++count;
    };
    // the final batch of the three kinds, joined in the workgroup
    const bool j3 = join && n_kind == 3 && !c->radix2 && use_narrow(c, 3ull * n_proof);
    auto add_join3 = [&](g16::Mode m, g16::BatchParams p) {
        p.n_kind = 3;
        p.vstride = vstride;
        p.h_mont = h_mont;
        p.h_std = h_std;
        out[count].mode = m;
        out[count].join = true;
        out[count].join3 = true;
        out[count].radix2 = false;
        out[count].narrow = true;
        out[count].p = p;
        out[count].n_vec = n_proof;
        ++count;
    };
    auto joined = [&](g16::BatchParams p) {
        p.src[0] = (nb == 1) ? srcs[n_kind - 1] : dsts[n_kind - 1];
        p.src[1] = p.src[2] = nullptr;
        p.dst[0] = p.dst[1] = p.dst[2] = nullptr;
        p.join_a = dsts[0];
        p.join_b = dsts[1];
        p.h_mont = h_mont;
        p.h_std = h_std;
        return p;
    };
    // Outputs that only further transform batches read are stored in [0, 2r) (lazy_out);
    // the last batch's outputs, and A' and B' that the join reads, are canonical.
    // inverse transform, high batches first (DIF), the first one reading the inputs
    for (uint32_t b = nb - 1; b >= 1; --b) {
        g16::BatchParams p = base_params(c);
        p.lazy_out = 1u;
        p.tw = c->tw_inv;
        p.s0 = batch_s0(c, b);
        p.k = c->batch_k[b];
        for (uint32_t v = 0; v < n_kind; ++v) {
            p.src[v] = (b == nb - 1) ? srcs[v] : dsts[v];
            p.dst[v] = dsts[v];
        }
        add(g16::Mode::InvStrided, false, p, n_kind);
    }
    // lowest batch of both transforms with the coset multiply between them; the forward
    // passes read the shifted table
    g16::BatchParams f = base_params(c);
    f.tw = c->tw_inv;
    f.tw_fwd = c->tw_coset;
    f.kappa = c->kappa;
    f.k = c->batch_k[0];
    f.lazy_out = nb > 1 ? 1u : 0u;
    for (uint32_t v = 0; v < n_kind; ++v) {
        f.src[v] = (nb == 1) ? srcs[v] : dsts[v];
        f.dst[v] = dsts[v];
    }
    if (nb == 1) {
        if (j3 && join3_fits<g16::Mode::Fused>(f.k, c->log_n)) {
            add_join3(g16::Mode::Fused, f);
            return count;
        }
        if (plain_kind) add(g16::Mode::Fused, false, f, plain_kind);
        if (join) add(g16::Mode::Fused, true, joined(f), 1);
        return count;
    }
    add(g16::Mode::Fused, false, f, n_kind);
    // forward transform, remaining batches (DIT), low to high
    for (uint32_t b = 1; b < nb; ++b) {
        g16::BatchParams p = base_params(c);
        p.tw = c->tw_coset;
        p.s0 = batch_s0(c, b);
        p.k = c->batch_k[b];
        p.lazy_out = b + 1 < nb ? 1u : 0u;
        for (uint32_t v = 0; v < n_kind; ++v) {
            p.src[v] = dsts[v];
            p.dst[v] = dsts[v];
        }
        if (b + 1 == nb && j3 && join3_fits<g16::Mode::FwdStrided>(p.k, c->log_n)) {
            add_join3(g16::Mode::FwdStrided, p);
        } else if (b + 1 == nb && join) {
            if (plain_kind) add(g16::Mode::FwdStrided, false, p, plain_kind);
            add(g16::Mode::FwdStrided, true, joined(p), 1);
        } else {
            add(g16::Mode::FwdStrided, false, p, n_kind);
        }
    }
    return count;
}

int run_plan(const Launch* ls, uint32_t count, hipStream_t s) {
    for (uint32_t i = 0; i < count; ++i) {
        int rc = exec_launch(ls[i], s);
        if (rc) return rc;
    }
    return G16_OK;
}

// Host checks shared by g16_h_compute, g16_h_stage and g16_h_compute_noalloc.
int check_h(g16_ctx* ctx, const void* a_mont, const void* b_mont, const void* c_mont,
            void* h_mont, void* h_std) {
    if (!ctx_ok(ctx)) return ctx ? G16_ESTATE : G16_EINVAL;
    if (!a_mont || !b_mont || !c_mont || !h_mont || !h_std) return G16_EINVAL;
    const size_t nbytes = vec_bytes(ctx);
    const void* ins[3] = {a_mont, b_mont, c_mont};
    const void* outs[2] = {h_mont, h_std};
    if (overlaps(h_mont, nbytes, h_std, nbytes)) return G16_EALIAS;
    for (const void* o : outs) {
        for (const void* i : ins)
            if (overlaps(o, nbytes, i, nbytes)) return G16_EALIAS;
        if (overlaps(o, nbytes, ctx->ws_begin, ctx->ws_bytes)) return G16_EALIAS;
    }
    for (const void* i : ins)
        if (overlaps(i, nbytes, ctx->ws_begin, ctx->ws_bytes)) return G16_EALIAS;
    for (const void* p : ins)
        if (!device_range(p, nbytes)) return G16_EINVAL;
    for (const void* p : outs)
        if (!device_range(p, nbytes)) return G16_EINVAL;
    return G16_OK;
}

// Host checks of g16_h_compute / g16_h_stage, then the launch list.
int plan_h(g16_ctx* ctx, const void* a_mont, const void* b_mont, const void* c_mont,
           void* h_mont, void* h_std, Launch* ls, uint32_t* count) {
    const int rc = check_h(ctx, a_mont, b_mont, c_mont, h_mont, h_std);
    if (rc) return rc;
    const size_t n = size_t(1) << ctx->log_n;
    const Fr* srcs[3] = {(const Fr*)a_mont, (const Fr*)b_mont, (const Fr*)c_mont};
    Fr* dsts[3] = {ctx->scratch, ctx->scratch + n, ctx->scratch + 2 * n};
    *count = plan_coset(ctx, srcs, dsts, 3, 1, 0, true, (Fr*)h_mont, (Fr*)h_std, ls);
    return G16_OK;
}

}  // namespace

// ---------------------------------------------------------------- no-allocation variant
//
// g16_h_compute_noalloc keeps C' between its launches in this array instead of the
// context's workspace scratch (A' and B' live in h_mont and h_std until the join
// overwrites them, as in g16_h_compute_batch), so a call allocates nothing and touches
// no caller memory beyond its arguments.  Every process that loads the library holds the
// array on each device it runs on until it exits.  Host code never uses the array's name
// as an address: the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[(size_t(1) << G16_NOALLOC_MAX_LOG_N) * 32];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each device

// The array's address on `device`, which must be the current device the first time
// (g16_h_prepare calls this for the device it prepares on).  G16_EHIP if the runtime
// cannot resolve it.
int static_scratch(int device, void** out) {
    if (device < 0 || device >= kMaxDevices) return G16_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != device) return G16_EHIP;
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return G16_EHIP;
        }
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return G16_OK;
}

}  // namespace

extern "C" {

uint32_t g16_abi_version(void) { return G16_ABI_VERSION; }

const char* g16_strerror(int code) {
    switch (code) {
        case G16_OK: return "ok";
        case G16_EINVAL: return "invalid argument";
        case G16_ERANGE: return "log_n out of range [1, 27]";
        case G16_ENOSPACE: return "workspace too small";
        case G16_EALIAS: return "buffers overlap";
        case G16_EHIP: return "HIP runtime or launch error";
        case G16_ESTATE: return "context released or not prepared";
        default: return "unknown status";
    }
}

int g16_batch_plan(uint32_t log_n, uint32_t kmax, uint32_t* ks, uint32_t cap) {
    if (log_n < G16_MIN_LOG_N || log_n > G16_MAX_LOG_N) return G16_ERANGE;
    if (kmax > 12 || (cap > 0 && !ks)) return G16_EINVAL;
    uint32_t tmp[kMaxBatches];
    uint32_t nb = plan_for(log_n, kmax, tmp);
    for (uint32_t i = 0; i < nb && i < cap; ++i) ks[i] = tmp[i];
    return (int)nb;
}

size_t g16_h_workspace_bytes(uint32_t log_n) {
    if (log_n < G16_MIN_LOG_N || log_n > G16_MAX_LOG_N) return 0;
    size_t n = size_t(1) << log_n;
    size_t tab = round_up(n * sizeof(g16::Tw29));
    size_t full = round_up(n * sizeof(Fr));
    return 3 * tab + 3 * full + round_up(4 * sizeof(g16::Tw29));
}

int g16_h_prepare(uint32_t log_n, void* workspace, size_t workspace_bytes, void* stream,
                  g16_ctx** out_ctx) {
    if (!out_ctx || !workspace) return G16_EINVAL;
    if (log_n < G16_MIN_LOG_N || log_n > G16_MAX_LOG_N) return G16_ERANGE;
    if ((uintptr_t)workspace % kAlign) return G16_EINVAL;
    if (workspace_bytes < g16_h_workspace_bytes(log_n)) return G16_ENOSPACE;
    if (!device_range(workspace, g16_h_workspace_bytes(log_n))) return G16_EINVAL;
    g16_ctx* c = new (std::nothrow) g16_ctx;
    if (!c) return G16_EINVAL;
    std::memset(c, 0, sizeof *c);
    c->log_n = log_n;
    if (hipGetDevice(&c->device) != hipSuccess) {
        delete c;
        return G16_EHIP;
    }
    const size_t n = size_t(1) << log_n;
    uint8_t* ws = (uint8_t*)workspace;
    size_t tab = round_up(n * sizeof(g16::Tw29));
    c->tw_fwd = g16::TwTab{(uint4*)ws, (uint32_t)n};
    c->tw_inv = g16::TwTab{(uint4*)(ws + tab), (uint32_t)n};
    c->tw_coset = g16::TwTab{(uint4*)(ws + 2 * tab), (uint32_t)n};
    c->scratch = (Fr*)(ws + 3 * tab);
    c->kappa = g16::TwTab{(uint4*)(ws + 3 * tab + 3 * round_up(n * sizeof(Fr))), 4u};
    c->ws_begin = ws;
    c->ws_bytes = g16_h_workspace_bytes(log_n);
    domain_roots(log_n, &c->omega, &c->shift, &c->size_inv);
    c->omega_inv = g16::fr_inv(c->omega);
    c->size_inv_entry = g16::tw29_entry(c->size_inv);
    c->n_batches = plan_for(log_n, 0u, c->batch_k);
    c->radix2 = std::getenv("G16_RADIX2") != nullptr;
    {
        const char* nw = std::getenv("G16_NARROW");
        c->narrow = nw ? (std::atoi(nw) != 0 ? 1 : 0) : -1;
    }
    {
        // the no-allocation entry point's scratch on this device (resolved here, with the
        // device current; a failure only disables that entry point, which reports it)
        void* unused = nullptr;
        (void)static_scratch(c->device, &unused);
    }

    // bits where the plan's batches start (the forward table's layout follows them)
    uint32_t starts = 0, bit = 0;
    for (uint32_t i = 0; i < c->n_batches; ++i) {
        starts |= 1u << bit;
        bit += c->batch_k[i];
    }

    hipStream_t s = (hipStream_t)stream;
    const uint32_t blocks = 2048;
    Fr one = g16::fr_mont_one();
    hipLaunchKernelGGL(g16::table_kernel, dim3(blocks), dim3(kThreads), 0, s, c->tw_fwd,
                       c->omega, one, (uint64_t)(n - 1), log_n, 0, starts);
    hipLaunchKernelGGL(g16::table_kernel, dim3(blocks), dim3(kThreads), 0, s, c->tw_inv,
                       c->omega_inv, one, (uint64_t)(n - 1), log_n, 2, starts);
    hipLaunchKernelGGL(g16::table_kernel, dim3(blocks), dim3(kThreads), 0, s, c->tw_coset,
                       c->omega, c->shift, (uint64_t)(n - 1), log_n, 3, starts);
    hipLaunchKernelGGL(g16::table_kernel, dim3(1), dim3(kThreads), 0, s, c->kappa, c->shift,
                       c->size_inv, (uint64_t)4, log_n, 1, starts);
    int rc = launch_status();
    if (rc) {
        delete c;
        return rc;
    }
    c->magic = kMagic;
    {
        std::lock_guard<std::mutex> lock(g_live_mu);
        g_live.insert(c);
    }
    *out_ctx = c;
    return G16_OK;
}

int g16_release(g16_ctx* ctx) {
    if (!ctx) return G16_EINVAL;
    {
        // a pointer that is not a live context (released before, or never handed out) is
        // refused without being read
        std::lock_guard<std::mutex> lock(g_live_mu);
        if (g_live.erase(ctx) == 0) return G16_ESTATE;
    }
    ctx->magic = kDead;
    delete ctx;
    return G16_OK;
}

uint32_t g16_ctx_log_n(const g16_ctx* ctx) { return ctx_ok(ctx) ? ctx->log_n : 0u; }

int g16_domain_roots(const g16_ctx* ctx, uint8_t omega_mont[32], uint8_t shift_mont[32],
                     uint8_t size_inv_mont[32]) {
    if (!ctx_ok(ctx)) return ctx ? G16_ESTATE : G16_EINVAL;
    if (omega_mont) std::memcpy(omega_mont, ctx->omega.w, 32);
    if (shift_mont) std::memcpy(shift_mont, ctx->shift.w, 32);
    if (size_inv_mont) std::memcpy(size_inv_mont, ctx->size_inv.w, 32);
    return G16_OK;
}

int g16_ntt_forward(g16_ctx* ctx, const void* in_mont, void* out_mont, void* stream) {
    return run_ntt(ctx, in_mont, out_mont, stream, false);
}

int g16_ntt_inverse(g16_ctx* ctx, const void* in_mont, void* out_mont, void* stream) {
    return run_ntt(ctx, in_mont, out_mont, stream, true);
}



int g16_coset_eval(g16_ctx* ctx, const void* in_mont, void* out_mont, void* stream) {
    if (!ctx_ok(ctx)) return ctx ? G16_ESTATE : G16_EINVAL;
    if (!in_mont || !out_mont) return G16_EINVAL;
    const size_t nbytes = vec_bytes(ctx);
    if (in_mont != out_mont && overlaps(in_mont, nbytes, out_mont, nbytes)) return G16_EALIAS;
    if (overlaps(in_mont, nbytes, ctx->ws_begin, ctx->ws_bytes) ||
        overlaps(out_mont, nbytes, ctx->ws_begin, ctx->ws_bytes))
        return G16_EALIAS;
    if (!device_range(in_mont, nbytes) || !device_range(out_mont, nbytes)) return G16_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    const Fr* src = (const Fr*)in_mont;
    Launch ls[kMaxLaunches];
    if (ctx->n_batches == 1) {
        // one contiguous kernel: each workgroup reads its whole slice before writing it
        Fr* dst = (Fr*)out_mont;
        return run_plan(ls, plan_coset(ctx, &src, &dst, 1, 1, 0, false, nullptr, nullptr, ls), s);
    }
    // inverse batches write scratch first, the last forward batch writes scratch too
    Fr* tmp = ctx->scratch;
    int rc = run_plan(ls, plan_coset(ctx, &src, &tmp, 1, 1, 0, false, nullptr, nullptr, ls), s);
    if (rc) return rc;
    if (hipMemcpyAsync(out_mont, tmp, nbytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return G16_EHIP;
    return G16_OK;
}

int g16_h_compute(g16_ctx* ctx, const void* a_mont, const void* b_mont, const void* c_mont,
                  void* h_mont, void* h_std, void* stream) {
    Launch ls[kMaxLaunches];
    uint32_t count = 0;
    int rc = plan_h(ctx, a_mont, b_mont, c_mont, h_mont, h_std, ls, &count);
    if (rc) return rc;
    return run_plan(ls, count, (hipStream_t)stream);
}

int g16_h_compute_noalloc(g16_ctx* ctx, const void* a_mont, const void* b_mont,
                          const void* c_mont, void* h_mont, void* h_std, void* stream) {
    int rc = check_h(ctx, a_mont, b_mont, c_mont, h_mont, h_std);
    if (rc) return rc;
    if (ctx->log_n > G16_NOALLOC_MAX_LOG_N) return G16_ENOSPACE;
    void* scr = nullptr;
    rc = static_scratch(ctx->device, &scr);
    if (rc) return rc;
    const Fr* srcs[3] = {(const Fr*)a_mont, (const Fr*)b_mont, (const Fr*)c_mont};
    Fr* dsts[3] = {(Fr*)h_mont, (Fr*)h_std, (Fr*)scr};
    Launch ls[kMaxLaunches];
    const uint32_t count = plan_coset(ctx, srcs, dsts, 3, 1, uint64_t(1) << ctx->log_n, true,
                                      (Fr*)h_mont, (Fr*)h_std, ls);
    return run_plan(ls, count, (hipStream_t)stream);
}

size_t g16_h_batch_scratch_bytes(uint32_t log_n, uint64_t n_proofs) {
    if (log_n < G16_MIN_LOG_N || log_n > G16_MAX_LOG_N) return 0;
    if (n_proofs > G16_MAX_PROOFS || (n_proofs << log_n) > (1ull << 31)) return 0;
    return (size_t)(n_proofs << log_n) * sizeof(Fr);
}

int g16_h_compute_batch(g16_ctx* ctx, uint64_t n_proofs, const void* a_mont,
                        const void* b_mont, const void* c_mont, void* h_mont, void* h_std,
                        void* scratch, size_t scratch_bytes, void* stream) {
    if (!ctx_ok(ctx)) return ctx ? G16_ESTATE : G16_EINVAL;
    if (n_proofs == 0) return G16_OK;
    if (n_proofs > G16_MAX_PROOFS || (n_proofs << ctx->log_n) > (1ull << 31))
        return G16_EINVAL;
    if (!a_mont || !b_mont || !c_mont || !h_mont || !h_std || !scratch) return G16_EINVAL;
    const size_t bytes = (size_t)(n_proofs << ctx->log_n) * sizeof(Fr);
    if (scratch_bytes < bytes) return G16_ENOSPACE;
    const void* ins[3] = {a_mont, b_mont, c_mont};
    void* outs[3] = {h_mont, h_std, scratch};
    for (int o = 0; o < 3; ++o) {
        for (int j = o + 1; j < 3; ++j)
            if (overlaps(outs[o], bytes, outs[j], bytes)) return G16_EALIAS;
        for (const void* i : ins)
            if (overlaps(outs[o], bytes, i, bytes)) return G16_EALIAS;
        if (overlaps(outs[o], bytes, ctx->ws_begin, ctx->ws_bytes)) return G16_EALIAS;
        if (!device_range(outs[o], bytes)) return G16_EINVAL;
    }
    for (const void* i : ins) {
        if (overlaps(i, bytes, ctx->ws_begin, ctx->ws_bytes)) return G16_EALIAS;
        if (!device_range(i, bytes)) return G16_EINVAL;
    }
    // A' and B' live in h_mont and h_std until the join overwrites them element by
    // element; C' (only when there is more than one batch) lives in the scratch.
    const Fr* srcs[3] = {(const Fr*)a_mont, (const Fr*)b_mont, (const Fr*)c_mont};
    Fr* dsts[3] = {(Fr*)h_mont, (Fr*)h_std, (Fr*)scratch};
    Launch ls[kMaxLaunches];
    const uint32_t count = plan_coset(ctx, srcs, dsts, 3, (uint32_t)n_proofs,
                                      uint64_t(1) << ctx->log_n, true, (Fr*)h_mont,
                                      (Fr*)h_std, ls);
    return run_plan(ls, count, (hipStream_t)stream);
}

int g16_h_stage_count(const g16_ctx* ctx) {
    if (!ctx_ok(ctx)) return ctx ? G16_ESTATE : G16_EINVAL;
    // the single-proof plan (planning reads no buffer)
    Launch ls[kMaxLaunches];
    const Fr* srcs[3] = {nullptr, nullptr, nullptr};
    Fr* dsts[3] = {nullptr, nullptr, nullptr};
    return (int)plan_coset(ctx, srcs, dsts, 3, 1, 0, true, nullptr, nullptr, ls);
}

int g16_h_stage(g16_ctx* ctx, uint32_t stage, const void* a_mont, const void* b_mont,
                const void* c_mont, void* h_mont, void* h_std, void* stream) {
    Launch ls[kMaxLaunches];
    uint32_t count = 0;
    int rc = plan_h(ctx, a_mont, b_mont, c_mont, h_mont, h_std, ls, &count);
    if (rc) return rc;
    if (stage >= count) return G16_EINVAL;
    return exec_launch(ls[stage], (hipStream_t)stream);
}

static uint32_t ew_blocks(uint64_t n) {
    uint64_t b = (n + kThreads - 1) / kThreads;
    return (uint32_t)(b < 8192 ? b : 8192);
}

int g16_h_join(uint64_t n, const void* a_mont, const void* b_mont, const void* c_mont,
               void* h_mont, void* h_std, void* stream) {
    if (n == 0 || !a_mont || !b_mont || !c_mont || !h_mont || !h_std) return G16_EINVAL;
    const size_t nbytes = n * sizeof(Fr);
    const void* ins[3] = {a_mont, b_mont, c_mont};
    if (overlaps(h_mont, nbytes, h_std, nbytes)) return G16_EALIAS;
    for (const void* i : ins)
        if (overlaps(h_mont, nbytes, i, nbytes) || overlaps(h_std, nbytes, i, nbytes))
            return G16_EALIAS;
    for (const void* p : {a_mont, b_mont, c_mont, (const void*)h_mont, (const void*)h_std})
        if (!device_range(p, nbytes)) return G16_EINVAL;
    hipLaunchKernelGGL(g16::h_join_kernel, dim3(ew_blocks(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const Fr*)a_mont, (const Fr*)b_mont,
                       (const Fr*)c_mont, (Fr*)h_mont, (Fr*)h_std, n);
    return launch_status();
}

int g16_gather_abc(uint64_t n_rows, const uint32_t* row_ptr_a, const uint32_t* signal_a,
                   const void* value_a, uint64_t nnz_a, const uint32_t* row_ptr_b,
                   const uint32_t* signal_b, const void* value_b, uint64_t nnz_b,
                   const void* witness, uint64_t n_witness, void* out_a, void* out_b,
                   void* out_c, void* stream) {
    if (n_rows == 0 || n_rows >= 0xffffffffull || !row_ptr_a || !row_ptr_b || !witness ||
        n_witness == 0 || !out_a || !out_b || !out_c)
        return G16_EINVAL;
    if ((nnz_a && (!signal_a || !value_a)) || (nnz_b && (!signal_b || !value_b)))
        return G16_EINVAL;
    if (nnz_a > 0xffffffffull || nnz_b > 0xffffffffull) return G16_EINVAL;
    const size_t ob = n_rows * sizeof(Fr);
    void* outs[3] = {out_a, out_b, out_c};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], ob, outs[j], ob)) return G16_EALIAS;
    const void* ins[8] = {row_ptr_a, signal_a, value_a, row_ptr_b, signal_b, value_b, witness,
                          nullptr};
    const size_t in_bytes[7] = {(n_rows + 1) * 4, nnz_a * 4, nnz_a * sizeof(Fr),
                                (n_rows + 1) * 4, nnz_b * 4, nnz_b * sizeof(Fr),
                                n_witness * sizeof(Fr)};
    for (int o = 0; o < 3; ++o)
        for (int i = 0; i < 7; ++i)
            if (ins[i] && in_bytes[i] && overlaps(outs[o], ob, ins[i], in_bytes[i]))
                return G16_EALIAS;
    for (int i = 0; i < 7; ++i)
        if (ins[i] && in_bytes[i] && !device_range(ins[i], in_bytes[i])) return G16_EINVAL;
    for (int o = 0; o < 3; ++o)
        if (!device_range(outs[o], ob)) return G16_EINVAL;
    const uint32_t blocks = (uint32_t)((n_rows + g16::kGatherLanes - 1) / g16::kGatherLanes);
    hipLaunchKernelGGL(g16::gather_kernel, dim3(blocks), dim3(g16::kGatherLanes), 0,
                       (hipStream_t)stream,
                       row_ptr_a, signal_a, (const Fr*)value_a, nnz_a, row_ptr_b, signal_b,
                       (const Fr*)value_b, nnz_b, (const Fr*)witness, n_witness, (Fr*)out_a,
                       (Fr*)out_b, (Fr*)out_c, n_rows);
    return launch_status();
}

static int elementwise(uint64_t n, const void* a, const void* b, void* out, int op,
                       void* stream) {
    if (n == 0 || !a || !out || (op == 2 && !b)) return G16_EINVAL;
    const size_t nbytes = n * sizeof(Fr);
    if (a != out && overlaps(a, nbytes, out, nbytes)) return G16_EALIAS;
    if (op == 2 && b != out && overlaps(b, nbytes, out, nbytes)) return G16_EALIAS;
    if (!device_range(a, nbytes) || !device_range(out, nbytes) ||
        (op == 2 && !device_range(b, nbytes)))
        return G16_EINVAL;
    hipLaunchKernelGGL(g16::elementwise_kernel, dim3(ew_blocks(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const Fr*)a, (const Fr*)b, (Fr*)out, n, op);
    return launch_status();
}

int g16_to_mont(uint64_t n, const void* in_std, void* out_mont, void* stream) {
    return elementwise(n, in_std, nullptr, out_mont, 0, stream);
}

int g16_from_mont(uint64_t n, const void* in_mont, void* out_std, void* stream) {
    return elementwise(n, in_mont, nullptr, out_std, 1, stream);
}

int g16_fr_mul(uint64_t n, const void* a_mont, const void* b_mont, void* out_mont,
               void* stream) {
    return elementwise(n, a_mont, b_mont, out_mont, 2, stream);
}

}  // extern "C"
