// libg16.so: host side of the BabyBear transform (include/g16.h, "BabyBear NTT").
//
// g16_bb_prepare builds the twiddle levels once in a caller-owned workspace (the NTT_CU
// page's rule for the BN254 tables, kept here: tables built at prepare time, left
// resident); g16_bb_lde only enqueues the batches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "bb_ntt.hpp"
#include "g16.h"
#include "host_util.hpp"

struct g16_bb_ctx {
    uint32_t log_n;
    const uint2* tw;
    const uint32_t* twm;
    const uint8_t* ws_begin;
    size_t ws_bytes;
};

namespace {

constexpr size_t kAlign = 256;
constexpr uint32_t kMaxBatchK = 8;
// The later batches of matrices of at most 2^kMontMaxLogW columns take the 4-byte
// Montgomery-form twiddles: with one or two columns a twiddle serves only one or two
// elements of a row, so the table is as large as the data and its bytes bind; with more
// columns each entry is shared and the Shoup product's two fewer instructions win.
#ifndef G16_BB_MONT_MAX_LW
#define G16_BB_MONT_MAX_LW 1
#endif
constexpr int kMontMaxLogW = G16_BB_MONT_MAX_LW;

size_t round_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

std::mutex g_bb_mu;
std::unordered_set<const g16_bb_ctx*> g_bb_live;

bool bb_ok(const g16_bb_ctx* c) {
    if (!c) return false;
    std::lock_guard<std::mutex> lock(g_bb_mu);
    return g_bb_live.count(c) != 0;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

template <int K>
hipError_t launch_k(bool head, bool mont, const g16::BbParams& p, uint32_t blocks,
                    hipStream_t s) {
    const uint32_t spw = 1u << p.log_spw;
    const uint32_t threads = spw * ((1u << K) / g16::kBbE);
    const size_t lds = (size_t)(spw + 1u) * (1u << K) * 4u;
    if (head)
        hipLaunchKernelGGL((g16::bb_batch_kernel<K, true, false>), dim3(blocks), dim3(threads),
                           lds, s, p);
    else if (mont)
        hipLaunchKernelGGL((g16::bb_batch_kernel<K, false, true>), dim3(blocks), dim3(threads),
                           lds, s, p);
    else
        hipLaunchKernelGGL((g16::bb_batch_kernel<K, false, false>), dim3(blocks),
                           dim3(threads), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_batch(bool head, bool mont, const g16::BbParams& p, uint32_t blocks,
                        hipStream_t s) {
    switch (p.k) {
        case 4: return launch_k<4>(head, mont, p, blocks, s);
        case 5: return launch_k<5>(head, mont, p, blocks, s);
        case 6: return launch_k<6>(head, mont, p, blocks, s);
        case 7: return launch_k<7>(head, mont, p, blocks, s);
        case 8: return launch_k<8>(head, mont, p, blocks, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" {

size_t g16_bb_workspace_bytes(uint32_t log_n) {
    if (log_n < 1 || log_n > G16_BB_MAX_LOG_N) return 0;
    const size_t entries = (size_t(1) << log_n) - 1;
    return round_up(entries * sizeof(uint2)) + round_up(entries * sizeof(uint32_t));
}

int g16_bb_batch_plan(uint32_t log_n, uint32_t* ks, uint32_t cap) {
    if (log_n < 1 || log_n > G16_BB_MAX_LOG_N) return G16_ERANGE;
    if (cap > 0 && !ks) return G16_EINVAL;
    if (log_n <= 4) {  // one kernel does the whole transform per column
        if (cap > 0) ks[0] = log_n;
        return 1;
    }
    const uint32_t nb = (log_n + kMaxBatchK - 1) / kMaxBatchK;
    for (uint32_t i = 0; i < nb && i < cap; ++i)
        ks[i] = log_n / nb + (i < log_n % nb ? 1u : 0u);
    return (int)nb;
}

int g16_bb_prepare(uint32_t log_n, void* workspace, size_t workspace_bytes, void* stream,
                   g16_bb_ctx** out_ctx) {
    if (!out_ctx || !workspace) return G16_EINVAL;
    if (log_n < 1 || log_n > G16_BB_MAX_LOG_N) return G16_ERANGE;
    if ((uintptr_t)workspace % kAlign) return G16_EINVAL;
    const size_t need = g16_bb_workspace_bytes(log_n);
    if (workspace_bytes < need) return G16_ENOSPACE;
    if (!g16::device_range(workspace, need)) return G16_EINVAL;
    g16_bb_ctx* c = new (std::nothrow) g16_bb_ctx;
    if (!c) return G16_EINVAL;
    c->log_n = log_n;
    c->tw = (const uint2*)workspace;
    c->twm = (const uint32_t*)((const uint8_t*)workspace +
                               round_up(((size_t(1) << log_n) - 1) * sizeof(uint2)));
    c->ws_begin = (const uint8_t*)workspace;
    c->ws_bytes = need;
    hipLaunchKernelGGL(g16::bb_table_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream,
                       (uint2*)workspace, (uint32_t*)c->twm, log_n);
    if (hipGetLastError() != hipSuccess) {
        delete c;
        return G16_EHIP;
    }
    std::lock_guard<std::mutex> lock(g_bb_mu);
    g_bb_live.insert(c);
    *out_ctx = c;
    return G16_OK;
}

int g16_bb_release(g16_bb_ctx* ctx) {
    if (!ctx) return G16_EINVAL;
    {
        std::lock_guard<std::mutex> lock(g_bb_mu);
        if (g_bb_live.erase(ctx) == 0) return G16_ESTATE;
    }
    delete ctx;
    return G16_OK;
}

int g16_bb_lde(g16_bb_ctx* ctx, uint32_t log_in, uint32_t log_w, uint64_t count,
               const void* in_mont, void* out_mont, void* stream) {
    if (!bb_ok(ctx)) return ctx ? G16_ESTATE : G16_EINVAL;
    const uint32_t L = ctx->log_n;
    if (log_in > L || log_w > G16_BB_MAX_LOG_W || L + log_w > 30u) return G16_EINVAL;
    if (count == 0) return G16_OK;
    if (!in_mont || !out_mont || count > (1u << 20)) return G16_EINVAL;
    const size_t in_elems = (size_t(1) << (log_in + log_w)), out_elems = (size_t(1) << (L + log_w));
    const size_t in_bytes = count * in_elems * 4, out_bytes = count * out_elems * 4;
    if (overlaps(in_mont, in_bytes, out_mont, out_bytes)) return G16_EALIAS;
    if (overlaps(out_mont, out_bytes, ctx->ws_begin, ctx->ws_bytes)) return G16_EALIAS;
    if (!g16::device_range(in_mont, in_bytes) || !g16::device_range(out_mont, out_bytes))
        return G16_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    g16::BbParams p;
    std::memset(&p, 0, sizeof p);
    p.src = (const uint32_t*)in_mont;
    p.dst = (uint32_t*)out_mont;
    p.tw = ctx->tw;
    p.twm = ctx->twm;
    p.in_stride = in_elems;
    p.out_stride = out_elems;
    p.log_n = L;
    p.log_w = log_w;
    p.log_in = log_in;
    if (L <= 4) {
        const uint64_t columns = count << log_w;
        hipLaunchKernelGGL(g16::bb_small_kernel, dim3((uint32_t)((columns + 255) / 256)),
                           dim3(256), 0, s, p, columns);
        return hipGetLastError() == hipSuccess ? G16_OK : G16_EHIP;
    }
    uint32_t ks[8];
    const int nb = g16_bb_batch_plan(L, ks, 8);
    uint32_t s0 = 0;
    for (int b = 0; b < nb; ++b) {
        const uint32_t K = ks[b];
        const uint32_t slices = log_w + L - K;  // log2 of the slices of a matrix
        p.s0 = s0;
        p.k = K;
        p.log_spw = slices < 5u ? slices : 5u;
        p.groups = 1u << (slices - p.log_spw);
        if (b > 0) p.src = p.dst;
        const uint64_t blocks = (uint64_t)p.groups * count;
        if (blocks >= (1ull << 31)) return G16_EINVAL;
        const bool mont = (int)log_w <= kMontMaxLogW;
        if (launch_batch(b == 0, mont, p, (uint32_t)blocks, s) != hipSuccess) return G16_EHIP;
        s0 += K;
    }
    return G16_OK;
}

static int bb_scale(uint64_t n, const void* in, void* out, uint32_t m, void* stream) {
    if (n == 0) return G16_OK;
    if (!in || !out) return G16_EINVAL;
    const size_t bytes = n * 4;
    if (in != out && overlaps(in, bytes, out, bytes)) return G16_EALIAS;
    if (!g16::device_range(in, bytes) || !g16::device_range(out, bytes)) return G16_EINVAL;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(g16::bb_scale_kernel, dim3((uint32_t)(blocks < 8192 ? blocks : 8192)),
                       dim3(256), 0, (hipStream_t)stream, (const uint32_t*)in, (uint32_t*)out, n,
                       m, g16::bb_shoup_companion(m));
    return hipGetLastError() == hipSuccess ? G16_OK : G16_EHIP;
}

int g16_bb_to_mont(uint64_t n, const void* in_std, void* out_mont, void* stream) {
    return bb_scale(n, in_std, out_mont, (uint32_t)((1ull << 32) % g16::kBbP), stream);
}

int g16_bb_from_mont(uint64_t n, const void* in_mont, void* out_std, void* stream) {
    // 2^-32 mod p by Fermat
    const uint32_t r = (uint32_t)((1ull << 32) % g16::kBbP);
    return bb_scale(n, in_mont, out_std, g16::bb_pow_plain(r, g16::kBbP - 2u), stream);
}

}  // extern "C"
