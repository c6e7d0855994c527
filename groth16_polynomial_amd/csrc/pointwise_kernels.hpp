// Element-wise, table and gather kernels (non-template; included by g16.hip only).
#pragma once

#include "kernels.hpp"

namespace g16 {

// ------------------------------------------------------------------ element-wise kernels

__global__ void __launch_bounds__(256) h_join_kernel(const Fr* a, const Fr* b, const Fr* c,
                                                     Fr* h_mont, Fr* h_std, uint64_t n) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x) {
        Fr h = fr_sub(fr_mul(ld_global(a + i), ld_global(b + i)), ld_global(c + i));
        st_global(h_mont + i, h);
        st_global(h_std + i, fr_from_mont(h));
    }
}

// op 0: to Montgomery, 1: from Montgomery, 2: product with b
__global__ void __launch_bounds__(256) elementwise_kernel(const Fr* a, const Fr* b, Fr* out,
                                                          uint64_t n, int op) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x) {
        Fr x = ld_global(a + i);
        Fr y;
        if (op == 0) y = fr_to_mont(x);
        else if (op == 1) y = fr_from_mont(x);
        else y = fr_mul(x, ld_global(b + i));
        st_global(out + i, y);
    }
}

// Table builders.  Each thread raises the base to its own exponent (prepare time only)
// and stores the entry the table products take (fr29.hpp: the plain value and its
// Shoup companion floor(w 2^261 / r)).
//   kind 0: twiddles by level (see level_index): entry e = n - n/2^m + j of level m is
//           base^(2^m j), for the n - 1 entries of a 2^L domain
//   kind 2: the same levels bit-reversed: entry n - n/2^m + j is
//           base^(2^m bitrev_(L-1-m)(j))
//   kind 3: kind 0 with the coset shift folded in: the levels of the passes on bits
//           b = L-1-m >= 2 times factor^(2^m) (factor = s; the coset shift, kernels.hpp)
//   kind 1: the four kappa entries, q < 4: factor base^(2^(L-1) q_0 + 2^(L-2) q_1)
//           (base = s, factor = n^-1; q_1 only for L >= 2)
__device__ __forceinline__ void st_tw(const TwTab& tab, uint64_t e, const Tw29& t) {
    uint4* q = tab.base + e;
    const size_t s = tab.stride;
    q[0] = make_uint4(t.w[0], t.w[1], t.w[2], t.w[3]);
    q[s] = make_uint4(t.w[4], t.w[5], t.w[6], t.w[7]);
    q[2 * s] = make_uint4(t.w[8], t.wp[0], t.wp[1], t.wp[2]);
    q[3 * s] = make_uint4(t.wp[3], t.wp[4], t.wp[5], t.wp[6]);
    q[4 * s] = make_uint4(t.wp[7], t.wp[8], 0u, 0u);
}

// Tables, one 80-byte entry per thread (grid-stride loop) for the count entries (n - 1
// for the levels, 4 for kind 1).
//   kinds 0 and 3: forward levels (omega = base); entry positions follow fwd_tw_index,
//           for the batch plan whose start bits are set in batch_starts (bit 0 always);
//   kind 2: inverse levels (omega^-1 = base), bit-reversed within each level;
//   kind 1: the kappa entries.
__global__ void __launch_bounds__(256) table_kernel(TwTab out, Fr base, Fr factor,
                                                    uint64_t count, uint32_t log_n, int kind,
                                                    uint32_t batch_starts) {
    const uint64_t n = 1ull << log_n;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
         j += (uint64_t)gridDim.x * blockDim.x) {
        if (kind == 1) {
            uint64_t e = (j & 1u) << (log_n - 1u);
            if (log_n >= 2u) e += (j >> 1) << (log_n - 2u);
            st_tw(out, j, tw29_entry(fr_mul(factor, fr_pow_u64(base, e))));
            continue;
        }
        // level m spans [n - n/2^m, n - n/2^(m+1)) and has L-1-m index bits
        uint32_t m = 0;
        while (j >= n - (n >> (m + 1))) ++m;
        uint64_t jj = j - (n - (n >> m));
        const uint32_t bits = log_n - 1u - m;
        if (kind == 2 && bits > 0u) jj = bitrev_bits((uint32_t)jj, bits);
        if (kind != 2) {
            // position jm + low 2^t -> exponent low + jm 2^s0 (t = bits - s0)
            const uint32_t s0 = 31u - __builtin_clz(batch_starts & ((2u << bits) - 1u));
            const uint32_t t = bits - s0;
            const uint64_t low = jj >> t, jm = jj & ((1ull << t) - 1ull);
            jj = low + (jm << s0);
        }
        Fr v = fr_pow_u64(base, jj << m);
        // the pass on bit L-1-m >= 2 of the shifted forward table: times s^(2^m)
        if (kind == 3 && bits >= 2u) v = fr_mul(v, fr_pow_u64(factor, 1ull << m));
        st_tw(out, j, tw29_entry(v));
    }
}

// The CSR gather: 64 consecutive rows per workgroup of one wave (the GATHER_CU page puts
// a row on a lane: rows are short and ragged).  With a row per lane a wave would form as
// many products as its longest row has terms, while most rows have one or two; here the
// wave flattens its rows' terms instead, the terms of its A rows followed by those of its
// B rows, so that both matrices share each dependent load: the row pointers of A and B
// are read together, and in each round of 64 terms every lane forms one product (value
// times witness, from A or B).  Then every lane adds the products of its own A row and
// its own B row from LDS (additions only).  A row whose range or a signal is out of
// bounds is flagged and reads nothing out of bounds.
constexpr uint32_t kGatherLanes = 64;

__device__ __forceinline__ Fr fr_invalid() {
    Fr z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = 0xffffffffu;
    return z;
}

// Per row of the wave, A rows at [0, 64) and B rows at [64, 128).
struct GatherLds {
    uint64_t off[2 * kGatherLanes];  // the row's first term in the wave's flattened list
    uint32_t lo[2 * kGatherLanes];   // its first index in its matrix's CSR arrays
    uint32_t len[2 * kGatherLanes];  // its number of terms
    uint32_t bad[2 * kGatherLanes];  // it named a witness index out of range
    Fr prod[kGatherLanes];           // the round's products, by flattened term
};

// Row `row` of one matrix: its CSR range, or an empty range and false when the range is
// not within [0, nnz].
__device__ __forceinline__ bool gather_range(const uint32_t* row_ptr, uint64_t nnz,
                                             uint64_t row, bool in_rows, uint32_t& lo,
                                             uint32_t& len) {
    lo = 0;
    len = 0;
    if (!in_rows) return true;
    lo = row_ptr[row];
    const uint32_t hi = row_ptr[row + 1];
    const bool ok = lo <= hi && (uint64_t)hi <= nnz;
    len = ok ? hi - lo : 0u;
    return ok;
}

// The sum of this lane's row's products that fall in the round's window [t0, t0 + 64).
__device__ __forceinline__ void gather_add_round(Fr& acc, const GatherLds& sh, uint64_t off,
                                                 uint32_t len, uint64_t t0) {
    const uint64_t a0 = off > t0 ? off : t0;
    const uint64_t a1 = off + len < t0 + kGatherLanes ? off + len : t0 + kGatherLanes;
    for (uint64_t j = a0; j < a1; ++j) acc = fr_add(acc, sh.prod[j - t0]);
}

__global__ void __launch_bounds__(kGatherLanes) gather_kernel(
    const uint32_t* row_ptr_a, const uint32_t* signal_a, const Fr* value_a, uint64_t nnz_a,
    const uint32_t* row_ptr_b, const uint32_t* signal_b, const Fr* value_b, uint64_t nnz_b,
    const Fr* witness, uint64_t n_witness, Fr* out_a, Fr* out_b, Fr* out_c, uint64_t n_rows) {
    __shared__ GatherLds sh;
    const uint32_t l = threadIdx.x;
    const uint64_t row = (uint64_t)blockIdx.x * kGatherLanes + l;
    const bool in_rows = row < n_rows;
    uint32_t lo_a, len_a, lo_b, len_b;
    const bool ok_a = gather_range(row_ptr_a, nnz_a, row, in_rows, lo_a, len_a);
    const bool ok_b = gather_range(row_ptr_b, nnz_b, row, in_rows, lo_b, len_b);
    // exclusive prefixes of the lengths over the wave (64-bit: ranges of malformed row
    // pointers may overlap, and each is only checked against its nnz)
    uint64_t inc_a = len_a, inc_b = len_b;
#pragma unroll
    for (uint32_t d = 1; d < kGatherLanes; d <<= 1) {
        const uint64_t ya = __shfl_up(inc_a, d, kGatherLanes);
        const uint64_t yb = __shfl_up(inc_b, d, kGatherLanes);
        if (l >= d) {
            inc_a += ya;
            inc_b += yb;
        }
    }
    const uint64_t total_a = __shfl(inc_a, kGatherLanes - 1u, kGatherLanes);
    const uint64_t total = total_a + __shfl(inc_b, kGatherLanes - 1u, kGatherLanes);
    const uint64_t off_a = inc_a - len_a;
    const uint64_t off_b = total_a + inc_b - len_b;
    sh.off[l] = off_a;
    sh.off[kGatherLanes + l] = off_b;
    sh.lo[l] = lo_a;
    sh.lo[kGatherLanes + l] = lo_b;
    sh.len[l] = len_a;
    sh.len[kGatherLanes + l] = len_b;
    sh.bad[l] = 0u;
    sh.bad[kGatherLanes + l] = 0u;
    __syncthreads();
    Fr a = fr_zero(), b = fr_zero();
    for (uint64_t t0 = 0; t0 < total; t0 += kGatherLanes) {
        const uint64_t f = t0 + l;
        Fr p = fr_zero();
        if (f < total) {
            // the last row whose first term is at or before f (empty rows share their
            // successor's offset, so that row is the one holding f)
            uint32_t r = 0;
#pragma unroll
            for (uint32_t step = kGatherLanes; step > 0; step >>= 1)
                if (r + step < 2u * kGatherLanes && sh.off[r + step] <= f) r += step;
            const uint64_t j = f - sh.off[r];  // < len[r], so k < hi <= nnz
            if (j < sh.len[r]) {
                const bool in_b = r >= kGatherLanes;
                const uint32_t k = sh.lo[r] + (uint32_t)j;
                const uint32_t s = (in_b ? signal_b : signal_a)[k];
                const Fr v = ld_global((in_b ? value_b : value_a) + k);
                if ((uint64_t)s < n_witness)
                    p = fr_mul29(v, ld_global(witness + s));
                else
                    sh.bad[r] = 1u;
            }
        }
        sh.prod[l] = p;
        __syncthreads();
        gather_add_round(a, sh, off_a, len_a, t0);
        gather_add_round(b, sh, off_b, len_b, t0);
        __syncthreads();
    }
    if (!in_rows) return;
    if (ok_a && ok_b && sh.bad[l] == 0u && sh.bad[kGatherLanes + l] == 0u) {
        st_global(out_a + row, a);
        st_global(out_b + row, b);
        st_global(out_c + row, fr_mul29(a, b));
    } else {
        Fr bad = fr_invalid();
        st_global(out_a + row, bad);
        st_global(out_b + row, bad);
        st_global(out_c + row, bad);
    }
}

}  // namespace g16
