// Batched lossless speculative-sampling verification on CDNA4 (gfx950).
//
// What is computed ("breaking down dspark and its lineage", sections
// "Speculative decoding basics: drafting and verification" and "Preserving the
// target distribution during verification"; "UraionSpec", section "Speculative
// Decoding", Eq. (acceptance); "AngelSpec", sections 1 and 4.1): per request,
// the temperature softmax of every read target row, the accept test
// u < p(x)/q(x) for each draft, the first rejection j, and one inverse-CDF draw
// from max(p_j - q_j, 0) (a rejection) or from p_len (the bonus token).
// Temperature 0 is the exact argmax limit.
//
// How it maps to the chip
// -----------------------
// The work is a bandwidth-bound streaming reduction (no contraction, so no
// MFMA).  One launch handles the whole batch:
//
//   row-pass items   one workgroup per (request, row, chunk of the vocabulary):
//                    8 x 16-byte loads in flight per thread, held in registers,
//                    chunk maximum, then sum of 2^((z - m) * log2(e)/T); wave
//                    butterflies and LDS merge (max, sum) pairs.  The
//                    workgroup that finishes a request's last chunk (arrival
//                    counter) merges that request's chunk partials in fp64,
//                    runs the accept tests and the first-reject scan, writes
//                    the accepted prefix, and publishes a decision record.
//   draw items       a few workgroups per request, placed in the grid `lag`
//                    requests behind the request's row-pass items, wait for its
//                    decision, stream the one row the final token is drawn from
//                    (target row, plus the draft row on a rejection) in tiles of
//                    8192, and write per-tile masses; the last one to arrive
//                    locates the tile holding u * R by an fp64 prefix over tiles
//                    and re-scans only that tile to find the token.
//
// The draw items of request b only wait for row-pass items that precede them
// in the grid, and the host keeps the number of draw workgroups below half the
// device's resident capacity, so the waits always end (they are also bounded).
// When that bound cannot be met the host uses two launches (row pass, then
// draw pass) instead.  All counters are reset by their last user, so a zeroed
// workspace stays zeroed after every call.
//
// Determinism: no floating-point atomics; reductions run in a fixed order;
// the per-tile masses and the re-scan use the same code, so the tile the draw
// lands in is found exactly.  The library is compiled with -ffp-contract=off.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"

namespace sv {
namespace {

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Native 2^x (v_exp_f32).  Arguments here are <= 0; results below the fp32
// normal range flush to zero, which is far below every tolerance.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int ES>
__device__ __forceinline__ float load_elem(const void *base, size_t i) {
    if constexpr (ES == 2) {
        return __uint_as_float(uint32_t(static_cast<const uint16_t *>(base)[i]) << 16);
    } else {
        return static_cast<const float *>(base)[i];
    }
}

struct __align__(16) Smem {
    union {
        float ms[8];                      // (max, sum) per wave
        struct { float v[4]; int i[4]; int nan[4]; } am;   // argmax per wave
        double sc[8];                     // scan totals per wave
    } r;
    double S[kWG];                        // fp64 row sums (decision)
    float M[kWG];                         // row maxima (decision)
    int A[kWG];                           // greedy row argmax (decision)
    int jmin, bad, last, flag;
    double base, target, total, R;
    int tstar, mode, t1, y;
};

// ---------------------------------------------------------------- reductions

// Merge two (max, sum) partials of the same row; sums are relative to their max.
__device__ __forceinline__ void merge_ms(float &m, float &s, float m2, float s2, float c) {
    const float M = fmaxf(m, m2);
    if (M == neg_inf()) { m = M; s = s + s2; return; }
    const float a = (m == neg_inf()) ? 0.0f * s : s * exp2_fast((m - M) * c);
    const float b = (m2 == neg_inf()) ? 0.0f * s2 : s2 * exp2_fast((m2 - M) * c);
    m = M;
    s = a + b;
}

// Result valid in thread 0.
__device__ void wg_reduce_ms(float &m, float &s, float c, Smem &sh) {
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const float s2 = __shfl_xor(s, off);
        merge_ms(m, s, m2, s2, c);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) { sh.r.ms[2 * w] = m; sh.r.ms[2 * w + 1] = s; }
    __syncthreads();
    if (threadIdx.x == 0) {
        m = sh.r.ms[0]; s = sh.r.ms[1];
        for (int i = 1; i < 4; ++i) merge_ms(m, s, sh.r.ms[2 * i], sh.r.ms[2 * i + 1], c);
    }
}

// (value, index) with the larger value; equal values keep the lower index; index < 0 = none.
__device__ __forceinline__ void merge_am(float &v, int &i, float v2, int i2) {
    if (i2 < 0) return;
    if (i < 0 || v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ void wg_reduce_am(float &v, int &i, int &nan, Smem &sh) {
    for (int off = 32; off >= 1; off >>= 1) {
        const float v2 = __shfl_xor(v, off);
        const int i2 = __shfl_xor(i, off);
        const int n2 = __shfl_xor(nan, off);
        merge_am(v, i, v2, i2);
        nan |= n2;
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) { sh.r.am.v[w] = v; sh.r.am.i[w] = i; sh.r.am.nan[w] = nan; }
    __syncthreads();
    if (threadIdx.x == 0) {
        v = sh.r.am.v[0]; i = sh.r.am.i[0]; nan = sh.r.am.nan[0];
        for (int k = 1; k < 4; ++k) { merge_am(v, i, sh.r.am.v[k], sh.r.am.i[k]); nan |= sh.r.am.nan[k]; }
    }
}

// Exclusive prefix over the 256 threads in fp64, fixed association.
// Returns the exclusive prefix; `total` = inclusive prefix of the last thread,
// computed as (its exclusive prefix + its value), the same way every caller's
// inclusive value is formed.
__device__ double wg_excl_scan(double v, double &total, Smem &sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double x = v;
    for (int d = 1; d < 64; d <<= 1) {
        const double y = __shfl_up(x, d);
        if (lane >= d) x = x + y;
    }
    double xprev = __shfl_up(x, 1);
    if (lane == 0) xprev = 0.0;
    __syncthreads();
    if (lane == 63) sh.r.sc[w] = x;
    __syncthreads();
    double wbase = 0.0;
    for (int i = 0; i < w; ++i) wbase = wbase + sh.r.sc[i];
    const double excl = (lane == 0) ? wbase : wbase + xprev;
    if (threadIdx.x == kWG - 1) sh.total = excl + v;
    __syncthreads();
    total = sh.total;
    return excl;
}

// ------------------------------------------------------------- arrivals

// Returns true in every thread of the workgroup that arrives last; that
// workgroup resets the counter and acquires the other workgroups' writes.
__device__ bool arrive_last(unsigned *ctr, unsigned target, Smem &sh) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned old = atomicAdd(ctr, 1u);
        const int last = (old + 1 == target);
        if (last) *ctr = 0u;
        sh.last = last;
    }
    __syncthreads();
    const bool last = sh.last != 0;
    if (last) __threadfence();
    return last;
}

__device__ void write_error(const VerifyArgs &a, int b, bool diag) {
    const int G1 = a.G + 1;
    for (int t = threadIdx.x; t < G1; t += kWG) a.out_tok[size_t(b) * G1 + t] = -1;
    if (threadIdx.x == 0) a.out_acc[b] = -1;
    if (!diag) return;
    const float qnan = __builtin_nanf("");
    for (int t = threadIdx.x; t < G1; t += kWG) {
        if (a.d_lse) a.d_lse[size_t(b) * G1 + t] = qnan;
        if (t < a.G) {
            if (a.d_p) a.d_p[size_t(b) * a.G + t] = qnan;
            if (a.d_q) a.d_q[size_t(b) * a.G + t] = qnan;
        }
    }
    if (threadIdx.x == 0 && a.d_r) a.d_r[b] = qnan;
}

// Per-request counter slot at a fixed offset: [0] row-pass arrivals,
// [1] decision flag, [2] draw-pass arrivals.
__device__ __forceinline__ unsigned *slot(const VerifyArgs &a, int b) {
    return reinterpret_cast<unsigned *>(a.ws + size_t(b) * kSlotBytes);
}

// ------------------------------------------------------------- row pass

// (max, sum of 2^((z-max)*c)) over elements [beg, end) of one row, per thread.
template <int ES, bool AL>
__device__ void chunk_ms(const void *row, int beg, int end, float c, float &m_out, float &s_out) {
    float m = neg_inf();
    if constexpr (AL) {
        constexpr int EPV = 16 / ES;
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const char *>(row) + size_t(beg) * ES);
        const int nvec = (end - beg) / EPV;
        constexpr uint32_t fill = (ES == 2) ? 0xff80ff80u : 0xff800000u;   // -inf
        uint4 r[kVecPerThread];
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const int v = threadIdx.x + i * kWG;
            if (v < nvec) r[i] = p[v];
            else r[i] = make_uint4(fill, fill, fill, fill);
        }
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if constexpr (ES == 2) m = fmaxf(m, fmaxf(bf16_lo(w[d]), bf16_hi(w[d])));
                else m = fmaxf(m, __uint_as_float(w[d]));
            }
        }
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
        if (m == neg_inf()) {
            // Every element is -inf or NaN (fmaxf drops NaN): keep a NaN visible.
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if constexpr (ES == 2) {
                        if (bf16_lo(w[d]) != bf16_lo(w[d]) || bf16_hi(w[d]) != bf16_hi(w[d])) s0 = __builtin_nanf("");
                    } else {
                        if (__uint_as_float(w[d]) != __uint_as_float(w[d])) s0 = __builtin_nanf("");
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                if constexpr (ES == 2) {
                    s0 = s0 + exp2_fast((bf16_lo(w[0]) - m) * c);
                    s1 = s1 + exp2_fast((bf16_hi(w[0]) - m) * c);
                    s2 = s2 + exp2_fast((bf16_lo(w[1]) - m) * c);
                    s3 = s3 + exp2_fast((bf16_hi(w[1]) - m) * c);
                    s0 = s0 + exp2_fast((bf16_lo(w[2]) - m) * c);
                    s1 = s1 + exp2_fast((bf16_hi(w[2]) - m) * c);
                    s2 = s2 + exp2_fast((bf16_lo(w[3]) - m) * c);
                    s3 = s3 + exp2_fast((bf16_hi(w[3]) - m) * c);
                } else {
                    s0 = s0 + exp2_fast((__uint_as_float(w[0]) - m) * c);
                    s1 = s1 + exp2_fast((__uint_as_float(w[1]) - m) * c);
                    s2 = s2 + exp2_fast((__uint_as_float(w[2]) - m) * c);
                    s3 = s3 + exp2_fast((__uint_as_float(w[3]) - m) * c);
                }
            }
        }
        s_out = (s0 + s1) + (s2 + s3);
    } else {
        float s = 0.0f;
        for (int e = beg + threadIdx.x; e < end; e += kWG) {
            const float v = load_elem<ES>(row, size_t(e));
            if (v > m) { s = s * exp2_fast((m - v) * c); m = v; }
            if (m != neg_inf()) s = s + exp2_fast((v - m) * c);
            else if (v != v) s = v;                       // NaN among -inf: keep it visible
        }
        s_out = s;
    }
    m_out = m;
}

// (max, lowest index of max, any NaN) over [beg, end), per thread, ascending order.
template <int ES, bool AL>
__device__ void chunk_argmax(const void *row, int beg, int end, float &best, int &bi, int &nan) {
    best = neg_inf(); bi = -1; nan = 0;
    if constexpr (AL) {
        constexpr int EPV = 16 / ES;
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const char *>(row) + size_t(beg) * ES);
        const int nvec = (end - beg) / EPV;
        constexpr uint32_t fill = (ES == 2) ? 0xff80ff80u : 0xff800000u;   // -inf
        uint4 r[kVecPerThread];
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const int v = threadIdx.x + i * kWG;
            r[i] = (v < nvec) ? p[v] : make_uint4(fill, fill, fill, fill);
        }
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const int e0 = beg + (threadIdx.x + i * kWG) * EPV;
            const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if constexpr (ES == 2) {
                    const float lo = bf16_lo(w[d]), hi = bf16_hi(w[d]);
                    nan |= (lo != lo) | (hi != hi);
                    if (lo > best) { best = lo; bi = e0 + 2 * d; }
                    if (hi > best) { best = hi; bi = e0 + 2 * d + 1; }
                } else {
                    const float f = __uint_as_float(w[d]);
                    nan |= (f != f);
                    if (f > best) { best = f; bi = e0 + d; }
                }
            }
        }
    } else {
        for (int e = beg + threadIdx.x; e < end; e += kWG) {
            const float v = load_elem<ES>(row, size_t(e));
            nan |= (v != v);
            if (v > best) { best = v; bi = e; }
        }
    }
}

// ---------------------------------------------------------- decisions

// Workgroup that completed request b's row pass (T > 0).
template <int ES>
__device__ void decide_sampled(const VerifyArgs &a, int b, int n, Smem &sh) {
    const int G1 = a.G + 1;
    const float2 *part = reinterpret_cast<const float2 *>(a.ws + a.lay.part) + size_t(b) * G1 * a.nc1;
    const double c64 = double(a.c32);
    const double T64 = double(a.T);
    if (threadIdx.x == 0) { sh.jmin = n; sh.bad = 0; }
    __syncthreads();
    for (int r = threadIdx.x; r <= n; r += kWG) {
        const float2 *pp = part + size_t(r) * a.nc1;
        float M = neg_inf();
        for (int c = 0; c < a.nc1; ++c) M = fmaxf(M, pp[c].x);
        double S = 0.0;
        for (int c = 0; c < a.nc1; ++c) {
            const float2 v = pp[c];
            if (v.x == neg_inf() && v.y == 0.0f) continue;          // empty chunk
            S = S + double(v.y) * exp2((double(v.x) - double(M)) * c64);
        }
        const bool bad = !(S > 0.0 && S < INFINITY) || !(M > neg_inf() && M < INFINITY);
        if (bad) atomicOr(&sh.bad, 1);
        sh.M[r] = M;
        sh.S[r] = S;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < n; k += kWG) {
        const int xk = a.x[size_t(b) * a.G + k];
        if (xk < 0 || xk >= a.V) { atomicOr(&sh.bad, 1); continue; }
        const float zx = load_elem<ES>(a.logits, (size_t(b) * G1 + k) * size_t(a.V) + size_t(xk));
        const float qx = a.q[(size_t(b) * a.G + k) * size_t(a.V) + size_t(xk)];
        const double u = double(a.u[size_t(b) * G1 + k]);
        const double p = exp((double(zx) - double(sh.M[k])) / T64) / sh.S[k];
        const bool acc = (qx > 0.0f) ? (u < p / double(qx)) : (p > 0.0);
        if (!acc) atomicMin(&sh.jmin, k);
        if (a.d_p) a.d_p[size_t(b) * a.G + k] = float(p);
        if (a.d_q) a.d_q[size_t(b) * a.G + k] = qx;
    }
    __syncthreads();
    unsigned *flag = slot(a, b) + 1;
    const bool diag = a.d_lse || a.d_p || a.d_q || a.d_r;
    if (sh.bad) {
        write_error(a, b, diag);
        __syncthreads();
        if (threadIdx.x == 0) {
            __threadfence();
            __hip_atomic_store(flag, kFlagError, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    const int j = sh.jmin;
    const float qnan = __builtin_nanf("");
    for (int t = threadIdx.x; t < G1; t += kWG) {
        if (t < j) a.out_tok[size_t(b) * G1 + t] = a.x[size_t(b) * a.G + t];
        else if (t > j) a.out_tok[size_t(b) * G1 + t] = -1;
        if (a.d_lse) a.d_lse[size_t(b) * G1 + t] = (t <= n) ? float(double(sh.M[t]) / T64 + log(sh.S[t])) : qnan;
        if (t >= n && t < a.G) {
            if (a.d_p) a.d_p[size_t(b) * a.G + t] = qnan;
            if (a.d_q) a.d_q[size_t(b) * a.G + t] = qnan;
        }
    }
    if (threadIdx.x == 0) {
        a.out_acc[b] = j;
        const int row = (j < n) ? j : n;
        Decision d;
        d.j = j;
        d.row = row;
        d.resid = (j < n) ? 1 : 0;
        d.pad = 0;
        d.m = sh.M[row];
        d.s = sh.S[row];
        d.inv_s = float(1.0 / sh.S[row]);
        reinterpret_cast<Decision *>(a.ws + a.lay.dec)[b] = d;
        __threadfence();
        __hip_atomic_store(flag, kFlagReady, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Workgroup that completed request b's row pass (T == 0).
__device__ void decide_greedy(const VerifyArgs &a, int b, int n, Smem &sh) {
    const int G1 = a.G + 1;
    const int2 *part = reinterpret_cast<const int2 *>(a.ws + a.lay.part) + size_t(b) * G1 * a.nc1;
    if (threadIdx.x == 0) { sh.jmin = n; sh.bad = 0; }
    __syncthreads();
    for (int r = threadIdx.x; r <= n; r += kWG) {
        const int2 *pp = part + size_t(r) * a.nc1;
        float best = neg_inf();
        int bi = -1, nan = 0;
        for (int c = 0; c < a.nc1; ++c) {               // ascending chunks: first maximum wins
            const int2 v = pp[c];
            if (v.y == kNanIdx) { nan = 1; continue; }
            merge_am(best, bi, __int_as_float(v.x), v.y);
        }
        if (nan || bi < 0 || best == __builtin_inff()) atomicOr(&sh.bad, 1);
        sh.A[r] = bi;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < n; k += kWG) {
        const int xk = a.x[size_t(b) * a.G + k];
        if (xk < 0 || xk >= a.V) { atomicOr(&sh.bad, 1); continue; }
        if (xk != sh.A[k]) atomicMin(&sh.jmin, k);
    }
    __syncthreads();
    if (sh.bad) { write_error(a, b, false); return; }
    const int j = sh.jmin;
    for (int t = threadIdx.x; t < G1; t += kWG) {
        int v = -1;
        if (t < j) v = a.x[size_t(b) * a.G + t];
        else if (t == j) v = sh.A[j];
        a.out_tok[size_t(b) * G1 + t] = v;
    }
    if (threadIdx.x == 0) a.out_acc[b] = j;
}

// ---------------------------------------------------------- final draw

__device__ __forceinline__ void draw_term(float z, float q, const Decision &d, float c, bool resid,
                                          float &r, float &p) {
    const float e = exp2_fast((z - d.m) * c);
    p = e * d.inv_s;
    r = resid ? fmaxf(p - q, 0.0f) : p;
}

// Sums over one thread's run [e0, e0 + kRun) of a draw row: residual (or
// target) mass `rs` and target mass `ps`, accumulated in fp64 in index order.
template <int ES, bool ALZ, bool ALQ>
__device__ void run_sums(const void *zrow, const float *qrow, int V, int e0, const Decision &d,
                         float c, bool resid, double &rs, double &ps) {
    rs = 0.0; ps = 0.0;
    if (e0 >= V) return;
    const bool vec = ALZ && (!resid || ALQ) && (e0 + kRun <= V);
    if (vec) {
        float z[kRun], q[kRun];
        const uint4 *zp = reinterpret_cast<const uint4 *>(static_cast<const char *>(zrow) + size_t(e0) * ES);
        if constexpr (ES == 2) {
#pragma unroll
            for (int i = 0; i < kRun / 8; ++i) {
                const uint4 w = zp[i];
                z[8 * i + 0] = bf16_lo(w.x); z[8 * i + 1] = bf16_hi(w.x);
                z[8 * i + 2] = bf16_lo(w.y); z[8 * i + 3] = bf16_hi(w.y);
                z[8 * i + 4] = bf16_lo(w.z); z[8 * i + 5] = bf16_hi(w.z);
                z[8 * i + 6] = bf16_lo(w.w); z[8 * i + 7] = bf16_hi(w.w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kRun / 4; ++i) {
                const uint4 w = zp[i];
                z[4 * i + 0] = __uint_as_float(w.x); z[4 * i + 1] = __uint_as_float(w.y);
                z[4 * i + 2] = __uint_as_float(w.z); z[4 * i + 3] = __uint_as_float(w.w);
            }
        }
        if (resid) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(qrow + e0);
#pragma unroll
            for (int i = 0; i < kRun / 4; ++i) {
                const uint4 w = qp[i];
                q[4 * i + 0] = __uint_as_float(w.x); q[4 * i + 1] = __uint_as_float(w.y);
                q[4 * i + 2] = __uint_as_float(w.z); q[4 * i + 3] = __uint_as_float(w.w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kRun; ++i) q[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kRun; ++i) {
            float r, p;
            draw_term(z[i], q[i], d, c, resid, r, p);
            rs = rs + double(r);
            ps = ps + double(p);
        }
    } else {
        const int e1 = min(V, e0 + kRun);
        for (int e = e0; e < e1; ++e) {
            float r, p;
            draw_term(load_elem<ES>(zrow, size_t(e)), resid ? qrow[e] : 0.0f, d, c, resid, r, p);
            rs = rs + double(r);
            ps = ps + double(p);
        }
    }
}

// Last draw workgroup of request b: locate u * R and write the token.
template <int ES, bool ALZ, bool ALQ>
__device__ void final_select(const VerifyArgs &a, int b, const Decision &d, const void *zrow,
                             const float *qrow, Smem &sh) {
    const int G1 = a.G + 1;
    const double2 *mass = reinterpret_cast<const double2 *>(a.ws + a.lay.mass) + size_t(b) * a.ntiles;
    bool resid = d.resid != 0;
    if (threadIdx.x == 0) {
        double R = 0.0, Rp = 0.0;
        for (int t = 0; t < a.ntiles; ++t) { const double2 m = mass[t]; R = R + m.x; Rp = Rp + m.y; }
        int mode = resid ? 1 : 0;                       // 1: residual terms, 0: target terms
        if (resid && !(R > 0.0)) mode = 0;              // zero residual: draw from p_j
        const double total = mode ? R : (resid ? Rp : R);
        const double target = double(a.u[size_t(b) * G1 + a.G]) * total;
        double P = 0.0;
        int tstar = -1;
        for (int t = 0; t < a.ntiles; ++t) {
            const double2 m = mass[t];
            const double mt = mode ? m.x : (resid ? m.y : m.x);
            const double P1 = P + mt;
            if (P1 > target) { tstar = t; break; }
            P = P1;
        }
        int lastpos = 0;
        if (tstar < 0) {                                 // u * R at or beyond the top
            lastpos = 1;
            for (int t = a.ntiles - 1; t >= 0; --t) {
                const double2 m = mass[t];
                const double mt = mode ? m.x : (resid ? m.y : m.x);
                if (mt > 0.0) { tstar = t; break; }
            }
            if (tstar < 0) tstar = 0;
        }
        sh.mode = mode | (lastpos << 1);
        sh.tstar = tstar;
        sh.base = P;
        sh.target = target;
        sh.R = R;
        sh.t1 = kWG;
        sh.y = -1;
    }
    __syncthreads();
    const int mode = sh.mode & 1, lastpos = sh.mode >> 1;
    const int tstar = sh.tstar;
    const double base = sh.base, target = sh.target, R = sh.R;
    const bool use_resid = resid && mode;
    const int e0 = tstar * kTile + threadIdx.x * kRun;
    double rs, ps;
    run_sums<ES, ALZ, ALQ>(zrow, qrow, a.V, e0, d, a.c32, resid, rs, ps);
    const double mine = use_resid ? rs : (resid ? ps : rs);
    double tile_total;
    const double excl = wg_excl_scan(mine, tile_total, sh);
    const int e1 = min(a.V, e0 + kRun);
    if (lastpos) {
        int lp = -1;
        for (int e = e0; e < e1; ++e) {
            float r, p;
            draw_term(load_elem<ES>(zrow, size_t(e)), resid ? qrow[e] : 0.0f, d, a.c32, resid, r, p);
            if ((use_resid ? r : p) > 0.0f) lp = e;
        }
        atomicMax(&sh.y, lp);
        __syncthreads();
    } else {
        if (base + (excl + mine) > target) atomicMin(&sh.t1, int(threadIdx.x));
        __syncthreads();
        if (int(threadIdx.x) == sh.t1) {
            double acc = base + excl;
            int y = -1, lp = -1;
            for (int e = e0; e < e1; ++e) {
                float r, p;
                draw_term(load_elem<ES>(zrow, size_t(e)), resid ? qrow[e] : 0.0f, d, a.c32, resid, r, p);
                const float t = use_resid ? r : p;
                if (t > 0.0f) lp = e;
                acc = acc + double(t);
                if (acc > target) { y = e; break; }
            }
            sh.y = (y >= 0) ? y : lp;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.out_tok[size_t(b) * G1 + d.j] = sh.y;
        if (a.d_r) a.d_r[b] = resid ? float(R) : -1.0f;
    }
}

// One draw workgroup: tiles [w*tpw, (w+1)*tpw) of request b's draw row.
template <int ES, bool ALZ, bool ALQ>
__device__ void draw_item(const VerifyArgs &a, int b, int w, Smem &sh) {
    unsigned *flag = slot(a, b) + 1;
    unsigned *ctr2 = slot(a, b) + 2;
    if (threadIdx.x == 0) {
        unsigned f;
        uint32_t spins = 0;
        while ((f = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
            if (++spins > a.spin_limit) break;
            __builtin_amdgcn_s_sleep(2);
        }
        sh.flag = int(f);
    }
    __syncthreads();
    unsigned f = unsigned(sh.flag);
    if (f == 0u) {                                   // bounded wait expired: report, do not arrive
        write_error(a, b, false);
        return;
    }
    f = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if (f == kFlagError) {
        if (arrive_last(ctr2, unsigned(a.nc2), sh) && threadIdx.x == 0) *flag = 0u;
        return;
    }
    const Decision d = reinterpret_cast<const Decision *>(a.ws + a.lay.dec)[b];
    if (d.j < 0 || d.j > a.G || d.row != d.j || (d.resid != 0 && d.j >= a.G)) {
        // Not a record this call wrote (workspace not zero-filled before its
        // first use): report the request instead of following it.
        write_error(a, b, false);
        if (arrive_last(ctr2, unsigned(a.nc2), sh) && threadIdx.x == 0) *flag = 0u;
        return;
    }
    const bool resid = d.resid != 0;
    const int G1 = a.G + 1;
    const void *zrow = static_cast<const char *>(a.logits) + (size_t(b) * G1 + d.row) * size_t(a.V) * ES;
    const float *qrow = resid ? a.q + (size_t(b) * a.G + d.j) * size_t(a.V) : nullptr;
    double2 *mass = reinterpret_cast<double2 *>(a.ws + a.lay.mass) + size_t(b) * a.ntiles;
    const int t_end = min(a.ntiles, (w + 1) * a.tpw);
    for (int t = w * a.tpw; t < t_end; ++t) {
        double rs, ps, rtot, ptot;
        run_sums<ES, ALZ, ALQ>(zrow, qrow, a.V, t * kTile + threadIdx.x * kRun, d, a.c32, resid, rs, ps);
        wg_excl_scan(rs, rtot, sh);
        if (resid) wg_excl_scan(ps, ptot, sh);
        else ptot = rtot;
        if (threadIdx.x == 0) mass[t] = make_double2(rtot, ptot);
    }
    if (arrive_last(ctr2, unsigned(a.nc2), sh)) {
        final_select<ES, ALZ, ALQ>(a, b, d, zrow, qrow, sh);
        __syncthreads();
        if (threadIdx.x == 0) *flag = 0u;
    }
}

// ------------------------------------------------------------- kernels

__device__ __forceinline__ void map_item(const VerifyArgs &a, int i, int &phase, int &b, int &local) {
    const int g1 = (a.G + 1) * a.nc1, g2 = a.nc2;
    if (a.mode == 1) { phase = 1; b = i / g1; local = i - b * g1; return; }
    if (a.mode == 2) { phase = 2; b = i / g2; local = i - b * g2; return; }
    const int L = a.lag;
    const long head = long(L) * g1;
    if (i < head) { phase = 1; b = int(i / g1); local = int(i - long(b) * g1); return; }
    const long i2 = i - head;
    const int seg = g1 + g2;
    const long nseg = long(a.B - L);
    if (i2 < nseg * seg) {
        const long s = i2 / seg;
        const int r = int(i2 - s * seg);
        if (r < g1) { phase = 1; b = L + int(s); local = r; }
        else { phase = 2; b = int(s); local = r - g1; }
        return;
    }
    const long t = i2 - nseg * seg;
    phase = 2;
    b = (a.B - L) + int(t / g2);
    local = int(t % g2);
}

template <int ES, bool ALZ, bool ALQ>
__global__ __launch_bounds__(kWG) void k_verify_sampled(VerifyArgs a) {
    __shared__ Smem sh;
    int phase, b, local;
    map_item(a, int(blockIdx.x), phase, b, local);
    if (phase == 2) { draw_item<ES, ALZ, ALQ>(a, b, local, sh); return; }
    const int k = local / a.nc1, c = local - k * a.nc1;
    const int n = a.vlen ? a.vlen[b] : a.G;
    if (n < 0 || n > a.G) {
        if (k == 0 && c == 0) {
            write_error(a, b, a.d_lse || a.d_p || a.d_q || a.d_r);
            __syncthreads();
            if (threadIdx.x == 0) {
                __threadfence();
                __hip_atomic_store(slot(a, b) + 1, kFlagError, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        return;
    }
    if (k > n) return;
    const int G1 = a.G + 1;
    const void *row = static_cast<const char *>(a.logits) + (size_t(b) * G1 + k) * size_t(a.V) * ES;
    const int beg = c * a.ch1, end = min(a.V, beg + a.ch1);
    float m, s;
    chunk_ms<ES, ALZ>(row, beg, end, a.c32, m, s);
    wg_reduce_ms(m, s, a.c32, sh);
    if (threadIdx.x == 0)
        reinterpret_cast<float2 *>(a.ws + a.lay.part)[(size_t(b) * G1 + k) * a.nc1 + c] = make_float2(m, s);
    if (arrive_last(slot(a, b) + 0, unsigned((n + 1) * a.nc1), sh)) decide_sampled<ES>(a, b, n, sh);
}

template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_verify_greedy(VerifyArgs a) {
    __shared__ Smem sh;
    const int g1 = (a.G + 1) * a.nc1;
    const int b = int(blockIdx.x) / g1, local = int(blockIdx.x) - b * g1;
    const int k = local / a.nc1, c = local - k * a.nc1;
    const int n = a.vlen ? a.vlen[b] : a.G;
    if (n < 0 || n > a.G) {
        if (k == 0 && c == 0) write_error(a, b, false);
        return;
    }
    if (k > n) return;
    const int G1 = a.G + 1;
    const void *row = static_cast<const char *>(a.logits) + (size_t(b) * G1 + k) * size_t(a.V) * ES;
    const int beg = c * a.ch1, end = min(a.V, beg + a.ch1);
    float best;
    int bi, nan;
    chunk_argmax<ES, AL>(row, beg, end, best, bi, nan);
    wg_reduce_am(best, bi, nan, sh);
    if (threadIdx.x == 0)
        reinterpret_cast<int2 *>(a.ws + a.lay.part)[(size_t(b) * G1 + k) * a.nc1 + c] =
            make_int2(__float_as_int(best), nan ? kNanIdx : bi);
    if (arrive_last(slot(a, b) + 0, unsigned((n + 1) * a.nc1), sh)) decide_greedy(a, b, n, sh);
}

template <int ES, bool ALZ, bool ALQ>
int launch_s(const VerifyArgs &a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_verify_sampled<ES, ALZ, ALQ>), dim3(grid), dim3(kWG), 0, st, a);
    return int(hipGetLastError());
}

template <int ES, bool AL>
int launch_g(const VerifyArgs &a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_verify_greedy<ES, AL>), dim3(grid), dim3(kWG), 0, st, a);
    return int(hipGetLastError());
}

template <int ES, bool ALZ, bool ALQ>
int occ_s(int *n) {
    return int(hipOccupancyMaxActiveBlocksPerMultiprocessor(n, k_verify_sampled<ES, ALZ, ALQ>, kWG, 0));
}

}  // namespace

int launch_verify_sampled(const VerifyArgs &a, bool az, bool aq, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) {
        if (az && aq) return launch_s<2, true, true>(a, grid, st);
        if (az) return launch_s<2, true, false>(a, grid, st);
        return launch_s<2, false, false>(a, grid, st);
    }
    if (az && aq) return launch_s<4, true, true>(a, grid, st);
    if (az) return launch_s<4, true, false>(a, grid, st);
    return launch_s<4, false, false>(a, grid, st);
}

int launch_verify_greedy(const VerifyArgs &a, bool az, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) return az ? launch_g<2, true>(a, grid, st) : launch_g<2, false>(a, grid, st);
    return az ? launch_g<4, true>(a, grid, st) : launch_g<4, false>(a, grid, st);
}

int verify_sampled_occupancy(bool az, bool aq, int esize, int *n) {
    if (esize == 2) {
        if (az && aq) return occ_s<2, true, true>(n);
        if (az) return occ_s<2, true, false>(n);
        return occ_s<2, false, false>(n);
    }
    if (az && aq) return occ_s<4, true, true>(n);
    if (az) return occ_s<4, true, false>(n);
    return occ_s<4, false, false>(n);
}

}  // namespace sv
