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
// MFMA).  Temperature > 0 runs as two launches on the caller's stream:
//
//   row pass       one workgroup per (request, row, 16384-element chunk):
//                  8 x 16-byte loads in flight per thread, the chunk maximum,
//                  then the sum of 2^((z - m) * log2(e)/T), merged across the
//                  workgroup by wave butterflies and LDS; the (max, sum)
//                  partial is one 64-bit store.  Nothing else, so the kernel
//                  keeps few registers and full occupancy.
//   request pass   nc2 workgroups per request, one per pair of 2048-element
//                  sub-tiles of the draw row.  Each merges the request's chunk
//                  partials per row in fp64, runs the accept tests and finds the
//                  first rejection j (every workgroup of the request computes
//                  the same result), then streams its sub-tiles of the one row
//                  the final token is drawn from (target row j, plus draft row j
//                  on a rejection) and writes fp64 sub-tile masses.  The last of
//                  the request's workgroups to arrive (a counter) locates u * R
//                  by a prefix over the masses, re-scans that one sub-tile,
//                  writes the token, and zeroes every workspace word the
//                  request used.
//
// Nothing waits on anything inside a launch except the arrival counter, so
// there are no spin loops on this path.  Temperature 0 (argmax) is one launch:
// row items, then one item per request that polls its rows' partials (bounded
// wait) — the host keeps those below half the resident capacity, else it
// splits them into a second launch.
//
// Words handed between workgroups of one launch (sub-tile masses, the greedy
// partials) use coherent device-scope stores and loads instead of device-scope
// fences, which on this chip write back or invalidate the whole L2.
//
// Determinism: no floating-point atomics; every reduction has a fixed order;
// the sub-tile masses and the final re-scan run the same code, so the sub-tile
// the draw lands in is found exactly.  The library is compiled with
// -ffp-contract=off.

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
// normal range flush to zero, far below every tolerance.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b, c) in one instruction, without the NaN canonicalisation fmaxf
// needs: a NaN in the data reaches the row sum through its exp2 term anyway.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ bool finitef(float x) { return x > -__builtin_inff() && x < __builtin_inff(); }

// Sums are taken in scaled units y = z * c (c = log2(e)/T) against a
// reference R = fl(m * c) for the maximum m of the elements summed:
// 2^(fma(z, c, -R)) rounds only the difference, which is near 0 for the
// terms that dominate.  When R overflows (huge logits or a tiny T) the
// reference falls back to m itself: 2^((z - m) * c).
// Factor that rescales a sum taken against reference m1 to reference m0 >= m1.
__device__ __forceinline__ float rescale(float m1, float m0, float c) {
    if (m1 == -__builtin_inff()) return 0.0f;
    const float r1 = m1 * c, r0 = m0 * c;
    return (finitef(r1) && finitef(r0)) ? __builtin_amdgcn_exp2f(r1 - r0) : __builtin_amdgcn_exp2f((m1 - m0) * c);
}
__device__ __forceinline__ double rescale_d(float m1, float m0, float c) {
    if (m1 == -__builtin_inff()) return 0.0;
    const float r1 = m1 * c, r0 = m0 * c;
    return (finitef(r1) && finitef(r0)) ? exp2(double(r1) - double(r0))
                                        : exp2((double(m1) - double(m0)) * double(c));
}

template <int ES>
__device__ __forceinline__ float load_elem(const void *base, size_t i) {
    if constexpr (ES == 2) {
        return __uint_as_float(uint32_t(static_cast<const uint16_t *>(base)[i]) << 16);
    } else {
        return static_cast<const float *>(base)[i];
    }
}

// ------------------------------------------------ cross-workgroup publication
//
// Words one workgroup hands to another are written with coherent device-scope
// stores and read with coherent device-scope loads (no whole-cache write-back
// or invalidation, which a generic device-scope fence performs on every L2).
// A chunk partial carries its own valid bit, so it needs no ordering at all.
// Sub-tile masses are ordered before the arrival that publishes them by
// waiting for the stores to complete.
__device__ __forceinline__ void st_coherent(void *p, uint64_t v) {
    __hip_atomic_store(static_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const void *p) {
    return __hip_atomic_load(static_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);          // vmcnt = expcnt = lgkmcnt = 0
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Output words that a later workgroup may overwrite are written through to
// the coherence point, so the last write in time is the one that lands.
__device__ __forceinline__ void st_out(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_out(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float(uint32_t(v)); }
__device__ __forceinline__ uint32_t hi_u(uint64_t v) { return uint32_t(v >> 32); }
__device__ __forceinline__ bool valid(uint64_t v) { return (hi_u(v) & kValid) != 0u; }

struct __align__(16) Smem {
    union {
        float ms[8];                              // (max, sum) per wave
        struct { float v[4]; int i[4]; int nan[4]; } am;   // argmax per wave
        double sc[4][2 * kSubBatch];              // scan totals per wave
    } r;
    double S[kWG];                                // fp64 row sums
    float M[kWG];                                 // row maxima
    int A[kWG];                                   // greedy row argmax
    double mr[kStage], mp[kStage];                // staged sub-tile masses
    double tot[2 * kSubBatch];
    int jmin, bad, last;
    int sstar, mode, t1, y;
    double base, target, R;
};

// ---------------------------------------------------------------- reductions

// Merge two (max, sum) partials of the same row; each sum is taken against
// its own max (see rescale).
__device__ __forceinline__ void merge_ms(float &m, float &s, float m2, float s2, float c) {
    const float M = fmaxf(m, m2);
    if (M == neg_inf()) { m = M; s = s + s2; return; }
    const float a = (m == neg_inf()) ? 0.0f * s : s * rescale(m, M, c);
    const float b = (m2 == neg_inf()) ? 0.0f * s2 : s2 * rescale(m2, M, c);
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

// Exclusive prefix over the 256 threads of NS fp64 values at once.  Each value
// goes through the same fixed sequence of additions whatever NS is.  Writes
// the exclusive prefix to excl[]; the inclusive prefix of a thread is defined
// as excl + v, and total[] is that of the last thread.
template <int NS>
__device__ void wg_excl_scan(const double (&v)[NS], double (&excl)[NS], double (&total)[NS], Smem &sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double x[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) x[i] = v[i];
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const double y = __shfl_up(x[i], d);
            if (lane >= d) x[i] = x[i] + y;
        }
    }
    double xprev[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) xprev[i] = __shfl_up(x[i], 1);
    __syncthreads();
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < NS; ++i) sh.r.sc[w][i] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        double wbase = 0.0;
        for (int k = 0; k < w; ++k) wbase = wbase + sh.r.sc[k][i];
        excl[i] = (lane == 0) ? wbase : wbase + xprev[i];
        if (threadIdx.x == kWG - 1) sh.tot[i] = excl[i] + v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i) total[i] = sh.tot[i];
}

// ------------------------------------------------------------- arrivals

// Every thread's published stores complete, then one counted arrival.
// Returns true in every thread of the workgroup that arrives last; that
// workgroup resets the counter.
__device__ bool arrive_last(unsigned *ctr, unsigned target, Smem &sh) {
    stores_complete();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (old + 1 == target);
        if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.last = last;
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return sh.last != 0;
}

// Draw-workgroup counter of request b (fixed offset for every shape).
__device__ __forceinline__ unsigned *draw_counter(const VerifyArgs &a, int b) {
    return reinterpret_cast<unsigned *>(a.ws + size_t(b) * kSlotBytes) + 2;
}

__device__ __forceinline__ uint64_t *partials(const VerifyArgs &a, int b) {
    return reinterpret_cast<uint64_t *>(a.ws + a.lay.part) + size_t(b) * (a.G + 1) * a.nc1;
}

// A request with a data error: every output word -1 (diagnostics become NaN
// in the diagnostics kernel, which checks out_accepted).
__device__ void write_error(const VerifyArgs &a, int b) {
    const int G1 = a.G + 1;
    for (int t = threadIdx.x; t < G1; t += kWG) st_out(a.out_tok + size_t(b) * G1 + t, -1);
    if (threadIdx.x == 0) st_out(a.out_acc + b, -1);
}

// Wait until the chunk partials of rows 0..n are all written.  False if the
// bounded wait expired.
__device__ bool wait_partials(const VerifyArgs &a, int b, int n) {
    const uint64_t *part = partials(a, b);
    const int np = (n + 1) * a.nc1;
    for (uint32_t spins = 0;; ++spins) {
        bool ready = true;
        for (int i = threadIdx.x; i < np; i += kWG) ready &= valid(ld_coherent(part + i));   // no short circuit: loads overlap
        if (__syncthreads_and(ready)) return true;
        if (spins >= a.spin_limit) return false;
        __builtin_amdgcn_s_sleep(4);
    }
}

// ------------------------------------------------------------- row items

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
            if constexpr (ES == 2) {
#pragma unroll
                for (int d = 0; d < 4; ++d) m = max3(m, bf16_lo(w[d]), bf16_hi(w[d]));
            } else {
                m = max3(m, __uint_as_float(w[0]), __uint_as_float(w[1]));
                m = max3(m, __uint_as_float(w[2]), __uint_as_float(w[3]));
            }
        }
        // Keep only the raw words live between the two passes (re-converting a
        // bf16 is one instruction; holding 64 converted floats costs occupancy).
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i)
            asm volatile("" : "+v"(r[i].x), "+v"(r[i].y), "+v"(r[i].z), "+v"(r[i].w));
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
        } else if (finitef(m * c)) {
            const float nR = -(m * c);
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                if constexpr (ES == 2) {
                    s0 = s0 + exp2_fast(__builtin_fmaf(bf16_lo(w[0]), c, nR));
                    s1 = s1 + exp2_fast(__builtin_fmaf(bf16_hi(w[0]), c, nR));
                    s2 = s2 + exp2_fast(__builtin_fmaf(bf16_lo(w[1]), c, nR));
                    s3 = s3 + exp2_fast(__builtin_fmaf(bf16_hi(w[1]), c, nR));
                    s0 = s0 + exp2_fast(__builtin_fmaf(bf16_lo(w[2]), c, nR));
                    s1 = s1 + exp2_fast(__builtin_fmaf(bf16_hi(w[2]), c, nR));
                    s2 = s2 + exp2_fast(__builtin_fmaf(bf16_lo(w[3]), c, nR));
                    s3 = s3 + exp2_fast(__builtin_fmaf(bf16_hi(w[3]), c, nR));
                } else {
                    s0 = s0 + exp2_fast(__builtin_fmaf(__uint_as_float(w[0]), c, nR));
                    s1 = s1 + exp2_fast(__builtin_fmaf(__uint_as_float(w[1]), c, nR));
                    s2 = s2 + exp2_fast(__builtin_fmaf(__uint_as_float(w[2]), c, nR));
                    s3 = s3 + exp2_fast(__builtin_fmaf(__uint_as_float(w[3]), c, nR));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if constexpr (ES == 2) {
                        s0 = s0 + exp2_fast((bf16_lo(w[d]) - m) * c);
                        s1 = s1 + exp2_fast((bf16_hi(w[d]) - m) * c);
                    } else {
                        s0 = s0 + exp2_fast((__uint_as_float(w[d]) - m) * c);
                    }
                }
            }
        }
        s_out = (s0 + s1) + (s2 + s3);
    } else {
        float s = 0.0f;
        for (int e = beg + threadIdx.x; e < end; e += kWG) {
            const float v = load_elem<ES>(row, size_t(e));
            if (v > m) { s = s * rescale(m, v, c); m = v; }
            if (m != neg_inf()) {
                const float R = m * c;
                s = s + (finitef(R) ? exp2_fast(__builtin_fmaf(v, c, -R)) : exp2_fast((v - m) * c));
            } else if (v != v) {
                s = v;                                    // NaN among -inf: keep it visible
            }
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

__device__ __forceinline__ int verify_len(const VerifyArgs &a, int b) { return a.vlen ? a.vlen[b] : a.G; }

template <int ES, bool AL>
__device__ void row_item_sampled(const VerifyArgs &a, int b, int local, Smem &sh) {
    const int k = local / a.nc1, c = local - k * a.nc1;
    const int n = verify_len(a, b);
    if (n < 0 || n > a.G || k > n) return;
    const void *row = static_cast<const char *>(a.logits) + (size_t(b) * (a.G + 1) + k) * size_t(a.V) * ES;
    const int beg = c * a.ch1, end = min(a.V, beg + a.ch1);
    float m, s;
    chunk_ms<ES, AL>(row, beg, end, a.c32, m, s);
    wg_reduce_ms(m, s, a.c32, sh);
    if (threadIdx.x == 0)
        st_coherent(partials(a, b) + size_t(k) * a.nc1 + c,
                    uint64_t(__float_as_uint(m)) | (uint64_t(__float_as_uint(s) | kValid) << 32));
}

template <int ES, bool AL>
__device__ void row_item_greedy(const VerifyArgs &a, int b, int local, Smem &sh) {
    const int k = local / a.nc1, c = local - k * a.nc1;
    const int n = verify_len(a, b);
    if (n < 0 || n > a.G || k > n) return;
    const void *row = static_cast<const char *>(a.logits) + (size_t(b) * (a.G + 1) + k) * size_t(a.V) * ES;
    const int beg = c * a.ch1, end = min(a.V, beg + a.ch1);
    float best;
    int bi, nan;
    chunk_argmax<ES, AL>(row, beg, end, best, bi, nan);
    wg_reduce_am(best, bi, nan, sh);
    if (threadIdx.x == 0)
        st_coherent(partials(a, b) + size_t(k) * a.nc1 + c,
                    uint64_t(__float_as_uint(best)) | (uint64_t(uint32_t((nan ? kNanIdx : bi) + 2) | kValid) << 32));
}

// ---------------------------------------------------------- draw sub-tiles

// Target probability and residual of one element of the draw row; m is the
// row maximum (reference as in the row pass: fl(m * c) when finite).
__device__ __forceinline__ void draw_term(float z, float q, float m, float c, float inv_s, bool resid,
                                          float &r, float &p) {
    const float R = m * c;
    const float e = finitef(R) ? exp2_fast(__builtin_fmaf(z, c, -R)) : exp2_fast((z - m) * c);
    p = e * inv_s;
    r = resid ? fmaxf(p - q, 0.0f) : p;
}

// One thread's 8 contiguous elements of sub-tile `sub` of a draw row: the
// residual (or target) mass `rs` and the target mass `ps`, fp64 in index order.
template <int ES, bool ALZ, bool ALQ>
__device__ void sub_sums(const void *zrow, const float *qrow, int V, int sub, float m, float c, float inv_s,
                         bool resid, double &rs, double &ps) {
    rs = 0.0; ps = 0.0;
    const int e0 = sub * kSub + int(threadIdx.x) * kSubPerThread;
    if (e0 >= V) return;
    float z[kSubPerThread], q[kSubPerThread];
    if (ALZ && (!resid || ALQ) && e0 + kSubPerThread <= V) {
        const uint4 *zp = reinterpret_cast<const uint4 *>(static_cast<const char *>(zrow) + size_t(e0) * ES);
        if constexpr (ES == 2) {
            const uint4 w = zp[0];
            z[0] = bf16_lo(w.x); z[1] = bf16_hi(w.x); z[2] = bf16_lo(w.y); z[3] = bf16_hi(w.y);
            z[4] = bf16_lo(w.z); z[5] = bf16_hi(w.z); z[6] = bf16_lo(w.w); z[7] = bf16_hi(w.w);
        } else {
            const uint4 w0 = zp[0], w1 = zp[1];
            z[0] = __uint_as_float(w0.x); z[1] = __uint_as_float(w0.y);
            z[2] = __uint_as_float(w0.z); z[3] = __uint_as_float(w0.w);
            z[4] = __uint_as_float(w1.x); z[5] = __uint_as_float(w1.y);
            z[6] = __uint_as_float(w1.z); z[7] = __uint_as_float(w1.w);
        }
        if (resid) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(qrow + e0);
            const uint4 w0 = qp[0], w1 = qp[1];
            q[0] = __uint_as_float(w0.x); q[1] = __uint_as_float(w0.y);
            q[2] = __uint_as_float(w0.z); q[3] = __uint_as_float(w0.w);
            q[4] = __uint_as_float(w1.x); q[5] = __uint_as_float(w1.y);
            q[6] = __uint_as_float(w1.z); q[7] = __uint_as_float(w1.w);
        } else {
#pragma unroll
            for (int i = 0; i < kSubPerThread; ++i) q[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kSubPerThread; ++i) {
            float r, p;
            draw_term(z[i], q[i], m, c, inv_s, resid, r, p);
            rs = rs + double(r);
            ps = ps + double(p);
        }
    } else {
        const int e1 = min(V, e0 + kSubPerThread);
        for (int e = e0; e < e1; ++e) {
            float r, p;
            const float qv = resid ? qrow[e] : 0.0f;
            draw_term(load_elem<ES>(zrow, size_t(e)), qv, m, c, inv_s, resid, r, p);
            rs = rs + double(r);
            ps = ps + double(p);
        }
    }
}

// ------------------------------------------------------------- request items

// Per-request decision, computed identically by each of the request's workgroups.
struct Decision {
    int n, j;
    bool resid;
    float m, inv_s;
};

// Merge row r's chunk partials into sh.M[r] (max) and sh.S[r] (fp64 sum);
// marks the request bad for a bad row or a partial that was never written.
__device__ void merge_row_sampled(const VerifyArgs &a, const uint64_t *pp, int r, Smem &sh) {
    float M = neg_inf();
    bool ok = true;
    for (int c = 0; c < a.nc1; ++c) {
        const uint64_t v = pp[c];
        ok &= valid(v);
        M = fmaxf(M, lo_f(v));
    }
    double S = 0.0;
    for (int c = 0; c < a.nc1; ++c) {
        const uint64_t v = pp[c];
        const float vm = lo_f(v), vs = __uint_as_float(hi_u(v) & ~kValid);
        if (vm == neg_inf() && vs == 0.0f) continue;            // empty chunk
        S = S + double(vs) * rescale_d(vm, M, a.c32);
    }
    if (!ok || !(S > 0.0 && S < INFINITY) || !(M > neg_inf() && M < INFINITY)) atomicOr(&sh.bad, 1);
    sh.M[r] = M;
    sh.S[r] = S;
}

// Row r's chunk partials (greedy): lowest index of the maximum into sh.A[r].
__device__ void merge_row_greedy(const VerifyArgs &a, const uint64_t *pp, int r, Smem &sh) {
    float best = neg_inf();
    int bi = -1, nan = 0;
    bool ok = true;
    for (int c = 0; c < a.nc1; ++c) {               // ascending chunks: first maximum wins
        const uint64_t v = ld_coherent(pp + c);
        ok &= valid(v);
        const int vi = int(hi_u(v) & ~kValid) - 2;
        if (vi == kNanIdx) { nan = 1; continue; }
        merge_am(best, bi, lo_f(v), vi);
    }
    if (!ok || nan || bi < 0 || best == __builtin_inff()) atomicOr(&sh.bad, 1);
    sh.A[r] = bi;
}

// Unnormalised target probability 2^(z*c - R) of a value z in a row with
// maximum m, in fp64, against the same reference the row sum S used.
__device__ __forceinline__ double target_prob(float z, float m, float c) {
    const float R = m * c;
    return finitef(R) ? exp2(double(z) * double(c) - double(R)) : exp2((double(z) - double(m)) * double(c));
}
// log-sum-exp of the row at temperature T: ln sum_v e^(z_v/T) = R ln 2 + ln S.
__device__ __forceinline__ double row_lse(float m, double S, float c, double T) {
    const float R = m * c;
    return finitef(R) ? double(R) * 0.69314718055994530942 + log(S) : double(m) / T + log(S);
}

// All chunk partials of the request are complete (written by the previous
// launch): merge every row, run the accept tests, find the first rejection.
// Returns false (outputs reported by workgroup 0) for a data error or an
// invalid verify length (then *arrive is false: no workgroup counts itself).
template <int ES>
__device__ bool decide(const VerifyArgs &a, int b, int w, Decision &d, bool &arrive, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const int n = verify_len(a, b);
    d.n = n;
    arrive = false;
    if (n < 0 || n > G) {
        if (w == 0) write_error(a, b);
        return false;
    }
    arrive = true;
    const int k = threadIdx.x;
    int xk = 0;
    float zx = 0.0f, qx = 0.0f, uk = 0.0f;
    bool xbad = false;
    if (k < n) {
        xk = a.x[size_t(b) * G + k];
        xbad = xk < 0 || xk >= a.V;
        if (!xbad) {
            zx = load_elem<ES>(a.logits, (size_t(b) * G1 + k) * size_t(a.V) + size_t(xk));
            qx = a.q[(size_t(b) * G + k) * size_t(a.V) + size_t(xk)];
        }
        uk = a.u[size_t(b) * G1 + k];
    }
    if (threadIdx.x == 0) { sh.jmin = n; sh.bad = 0; }
    __syncthreads();
    const uint64_t *part = partials(a, b);
    for (int r = threadIdx.x; r <= n; r += kWG) merge_row_sampled(a, part + size_t(r) * a.nc1, r, sh);
    if (xbad) atomicOr(&sh.bad, 1);
    __syncthreads();
    if (k < n && !xbad) {
        const double pk = target_prob(zx, sh.M[k], a.c32) / sh.S[k];
        const bool acc = (qx > 0.0f) ? (double(uk) < pk / double(qx)) : (pk > 0.0);
        if (!acc) atomicMin(&sh.jmin, k);
    }
    __syncthreads();
    if (sh.bad) {
        if (w == 0) write_error(a, b);
        return false;
    }
    const int j = sh.jmin;
    d.j = j;
    d.resid = j < n;
    d.m = sh.M[j];
    d.inv_s = float(1.0 / sh.S[j]);
    if (w == 0) {
        for (int t = threadIdx.x; t < G1; t += kWG) {
            if (t < j) a.out_tok[size_t(b) * G1 + t] = a.x[size_t(b) * G + t];
            else if (t > j) a.out_tok[size_t(b) * G1 + t] = -1;
        }
        if (threadIdx.x == 0) a.out_acc[b] = j;
    }
    return true;
}

// Diagnostics of request b (only when requested), from the merged rows.
template <int ES>
__device__ void write_diag(const VerifyArgs &a, int b, bool ok, int n, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const float qnan = __builtin_nanf("");
    const double T64 = double(a.T);
    for (int t = threadIdx.x; t < G1; t += kWG) {
        float lse = qnan, pv = qnan, qv = qnan;
        if (ok && t <= n) {
            lse = float(row_lse(sh.M[t], sh.S[t], a.c32, T64));
            if (t < n) {
                const int xt = a.x[size_t(b) * G + t];
                const float zt = load_elem<ES>(a.logits, (size_t(b) * G1 + t) * size_t(a.V) + size_t(xt));
                qv = a.q[(size_t(b) * G + t) * size_t(a.V) + size_t(xt)];
                pv = float(target_prob(zt, sh.M[t], a.c32) / sh.S[t]);
            }
        }
        if (a.d_lse) a.d_lse[size_t(b) * G1 + t] = lse;
        if (t < G) {
            if (a.d_p) a.d_p[size_t(b) * G + t] = pv;
            if (a.d_q) a.d_q[size_t(b) * G + t] = qv;
        }
    }
    if (!ok && threadIdx.x == 0 && a.d_r) a.d_r[b] = qnan;
}

// Last workgroup of request b: locate u * R and write the token.
template <int ES, bool ALZ, bool ALQ>
__device__ void final_select(const VerifyArgs &a, int b, const Decision &d, const void *zrow, const float *qrow,
                             Smem &sh) {
    const int G1 = a.G + 1;
    const bool resid = d.resid;
    const uint64_t *mass = reinterpret_cast<const uint64_t *>(a.ws + a.lay.mass) + size_t(b) * a.nsub * 2;
    // Pass 1: totals, in sub-tile order.  mode 1 draws from the residual, mode 0 from p.
    double R = 0.0, Rp = 0.0;
    int last_r = -1, last_p = -1;
    for (int blk = 0; blk < a.nsub; blk += kStage) {
        const int cnt = min(kStage, a.nsub - blk);
        __syncthreads();
        if (int(threadIdx.x) < cnt) {
            sh.mr[threadIdx.x] = __longlong_as_double(ld_coherent(mass + 2 * (blk + threadIdx.x)));
            sh.mp[threadIdx.x] = __longlong_as_double(ld_coherent(mass + 2 * (blk + threadIdx.x) + 1));
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 0; i < cnt; ++i) {
                R = R + sh.mr[i];
                Rp = Rp + sh.mp[i];
                if (sh.mr[i] > 0.0) last_r = blk + i;
                if (sh.mp[i] > 0.0) last_p = blk + i;
            }
        }
    }
    if (threadIdx.x == 0) {
        const int mode = (resid && R > 0.0) ? 1 : 0;
        const double total = mode ? R : (resid ? Rp : R);
        sh.mode = mode;
        sh.target = double(a.u[size_t(b) * G1 + a.G]) * total;
        sh.R = R;
        sh.sstar = -1;
        sh.base = 0.0;
        sh.t1 = kWG;
        sh.y = -1;
        sh.jmin = (mode || !resid) ? last_r : last_p;   // for the no-crossing fallback
    }
    __syncthreads();
    const int mode = sh.mode;
    const bool use_r = resid && mode;          // else: terms are p (bonus draw or zero-residual fallback)
    const bool from_m = mode || !resid;        // which mass array holds those terms' sums
    // Pass 2: the first sub-tile whose running sum exceeds the target.
    double P = 0.0;
    for (int blk = 0; blk < a.nsub; blk += kStage) {
        const int cnt = min(kStage, a.nsub - blk);
        if (a.nsub > kStage) {
            __syncthreads();
            if (int(threadIdx.x) < cnt) {
                sh.mr[threadIdx.x] = __longlong_as_double(ld_coherent(mass + 2 * (blk + threadIdx.x)));
                sh.mp[threadIdx.x] = __longlong_as_double(ld_coherent(mass + 2 * (blk + threadIdx.x) + 1));
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 0; i < cnt; ++i) {
                const double P1 = P + (from_m ? sh.mr[i] : sh.mp[i]);
                if (P1 > sh.target) { sh.sstar = blk + i; sh.base = P; break; }
                P = P1;
            }
        }
        __syncthreads();
        if (sh.sstar >= 0) break;
    }
    const int lastpos = (sh.sstar < 0) ? 1 : 0;         // u * R at or beyond the top
    const int sstar = lastpos ? max(0, sh.jmin) : sh.sstar;
    const double base = sh.base, target = sh.target;
    double rs, ps;
    sub_sums<ES, ALZ, ALQ>(zrow, qrow, a.V, sstar, d.m, a.c32, d.inv_s, resid, rs, ps);
    const double v1[1] = {use_r ? rs : ps};
    double ex[1], tot[1];
    wg_excl_scan<1>(v1, ex, tot, sh);
    const int e0 = sstar * kSub + int(threadIdx.x) * kSubPerThread;
    const int e1 = min(a.V, e0 + kSubPerThread);
    if (lastpos) {
        int lp = -1;
        for (int e = e0; e < e1; ++e) {
            float r, p;
            draw_term(load_elem<ES>(zrow, size_t(e)), resid ? qrow[e] : 0.0f, d.m, a.c32, d.inv_s, resid, r, p);
            if ((use_r ? r : p) > 0.0f) lp = e;
        }
        atomicMax(&sh.y, lp);
        __syncthreads();
    } else {
        if (base + (ex[0] + v1[0]) > target) atomicMin(&sh.t1, int(threadIdx.x));
        __syncthreads();
        if (int(threadIdx.x) == sh.t1) {
            double acc = base + ex[0];
            int y = -1, lp = -1;
            for (int e = e0; e < e1; ++e) {
                float r, p;
                draw_term(load_elem<ES>(zrow, size_t(e)), resid ? qrow[e] : 0.0f, d.m, a.c32, d.inv_s, resid, r, p);
                const float t = use_r ? r : p;
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
        if (a.d_r) a.d_r[b] = resid ? float(sh.R) : -1.0f;
    }
}

// Request pass (after the row pass has completed): workgroup w of request b
// decides the request, streams sub-tiles [w*spw, (w+1)*spw) of the draw row,
// and the last of the request's nc2 workgroups selects the token and zeroes
// the request's partials and masses.
template <int ES, bool ALZ, bool ALQ>
__device__ void request_item_sampled(const VerifyArgs &a, int b, int w, Smem &sh) {
    Decision d;
    bool arrive;
    const bool ok = decide<ES>(a, b, w, d, arrive, sh);
    if (!arrive) return;
    const int G1 = a.G + 1;
    const bool diag = a.d_lse || a.d_p || a.d_q || a.d_r;
    const void *zrow = nullptr;
    const float *qrow = nullptr;
    if (ok) {
        zrow = static_cast<const char *>(a.logits) + (size_t(b) * G1 + d.j) * size_t(a.V) * ES;
        qrow = d.resid ? a.q + (size_t(b) * a.G + d.j) * size_t(a.V) : nullptr;
        uint64_t *mass = reinterpret_cast<uint64_t *>(a.ws + a.lay.mass) + size_t(b) * a.nsub * 2;
        const int s_end = min(a.nsub, (w + 1) * a.spw);
        for (int s0 = w * a.spw; s0 < s_end; s0 += kSubBatch) {
            double v[2 * kSubBatch], ex[2 * kSubBatch], tot[2 * kSubBatch];
#pragma unroll
            for (int i = 0; i < kSubBatch; ++i) {
                double rs = 0.0, ps = 0.0;
                if (s0 + i < s_end) sub_sums<ES, ALZ, ALQ>(zrow, qrow, a.V, s0 + i, d.m, a.c32, d.inv_s, d.resid, rs, ps);
                v[i] = rs;
                v[kSubBatch + i] = ps;
            }
            wg_excl_scan<2 * kSubBatch>(v, ex, tot, sh);
            if (int(threadIdx.x) < kSubBatch && s0 + int(threadIdx.x) < s_end) {
                const int i = threadIdx.x;
                st_coherent(mass + 2 * (s0 + i), uint64_t(__double_as_longlong(tot[i])));
                st_coherent(mass + 2 * (s0 + i) + 1, uint64_t(__double_as_longlong(tot[kSubBatch + i])));
            }
        }
    }
    if (!arrive_last(draw_counter(a, b), unsigned(a.nc2), sh)) return;
    if (ok) {
        final_select<ES, ALZ, ALQ>(a, b, d, zrow, qrow, sh);
        uint64_t *m = reinterpret_cast<uint64_t *>(a.ws + a.lay.mass) + size_t(b) * a.nsub * 2;
        for (int i = threadIdx.x; i < 2 * a.nsub; i += kWG) st_coherent(m + i, 0ull);
    }
    if (diag) write_diag<ES>(a, b, ok, d.n, sh);
    uint64_t *part = partials(a, b);
    for (int i = threadIdx.x; i < (d.n + 1) * a.nc1; i += kWG) part[i] = 0ull;
}

// One workgroup per request (T == 0), after the request's row items: waits
// for every read row, emits the argmax match, and zeroes the partials.
__device__ void request_item_greedy(const VerifyArgs &a, int b, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const int n = verify_len(a, b);
    if (n < 0 || n > G) { write_error(a, b); return; }
    const int k = threadIdx.x;
    int xk = 0;
    if (k < n) xk = a.x[size_t(b) * G + k];
    if (threadIdx.x == 0) { sh.jmin = n; sh.bad = 0; }
    if (!wait_partials(a, b, n)) { write_error(a, b); return; }
    const uint64_t *part = partials(a, b);
    for (int r = threadIdx.x; r <= n; r += kWG) merge_row_greedy(a, part + size_t(r) * a.nc1, r, sh);
    __syncthreads();
    if (k < n) {
        if (xk < 0 || xk >= a.V) atomicOr(&sh.bad, 1);
        else if (xk != sh.A[k]) atomicMin(&sh.jmin, k);
    }
    __syncthreads();
    if (sh.bad) {
        write_error(a, b);
    } else {
        const int j = sh.jmin;
        for (int t = threadIdx.x; t < G1; t += kWG) {
            int v = -1;
            if (t < j) v = a.x[size_t(b) * G + t];
            else if (t == j) v = sh.A[j];
            a.out_tok[size_t(b) * G1 + t] = v;
        }
        if (threadIdx.x == 0) a.out_acc[b] = j;
    }
    __syncthreads();
    uint64_t *pw = partials(a, b);
    for (int i = threadIdx.x; i < (n + 1) * a.nc1; i += kWG) st_coherent(pw + i, 0ull);
}

// ------------------------------------------------------------- kernels

// Row pass of a sampled verify: one workgroup per (request, row, chunk).
template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_rows_sampled(VerifyArgs a) {
    __shared__ Smem sh;
    const int g1 = (a.G + 1) * a.nc1;
    const int b = int(blockIdx.x) / g1;
    row_item_sampled<ES, AL>(a, b, int(blockIdx.x) - b * g1, sh);
}

// Request pass of a sampled verify: nc2 workgroups per request.
template <int ES, bool ALZ, bool ALQ>
__global__ __launch_bounds__(kWG) void k_requests_sampled(VerifyArgs a) {
    __shared__ Smem sh;
    const int b = int(blockIdx.x) / a.nc2;
    request_item_sampled<ES, ALZ, ALQ>(a, b, int(blockIdx.x) - b * a.nc2, sh);
}

// Greedy verify: row items (request-major), then one request item per
// request (mode 0); or only the row items (mode 1) / request items (mode 2).
template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_verify_greedy(VerifyArgs a) {
    __shared__ Smem sh;
    const int g1 = (a.G + 1) * a.nc1;
    const long rows = long(a.B) * g1;
    const long i = blockIdx.x;
    if (a.mode == 2 || (a.mode == 0 && i >= rows)) {
        request_item_greedy(a, int(a.mode == 2 ? i : i - rows), sh);
    } else {
        const int b = int(i / g1);
        row_item_greedy<ES, AL>(a, b, int(i - long(b) * g1), sh);
    }
}

template <typename K>
int occ(K kernel, int *n) {
    return int(hipOccupancyMaxActiveBlocksPerMultiprocessor(n, kernel, kWG, 0));
}

}  // namespace

int launch_rows_sampled(const VerifyArgs &a, bool az, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) {
        if (az) hipLaunchKernelGGL((k_rows_sampled<2, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_rows_sampled<2, false>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az) hipLaunchKernelGGL((k_rows_sampled<4, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_rows_sampled<4, false>), dim3(grid), dim3(kWG), 0, st, a);
    }
    return int(hipGetLastError());
}

int launch_requests_sampled(const VerifyArgs &a, bool az, bool aq, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) {
        if (az && aq) hipLaunchKernelGGL((k_requests_sampled<2, true, true>), dim3(grid), dim3(kWG), 0, st, a);
        else if (az) hipLaunchKernelGGL((k_requests_sampled<2, true, false>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_requests_sampled<2, false, false>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az && aq) hipLaunchKernelGGL((k_requests_sampled<4, true, true>), dim3(grid), dim3(kWG), 0, st, a);
        else if (az) hipLaunchKernelGGL((k_requests_sampled<4, true, false>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_requests_sampled<4, false, false>), dim3(grid), dim3(kWG), 0, st, a);
    }
    return int(hipGetLastError());
}

int launch_verify_greedy(const VerifyArgs &a, bool az, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) {
        if (az) hipLaunchKernelGGL((k_verify_greedy<2, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_verify_greedy<2, false>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az) hipLaunchKernelGGL((k_verify_greedy<4, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_verify_greedy<4, false>), dim3(grid), dim3(kWG), 0, st, a);
    }
    return int(hipGetLastError());
}

int greedy_occupancy(bool az, int esize, int *n) {
    if (esize == 2) return az ? occ(k_verify_greedy<2, true>, n) : occ(k_verify_greedy<2, false>, n);
    return az ? occ(k_verify_greedy<4, true>, n) : occ(k_verify_greedy<4, false>, n);
}

}  // namespace sv
