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
// MFMA).  With draft probabilities and the full [B, G+1, V] row layout a
// temperature > 0 call is one launch, k_verify_sampled, whose grid holds three
// kinds of workgroup:
//
//   row groups     one per (request, row, 8192-element group), one wave per
//                  2048-element chunk: four 16-byte streaming loads per lane,
//                  the chunk maximum, then the sum of 2^((z - m) * log2(e)/T),
//                  both reduced across the wave with DPP; the four waves'
//                  (max, sum) pairs merge in LDS into one 64-bit partial per
//                  group, published with its written bit.  The wave whose chunk
//                  holds draft token x_k also publishes z(x_k) and q(x_k).
//   decisions      one per request, placed in grid order one request after its
//                  row groups (on the same XCD): polls the request's partials
//                  and gathers, merges each row (fp64) as it completes and runs
//                  its accept test, and publishes a decision record (j, m_j,
//                  1/S_j) as soon as rows 0..j settle the first rejection j;
//                  once every row is in, it states whether the request holds
//                  a data error anywhere and writes the accepted prefix.
//   request pass   after every row group and decision: nc2 workgroups per
//                  request (about 2048 in all), each polling the record and
//                  streaming its sub-tiles of the one row the final token is
//                  drawn from (target row j, plus draft row j on a rejection),
//                  writing fp64 sub-tile masses, each word marked as written.
//                  The request's last workgroup in grid order polls the masses
//                  and the decision's error check, locates u * R by a parallel
//                  prefix over the masses, re-scans that one sub-tile, writes
//                  the token, and zeroes the words the request used.
//
// Every wait is on workgroups earlier in grid order that never wait on later
// ones, so the launch completes whatever the device holds at once.  With B a
// multiple of 8 each XCD (workgroup i runs on XCD i mod 8) serves whole
// requests: their row groups as a contiguous stream, their decisions while
// it streams the next request, their request workgroups at the end.
// With verify lengths at B <= 256, or with draft logits, the call is two
// launches instead: a row pass (k_rows_sampled_vl visits only the read row
// groups; k_rows_sampled otherwise), then k_requests_sampled, whose every
// workgroup makes the decision itself from the completed partials.
//
// Temperature 0 (argmax) is one launch: row workgroups of four chunks, then
// one workgroup per request that polls its rows' partials (bounded wait) --
// the host keeps those below half the resident capacity, else it splits them
// into a second launch.
//
// Words handed between workgroups of one launch (row partials, gathers and
// decision records of the one-launch verify, sub-tile masses, the greedy
// partials) use coherent device-scope stores and loads instead of device-scope
// fences, which on this chip write back or invalidate the whole L2; each such
// word carries its own written bit, so none needs ordering.
//
// Determinism: no floating-point atomics; every reduction has a fixed order.
// A sub-tile mass is the butterfly sum of its wave totals, which is bitwise the
// total of the prefix scan the final re-scan runs over the same terms, so the
// sub-tile the draw lands in is located exactly.  The library is compiled with
// -ffp-contract=off.

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"
#include "sv_wave.h"

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
    return (finitef(r1) && finitef(r0)) ? exp2_fast(r1 - r0) : exp2_fast((m1 - m0) * c);
}

template <int ES>
__device__ __forceinline__ float load_elem(const void *base, size_t i) {
    if constexpr (ES == 2) {
        return __uint_as_float(uint32_t(static_cast<const uint16_t *>(base)[i]) << 16);
    } else {
        return static_cast<const float *>(base)[i];
    }
}

// Streaming 16-byte load: the logits are read once, so keep them from
// displacing the cached workspace and draft rows.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// ------------------------------------------------ cross-workgroup publication
//
// Words one workgroup hands to another inside a launch are written with
// coherent device-scope stores and read with coherent device-scope loads (no
// whole-cache write-back or invalidation, which a generic device-scope fence
// performs on every L2).  Greedy chunk partials and sub-tile masses carry
// their own written bits, so they need no ordering at all.
__device__ __forceinline__ void st_coherent(void *p, uint64_t v) {
    __hip_atomic_store(static_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const void *p) {
    return __hip_atomic_load(static_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Output words that a later workgroup may overwrite are written through to
// the coherence point, so the last write in time is the one that lands.
__device__ __forceinline__ void st_out(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float(uint32_t(v)); }
__device__ __forceinline__ uint32_t hi_u(uint64_t v) { return uint32_t(v >> 32); }
__device__ __forceinline__ bool valid(uint64_t v) { return (hi_u(v) & kValid) != 0u; }


struct __align__(16) Smem {
    union {
        double sc[kWaves][2];                     // scan: wave totals
        double wt[kWaves][2 * kSubBatch];         // draw: wave totals of the sub-tile masses
    } r;
    double S[kWG];                                // fp64 row sums
    float M[kWG];                                 // row maxima
    double Sq[kWG];                               // draft logits: the draft rows' sums and maxima
    float Mq[kWG];
    int A[kWG];                                   // greedy row argmax
    int last;
    int q[6][kWaves];                             // per-wave results of ballot searches
    double base, R, Rp;
    int fsel[2];                                  // final select: first sub-tile, flags
    float gm[kWaves];                             // greedy row group: the waves' (max, index, NaN)
    int gi[kWaves], gn[kWaves];
    uint64_t pw[2];                               // a polled record, shared from one lane
    int pok;
    int rst[kWG / 16];                            // early decision: each row's status
    int pub;                                      // early decision: the record is out
};

// ---------------------------------------------------------------- merges

// (value, index) with the larger value; equal values keep the lower index; index < 0 = none.
__device__ __forceinline__ void merge_am(float &v, int &i, float v2, int i2) {
    if (i2 < 0) return;
    if (i < 0 || v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

template <int C> __device__ __forceinline__ void am_step(float &v, int &i, int &nan) {
    const float v2 = dpp_f<C>(v);
    const int i2 = dpp_i<C>(i);
    nan |= dpp_i<C>(nan);
    merge_am(v, i, v2, i2);
}
__device__ __forceinline__ void row16_argmax(float &v, int &i, int &nan) {
    am_step<kXor1>(v, i, nan);
    am_step<kXor2>(v, i, nan);
    am_step<kHalfMirror>(v, i, nan);
    am_step<kMirror>(v, i, nan);
}

// Ballot searches over the workgroup's threads.  Each wave reduces its
// ballot (first or last set lane); lane 0 posts the wave's result in slot q
// of sh.q; after the caller's barrier, wg_first / wg_last combine the four.
// (A shared-memory atomic here would become a loop over the active lanes.)
__device__ __forceinline__ void post_first(bool pred, int q, Smem &sh) {
    const uint64_t m = __ballot(pred);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh.q[q][w] = m ? w * 64 + __builtin_ctzll(m) : INT_MAX;
}
__device__ __forceinline__ void post_last(bool pred, int q, Smem &sh) {
    const uint64_t m = __ballot(pred);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh.q[q][w] = m ? w * 64 + 63 - __builtin_clzll(m) : -1;
}
// Whether any thread's predicate holds, through ballot slot q (one barrier;
// cheaper than __syncthreads_or).  Slot q must not be posted again before
// every thread has read it.
__device__ __forceinline__ bool wg_any(bool pred, int q, Smem &sh);
// Lowest thread with the posted predicate (INT_MAX if none) / highest (-1).
__device__ __forceinline__ int wg_first(int q, const Smem &sh) {
    return min(min(sh.q[q][0], sh.q[q][1]), min(sh.q[q][2], sh.q[q][3]));
}
__device__ __forceinline__ int wg_last(int q, const Smem &sh) {
    return max(max(sh.q[q][0], sh.q[q][1]), max(sh.q[q][2], sh.q[q][3]));
}
__device__ __forceinline__ bool wg_any(bool pred, int q, Smem &sh) {
    post_first(pred, q, sh);
    __syncthreads();
    return wg_first(q, sh) != INT_MAX;
}

// Inclusive prefix over the 256 threads of NS fp64 values at once: the DPP
// wave prefix x, then the wave totals W (x of lane 63) added in wave order
// (wbase).  incl = wbase + x; excl = the previous thread's incl (wbase for
// lane 0); total = incl of the last thread = ((W0 + W1) + W2) + W3, which is
// what a sum of the four wave_sum_d results in that order gives.
template <int NS>
__device__ void wg_scan(const double (&v)[NS], double (&excl)[NS], double (&incl)[NS], double (&total)[NS],
                        Smem &sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double x[NS], xp[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        x[i] = wave_scan_d(v[i]);
        xp[i] = dpp_d<kWaveShr1>(x[i]);          // lane - 1's prefix (0 in lane 0)
    }
    __syncthreads();
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < NS; ++i) sh.r.sc[w][i] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        double wb = 0.0;
        for (int k = 0; k < w; ++k) wb = wb + sh.r.sc[k][i];
        incl[i] = wb + x[i];
        excl[i] = (lane == 0) ? wb : wb + xp[i];
        total[i] = ((sh.r.sc[0][i] + sh.r.sc[1][i]) + sh.r.sc[2][i]) + sh.r.sc[3][i];
    }
}

// ------------------------------------------------------------- workspace

__device__ __forceinline__ uint64_t *partials(const VerifyArgs &a, int b) {
    return reinterpret_cast<uint64_t *>(a.ws + size_t(a.lay.part) * 256) + size_t(b) * (a.G + 1) * a.np1;
}
__device__ __forceinline__ uint64_t *partials_d(const VerifyArgs &a, int b) {
    return reinterpret_cast<uint64_t *>(a.ws + size_t(a.lay.partd) * 256) + size_t(b) * a.G * a.np1;
}
__device__ __forceinline__ uint64_t *masses(const VerifyArgs &a, int b) {
    return reinterpret_cast<uint64_t *>(a.ws + size_t(a.lay.mass) * 256) + size_t(b) * a.nsub * 2;
}
__device__ __forceinline__ uint64_t *gathered(const VerifyArgs &a, int b) {
    return reinterpret_cast<uint64_t *>(a.ws + size_t(a.lay.gx) * 256) + size_t(b) * a.G;
}
// A sub-tile mass word: the fp64 mass (>= 0) with bit 63 set once written.
constexpr uint64_t kMassWritten = uint64_t(1) << 63;
__device__ __forceinline__ uint64_t mass_word(double m) { return uint64_t(__double_as_longlong(m)) | kMassWritten; }
__device__ __forceinline__ double mass_value(uint64_t w) { return __longlong_as_double((long long)(w & ~kMassWritten)); }

// A request with a data error: every output word -1 (diagnostics NaN).
__device__ void write_error(const VerifyArgs &a, int b) {
    const int G1 = a.G + 1;
    for (int t = threadIdx.x; t < G1; t += kWG) st_out(a.out_tok + size_t(b) * G1 + t, -1);
    if (threadIdx.x == 0) st_out(a.out_acc + b, -1);
}

// Inputs no kernel writes, read through the constant address space so that
// uniform reads stay scalar loads even after the kernel's own stores.
typedef const __attribute__((address_space(4))) int32_t ci32;
__device__ __forceinline__ int32_t ld_const(const int32_t *p, size_t i) {
    return reinterpret_cast<ci32 *>(reinterpret_cast<uintptr_t>(p))[i];
}
// Verify length of request b (-1 when its packed rows are invalid).  Packed
// target rows: request b owns rows roff[b] .. roff[b+1]-1 of a buffer of
// `rows` rows, its positions 0..n in order.
__device__ __forceinline__ int verify_len(const VerifyArgs &a, int b) {
    if (a.roff) {
        const int lo = ld_const(a.roff, b), hi = ld_const(a.roff, size_t(b) + 1);
        return (lo >= 0 && hi > lo && hi <= a.rows && hi - lo - 1 <= a.G) ? hi - lo - 1 : -1;
    }
    return a.vlen ? ld_const(a.vlen, b) : a.G;
}
// Element offset of target row k of request b ([B, G+1, V], or packed rows).
__device__ __forceinline__ size_t row_elem(const VerifyArgs &a, int b, int k) {
    const size_t r = a.roff ? size_t(ld_const(a.roff, b)) + size_t(k) : size_t(b) * size_t(a.G + 1) + size_t(k);
    return r * size_t(a.V);
}

// ------------------------------------------------------------- row waves

template <int ES> constexpr int kEPL = kRowVec * (16 / ES);   // elements per lane of a chunk

// Lane `lane`'s values of the chunk that starts at element beg of a row of V
// elements; positions past the row end read as -inf.  Aligned rows use four
// 16-byte loads per lane (vector v = lane + 64 i); others one element per load
// (element beg + lane + 64 i).
template <int ES, bool AL>
__device__ __forceinline__ void load_chunk(const void *row, int beg, int V, int lane, float (&f)[kEPL<ES>]) {
    if constexpr (AL) {
        constexpr int EPV = 16 / ES;
        constexpr uint32_t fill = (ES == 2) ? 0xff80ff80u : 0xff800000u;   // -inf
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const char *>(row) + size_t(beg) * ES);
        const int nvec = (V - beg) / EPV;
        uint4 r[kRowVec];
        if (nvec >= 64 * kRowVec) {
#pragma unroll
            for (int i = 0; i < kRowVec; ++i) r[i] = ld_stream(p + lane + 64 * i);
        } else {
#pragma unroll
            for (int i = 0; i < kRowVec; ++i) {
                const int v = lane + 64 * i;
                r[i] = (v < nvec) ? ld_stream(p + v) : make_uint4(fill, fill, fill, fill);
            }
        }
#pragma unroll
        for (int i = 0; i < kRowVec; ++i) {
            if constexpr (ES == 2) {
                f[8 * i + 0] = bf16_lo(r[i].x); f[8 * i + 1] = bf16_hi(r[i].x);
                f[8 * i + 2] = bf16_lo(r[i].y); f[8 * i + 3] = bf16_hi(r[i].y);
                f[8 * i + 4] = bf16_lo(r[i].z); f[8 * i + 5] = bf16_hi(r[i].z);
                f[8 * i + 6] = bf16_lo(r[i].w); f[8 * i + 7] = bf16_hi(r[i].w);
            } else {
                f[4 * i + 0] = __uint_as_float(r[i].x); f[4 * i + 1] = __uint_as_float(r[i].y);
                f[4 * i + 2] = __uint_as_float(r[i].z); f[4 * i + 3] = __uint_as_float(r[i].w);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kEPL<ES>; ++i) {
            const int e = beg + lane + 64 * i;
            f[i] = (e < V) ? load_elem<ES>(row, size_t(e)) : neg_inf();
        }
    }
}
// Row index of f[i] in load_chunk's layout (ascending in i for a fixed lane).
template <int ES, bool AL>
__device__ __forceinline__ int chunk_index(int beg, int lane, int i) {
    constexpr int EPV = 16 / ES;
    return AL ? beg + (lane + 64 * (i / EPV)) * EPV + (i % EPV) : beg + lane + 64 * i;
}

// Sampled row pass, one wave: (max M, sum S of 2^((z - M) * c)) of chunk c
// of row k of request b (n = the request's verify length), uniform across
// the wave; of draft row k when `draft` (draft logits).  The chunk holding
// draft token x_k also stores z(x_k) and q(x_k) for the request pass's accept
// test (with draft logits: z(x_k) from the target row, d(x_k) from the draft
// row, each into its half of the gather word).  With `published` (the
// one-launch verify, draft probabilities) the gather word is stored
// coherently and carries its own written bit in place of q's sign: q(x_k) is
// stored as max(q, 0) (NaN as 0), which the accept test treats alike (a q
// that is not positive accepts iff p(x_k) > 0).
template <int ES, bool AL>
__device__ void row_chunk_sampled(const VerifyArgs &a, int b, int k, int chunk, int n, bool draft, int lane,
                                  float &M_out, float &S_out, long trow = -1, bool published = false) {
    constexpr int EPL = kEPL<ES>;
    // trow: the target row's index when the caller already holds it
    const size_t zoff = (trow >= 0) ? size_t(trow) * size_t(a.V) : row_elem(a, b, k);
    const void *row = draft ? static_cast<const void *>(static_cast<const char *>(a.dl) +
                                                        (size_t(b) * a.G + k) * size_t(a.V) * ES)
                            : static_cast<const void *>(static_cast<const char *>(a.logits) + zoff * ES);
    const int beg = chunk * a.ch1;
    float f[EPL];
    load_chunk<ES, AL>(row, beg, a.V, lane, f);
    // The chunk holding draft token x_k gathers z(x_k) and q(x_k) for the
    // accept test (an x_k out of range is never gathered).
    const int xk = (k < n) ? ld_const(a.x, size_t(b) * a.G + k) : -1;
    const bool gather = xk >= beg && xk < beg + a.ch1 && xk < a.V;
    float gz = 0.0f, gq = 0.0f;
    if (gather && lane == 0) {
        gz = load_elem<ES>(row, size_t(xk));
        if (!a.dl) gq = a.q[(size_t(b) * a.G + k) * size_t(a.V) + size_t(xk)];
    }
    const float c = a.c32;
    float m = f[0];
#pragma unroll
    for (int i = 1; i + 1 < EPL; i += 2) m = max3(m, f[i], f[i + 1]);
    m = fmaxf(m, f[EPL - 1]);
    const float M = wave_max(m);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    if (M == neg_inf()) {
        // Every element is -inf or NaN (the maximum drops NaN): keep a NaN visible.
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (f[i] != f[i]) s0 = __builtin_nanf("");
    } else if (finitef(M * c)) {
        const float nR = -(M * c);
#pragma unroll
        for (int i = 0; i < EPL; i += 4) {
            s0 = s0 + exp2_fast(__builtin_fmaf(f[i + 0], c, nR));
            s1 = s1 + exp2_fast(__builtin_fmaf(f[i + 1], c, nR));
            s2 = s2 + exp2_fast(__builtin_fmaf(f[i + 2], c, nR));
            s3 = s3 + exp2_fast(__builtin_fmaf(f[i + 3], c, nR));
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPL; i += 4) {
            s0 = s0 + exp2_fast((f[i + 0] - M) * c);
            s1 = s1 + exp2_fast((f[i + 1] - M) * c);
            s2 = s2 + exp2_fast((f[i + 2] - M) * c);
            s3 = s3 + exp2_fast((f[i + 3] - M) * c);
        }
    }
    M_out = M;
    S_out = wave_sum((s0 + s1) + (s2 + s3));
    if (gather && lane == 0) {
        if (published) {
            const uint32_t qb = (gq > 0.0f) ? __float_as_uint(gq) : 0u;
            st_coherent(gathered(a, b) + k, uint64_t(__float_as_uint(gz)) | (uint64_t(qb | kValid) << 32));
        } else if (!a.dl) {
            gathered(a, b)[k] = uint64_t(__float_as_uint(gz)) | (uint64_t(__float_as_uint(gq)) << 32);
        } else {
            reinterpret_cast<uint32_t *>(gathered(a, b) + k)[draft ? 1 : 0] = __float_as_uint(gz);
        }
    }
}

// Greedy row pass, one wave: (max M, lowest index of the max, any NaN) of
// chunk `chunk` of row k of request b, uniform across the wave.  The maximum
// comes first (v_max3, which drops NaN); a NaN anywhere shows in a running
// fp32 sum of the chunk (which also turns NaN when +inf meets -inf, a row
// whose maximum is +inf and so bad anyway); then each lane finds its lowest
// position holding the maximum and the wave takes the lowest such index.  An
// all -inf chunk has no argmax (index -1).
template <int ES, bool AL>
__device__ void row_chunk_greedy(const VerifyArgs &a, int b, int k, int chunk, int lane, float &M_out, int &idx_out,
                                 bool &nan_out) {
    constexpr int EPL = kEPL<ES>;
    const void *row = static_cast<const char *>(a.logits) + row_elem(a, b, k) * ES;
    const int beg = chunk * a.ch1;
    float f[EPL];
    load_chunk<ES, AL>(row, beg, a.V, lane, f);
    float m = f[0];
#pragma unroll
    for (int i = 1; i + 1 < EPL; i += 2) m = max3(m, f[i], f[i + 1]);
    m = fmaxf(m, f[EPL - 1]);
    const float M = wave_max(m);
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; i += 2) { s0 = s0 + f[i]; s1 = s1 + f[i + 1]; }
    const float sum = s0 + s1;
    nan_out = __ballot(sum != sum) != 0ull;
    int bi = -1;
    if (M != neg_inf()) {                         // uniform
        int bo = -1;
#pragma unroll
        for (int i = EPL - 1; i >= 0; --i) bo = (f[i] == M) ? i : bo;
        bi = wave_min_i((bo >= 0) ? chunk_index<ES, AL>(beg, lane, bo) : INT_MAX);
    }
    M_out = M;
    idx_out = bi;
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

// Eight values from one (bf16) or two (fp32) 16-byte words.
template <int ES> __device__ __forceinline__ void unpack8(const uint4 (&w)[ES == 2 ? 1 : 2], float (&f)[kSubPerThread]) {
    if constexpr (ES == 2) {
        f[0] = bf16_lo(w[0].x); f[1] = bf16_hi(w[0].x); f[2] = bf16_lo(w[0].y); f[3] = bf16_hi(w[0].y);
        f[4] = bf16_lo(w[0].z); f[5] = bf16_hi(w[0].z); f[6] = bf16_lo(w[0].w); f[7] = bf16_hi(w[0].w);
    } else {
        f[0] = __uint_as_float(w[0].x); f[1] = __uint_as_float(w[0].y);
        f[2] = __uint_as_float(w[0].z); f[3] = __uint_as_float(w[0].w);
        f[4] = __uint_as_float(w[1].x); f[5] = __uint_as_float(w[1].y);
        f[6] = __uint_as_float(w[1].z); f[7] = __uint_as_float(w[1].w);
    }
}

// One thread's 8 contiguous elements of sub-tile `sub` of a draw row: the
// residual (or target) mass `rs` and the target mass `ps`, fp64 in index
// order, and the terms t (residual if use_r, else target; 0 past the row end).
// qrow is the draft row (resid) or a block of zeros (bonus draw), so the z
// and q loads are all issued before any is waited for.  With draft logits
// (DL) qrow holds logits of the target's element size, and q is their
// softmax from the draft row's maximum mq and 1 / sum inv_sq.  The mass pass
// and the final re-scan both call this, so their sums agree bitwise.
template <int ES, bool ALZ, bool ALQ, bool DL>
__device__ __forceinline__ void sub_tile(const void *zrow, const void *qrow, int V, int sub, float m, float c,
                                         float inv_s, float mq, float inv_sq, bool resid, bool use_r,
                                         float (&t)[kSubPerThread], double &rs, double &ps) {
    rs = 0.0; ps = 0.0;
#pragma unroll
    for (int i = 0; i < kSubPerThread; ++i) t[i] = 0.0f;
    const int e0 = sub * kSub + int(threadIdx.x) * kSubPerThread;
    if (e0 >= V) return;
    const int qo = resid ? e0 : 0;          // the zero block is read from its start
    float z[kSubPerThread], q[kSubPerThread];
    constexpr int QS = DL ? ES : 4;          // element size of the draft row
    if (ALZ && (!resid || ALQ) && e0 + kSubPerThread <= V) {
        const uint4 *zp = reinterpret_cast<const uint4 *>(static_cast<const char *>(zrow) + size_t(e0) * ES);
        const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const char *>(qrow) + size_t(qo) * QS);
        uint4 zw[ES == 2 ? 1 : 2], qw[QS == 2 ? 1 : 2];
        zw[0] = zp[0];
        if constexpr (ES == 4) zw[1] = zp[1];
        qw[0] = qp[0];
        if constexpr (QS == 4) qw[1] = qp[1];
        unpack8<ES>(zw, z);
        unpack8<QS>(qw, q);
    } else {
        // Element loads at clamped indices (all in bounds, all issued at once);
        // positions past the row end are dropped below.
#pragma unroll
        for (int i = 0; i < kSubPerThread; ++i) {
            const int e = min(e0 + i, V - 1);
            z[i] = load_elem<ES>(zrow, size_t(e));
            q[i] = load_elem<QS>(qrow, size_t(resid ? e : 0));
        }
    }
    if constexpr (DL) {
        // q from the draft logits (its reference as in the row pass: fl(mq * c) when finite)
        const float Rq = mq * c;
#pragma unroll
        for (int i = 0; i < kSubPerThread; ++i)
            q[i] = (finitef(Rq) ? exp2_fast(__builtin_fmaf(q[i], c, -Rq)) : exp2_fast((q[i] - mq) * c)) * inv_sq;
    }
#pragma unroll
    for (int i = 0; i < kSubPerThread; ++i) {
        if (e0 + i < V) {
            float r, p;
            draw_term(z[i], q[i], m, c, inv_s, resid, r, p);
            rs = rs + double(r);
            ps = ps + double(p);
            t[i] = use_r ? r : p;
        }
    }
}

// ------------------------------------------------------------- request items

// Per-request decision, computed identically by each of the request's workgroups.
struct Decision {
    int n, j;
    bool resid;
    float m, inv_s;
    float mq, inv_sq;  // draft logits: the draft row j's maximum and 1 / sum
    float u_final;    // u[b, G], the final draw's uniform
};

// Merge each read row's partials into sh.M[r] (max) and sh.S[r] (fp64 sum
// against the reference of sh.M[r]): 16 lanes per row, each lane's partials
// rescaled once, then a fixed 16-lane tree.  The partials were written by the
// previous launch.  Returns true in some thread if a read row is bad or has a
// partial that was never written.
constexpr int kRowBad = 1;
// Rows 0..nrows-1 of `part` (np1 partials each): fp32 maximum and fp64 sum
// per row into Mo / So.  Returns whether any row is bad or not yet written.
__device__ bool merge_rows_sampled(const VerifyArgs &a, const uint64_t *part, int nrows, float *Mo, double *So) {
    bool bad = false;
    constexpr int kRegs = 4;   // partials held per lane when np1 <= 64
    const int n = nrows - 1;
    const int l = threadIdx.x & 15, g = threadIdx.x >> 4;
    const float c = a.c32;
    const uint64_t empty = uint64_t(0xff800000u) | (uint64_t(kValid) << 32);   // (-inf, 0), written
    for (int r0 = 0; r0 <= n; r0 += kWG / 16) {
        const int r = r0 + g;
        const bool live = r <= n;
        const uint64_t *pp = part + size_t(live ? r : 0) * a.np1;
        float M = neg_inf();
        double S = 0.0;
        int ok = 1;
        if (a.np1 <= 16 * kRegs) {
            uint64_t v[kRegs];
#pragma unroll
            for (int i = 0; i < kRegs; ++i) {
                const int cc = l + 16 * i;
                v[i] = (live && cc < a.np1) ? pp[cc] : empty;
            }
#pragma unroll
            for (int i = 0; i < kRegs; ++i) {
                ok &= int(valid(v[i]));
                M = fmaxf(M, lo_f(v[i]));
            }
            M = row16_max(M);
#pragma unroll
            for (int i = 0; i < kRegs; ++i)
                S = S + double(__uint_as_float(hi_u(v[i]) & ~kValid)) * double(rescale(lo_f(v[i]), M, c));
        } else {
            if (live)
                for (int cc = l; cc < a.np1; cc += 16) {
                    const uint64_t v = pp[cc];
                    ok &= int(valid(v));
                    M = fmaxf(M, lo_f(v));
                }
            M = row16_max(M);
            if (live)
                for (int cc = l; cc < a.np1; cc += 16) {
                    const uint64_t v = pp[cc];
                    S = S + double(__uint_as_float(hi_u(v) & ~kValid)) * double(rescale(lo_f(v), M, c));
                }
        }
        S = row16_sum_d(S);
        ok = row16_and(ok);
        if (l == 0 && live) {
            bad |= !ok || !(S > 0.0 && S < INFINITY) || !(M > neg_inf() && M < __builtin_inff());
            Mo[r] = M;
            So[r] = S;
        }
    }
    return bad;
}

// merge_rows_sampled for partials that row workgroups of the same launch are
// still writing (the one-launch verify): each lane reloads those of its words
// that do not yet carry their written bit until all do (a bounded wait; an
// expired one reports the request as bad), with no workgroup-wide step per
// attempt.  The merge itself is merge_rows_sampled's, in the same order, so
// its results are bitwise the same.  `extra` issues the lane's own polled
// loads with every attempt and reports whether they are complete; the lane is
// done when both are.
template <typename F>
__device__ bool merge_rows_sampled_poll(const VerifyArgs &a, const uint64_t *part, int nrows, float *Mo,
                                        double *So, F extra) {
    bool bad = false;
    constexpr int kRegs = 4;
    const int n = nrows - 1;
    const int l = threadIdx.x & 15, g = threadIdx.x >> 4;
    const float c = a.c32;
    const uint64_t empty = uint64_t(0xff800000u) | (uint64_t(kValid) << 32);   // (-inf, 0), written
    for (int r0 = 0; r0 <= n; r0 += kWG / 16) {
        const int r = r0 + g;
        const bool live = r <= n;
        const uint64_t *pp = part + size_t(live ? r : 0) * a.np1;
        float M = neg_inf();
        double S = 0.0;
        int ok = 1;
        if (a.np1 <= 16 * kRegs) {
            uint64_t v[kRegs];
#pragma unroll
            for (int i = 0; i < kRegs; ++i) v[i] = 0ull;
            for (uint32_t spins = 0;; ++spins) {
#pragma unroll
                for (int i = 0; i < kRegs; ++i) {
                    const int cc = l + 16 * i;
                    if (!valid(v[i])) v[i] = (live && cc < a.np1) ? ld_coherent(pp + cc) : empty;
                }
                ok = int(extra());
#pragma unroll
                for (int i = 0; i < kRegs; ++i) ok &= int(valid(v[i]));
                if (ok || spins >= a.spin_limit) break;
            }
#pragma unroll
            for (int i = 0; i < kRegs; ++i) M = fmaxf(M, lo_f(v[i]));
            M = row16_max(M);
#pragma unroll
            for (int i = 0; i < kRegs; ++i)
                S = S + double(__uint_as_float(hi_u(v[i]) & ~kValid)) * double(rescale(lo_f(v[i]), M, c));
        } else {
            for (uint32_t spins = 0;; ++spins) {
                ok = int(extra());
                if (__syncthreads_and(ok) || spins >= a.spin_limit) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (live)
                for (int cc = l; cc < a.np1; cc += 16) {
                    uint64_t v = ld_coherent(pp + cc);
                    for (uint32_t spins = 0; !valid(v) && spins < a.spin_limit; ++spins) {
                        __builtin_amdgcn_s_sleep(2);
                        v = ld_coherent(pp + cc);
                    }
                    ok &= int(valid(v));
                    M = fmaxf(M, lo_f(v));
                }
            M = row16_max(M);
            if (live)
                for (int cc = l; cc < a.np1; cc += 16) {
                    const uint64_t v = ld_coherent(pp + cc);      // written by now (or the request is bad)
                    S = S + double(__uint_as_float(hi_u(v) & ~kValid)) * double(rescale(lo_f(v), M, c));
                }
        }
        S = row16_sum_d(S);
        ok = row16_and(ok);
        if (l == 0 && live) {
            bad |= !ok || !(S > 0.0 && S < INFINITY) || !(M > neg_inf() && M < __builtin_inff());
            Mo[r] = M;
            So[r] = S;
        }
    }
    return bad;
}


// Rows 0..n's chunk partials (greedy): lowest index of the maximum into
// sh.A[r], 16 lanes per row.  The partials are written by row waves of the
// same launch: they are loaded in one batch per attempt (up to 8 per lane,
// every vocabulary up to 2^18 bf16 or 2^17 fp32), and the batch repeats
// (bounded) until all are written.  Returns kRowBad in some thread for a bad
// row or a wait that expired.
// Merged argmax of rows 0..n into sh.A (kBadRowArgmax for a bad row: a NaN,
// maximum +inf, all -inf, or a partial never written); returns kRowBad if any.
constexpr int kBadRowArgmax = -3;
__device__ int merge_rows_greedy(const VerifyArgs &a, int b, int n, Smem &sh) {
    constexpr int kRegs = 8;
    const uint64_t *part = partials(a, b);
    const int l = threadIdx.x & 15, g = threadIdx.x >> 4;
    int flags = 0;
    for (int r0 = 0; r0 <= n; r0 += kWG / 16) {
        const int r = r0 + g;
        const bool live = r <= n;
        const uint64_t *pp = part + size_t(live ? r : 0) * a.np1;
        float best = neg_inf();
        int bi = -1, nan = 0, ok = 1;
        if (a.np1 <= 16 * kRegs) {
            uint64_t v[kRegs];
#pragma unroll
            for (int i = 0; i < kRegs; ++i) v[i] = 0ull;
            for (uint32_t spins = 0;; ++spins) {
#pragma unroll
                for (int i = 0; i < kRegs; ++i) {
                    const int cc = l + 16 * i;
                    if (!valid(v[i]))
                        v[i] = (live && cc < a.np1) ? ld_coherent(pp + cc) : (uint64_t(1) << 32 | uint64_t(kValid) << 32);
                }
                ok = 1;
#pragma unroll
                for (int i = 0; i < kRegs; ++i) ok &= int(valid(v[i]));
                if (ok || spins >= a.spin_limit) break;
            }
#pragma unroll
            for (int i = 0; i < kRegs; ++i) {          // ascending chunks: the first maximum wins
                const int vi = int(hi_u(v[i]) & ~kValid) - 2;
                if (vi == kNanIdx) nan = 1;
                else merge_am(best, bi, lo_f(v[i]), vi);
            }
        } else if (live) {
            for (int cc = l; cc < a.np1; cc += 16) {
                uint64_t v = ld_coherent(pp + cc);
                for (uint32_t spins = 0; !valid(v) && spins < a.spin_limit; ++spins) {
                    __builtin_amdgcn_s_sleep(4);
                    v = ld_coherent(pp + cc);
                }
                ok &= int(valid(v));
                const int vi = int(hi_u(v) & ~kValid) - 2;
                if (vi == kNanIdx) nan = 1;
                else merge_am(best, bi, lo_f(v), vi);
            }
        }
        row16_argmax(best, bi, nan);
        ok = row16_and(ok);
        if (l == 0 && live) {
            const bool rb = !ok || nan || bi < 0 || best == __builtin_inff();
            if (rb) flags |= kRowBad;
            sh.A[r] = rb ? kBadRowArgmax : bi;
        }
    }
    return flags;
}

// Unnormalised target probability 2^(z*c - R) of a value z in a row with
// maximum m, in fp64, against the same reference the row sum S used.
__device__ __forceinline__ double target_prob(float z, float m, float c) {
    const float R = m * c;
    return finitef(R) ? exp2(double(z) * double(c) - double(R)) : exp2((double(z) - double(m)) * double(c));
}

// Diagnostics of request b (only when requested), from the merged rows.  In
// fp32 (their tolerance is far above fp32 rounding), so this path costs the
// kernel no registers beyond the hot path's.
template <int ES>
__device__ void write_diag(const VerifyArgs &a, int b, bool ok, int n, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const float qnan = __builtin_nanf("");
    for (int t = threadIdx.x; t < G1; t += kWG) {
        float lse = qnan, pv = qnan, qv = qnan;
        if (ok && t <= n) {
            const float m = sh.M[t], S = float(sh.S[t]), R = m * a.c32;
            lse = finitef(R) ? R * 0.6931471805599453f + logf(S) : m / a.T + logf(S);
            if (t < n) {
                const int xt = a.x[size_t(b) * G + t];
                const float zt = load_elem<ES>(a.logits, row_elem(a, b, t) + size_t(xt));
                if (a.dl) {
                    // the draft probability from the draft row's logits and normaliser
                    const float dt = load_elem<ES>(a.dl, (size_t(b) * G + t) * size_t(a.V) + size_t(xt));
                    const float mq = sh.Mq[t], Rq = mq * a.c32;
                    const float eq = finitef(Rq) ? exp2_fast(__builtin_fmaf(dt, a.c32, -Rq)) : exp2_fast((dt - mq) * a.c32);
                    qv = eq / float(sh.Sq[t]);
                } else {
                    qv = a.q[(size_t(b) * G + t) * size_t(a.V) + size_t(xt)];
                }
                const float e = finitef(R) ? exp2_fast(__builtin_fmaf(zt, a.c32, -R)) : exp2_fast((zt - m) * a.c32);
                pv = e / S;
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

// All partials and gathers of the request are complete (written by the
// previous launch): merge every read row, run the accept tests, find the first
// rejection.  Returns false (outputs reported by workgroup 0) for a data error
// or an invalid verify length (then *proceed is false: the request's
// workgroups do nothing more, since the row pass read none of its rows).
// Every load is issued before the first barrier (a barrier waits for
// outstanding loads), so the whole decision costs one memory round trip.
template <int ES>
__device__ bool decide(const VerifyArgs &a, int b, int w, Decision &d, bool &proceed, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const int k = threadIdx.x;
    const int n = verify_len(a, b);
    d.n = n;
    d.j = 0;
    d.resid = false;
    d.m = 0.0f;
    d.inv_s = 0.0f;
    d.mq = 0.0f;
    d.inv_sq = 0.0f;
    d.u_final = 0.0f;
    proceed = false;
    if (n < 0 || n > G) {
        if (w == 0) write_error(a, b);
        return false;
    }
    proceed = true;
    int xk = 0;
    uint64_t gk = 0;
    float uk = 0.0f;
    if (k < n) {
        xk = a.x[size_t(b) * G + k];
        gk = gathered(a, b)[k];
        uk = a.u[size_t(b) * G1 + k];
    }
    d.u_final = a.u[size_t(b) * G1 + G];
    bool bad = merge_rows_sampled(a, partials(a, b), n + 1, sh.M, sh.S);
    if (a.dl) bad |= merge_rows_sampled(a, partials_d(a, b), n, sh.Mq, sh.Sq);
    // Keep the uses of the per-draft loads below the partials' loads (the
    // compiler would otherwise wait for them before issuing the partials).
    asm volatile("" : "+v"(xk), "+v"(uk), "+v"(gk));
    bad |= k < n && (xk < 0 || xk >= a.V);
    if (__syncthreads_or(bad)) {
        if (w == 0) write_error(a, b);
        return false;
    }
    bool rej = false;
    if (k < n) {
        const float zx = lo_f(gk), hx = __uint_as_float(hi_u(gk));
        const double pk = target_prob(zx, sh.M[k], a.c32) / sh.S[k];
        // q(x_k): as read, or from the draft row's normaliser (draft logits)
        const double qx = a.dl ? target_prob(hx, sh.Mq[k], a.c32) / sh.Sq[k] : double(hx);
        const bool acc = (qx > 0.0) ? (double(uk) < pk / qx) : (pk > 0.0);
        rej = !acc;
    }
    post_first(rej, 0, sh);
    __syncthreads();
    const int jf = wg_first(0, sh);
    const int j = (jf == INT_MAX) ? n : jf;
    d.j = j;
    d.resid = j < n;
    d.m = sh.M[j];
    d.inv_s = float(1.0 / sh.S[j]);
    if (a.dl && j < n) {
        d.mq = sh.Mq[j];
        d.inv_sq = float(1.0 / sh.Sq[j]);
    }
    if (w == 0) {
        for (int t = threadIdx.x; t < G1; t += kWG) {
            if (t < j) st_out(a.out_tok + size_t(b) * G1 + t, a.x[size_t(b) * G + t]);
            else if (t > j) st_out(a.out_tok + size_t(b) * G1 + t, -1);
        }
        if (threadIdx.x == 0) st_out(a.out_acc + b, j);
    }
    return true;
}

// ------------------------------------------------- one-launch decision record

__device__ __forceinline__ uint64_t *decision(const VerifyArgs &a, int b) {
    return reinterpret_cast<uint64_t *>(a.ws + size_t(a.lay.dec) * 256) + size_t(b) * 4;
}
constexpr uint32_t kDecResid = 1u << 15, kDecOk = 1u << 16, kDecJ = 0x7fffu;
// Word 2 of the record: every read row and gather checked; ok or a data error.
constexpr uint64_t kFinWritten = uint64_t(kValid) << 32, kFinOk = 1ull;

// The decision workgroup of request b in the one-launch verify, after the
// request's row workgroups in grid order.  It polls the row partials and the
// flagged gathers until written and decides exactly as decide() does (the
// same merge and accept tests), in two steps:
//  - the record (words 0 and 1: j, the residual flag, m_j and 1 / S_j) goes
//    out as soon as the rows it depends on are in: rows 0..j merged, rows
//    0..j-1 accepted and row j rejected (or, with every draft accepted, row
//    n merged).  Row workgroups finish roughly in row order and most
//    requests reject early, so the request workgroups start the draw while
//    the later rows are still being read.  A bad row, or an id out of range,
//    among those rows publishes a record with ok = 0;
//  - once every read row and gather is in, word 2 states whether the request
//    holds a data error anywhere (the request's last workgroup waits for it
//    before writing the drawn token); then the accepted prefix, the -1
//    padding and out_accepted (or the error outputs) and the diagnostics go
//    out, and the partials and gathers, which nothing reads after it, are
//    cleared.
// An invalid verify length publishes nothing: the request workgroups see the
// length themselves.

// The record of a decision (one thread).
__device__ __forceinline__ void put_record(uint64_t *rec, int j, int n, bool err, float m, float inv_s) {
    const uint32_t h = uint32_t(j) | (j < n ? kDecResid : 0u) | (err ? 0u : kDecOk) | kValid;
    st_coherent(rec + 1, uint64_t(__float_as_uint(inv_s)) | (uint64_t(kValid) << 32));
    st_coherent(rec, uint64_t(__float_as_uint(m)) | (uint64_t(h) << 32));
}

// After every read row is in: the accepted prefix, the padding and
// out_accepted (the token at j is left to the request workgroups), or the
// error outputs; the diagnostics; the clearing of the partials and gathers.
template <int ES>
__device__ void decision_outputs(const VerifyArgs &a, int b, int n, int j, bool err, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    if (!err) {
        for (int t = threadIdx.x; t < G1; t += kWG) {
            if (t < j) st_out(a.out_tok + size_t(b) * G1 + t, a.x[size_t(b) * G + t]);
            else if (t > j) st_out(a.out_tok + size_t(b) * G1 + t, -1);
        }
        if (threadIdx.x == 0) st_out(a.out_acc + b, j);
    } else {
        write_error(a, b);
    }
    if (a.d_lse || a.d_p || a.d_q || a.d_r) write_diag<ES>(a, b, !err, n, sh);
    uint64_t *part = partials(a, b);
    for (int i = threadIdx.x; i < (n + 1) * a.np1; i += kWG) st_coherent(part + i, 0ull);
    for (int i = threadIdx.x; i < n; i += kWG) st_coherent(gathered(a, b) + i, 0ull);
}

// More rows than 16-lane groups, or more partials per row than a lane holds:
// every row merged first, then the record and word 2 together.
template <int ES>
__device__ void decide_publish_whole(const VerifyArgs &a, int b, int n, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const int k = threadIdx.x;
    int xk = 0;
    float uk = 0.0f;
    uint64_t gk = 0;
    if (k < n) {
        xk = a.x[size_t(b) * G + k];
        uk = a.u[size_t(b) * G1 + k];
    }
    // The gather word of draft k is written (its bit set) by the row
    // workgroup whose chunk holds x_k; an id out of range is never gathered
    // and is a data error.  It is polled with the partials.
    bool gready = !(k < n);
    const uint64_t *gxp = gathered(a, b) + (k < n ? k : 0);
    bool bad = merge_rows_sampled_poll(a, partials(a, b), n + 1, sh.M, sh.S, [&]() -> bool {
        if (!gready) {
            gk = ld_coherent(gxp);
            gready = (hi_u(gk) & kValid) != 0u || xk < 0 || xk >= a.V;
        }
        return gready;
    });
    bad |= k < n && (xk < 0 || xk >= a.V);
    const bool err = wg_any(bad, 1, sh);
    int j = n;
    float m = 0.0f, inv_s = 0.0f;
    if (!err) {
        bool rej = false;
        if (k < n) {
            const float zx = lo_f(gk), qx32 = __uint_as_float(hi_u(gk) & ~kValid);
            const double pk = target_prob(zx, sh.M[k], a.c32) / sh.S[k];
            const double qx = double(qx32);
            const bool acc = (qx > 0.0) ? (double(uk) < pk / qx) : (pk > 0.0);
            rej = !acc;
        }
        post_first(rej, 0, sh);
        __syncthreads();
        const int jf = wg_first(0, sh);
        j = (jf == INT_MAX) ? n : jf;
        m = sh.M[j];
        inv_s = float(1.0 / sh.S[j]);
    }
    if (threadIdx.x == 0) {
        uint64_t *rec = decision(a, b);
        put_record(rec, j, n, err, m, inv_s);
        st_coherent(rec + 2, kFinWritten | (err ? 0ull : kFinOk));
    }
    decision_outputs<ES>(a, b, n, j, err, sh);
}

// A row's status in the early decision.
constexpr int kRowWait = 0, kRowAcc = 1, kRowRej = 2, kRowBadSt = 3;

// What the statuses settle (uniform across the wave; lane r <= n holds row
// r's status s): the first row not accepted decides (rejected: j; bad: a data
// error; still waiting: nothing yet); with none, every draft is accepted and
// j = n.
struct Settled {
    bool known, err;
    int j;
};
__device__ __forceinline__ Settled settle(int n, int lane, int s) {
    const uint64_t notacc = __ballot(lane <= n && s != kRowAcc);
    const int f = notacc ? __builtin_ctzll(notacc) : n;
    const int sf = notacc ? __builtin_amdgcn_readlane(s, f) : kRowAcc;
    return Settled{sf != kRowWait, sf == kRowBadSt, f};
}

template <int ES>
__device__ void decide_publish(const VerifyArgs &a, int b, Smem &sh) {
    constexpr int kRegs = 4;      // partials held per lane (np1 <= 64)
    constexpr int kRows = kWG / 16;
    const int G = a.G, G1 = G + 1;
    const int n = verify_len(a, b);
    if (n < 0 || n > G) {
        write_error(a, b);
        if (a.d_lse || a.d_p || a.d_q || a.d_r) write_diag<ES>(a, b, false, n, sh);
        return;
    }
    if (n + 1 > kRows || a.np1 > 16 * kRegs) {
        decide_publish_whole<ES>(a, b, n, sh);
        return;
    }
    // Row r = t / 16 is merged by the 16 lanes of group r; the group's lane 0
    // also holds draft r (its id, uniform and gather word) for the accept test.
    // The statuses are cleared before any load is issued (a barrier waits for
    // outstanding loads), and no barrier follows until every row is in.
    const int t = threadIdx.x, l = t & 15, r = t >> 4, lane = t & 63;
    if (t < kRows) sh.rst[t] = kRowWait;
    if (t == 0) sh.pub = 0;
    __syncthreads();
    const bool live = r <= n, drafted = r < n;
    const bool lead = l == 0 && drafted;
    int xr = 0;
    float ur = 0.0f;
    if (lead) {
        xr = a.x[size_t(b) * G + r];
        ur = a.u[size_t(b) * G1 + r];
    }
    const bool xbad = lead && (xr < 0 || xr >= a.V);
    const uint64_t *pp = partials(a, b) + size_t(live ? r : 0) * a.np1;
    const uint64_t *gxp = gathered(a, b) + (drafted ? r : 0);
    const uint64_t empty = uint64_t(0xff800000u) | (uint64_t(kValid) << 32);   // (-inf, 0), written
    const float c = a.c32;
    uint64_t v[kRegs], gk = 0;
#pragma unroll
    for (int i = 0; i < kRegs; ++i) v[i] = 0ull;
    bool gready = !lead;
    bool merged = !live;                    // uniform in the group
    bool settled = false;                   // uniform in the wave: the record is out
    for (uint32_t spins = 0;; ++spins) {
        // Each lane reloads only its words not yet written (a bounded wait:
        // a row whose wait expires stays waiting, a data error).
#pragma unroll
        for (int i = 0; i < kRegs; ++i) {
            const int cc = l + 16 * i;
            if (!valid(v[i])) v[i] = (live && cc < a.np1) ? ld_coherent(pp + cc) : empty;
        }
        if (!gready) {
            gk = ld_coherent(gxp);
            gready = valid(gk) || xbad;     // an id out of range is never gathered
        }
        int ok = int(gready);
#pragma unroll
        for (int i = 0; i < kRegs; ++i) ok &= int(valid(v[i]));
        ok = row16_and(ok);
        const bool fresh = ok && !merged;
        if (__ballot(fresh) != 0ull) {
            // Rows complete in this attempt: merge_rows_sampled's merge (the
            // same order, so bitwise the same M and S), the accept test, and
            // the row's status, stored after its M and S.
            float M = neg_inf();
#pragma unroll
            for (int i = 0; i < kRegs; ++i) M = fmaxf(M, lo_f(v[i]));
            M = row16_max(M);
            double S = 0.0;
#pragma unroll
            for (int i = 0; i < kRegs; ++i)
                S = S + double(__uint_as_float(hi_u(v[i]) & ~kValid)) * double(rescale(lo_f(v[i]), M, c));
            S = row16_sum_d(S);
            if (fresh && l == 0) {
                int st;
                if (xbad || !(S > 0.0 && S < INFINITY) || !(M > neg_inf() && M < __builtin_inff())) {
                    st = kRowBadSt;
                } else if (!drafted) {
                    st = kRowAcc;                   // row n: merged and good
                } else {
                    const float zx = lo_f(gk), qx32 = __uint_as_float(hi_u(gk) & ~kValid);
                    const double pk = target_prob(zx, M, c) / S;
                    const double qx = double(qx32);
                    float u = ur;
                    asm volatile("" : "+v"(u));     // widened here, not held widened through the wait
                    st = ((qx > 0.0) ? (double(u) < pk / qx) : (pk > 0.0)) ? kRowAcc : kRowRej;
                }
                sh.M[r] = M;
                sh.S[r] = S;
                __hip_atomic_store(&sh.rst[r], st, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            merged = merged || ok;
            // Publish once the statuses settle the decision; the first wave
            // to claim sh.pub writes the record.  (Sequentially consistent
            // status stores and loads: of two waves completing rows at once,
            // at least one sees both.)
            if (!settled) {
                const int s = (lane <= n) ? __hip_atomic_load(&sh.rst[lane], __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_WORKGROUP)
                                          : kRowAcc;
                const Settled d = settle(n, lane, s);
                if (d.known) {
                    settled = true;
                    if (lane == 0 && atomicCAS(&sh.pub, 0, 1) == 0) {
                        float m = 0.0f, inv_s = 0.0f;
                        if (!d.err) {
                            m = sh.M[d.j];
                            inv_s = float(1.0 / sh.S[d.j]);
                        }
                        put_record(decision(a, b), d.j, n, d.err, m, inv_s);
                    }
                }
            }
        }
        if (__ballot(!merged) == 0ull || spins >= a.spin_limit) break;
    }
    __syncthreads();
    // Every row in (or its wait expired): a row still waiting or bad anywhere
    // is a data error; otherwise the decision is the one already published.
    const int s = (lane <= n) ? sh.rst[lane] : kRowAcc;
    const bool err = __ballot(lane <= n && s != kRowAcc && s != kRowRej) != 0ull;
    const Settled d = settle(n, lane, s);
    const int j = err ? n : d.j;
    if (t == 0) {
        uint64_t *rec = decision(a, b);
        if (sh.pub == 0) put_record(rec, j, n, err, err ? 0.0f : sh.M[j], err ? 0.0f : float(1.0 / sh.S[j]));
        st_coherent(rec + 2, kFinWritten | (err ? 0ull : kFinOk));
    }
    decision_outputs<ES>(a, b, n, j, err, sh);
}

// A request workgroup of the one-launch verify: request b's decision, from its
// record (a bounded wait: one lane polls, keeping its next load in flight
// while it examines the last, and shares the record through LDS).  Returns false for a
// data error; *proceed is false for an invalid verify length (the decision
// workgroup reports it).  An expired wait reports the request as bad (the
// request's last workgroup writes the error).
__device__ bool await_decision(const VerifyArgs &a, int b, int w, Decision &d, bool &proceed, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const int n = verify_len(a, b);
    d.n = n;
    d.j = 0;
    d.resid = false;
    d.m = 0.0f;
    d.inv_s = 0.0f;
    d.mq = 0.0f;
    d.inv_sq = 0.0f;
    proceed = n >= 0 && n <= G;
    if (!proceed) return false;
    d.u_final = a.u[size_t(b) * G1 + G];
    const uint64_t *rec = decision(a, b);
    if (threadIdx.x == 0) {
        // one lane polls, with the next poll in flight while it examines the last
        uint64_t p0 = ld_coherent(rec), p1 = ld_coherent(rec + 1);
        bool r = false;
        for (uint32_t spins = 0;; ++spins) {
            const uint64_t n0 = ld_coherent(rec), n1 = ld_coherent(rec + 1);
            if (((p0 & p1) >> 63) != 0) { r = true; break; }
            if (spins >= a.spin_limit) break;
            p0 = n0;
            p1 = n1;
        }
        sh.pw[0] = p0;
        sh.pw[1] = p1;
        sh.pok = r ? 1 : 0;
    }
    __syncthreads();
    const uint64_t w0 = sh.pw[0], w1 = sh.pw[1];
    const bool ready = sh.pok != 0;
    if (!ready) {
        if (w == a.nc2 - 1) write_error(a, b);
        return false;
    }
    const uint32_t h = hi_u(w0);
    d.j = int(h & kDecJ);
    d.resid = (h & kDecResid) != 0u;
    d.m = lo_f(w0);
    d.inv_s = lo_f(w1);
    return (h & kDecOk) != 0u;
}

// Wait until every sub-tile mass word of request b is written and, with fin
// (the one-launch verify: word 2 of the decision record), until the decision
// workgroup has checked every read row; *fin_ok is then whether it found no
// data error.  With at most kWG sub-tiles thread s polls sub-tile s's two
// words on its own (thread 0 also polls fin) and returns its (residual,
// target) masses in v (zeros past the end), and one barrier ends the wait.
// False if a bounded wait expired.
__device__ bool wait_masses(const VerifyArgs &a, int b, double (&v)[2], const uint64_t *fin, bool &fin_ok,
                            Smem &sh) {
    const uint64_t *mass = masses(a, b);
    const int nsub = a.nsub;
    const bool pf = fin != nullptr && threadIdx.x == 0;
    if (nsub <= kWG) {
        const int s = threadIdx.x;
        uint64_t w0 = kMassWritten, w1 = kMassWritten, wf = kFinWritten | kFinOk;
        bool mine = true;
        if (s < nsub) {
            for (uint32_t spins = 0;; ++spins) {
                w0 = ld_coherent(mass + 2 * s);
                w1 = ld_coherent(mass + 2 * s + 1);
                if (pf) wf = ld_coherent(fin);
                if ((w0 & w1 & kMassWritten) != 0 && (wf & kFinWritten) != 0) break;
                if (spins >= a.spin_limit) { mine = false; break; }
            }
        }
        if (pf) sh.pok = int((wf & kFinOk) != 0);
        v[0] = mass_value(w0);
        v[1] = mass_value(w1);
        const bool all = !wg_any(!mine, 2, sh);
        fin_ok = fin == nullptr || sh.pok != 0;
        return all;
    }
    for (uint32_t spins = 0;; ++spins) {
        bool ready = true;
        for (int i = threadIdx.x; i < 2 * nsub; i += kWG) ready &= (ld_coherent(mass + i) & kMassWritten) != 0;
        if (pf) {
            const uint64_t wf = ld_coherent(fin);
            ready &= (wf & kFinWritten) != 0;
            sh.pok = int((wf & kFinOk) != 0);
        }
        if (__syncthreads_and(ready)) {
            fin_ok = fin == nullptr || sh.pok != 0;
            return true;
        }
        if (spins >= a.spin_limit) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Last workgroup of request b: locate u * R and write the token.
//
// The draw follows the inverse-CDF definition: y is the first index whose
// running sum of terms exceeds u times their total.  Sums are hierarchical
// (sub-tile masses, then 8-element thread sums, then the elements), so the
// search takes the first sub-tile, then the first thread, then the first
// element whose running sum passes the target, each level restricted to
// positive mass.  Where rounding between the levels leaves no crossing, the
// last positive term before the target is taken, which differs from the exact
// draw only when u * R lies within rounding of a cumulative sum.
template <int ES, bool ALZ, bool ALQ, bool DL>
__device__ void final_select(const VerifyArgs &a, int b, const Decision &d, const void *zrow, const void *qrow,
                             const double (&polled)[2], Smem &sh) {
    const int G1 = a.G + 1;
    const bool resid = d.resid;
    const uint64_t *mass = masses(a, b);
    const int nsub = a.nsub;
    double R = 0.0, Rp = 0.0, target = 0.0, base = 0.0;
    int sstar = INT_MAX, sel = 0;
    bool use_r = false, lastpos = false;
    if (nsub <= 64) {
        // Wave 0 holds every sub-tile's masses (the polled values): both
        // prefixes, the last positive sub-tiles and the first sub-tile past
        // u * R come from DPP scans and ballots, with one barrier to share
        // them.  The prefixes are bitwise those of the workgroup scan below,
        // to which waves 1..3 would only add zeros.
        if (threadIdx.x < 64) {
            const int s = threadIdx.x;
            const double x0 = wave_scan_d(polled[0]);
            const double tR = lane_d(x0, 63);
            const bool ur = resid && tR > 0.0;
            const int sl = (resid && !ur) ? 1 : 0;
            // the target masses' prefix only when the draw falls back to them
            // (a residual of zero mass; uniform across the wave)
            double x1 = 0.0, tRp = 0.0;
            if (sl) {
                x1 = wave_scan_d(polled[1]);
                tRp = lane_d(x1, 63);
            }
            const double tg = double(d.u_final) * (sl ? tRp : tR);
            const double vs = sl ? polled[1] : polled[0], xs = sl ? x1 : x0;
            const double ps = dpp_d<kWaveShr1>(xs), bs = (s == 0) ? 0.0 : ps;
            const uint64_t mp = __ballot(vs > 0.0);
            const uint64_t mf = __ballot(s < nsub && vs > 0.0 && bs + vs > tg);
            const int ss = mf ? __builtin_ctzll(mf) : (mp ? 63 - __builtin_clzll(mp) : 0);
            const double bb = mf ? lane_d(bs, ss) : 0.0;
            if (s == 0) {
                sh.R = tR;
                sh.Rp = tRp;
                sh.base = bb;
                sh.fsel[0] = ss;
                sh.fsel[1] = int(mf == 0) | (int(ur) << 1) | (sl << 2);
            }
        }
        __syncthreads();
        R = sh.R;
        Rp = sh.Rp;
        base = sh.base;
        sstar = sh.fsel[0];
        lastpos = (sh.fsel[1] & 1) != 0;
        use_r = (sh.fsel[1] & 2) != 0;
        sel = sh.fsel[1] >> 2;
        target = double(d.u_final) * (sel ? Rp : R);
    } else {
        // More than 64 sub-tiles: wave 0 walks them in blocks of 64 with the DPP
        // scans and ballots of the path above and a running base (the words are
        // complete: wait_masses saw every written bit).  Pass 1 forms both totals
        // and the last positive sub-tile of each array; pass 2 finds the first
        // sub-tile with positive mass whose running total passes u * R.  Both
        // passes add the same block totals in the same order, so the located
        // sub-tile is consistent with R.
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            double tR = 0.0, tRp = 0.0;
            int lr = -1, lp = -1;
            for (int blk = 0; blk < nsub; blk += 64) {
                const int s = blk + lane;
                double v0 = 0.0, v1 = 0.0;
                if (s < nsub) {
                    v0 = mass_value(ld_coherent(mass + 2 * s));
                    v1 = mass_value(ld_coherent(mass + 2 * s + 1));
                }
                const double x0 = wave_scan_d(v0), x1 = wave_scan_d(v1);
                tR = tR + lane_d(x0, 63);
                tRp = tRp + lane_d(x1, 63);
                const uint64_t m0 = __ballot(v0 > 0.0), m1 = __ballot(v1 > 0.0);
                if (m0) lr = blk + 63 - __builtin_clzll(m0);
                if (m1) lp = blk + 63 - __builtin_clzll(m1);
            }
            const bool ur = resid && tR > 0.0;
            const int sl = (resid && !ur) ? 1 : 0;
            const double tg = double(d.u_final) * (sl ? tRp : tR);
            double P = 0.0, bb = 0.0;
            int ss = INT_MAX;
            for (int blk = 0; blk < nsub; blk += 64) {
                const int s = blk + lane;
                const double vs = (s < nsub) ? mass_value(ld_coherent(mass + 2 * s + sl)) : 0.0;
                const double xs = wave_scan_d(vs);
                const double ps = dpp_d<kWaveShr1>(xs), bs = P + ((lane == 0) ? 0.0 : ps);
                const uint64_t mf = __ballot(s < nsub && vs > 0.0 && bs + vs > tg);
                if (mf) {
                    const int f = __builtin_ctzll(mf);
                    ss = blk + f;
                    bb = lane_d(bs, f);
                    break;
                }
                P = P + lane_d(xs, 63);
            }
            if (lane == 0) {
                sh.R = tR;
                sh.Rp = tRp;
                sh.base = bb;
                sh.fsel[0] = (ss == INT_MAX) ? max(0, sl ? lp : lr) : ss;
                sh.fsel[1] = int(ss == INT_MAX) | (int(ur) << 1) | (sl << 2);
            }
        }
        __syncthreads();
        R = sh.R;
        Rp = sh.Rp;
        base = sh.base;
        sstar = sh.fsel[0];
        lastpos = (sh.fsel[1] & 1) != 0;
        use_r = (sh.fsel[1] & 2) != 0;
        sel = sh.fsel[1] >> 2;
        target = double(d.u_final) * (sel ? Rp : R);
    }
    float t[kSubPerThread];
    double rs, ps;
    sub_tile<ES, ALZ, ALQ, DL>(zrow, qrow, a.V, sstar, d.m, a.c32, d.inv_s, d.mq, d.inv_sq, resid, use_r, t, rs, ps);
    const double v1[1] = {sel ? ps : rs};
    double ex1[1], in1[1], tot1[1];
    wg_scan<1>(v1, ex1, in1, tot1, sh);
    const int e0 = sstar * kSub + int(threadIdx.x) * kSubPerThread;
    int lp = -1;
#pragma unroll
    for (int i = 0; i < kSubPerThread; ++i)
        if (t[i] > 0.0f) lp = e0 + i;
    // The draw lies in the first thread with positive mass whose running total
    // passes the target.  A thread's exclusive prefix is bitwise its
    // predecessor's inclusive one, so that thread is the one whose interval
    // [base + excl, base + incl) holds the target: each thread tests its own,
    // with no barrier.  Whether one does is uniform: the sub-tile was chosen
    // with base <= target < base + its mass, which equals the scan's total
    // bitwise; only when no sub-tile passed (lastpos) does none, and the last
    // thread with positive mass takes its last positive term.
    const bool none = lastpos || !(base + tot1[0] > target);
    int y = -2;
    if (none) {
        post_last(v1[0] > 0.0, 4, sh);
        __syncthreads();
        const int tl = wg_last(4, sh);
        if (int(threadIdx.x) == max(tl, 0)) y = lp;   // tl < 0 cannot happen: p(argmax) >= 1/V
    } else if (base + ex1[0] <= target && base + in1[0] > target) {
        // The thread holding the draw writes it.
        double acc = base + ex1[0];
        int yc = -1;
#pragma unroll
        for (int i = 0; i < kSubPerThread; ++i) {
            acc = acc + double(t[i]);
            if (yc < 0 && t[i] > 0.0f && acc > target) yc = e0 + i;
        }
        y = (yc >= 0) ? yc : lp;
    }
    if (y != -2) {
        st_out(a.out_tok + size_t(b) * G1 + d.j, y);
        if (a.d_r) a.d_r[b] = resid ? float(R) : -1.0f;
    }
}

// Request pass (after the row pass has completed): workgroup w of request b
// decides the request, streams sub-tiles [w*spw, (w+1)*spw) of the draw row
// and writes their masses (on a data error, marks them done); the request's
// last workgroup (w = nc2 - 1) waits for every mass word, selects the token,
// writes the diagnostics and zeroes the request's partials, gathers and
// masses.  FUSED: the same, in the launch that also runs the row workgroups
// (the decision polls the partials; nothing was gathered).
template <int ES, bool ALZ, bool ALQ, bool DL, bool FUSED = false>
__device__ void request_item_sampled(const VerifyArgs &a, int b, int w, Smem &sh) {
    static_assert(!(FUSED && DL), "the one-launch verify reads draft probabilities");
    Decision d;
    bool proceed;
    const bool ok = FUSED ? await_decision(a, b, w, d, proceed, sh) : decide<ES>(a, b, w, d, proceed, sh);
    if (!proceed) {
        if (!FUSED && w == 0 && (a.d_lse || a.d_p || a.d_q || a.d_r)) write_diag<ES>(a, b, false, d.n, sh);
        return;
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t *mass = masses(a, b);
    const void *zrow = static_cast<const char *>(a.logits) + row_elem(a, b, d.j) * ES;
    // the draft row j (probabilities, or logits with DL) on a rejection, else the zero block
    const size_t qe = (size_t(b) * a.G + d.j) * size_t(a.V);
    const void *qrow = !d.resid ? static_cast<const void *>(a.ws + size_t(a.lay.zero) * 256)
                       : DL    ? static_cast<const void *>(static_cast<const char *>(a.dl) + qe * ES)
                               : static_cast<const void *>(a.q + qe);
    if (!ok) {
        const int s_beg = w * a.spw, s_end = min(a.nsub, (w + 1) * a.spw);
        for (int i = 2 * s_beg + int(threadIdx.x); i < 2 * s_end; i += kWG) st_coherent(mass + i, kMassWritten);
    } else {
        const int s_end = min(a.nsub, (w + 1) * a.spw);
        for (int s0 = w * a.spw; s0 < s_end; s0 += kSubBatch) {
            double rs[kSubBatch], ps[kSubBatch];
#pragma unroll
            for (int i = 0; i < kSubBatch; ++i) {
                float t[kSubPerThread];
                rs[i] = 0.0; ps[i] = 0.0;
                if (s0 + i < s_end)
                    sub_tile<ES, ALZ, ALQ, DL>(zrow, qrow, a.V, s0 + i, d.m, a.c32, d.inv_s, d.mq, d.inv_sq, d.resid,
                                               true, t, rs[i], ps[i]);
            }
#pragma unroll
            for (int i = 0; i < kSubBatch; ++i) {
                rs[i] = wave_sum_d(rs[i]);
                ps[i] = wave_sum_d(ps[i]);
            }
            __syncthreads();
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < kSubBatch; ++i) {
                    sh.r.wt[wv][i] = rs[i];
                    sh.r.wt[wv][kSubBatch + i] = ps[i];
                }
            }
            __syncthreads();
            if (int(threadIdx.x) < 2 * kSubBatch) {
                const int q = threadIdx.x, i = q % kSubBatch, which = q / kSubBatch;   // which: 0 residual, 1 target
                const double m4 = ((sh.r.wt[0][q] + sh.r.wt[1][q]) + sh.r.wt[2][q]) + sh.r.wt[3][q];
                if (s0 + i < s_end) st_coherent(mass + 2 * (s0 + i) + which, mass_word(m4));
            }
        }
    }
    // The request's last workgroup in grid order selects the token: it waits
    // only for workgroups dispatched before it, which never wait themselves.
    // A mass word is written after its workgroup's decision, so once all are
    // written no workgroup of the request reads the partials any more.
    if (w != a.nc2 - 1) return;
    // The diagnostics need only the merged rows, so they go out before the wait
    // (in the one-launch verify the decision workgroup writes them).
    if (!FUSED && (a.d_lse || a.d_p || a.d_q || a.d_r)) write_diag<ES>(a, b, ok, d.n, sh);
    // In the one-launch verify the token waits also for the decision
    // workgroup's check of every read row (word 2 of the record): on a data
    // error that workgroup writes the error outputs instead.
    double polled[2];
    bool fin_ok = true;
    const bool all = wait_masses(a, b, polled, FUSED ? decision(a, b) + 2 : nullptr, fin_ok, sh);
    if (ok && all && fin_ok) final_select<ES, ALZ, ALQ, DL>(a, b, d, zrow, qrow, polled, sh);
    else if (ok && !all) write_error(a, b);      // an expired wait
    // Every read of the mass words and of the record came before a barrier
    // of the wait or of the select.
    for (int i = threadIdx.x; i < 2 * a.nsub; i += kWG) st_coherent(mass + i, 0ull);
    if constexpr (FUSED) {
        // every request workgroup has read the record before writing its
        // masses, and word 2 is the decision workgroup's last write to it
        if (threadIdx.x < 3) st_coherent(decision(a, b) + threadIdx.x, 0ull);
        return;
    }
    uint64_t *part = partials(a, b);
    for (int i = threadIdx.x; i < (d.n + 1) * a.np1; i += kWG) part[i] = 0ull;
    if (DL) {
        uint64_t *pd = partials_d(a, b);
        for (int i = threadIdx.x; i < d.n * a.np1; i += kWG) pd[i] = 0ull;
    }
    uint64_t *gx = gathered(a, b);
    for (int i = threadIdx.x; i < d.n; i += kWG) gx[i] = 0ull;
}

// One workgroup per request (T == 0), after the request's row waves: waits
// for every read row, emits the argmax match, and zeroes the partials.
__device__ void request_item_greedy(const VerifyArgs &a, int b, Smem &sh) {
    const int G = a.G, G1 = G + 1;
    const int n = verify_len(a, b);
    if (n < 0 || n > G) { write_error(a, b); return; }
    const int k = threadIdx.x;
    int xk = 0;
    if (k < n) xk = a.x[size_t(b) * G + k];
    // Every lane polls its partials directly (a batch per attempt): request
    // workgroups are dispatched after the last row workgroup, so this polling
    // overlaps only the row pass's final workgroups, and the last partial is
    // seen one round trip earlier than behind a one-lane wait on it.
    bool bad = merge_rows_greedy(a, b, n, sh) != 0;
    bad |= k < n && (xk < 0 || xk >= a.V);
    if (wg_any(bad, 1, sh)) {
        write_error(a, b);
    } else if (G1 <= 64) {
        // every draft and output position lies in wave 0: the first mismatch
        // by one ballot, with no further barrier
        if (threadIdx.x < 64) {
            const uint64_t mm = __ballot(k < n && xk != sh.A[k]);
            const int j = mm ? __builtin_ctzll(mm) : n;
            if (k < G1) a.out_tok[size_t(b) * G1 + k] = (k < j) ? xk : (k == j) ? sh.A[j] : -1;
            if (k == 0) a.out_acc[b] = j;
        }
    } else {
        post_first(k < n && xk != sh.A[k], 0, sh);
        __syncthreads();
        const int jf = wg_first(0, sh);
        const int j = (jf == INT_MAX) ? n : jf;
        for (int t = threadIdx.x; t < G1; t += kWG) {
            int v = -1;
            if (t < j) v = a.x[size_t(b) * G + t];
            else if (t == j) v = sh.A[j];
            a.out_tok[size_t(b) * G1 + t] = v;
        }
        if (threadIdx.x == 0) a.out_acc[b] = j;
    }
    // Every lane finished reading the partials before wg_any's barrier.
    uint64_t *pw = partials(a, b);
    for (int i = threadIdx.x; i < (n + 1) * a.np1; i += kWG) st_coherent(pw + i, 0ull);
}

// ------------------------------------------------------------- kernels

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6); }

// Row group (request b, row k <= n, group g of kWaves consecutive chunks) of
// a sampled verify, one wave per chunk.  The group's partial merges its
// waves' (max, sum) pairs in wave order, so the request pass reads a quarter
// as many partials.
// With `published` (the one-launch verify) the partial and the gather are
// stored coherently, for request workgroups of the same launch that poll them.
template <int ES, bool AL>
__device__ __forceinline__ void row_group_sampled(const VerifyArgs &a, int b, int k, int g, int n, bool draft,
                                                  float *gm, float *gs, long trow = -1, bool published = false) {
    const int w = wave_id(), lane = int(threadIdx.x) & 63;
    const int c = g * kWaves + w;
    float M = neg_inf(), S = 0.0f;
    if (c < a.nc1) row_chunk_sampled<ES, AL>(a, b, k, c, n, draft, lane, M, S, trow, published);
    if (lane == 0) {
        gm[w] = M;
        gs[w] = S;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const float m = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
        float t = 0.0f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) t = t + gs[v] * rescale(gm[v], m, a.c32);
        uint64_t *dst = (draft ? partials_d(a, b) : partials(a, b)) + size_t(k) * a.np1 + g;
        const uint64_t word = uint64_t(__float_as_uint(m)) | (uint64_t(__float_as_uint(t) | kValid) << 32);
        if (published) st_coherent(dst, word);
        else *dst = word;
    }
}

// Row pass of a sampled verify: one workgroup per (request, row, group).
template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_rows_sampled(VerifyArgs a) {
    __shared__ float gm[kWaves], gs[kWaves];
    // Rows of a request: target rows 0..G, then (draft logits) draft rows 0..G-1.
    const int per = ((a.G + 1) + (a.dl ? a.G : 0)) * a.np1;
    const int i = blockIdx.x;
    // With B a multiple of 8, workgroup i (on XCD i mod 8) serves request
    // ((i / 8) / per) * 8 + i mod 8: each XCD streams whole requests, a
    // contiguous block of rows (faster than interleaving every request's row
    // groups over all eight XCDs).
    int b, rem;
    if ((a.B & 7) == 0) {
        const int x = i & 7, j = i >> 3;
        b = (j / per) * 8 + x;
        rem = j - (j / per) * per;
    } else {
        b = i / per;
        rem = i - b * per;
    }
    const int rr = rem / a.np1, g = rem - rr * a.np1;
    const bool draft = rr > a.G;
    const int k = draft ? rr - a.G - 1 : rr;
    const int n = verify_len(a, b);
    if (n < 0 || n > a.G || (draft ? k >= n : k > n)) return;   // row not read: the whole workgroup leaves
    row_group_sampled<ES, AL>(a, b, k, g, n, draft, gm, gs);
}

// Row pass with verify lengths and at most kWG requests, where most rows may
// be unread: a grid sized to the device whose workgroups visit only the read
// row groups.  Each workgroup first forms, in LDS, the prefix over requests of
// their read row groups ((n_b + 1) * np1; none for an invalid length), then
// takes jobs first, first + nwg, ... of that list (first = its index among the
// nwg row workgroups) and finds each job's request by binary search.
// `published` as for row_group_sampled (the one-launch verify).
struct VlSmem {
    float gm[kWaves], gs[kWaves];
    int off[kWG + 1];
    int wtot[kWaves];
    int nlen[kWG], row0[kWG];                 // each request's length and first target row
};
template <int ES, bool AL>
__device__ void rows_vl(const VerifyArgs &a, int first, int nwg, bool published, VlSmem &v) {
    const int t = int(threadIdx.x), lane = t & 63, w = wave_id();
    int cnt = 0;
    if (t < a.B) {
        const int n = verify_len(a, t);
        cnt = (n >= 0 && n <= a.G) ? ((n + 1) + (a.dl ? n : 0)) * a.np1 : 0;   // target rows, then draft rows
        v.nlen[t] = n;
        v.row0[t] = a.roff ? ld_const(a.roff, t) : t * (a.G + 1);
    }
    const int x = wave_scan_i(cnt);
    if (lane == 63) v.wtot[w] = x;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        base += (q < w) ? v.wtot[q] : 0;
        total += v.wtot[q];
    }
    v.off[t] = base + x - cnt;                        // exclusive: first job of request t
    if (t == 0) v.off[kWG] = total;
    __syncthreads();
    for (int job = first; job < total; job += nwg) {
        int lo = 0, hi = a.B - 1;                     // the last request whose first job is <= job
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (v.off[mid] <= job) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo, local = job - v.off[b];
        const int n = v.nlen[b];
        const int rr = local / a.np1, g = local - rr * a.np1;
        const bool draft = rr > n;
        const int k = draft ? rr - n - 1 : rr;
        row_group_sampled<ES, AL>(a, b, k, g, n, draft, v.gm, v.gs, long(v.row0[b]) + k, published);
        __syncthreads();                              // gm / gs are reused by the next job
    }
}
template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_rows_sampled_vl(VerifyArgs a) {
    __shared__ VlSmem v;
    rows_vl<ES, AL>(a, int(blockIdx.x), int(gridDim.x), false, v);
}

// Request pass of a sampled verify: nc2 workgroups per request.
template <int ES, bool ALZ, bool ALQ, bool DL>
// Draft logits need more registers (the draft normalisers and the logit
// conversion); 4 waves per SIMD still hold 1024 draw workgroups at once.
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(DL ? 4 : 8, DL ? 4 : 8))) void k_requests_sampled(VerifyArgs a) {
    __shared__ Smem sh;
    // With B a multiple of the XCD count, workgroup i (placed on XCD i mod 8)
    // serves request ((i / 8) / nc2) * 8 + i mod 8: a request's workgroups
    // share one XCD and its L2, in increasing grid order.
    const int i = int(blockIdx.x);
    int b, w;
    if ((a.B & 7) == 0) {
        const int x = i & 7, j = i >> 3;
        b = (j / a.nc2) * 8 + x;
        w = j - (j / a.nc2) * a.nc2;
    } else {
        b = i / a.nc2;
        w = i - b * a.nc2;
    }
    request_item_sampled<ES, ALZ, ALQ, DL>(a, b, w, sh);
}

// One-launch sampled verify (draft probabilities).  Three kinds of workgroup
// share one grid:
//   rows(b)    request b's row workgroups (k_rows_sampled's, with partials and
//              gathers published coherently, each word with its written bit);
//   dec(b)     one decision workgroup (decide_publish): polls rows(b)'s words,
//              publishes a decision record once rows 0..j settle it, then,
//              with every row in, the error check and the accepted prefix;
//   draws(b)   request b's nc2 request workgroups (k_requests_sampled's),
//              which poll the record instead of the partials, stream the draw
//              row and select the token.
// Every wait is on workgroups earlier in grid order that never wait on later
// ones (dec(b) on rows(b), draws(b) on dec(b) and, for the last of them, on
// draws(b)'s earlier ones), so the launch completes whatever the device holds
// at once.
//
// Grid order.  With B a multiple of 8, workgroup i runs on XCD x = i mod 8 and
// is the (i / 8)-th of that XCD's sequence, which serves requests b = 8t + x,
// t = 0..R-1 (R = B / 8):
//   rows(0) .. rows(lag-1), then rows(t) followed by dec(t - lag) for
//   t = lag..R-1, then dec(R-lag) .. dec(R-1), then draws(0) .. draws(R-1).
// A request is decided while the XCD streams the next request's rows, so when
// the request workgroups are dispatched (after every row workgroup) all but
// the last requests' records are ready and their draw streams start at once,
// filling the row pass's drain.  Otherwise: every rows(b), then every dec(b),
// then every draws(b).
//
// VL (verify lengths or packed rows, at most kWG requests): the first a.vlrows
// workgroups are k_rows_sampled_vl's (visiting only the read row groups),
// then one decision workgroup per request, then the request workgroups.
template <int ES, bool ALZ, bool ALQ, bool VL>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_verify_sampled(VerifyArgs a) {
    __shared__ Smem sh;
    __shared__ float gm[kWaves], gs[kWaves];
    const int per = (a.G + 1) * a.np1, nc2 = a.nc2;
    const int i = int(blockIdx.x);
    if constexpr (VL) {
        __shared__ VlSmem v;
        if (i < a.vlrows) {
            rows_vl<ES, ALZ>(a, i, a.vlrows, /*published=*/true, v);
        } else if (i < a.vlrows + a.B) {
            decide_publish<ES>(a, i - a.vlrows, sh);
        } else {
            // with vlrows and B multiples of 8, request b's workgroups share an XCD
            const int j = i - a.vlrows - a.B;
            int b, w;
            if ((a.B & 7) == 0 && (a.vlrows & 7) == 0) {
                const int x = j & 7, jj = j >> 3;
                b = (jj / nc2) * 8 + x;
                w = jj - (jj / nc2) * nc2;
            } else {
                b = j / nc2;
                w = j - b * nc2;
            }
            request_item_sampled<ES, ALZ, ALQ, false, true>(a, b, w, sh);
        }
        return;
    }
    int kind, b, loc;                                 // kind: 0 rows, 1 decision, 2 draws
    if ((a.B & 7) == 0) {
        const int x = i & 7;
        int s = i >> 3;
        const int R = a.B >> 3, L = min(a.lag, R);
        int t;
        if (s < L * per) {                            // rows(0) .. rows(L-1)
            t = s / per;
            kind = 0;
            loc = s - t * per;
        } else if ((s -= L * per) < (R - L) * (per + 1)) {   // rows(t), dec(t - L)
            const int q = s / (per + 1), o = s - q * (per + 1);
            kind = (o < per) ? 0 : 1;
            t = (o < per) ? L + q : q;
            loc = o;
        } else if ((s -= (R - L) * (per + 1)) < L) {  // dec(R-L) .. dec(R-1)
            kind = 1;
            t = R - L + s;
            loc = 0;
        } else {                                      // draws(0) .. draws(R-1)
            s -= L;
            kind = 2;
            t = s / nc2;
            loc = s - t * nc2;
        }
        b = 8 * t + x;
    } else {
        const int groups = a.B * per;
        if (i < groups) {
            kind = 0;
            b = i / per;
            loc = i - b * per;
        } else if (i < groups + a.B) {
            kind = 1;
            b = i - groups;
            loc = 0;
        } else {
            const int j = i - groups - a.B;
            kind = 2;
            b = j / nc2;
            loc = j - b * nc2;
        }
    }
    if (kind == 0) {
        const int k = loc / a.np1, g = loc - k * a.np1;
        const int n = verify_len(a, b);
        if (n < 0 || n > a.G || k > n) return;        // row not read: the whole workgroup leaves
        row_group_sampled<ES, ALZ>(a, b, k, g, n, false, gm, gs, -1, /*published=*/true);
    } else if (kind == 1) {
        decide_publish<ES>(a, b, sh);
    } else {
        request_item_sampled<ES, ALZ, ALQ, false, true>(a, b, loc, sh);
    }
}

// Greedy row workgroup gi: (request b, row k, group g of kWaves consecutive
// chunks), one wave per chunk.  The group's partial is the largest of the
// waves' maxima with the lowest index holding it (waves in chunk order, so the
// first wave to reach the maximum holds the lowest index), and whether any
// wave saw a NaN.  Stored coherently: the request items of the same launch
// read it.
template <int ES, bool AL>
__device__ void row_group_greedy(const VerifyArgs &a, int gi, Smem &sh) {
    const int per = (a.G + 1) * a.np1;
    // Request-per-XCD placement as in the sampled row pass (B a multiple of 8).
    int b, rem;
    if ((a.B & 7) == 0) {
        const int x = gi & 7, j = gi >> 3;
        b = (j / per) * 8 + x;
        rem = j - (j / per) * per;
    } else {
        b = gi / per;
        rem = gi - b * per;
    }
    const int k = rem / a.np1, g = rem - k * a.np1;
    const int n = verify_len(a, b);
    if (n < 0 || n > a.G || k > n) return;           // row not read: the whole workgroup leaves
    const int w = wave_id(), lane = int(threadIdx.x) & 63;
    const int c = g * kWaves + w;
    float M = neg_inf();
    int idx = -1;
    bool nan = false;
    if (c < a.nc1) row_chunk_greedy<ES, AL>(a, b, k, c, lane, M, idx, nan);
    if (lane == 0) {
        sh.gm[w] = M;
        sh.gi[w] = idx;
        sh.gn[w] = int(nan);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = neg_inf();
        int bi = -1, any_nan = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            any_nan |= sh.gn[v];
            if (sh.gi[v] >= 0 && (bi < 0 || sh.gm[v] > m)) {
                m = sh.gm[v];
                bi = sh.gi[v];
            }
        }
        st_coherent(partials(a, b) + size_t(k) * a.np1 + g,
                    uint64_t(__float_as_uint(m)) | (uint64_t(uint32_t((any_nan ? kNanIdx : bi) + 2) | kValid) << 32));
    }
}

// Greedy verify: row workgroups (request-major), then one request workgroup
// per request (mode 0); or only the row workgroups (mode 1) / request
// workgroups (mode 2).
template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_verify_greedy(VerifyArgs a) {
    __shared__ Smem sh;
    const int groups = a.B * (a.G + 1) * a.np1;
    const int i = blockIdx.x;
    if (a.mode == 2 || (a.mode == 0 && i >= groups)) request_item_greedy(a, a.mode == 2 ? i : i - groups, sh);
    else row_group_greedy<ES, AL>(a, i, sh);
}

// Merged argmax of rows 0..n into sh.A for the tree walk: four lanes per row
// (a row's partials interleaved over them, all loads issued together), so 64
// rows per pass.  POLL: the row workgroups of the same launch are still
// writing the partials, so each lane reloads those of its words not yet
// written until all are (a bounded wait; a word never written makes its row
// bad); otherwise they are complete (written by the previous launch).  No
// barrier inside; the caller synchronises.
template <bool POLL>
__device__ void merge_rows_greedy4(const VerifyArgs &a, int b, int n, Smem &sh) {
    constexpr int kR = 8;                  // partials per lane when np1 <= 32
    const uint64_t *part = partials(a, b);
    const int l = threadIdx.x & 3, g = threadIdx.x >> 2;
    const uint64_t empty = uint64_t(1) << 32 | uint64_t(kValid) << 32;   // (0.0, index -1), written
    for (int r0 = 0; r0 <= n; r0 += kWG / 4) {
        const int r = r0 + g;
        const bool live = r <= n;
        const uint64_t *pp = part + size_t(live ? r : 0) * a.np1;
        float best = neg_inf();
        int bi = -1, nan = 0, ok = 1;
        if (a.np1 <= 4 * kR) {
            uint64_t v[kR];
            if constexpr (POLL) {
#pragma unroll
                for (int i = 0; i < kR; ++i) v[i] = 0ull;
                for (uint32_t spins = 0;; ++spins) {
                    int all = 1;
#pragma unroll
                    for (int i = 0; i < kR; ++i) {
                        const int cc = l + 4 * i;
                        if (!valid(v[i])) v[i] = (live && cc < a.np1) ? ld_coherent(pp + cc) : empty;
                        all &= int(valid(v[i]));
                    }
                    if (all || spins >= a.spin_limit) break;
                }
            } else {
#pragma unroll
                for (int i = 0; i < kR; ++i) {
                    const int cc = l + 4 * i;
                    v[i] = (live && cc < a.np1) ? pp[cc] : empty;
                }
            }
#pragma unroll
            for (int i = 0; i < kR; ++i) {
                ok &= int(valid(v[i]));
                const int vi = int(hi_u(v[i]) & ~kValid) - 2;
                if (vi == kNanIdx) nan = 1;
                else merge_am(best, bi, lo_f(v[i]), vi);
            }
        } else if (live) {
            for (int cc = l; cc < a.np1; cc += 4) {
                uint64_t v = POLL ? ld_coherent(pp + cc) : pp[cc];
                if constexpr (POLL) {
                    for (uint32_t spins = 0; !valid(v) && spins < a.spin_limit; ++spins) v = ld_coherent(pp + cc);
                }
                ok &= int(valid(v));
                const int vi = int(hi_u(v) & ~kValid) - 2;
                if (vi == kNanIdx) nan = 1;
                else merge_am(best, bi, lo_f(v), vi);
            }
        }
        am_step<kXor1>(best, bi, nan);
        am_step<kXor2>(best, bi, nan);
        ok = ok & dpp_i<kXor1>(ok);
        ok = ok & dpp_i<kXor2>(ok);
        if (l == 0 && live) {
            const bool rb = !ok || nan || bi < 0 || best == __builtin_inff();
            sh.A[r] = rb ? kBadRowArgmax : bi;
        }
    }
}

// Greedy tree walk ("breaking down dspark and its lineage", section "Tree
// attention"): one workgroup per request, after the greedy row pass over its
// G + 1 node rows.  Every row's argmax is merged; each node that carries its
// parent's argmax offers itself to the parent (LDS minimum: the lowest such
// child); the walk from the root is then a pointer chase in LDS.  A visited
// bad row, a parent outside [0, i) or a token outside [0, V) is a data error.
// POLL: the row workgroups of the same launch (earlier in grid order) are
// still writing the partials.
struct TreeSmem {
    int match[kWG];
    int emit[kWG + 1], path[kWG];
    int acc_n;
};
template <bool POLL>
__device__ void tree_walk_item(const VerifyArgs &a, int b, Smem &sh, TreeSmem &ts) {
    const int t = int(threadIdx.x), M = a.G + 1;
    const int32_t *par = a.tpar + size_t(b) * M, *tok = a.ttok + size_t(b) * M;
    bool bad = false;
    int p = 0, tk = 0;
    if (t < M) {
        ts.match[t] = INT_MAX;
        if (t >= 1) {
            p = par[t];
            tk = tok[t];
            bad = !(p >= 0 && p < t) || !(tk >= 0 && tk < a.V);
        }
    }
    merge_rows_greedy4<POLL>(a, b, a.G, sh);
    bad = __syncthreads_or(bad);
    if (!bad && t >= 1 && t < M && tk == sh.A[p]) atomicMin(&ts.match[p], t);
    __syncthreads();
    if (t == 0) {
        int n = -1;
        if (!bad) {
            int cur = 0;
            n = 0;
            for (;;) {
                const int am = sh.A[cur];
                if (am < 0) {                             // a visited bad row
                    n = -1;
                    break;
                }
                ts.emit[n] = am;
                const int nx = ts.match[cur];
                if (nx == INT_MAX) break;
                ts.path[n++] = nx;
                cur = nx;
            }
        }
        ts.acc_n = n;
    }
    __syncthreads();
    const int n = ts.acc_n;
    for (int i = t; i < M; i += kWG) {
        a.out_tok[size_t(b) * M + i] = (n >= 0 && i <= n) ? ts.emit[i] : -1;
        a.out_path[size_t(b) * M + i] = (n >= 0 && i < n) ? ts.path[i] : -1;
    }
    if (t == 0) a.out_acc[b] = n;
    uint64_t *pw = partials(a, b);
    for (int i = t; i < M * a.np1; i += kWG) st_coherent(pw + i, 0ull);
}

// The walk after a separate row launch: one workgroup per request.
__global__ __launch_bounds__(kWG) void k_tree_walk(VerifyArgs a) {
    __shared__ Smem sh;
    __shared__ TreeSmem ts;
    tree_walk_item<false>(a, int(blockIdx.x), sh, ts);
}

// Tree verification in one launch: the greedy row workgroups over every node
// row (row_group_greedy's placement), then one walk workgroup per request,
// which polls its rows' partials (every wait is on workgroups earlier in grid
// order; the host keeps the walk workgroups below half the resident capacity).
template <int ES, bool AL>
__global__ __launch_bounds__(kWG) void k_tree_fused(VerifyArgs a) {
    __shared__ Smem sh;
    __shared__ TreeSmem ts;
    const int groups = a.B * (a.G + 1) * a.np1;
    const int i = blockIdx.x;
    if (i >= groups) tree_walk_item<true>(a, i - groups, sh, ts);
    else row_group_greedy<ES, AL>(a, i, sh);
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

int launch_rows_sampled_vl(const VerifyArgs &a, bool az, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) {
        if (az) hipLaunchKernelGGL((k_rows_sampled_vl<2, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_rows_sampled_vl<2, false>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az) hipLaunchKernelGGL((k_rows_sampled_vl<4, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_rows_sampled_vl<4, false>), dim3(grid), dim3(kWG), 0, st, a);
    }
    return int(hipGetLastError());
}

template <bool DL>
void launch_requests_dl(const VerifyArgs &a, bool az, bool aq, int esize, int grid, hipStream_t st) {
    if (esize == 2) {
        if (az && aq) hipLaunchKernelGGL((k_requests_sampled<2, true, true, DL>), dim3(grid), dim3(kWG), 0, st, a);
        else if (az) hipLaunchKernelGGL((k_requests_sampled<2, true, false, DL>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_requests_sampled<2, false, false, DL>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az && aq) hipLaunchKernelGGL((k_requests_sampled<4, true, true, DL>), dim3(grid), dim3(kWG), 0, st, a);
        else if (az) hipLaunchKernelGGL((k_requests_sampled<4, true, false, DL>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_requests_sampled<4, false, false, DL>), dim3(grid), dim3(kWG), 0, st, a);
    }
}

int launch_requests_sampled(const VerifyArgs &a, bool az, bool aq, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.dl) launch_requests_dl<true>(a, az, aq, esize, grid, st);
    else launch_requests_dl<false>(a, az, aq, esize, grid, st);
    return int(hipGetLastError());
}

template <bool VL>
void launch_verify_sampled_t(const VerifyArgs &a, bool az, bool aq, int esize, int grid, hipStream_t st) {
    if (esize == 2) {
        if (az && aq) hipLaunchKernelGGL((k_verify_sampled<2, true, true, VL>), dim3(grid), dim3(kWG), 0, st, a);
        else if (az) hipLaunchKernelGGL((k_verify_sampled<2, true, false, VL>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_verify_sampled<2, false, false, VL>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az && aq) hipLaunchKernelGGL((k_verify_sampled<4, true, true, VL>), dim3(grid), dim3(kWG), 0, st, a);
        else if (az) hipLaunchKernelGGL((k_verify_sampled<4, true, false, VL>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_verify_sampled<4, false, false, VL>), dim3(grid), dim3(kWG), 0, st, a);
    }
}

int launch_verify_sampled(const VerifyArgs &a, bool az, bool aq, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.vlrows > 0) launch_verify_sampled_t<true>(a, az, aq, esize, grid, st);
    else launch_verify_sampled_t<false>(a, az, aq, esize, grid, st);
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

int launch_tree_fused(const VerifyArgs &a, bool az, int esize, int grid, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esize == 2) {
        if (az) hipLaunchKernelGGL((k_tree_fused<2, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_tree_fused<2, false>), dim3(grid), dim3(kWG), 0, st, a);
    } else {
        if (az) hipLaunchKernelGGL((k_tree_fused<4, true>), dim3(grid), dim3(kWG), 0, st, a);
        else hipLaunchKernelGGL((k_tree_fused<4, false>), dim3(grid), dim3(kWG), 0, st, a);
    }
    return int(hipGetLastError());
}

int launch_tree_walk(const VerifyArgs &a, int grid, void *stream) {
    hipLaunchKernelGGL(k_tree_walk, dim3(grid), dim3(kWG), 0, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

int greedy_occupancy(bool az, int esize, int *n) {
    if (esize == 2) return az ? occ(k_verify_greedy<2, true>, n) : occ(k_verify_greedy<2, false>, n);
    return az ? occ(k_verify_greedy<4, true>, n) : occ(k_verify_greedy<4, false>, n);
}

}  // namespace sv
