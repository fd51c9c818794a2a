// Per-position acceptance overlap on CDNA4 (gfx950).
//
// What is computed ("AngelSpec", section 2, Eq. 2, 4 and 5; "UraionSpec", the
// confidence head's target c* = 1 - TV): for every tested draft position
// (b, k < n_b), alpha_k = sum_v min(p_k(v), q_k(v)) with p_k = softmax(z_k / T)
// and q_k the draft distribution (given, or softmax(d_k / T) of draft logits).
// alpha is the expected acceptance probability of the position, 1 - TV(p, q).
//
// One workgroup of 512 threads per position, two 16-byte loads in flight per
// row per thread.  At B = 64, gamma = 15, V = 129280 (draft logits) this shape
// left the most of each row pair cached for its second read:
//   256 threads: 188 us with two loads in flight, 185 us with four;
//   512 threads: 155.5 us with two, 155.6 us with one, 185.5 us with four;
//   1024 threads: 198 us with two, 202 us with one.
// The exact overlap needs both rows' normalisers before any min(p, q), so the
// workgroup reads its row pair twice:
//   pass 1  per thread an online (max, sum of 2^((z - m) log2(e)/T)) over
//           16-byte loads (eight elements per load, two loads in flight per
//           row), merged across the wave with DPP and across the eight waves in
//           LDS; the draft row too in draft-logits mode.  These loads are
//           ordinary (cache-allocating) ones, so part of the row pair is still
//           cached when pass 2 reads it (7.7% faster than streaming loads at
//           B = 64, gamma = 15, V = 129280 with draft logits);
//   pass 2  sum of min(p, q) per thread (fp32 per eight elements, fp64 across
//           them), then a DPP and LDS sum in fp64; each term's exponent is
//           fma(z, c, -fl(m c)) - log2 S, and with draft logits a term is
//           2^min(a, b), one v_exp_f32.  The row pair is not read again, so
//           these loads are nontemporal.
// Both passes are bound by the two reads of the row pair once the terms cost
// two instructions each.
// A row holding a NaN, whose maximum is +inf, or which is entirely -inf gives
// NaN, as does every untested position.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"
#include "sv_wave.h"

namespace sv {
namespace {

constexpr int kAT = 512;                 // threads per workgroup
constexpr int kAW = kAT / 64;            // waves
constexpr int kAE = 8;                   // elements per thread per load
constexpr int kAU = 2;                   // loads in flight per row per thread
constexpr int kAStep = kAT * kAE;        // elements per workgroup step (4096)

__device__ __forceinline__ float ninf() { return -__builtin_inff(); }
__device__ __forceinline__ float exp2n(float x) { return __builtin_amdgcn_exp2f(x); }   // v_exp_f32
__device__ __forceinline__ bool fin(float x) { return __builtin_isfinite(x); }

typedef uint32_t au32x4 __attribute__((ext_vector_type(4)));
// A 16-byte load for data read for the last time (nontemporal).
__device__ __forceinline__ uint4 ld_once(const uint4 *p) {
    const au32x4 v = __builtin_nontemporal_load(reinterpret_cast<const au32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int ES> __device__ __forceinline__ float elem(const void *row, size_t i) {
    if constexpr (ES == 2) {
        const uint16_t h = static_cast<const uint16_t *>(row)[i];
        return __uint_as_float(uint32_t(h) << 16);
    } else {
        return static_cast<const float *>(row)[i];
    }
}

// Eight consecutive elements e0 .. e0+7 of a row (positions >= V read as
// `fill`).  Aligned rows take one (bf16) or two (fp32) 16-byte loads,
// nontemporal (NT) or ordinary.
template <bool NT> __device__ __forceinline__ uint4 ld16(const uint4 *p) { return NT ? ld_once(p) : *p; }
template <int ES, bool AL, bool NT>
__device__ __forceinline__ void load8(const void *row, int e0, int V, float fill, float (&f)[kAE]) {
    if (AL && e0 + kAE <= V) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const char *>(row) + size_t(e0) * ES);
        if constexpr (ES == 2) {
            const uint4 w = ld16<NT>(p);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[2 * i] = __uint_as_float(u[i] << 16);
                f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
            }
        } else {
            const uint4 w0 = ld16<NT>(p), w1 = ld16<NT>(p + 1);
            f[0] = __uint_as_float(w0.x); f[1] = __uint_as_float(w0.y);
            f[2] = __uint_as_float(w0.z); f[3] = __uint_as_float(w0.w);
            f[4] = __uint_as_float(w1.x); f[5] = __uint_as_float(w1.y);
            f[6] = __uint_as_float(w1.z); f[7] = __uint_as_float(w1.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kAE; ++i) f[i] = (e0 + i < V) ? elem<ES>(row, size_t(e0 + i)) : fill;
    }
}

// (max, sum) pair: sum of 2^((x - m) c) over the elements seen.
struct MS {
    float m, s;
    bool nan;
};
// s, a sum taken against reference m_from, rescaled to reference m_to >=
// m_from.  Sums use the rounded reference R = fl(m c) (see ms_add8), so the
// factor is 2^(fl(m_from c) - fl(m_to c)) (an exact difference of the two
// references), which makes the references' rounding cancel; where m c
// overflows, 2^((m_from - m_to) c).
__device__ __forceinline__ float rescale(float s, float m_from, float m_to, float c) {
    if (m_from == ninf()) return 0.0f;
    const float r_from = m_from * c, r_to = m_to * c;
    return s * ((fin(r_from) && fin(r_to)) ? exp2n(r_from - r_to) : exp2n((m_from - m_to) * c));
}
__device__ __forceinline__ void ms_add8(MS &a, const float (&f)[kAE], float c) {
    float cm = f[0];
    bool nan = f[0] != f[0];
#pragma unroll
    for (int i = 1; i < kAE; ++i) {
        cm = fmaxf(cm, f[i]);               // drops NaN
        nan |= f[i] != f[i];
    }
    a.nan |= nan;
    if (cm > a.m) {
        a.s = rescale(a.s, a.m, cm, c);
        a.m = cm;
    }
    // Terms 2^(fma(x, c, -R)) with R = fl(m c) (as the verify row pass), or
    // 2^((x - m) c) where m c overflows; -inf elements give 0 either way.
    if (fin(a.m)) {
        const float R = a.m * c;
        float t = 0.0f;
        if (fin(R)) {
#pragma unroll
            for (int i = 0; i < kAE; ++i) t = t + exp2n(__builtin_fmaf(f[i], c, -R));
        } else {
#pragma unroll
            for (int i = 0; i < kAE; ++i) t = t + exp2n((f[i] - a.m) * c);
        }
        a.s = a.s + t;
    }
}
__device__ __forceinline__ void ms_merge(MS &a, float m2, float s2, bool nan2, float c) {
    const float m = fmaxf(a.m, m2);
    a.s = rescale(a.s, a.m, m, c) + rescale(s2, m2, m, c);
    a.m = m;
    a.nan |= nan2;
}

template <int C> __device__ __forceinline__ void ms_dpp(MS &a, float c) {
    const float m2 = dpp_f<C>(a.m), s2 = dpp_f<C>(a.s);
    const int n2 = dpp_i<C>(int(a.nan));
    ms_merge(a, m2, s2, n2 != 0, c);
}

struct ASmem {
    float m[kAW][2], s[kAW][2];
    int nan[kAW][2];
    double acc[kAW];
};

// Whole-workgroup (max, sum) of up to two rows; every thread gets the result.
// (DPP steps combine a lane with a partner in its row of 16 through a
// commutative merge, so all 16 lanes agree; rows then merge in lane order.)
__device__ void ms_block(MS (&v)[2], int nrow, float c, ASmem &sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int r = 0; r < nrow; ++r) {
        MS a = v[r];
        ms_dpp<kXor1>(a, c);
        ms_dpp<kXor2>(a, c);
        ms_dpp<kHalfMirror>(a, c);
        ms_dpp<kMirror>(a, c);
        MS t = {lane_f(a.m, 0), lane_f(a.s, 0), lane_i(int(a.nan), 0) != 0};
#pragma unroll
        for (int l = 16; l < 64; l += 16) ms_merge(t, lane_f(a.m, l), lane_f(a.s, l), lane_i(int(a.nan), l) != 0, c);
        if (lane == 0) {
            sh.m[w][r] = t.m;
            sh.s[w][r] = t.s;
            sh.nan[w][r] = int(t.nan);
        }
    }
    __syncthreads();
    for (int r = 0; r < nrow; ++r) {
        MS t = {sh.m[0][r], sh.s[0][r], sh.nan[0][r] != 0};
#pragma unroll
        for (int q = 1; q < kAW; ++q) ms_merge(t, sh.m[q][r], sh.s[q][r], sh.nan[q][r] != 0, c);
        v[r] = t;
    }
}

// Pass 2 over the row pair: sum of min(p, q) per thread.  The exponent of p
// is a = fma(z, c, -fl(mp c)) - log2 Sp: the reference is subtracted before
// log2 Sp, so the exponent's rounding is relative to |a| (small for the terms
// that carry the mass), not to |mp c|.  With draft logits b is formed the same
// way and min(p, q) = 2^min(a, b) (2^x is monotone), one exp per term.  Where
// m c overflows (a tiny T), a = (z - mp) c - log2 Sp (FAST false).
template <int ES, bool AL, bool QL, bool FAST>
__device__ double overlap_rows(const void *zrow, const void *drow, int V, int t, float c, float mp, float lsp,
                               float mq, float lsq) {
    const float Rp = mp * c, Rq = mq * c;
    double acc = 0.0;
    for (int base = 0; base < V; base += kAStep * kAU) {
        float fz[kAU][kAE], fd[kAU][kAE];
#pragma unroll
        for (int u = 0; u < kAU; ++u) {
            const int e0 = base + u * kAStep + t * kAE;
            load8<ES, AL, true>(zrow, e0, V, ninf(), fz[u]);
            if constexpr (QL) load8<ES, AL, true>(drow, e0, V, ninf(), fd[u]);
            else load8<4, AL, true>(drow, e0, V, 0.0f, fd[u]);
        }
#pragma unroll
        for (int u = 0; u < kAU; ++u) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < kAE; ++i) {
                const float ea = (FAST ? __builtin_fmaf(fz[u][i], c, -Rp) : (fz[u][i] - mp) * c) - lsp;
                if constexpr (QL) {
                    const float eb = (FAST ? __builtin_fmaf(fd[u][i], c, -Rq) : (fd[u][i] - mq) * c) - lsq;
                    s = s + exp2n(fminf(ea, eb));
                } else {
                    s = s + fminf(exp2n(ea), fd[u][i]);
                }
            }
            acc = acc + double(s);
        }
    }
    return acc;
}

// QL: draft logits (of the target's element size) instead of probabilities.
template <int ES, bool AL, bool QL>
__global__ __launch_bounds__(kAT) void k_acceptance(AcceptArgs a) {
    __shared__ ASmem sh;
    // With B * G a multiple of 8, the workgroups on XCD x (= blockIdx mod 8)
    // take the x-th eighth of the positions: contiguous row pairs per XCD.
    const int npos = a.B * a.G;
    int pos = int(blockIdx.x);
    if ((npos & 7) == 0) pos = (pos & 7) * (npos >> 3) + (pos >> 3);
    const int b = pos / a.G, k = pos - b * a.G;
    const int n = a.vlen ? a.vlen[b] : a.G;
    float *out = a.out + size_t(b) * a.G + k;
    if (n < 0 || n > a.G || k >= n) {
        if (threadIdx.x == 0) *out = __builtin_nanf("");
        return;
    }
    const int V = a.V, t = threadIdx.x;
    const float c = a.c32;
    const void *zrow = static_cast<const char *>(a.z) + (size_t(b) * (a.G + 1) + k) * size_t(V) * ES;
    const size_t drow_elem = (size_t(b) * a.G + k) * size_t(V);
    const void *drow = QL ? static_cast<const void *>(static_cast<const char *>(a.d) + drow_elem * ES)
                          : static_cast<const void *>(static_cast<const float *>(a.d) + drow_elem);

    // Pass 1: normalisers.
    MS v[2] = {{ninf(), 0.0f, false}, {ninf(), 0.0f, false}};
    for (int base = 0; base < V; base += kAStep * kAU) {
        float fz[kAU][kAE], fd[kAU][kAE];
#pragma unroll
        for (int u = 0; u < kAU; ++u) {
            const int e0 = base + u * kAStep + t * kAE;
            load8<ES, AL, false>(zrow, e0, V, ninf(), fz[u]);
            if constexpr (QL) load8<ES, AL, false>(drow, e0, V, ninf(), fd[u]);
        }
#pragma unroll
        for (int u = 0; u < kAU; ++u) {
            ms_add8(v[0], fz[u], c);
            if constexpr (QL) ms_add8(v[1], fd[u], c);
        }
    }
    ms_block(v, QL ? 2 : 1, c, sh);
    bool bad = false;
#pragma unroll
    for (int r = 0; r < (QL ? 2 : 1); ++r) bad |= v[r].nan || v[r].m == ninf() || v[r].m == __builtin_inff();
    if (bad) {
        if (t == 0) *out = __builtin_nanf("");
        return;
    }
    // log2 of the sums, correctly rounded (once per workgroup)
    const float mp = v[0].m, lsp = float(log2(double(v[0].s)));
    const float mq = QL ? v[1].m : 0.0f, lsq = QL ? float(log2(double(v[1].s))) : 0.0f;

    // Pass 2: sum of min(p, q).
    const bool fast = fin(mp * c) && (!QL || fin(mq * c));
    double acc = fast ? overlap_rows<ES, AL, QL, true>(zrow, drow, V, t, c, mp, lsp, mq, lsq)
                      : overlap_rows<ES, AL, QL, false>(zrow, drow, V, t, c, mp, lsp, mq, lsq);
    acc = wave_sum_d(acc);
    if ((t & 63) == 0) sh.acc[t >> 6] = acc;
    __syncthreads();
    if (t == 0) {
        double tot = 0.0;
#pragma unroll
        for (int q = 0; q < kAW; ++q) tot = tot + sh.acc[q];
        *out = float(tot);
    }
}

}  // namespace

int launch_acceptance(const AcceptArgs &a, bool aligned, int esize, bool draft_logits, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(unsigned(a.B) * unsigned(a.G)), block(kAT);
    if (esize == 2) {
        if (draft_logits) {
            if (aligned) hipLaunchKernelGGL((k_acceptance<2, true, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_acceptance<2, false, true>), grid, block, 0, st, a);
        } else {
            if (aligned) hipLaunchKernelGGL((k_acceptance<2, true, false>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_acceptance<2, false, false>), grid, block, 0, st, a);
        }
    } else {
        if (draft_logits) {
            if (aligned) hipLaunchKernelGGL((k_acceptance<4, true, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_acceptance<4, false, true>), grid, block, 0, st, a);
        } else {
            if (aligned) hipLaunchKernelGGL((k_acceptance<4, true, false>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_acceptance<4, false, false>), grid, block, 0, st, a);
        }
    }
    return int(hipGetLastError());
}

}  // namespace sv
