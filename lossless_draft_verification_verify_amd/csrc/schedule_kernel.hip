// Confidence-scheduled verification depth on CDNA4 (gfx950): one workgroup.
//
// What is computed ("AngelSpec", section 4.2, Eq. 19-21 and the shallow-tie
// rule that follows them; "UraionSpec", section "Hardware-Aware Prefix
// Scheduler", Algorithm 1): survival s[b,k] = prod_{t<=k} c[b,t]; candidates
// with s > eps in the order (s desc, k asc, b asc); starting from one anchor per
// request, extend a request's prefix (contiguously) while the throughput
// tau / cost[T] strictly improves and T stays within the token budget.
//
// The result is bit-identical to the sequential float64 loop: the survival
// products and the running sum tau are formed in exactly that loop's order;
// only the independent parts (sorting, the theta comparisons, the length
// tally) run in parallel.
//
//   1. one thread per request: fp64 CumProd; detect whether survival is
//      non-increasing along the request (always true for c in [0, 1]);
//   2. bitonic sort of (s, k, b) keys in LDS, candidates first;
//   3. contiguity: a candidate can be kept only if all shallower positions of
//      its request are candidates placed before it (true for every candidate
//      when survival is non-increasing);
//   4. one wave forms tau_m = B + s_(0) + ... + s_(m-1) sequentially over the
//      kept-able candidates (at most budget - B of them can be kept);
//   5. all threads test theta_{m+1} > theta_m and T <= budget in parallel; the
//      first failure m* ends the scan; lengths are tallied from the first m*.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"

namespace sv {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kMaxCand = 4096;

struct SchedSmem {
    double key[kMaxCand];      // survival (sort key), then tau_m
    int id[kMaxCand];          // b * G + k, or INT_MAX for padding
    int pos[kMaxCand];         // sorted position of each candidate id (or -1)
    int len[kMaxCand];         // per request kept length (B <= kMaxCand)
    int nonincr, ncand, nvalid, mstar;
};

// Order: larger survival first; equal survival -> smaller k, then smaller b.
__device__ __forceinline__ bool before(double s1, int id1, double s2, int id2, int G, int B) {
    if (s1 != s2) return s1 > s2;
    if (id1 == id2) return false;
    if (id2 == 0x7fffffff) return true;
    if (id1 == 0x7fffffff) return false;
    const int k1 = id1 % G, k2 = id2 % G;
    if (k1 != k2) return k1 < k2;
    return id1 / G < id2 / G;
}

__global__ __launch_bounds__(kSchedThreads) void k_schedule(ScheduleArgs a) {
    __shared__ SchedSmem sh;
    const int tid = threadIdx.x;
    const int B = a.B, G = a.G, N = B * G;
    const double eps = double(a.eps);
    if (tid == 0) { sh.nonincr = 1; sh.ncand = 0; sh.mstar = 0x7fffffff; }
    __syncthreads();

    // 1. survival, sequential product per request.
    for (int b = tid; b < B; b += kSchedThreads) {
        double acc = 1.0, prev = 1.0;
        bool ok = true;
        for (int k = 0; k < G; ++k) {
            acc = acc * double(a.conf[size_t(b) * G + k]);
            if (k > 0 && !(acc <= prev)) ok = false;
            prev = acc;
            sh.key[b * G + k] = acc;
        }
        sh.len[b] = 0;
        if (!ok) atomicAnd(&sh.nonincr, 0);
    }
    __syncthreads();

    // 2. bitonic sort of candidates; non-candidates become -inf padding.
    int Np = 1;
    while (Np < N) Np <<= 1;
    for (int i = tid; i < Np; i += kSchedThreads) {
        if (i < N && sh.key[i] > eps) {
            sh.id[i] = i;
        } else {
            sh.key[i] = -__builtin_inf();
            sh.id[i] = 0x7fffffff;
        }
    }
    __syncthreads();
    for (int size = 2; size <= Np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < Np / 2; t += kSchedThreads) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool up = ((lo & size) == 0);         // this block sorts "before" first
                const double s1 = sh.key[lo], s2 = sh.key[hi];
                const int i1 = sh.id[lo], i2 = sh.id[hi];
                const bool swap = up ? before(s2, i2, s1, i1, G, B) : before(s1, i1, s2, i2, G, B);
                if (swap) { sh.key[lo] = s2; sh.key[hi] = s1; sh.id[lo] = i2; sh.id[hi] = i1; }
            }
            __syncthreads();
        }
    }

    // 3. candidates and contiguity.
    for (int i = tid; i < N; i += kSchedThreads) sh.pos[i] = -1;
    __syncthreads();
    for (int p = tid; p < Np; p += kSchedThreads) {
        const int id = sh.id[p];
        if (id != 0x7fffffff) { sh.pos[id] = p; atomicAdd(&sh.ncand, 1); }
    }
    __syncthreads();
    const int ncand = sh.ncand;
    if (!sh.nonincr) {
        for (int p = tid; p < ncand; p += kSchedThreads) {
            const int id = sh.id[p];
            const int b = id / G, k = id - b * G;
            bool valid = true;
            int prevp = -1;
            for (int kk = 0; kk <= k; ++kk) {
                const int pp = sh.pos[b * G + kk];
                if (pp < 0 || pp <= prevp) { valid = false; break; }
                prevp = pp;
            }
            if (!valid) sh.id[p] = -1 - id;           // keep order, mark as skipped
        }
        __syncthreads();
        // Compact the valid candidates in order (single wave, ordered).
        if (tid < 64) {
            int w = 0;
            for (int base = 0; base < ncand; base += 64) {
                const int p = base + tid;
                const bool v = (p < ncand) && sh.id[p] >= 0;
                const double kv = (p < ncand) ? sh.key[p] : 0.0;
                const int iv = (p < ncand) ? sh.id[p] : 0;
                const unsigned long long m = __ballot(v);
                const int off = __popcll(m & ((1ull << tid) - 1ull));
                // Writes land at w + off <= p: never past an entry not yet read.
                if (v) { sh.key[w + off] = kv; sh.id[w + off] = iv; }
                w += __popcll(m);
            }
            if (tid == 0) sh.nvalid = w;
        }
        __syncthreads();
    } else {
        if (tid == 0) sh.nvalid = ncand;
        __syncthreads();
    }
    const int nvalid = sh.nvalid;

    // 4. tau_m for m = 0..mt, sequential fp64 in candidate order (key[m] = s_(m)).
    const int mt = min(nvalid, a.budget - B);        // at most budget - B can be kept
    __shared__ double tau[kMaxCand + 1];
    if (tid < 64) {
        double t = double(B);
        if (tid == 0) tau[0] = t;
        for (int base = 0; base < mt; base += 64) {
            const double v = (base + tid < mt) ? sh.key[base + tid] : 0.0;
            const int cnt = min(64, mt - base);
            for (int i = 0; i < cnt; ++i) {
                const double si = __shfl(v, i);
                t = t + si;
                if (tid == 0) tau[base + i + 1] = t;
            }
        }
    }
    __syncthreads();

    // 5. first failure of "theta improves" (the budget caps m at mt).
    for (int m = tid; m < mt; m += kSchedThreads) {
        const int T = B + m;
        const double th0 = tau[m] / double(a.cost[T]);
        const double th1 = tau[m + 1] / double(a.cost[T + 1]);
        if (!(th1 > th0)) atomicMin(&sh.mstar, m);
    }
    __syncthreads();
    const int mstar = min(sh.mstar, mt);
    for (int m = tid; m < mstar; m += kSchedThreads) {
        const int id = sh.id[m];
        const int b = id / G, k = id - b * G;
        atomicMax(&sh.len[b], k + 1);
    }
    __syncthreads();
    for (int b = tid; b < B; b += kSchedThreads) a.out_len[b] = sh.len[b];
    if (tid == 0) {
        a.out_T[0] = B + mstar;
        if (a.out_tau) a.out_tau[0] = float(tau[mstar]);
    }
}

}  // namespace

int launch_schedule(const ScheduleArgs &a, void *stream) {
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

}  // namespace sv
