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
// tally) run in parallel.  The work is a chain of dependent steps on one
// workgroup, so the design minimises round trips and serial steps:
//
//   1. every confidence and every cost entry the scan can reach is loaded into
//      LDS at once (one memory round trip);
//   2. one thread per request: the fp64 running product of its confidences
//      (the sequential loop's order), and whether survival is non-increasing
//      along every request (always true for c in [0, 1]);
//   3. bitonic sort of (s, k*B + b) keys, candidates first (the key's second
//      half orders equal survivals by k, then b, with no division).  With at
//      most 1024 slots each thread holds one in registers and the network is
//      unrolled: partners closer than a wave are read across lanes with DPP
//      (strides 1, 2, 4, 8) and the row-swap permutes (16, 32), farther ones
//      through LDS, two strides per barrier where two remain.  The network
//      compares one 64-bit key (fp32-rounded survival above the id); runs of
//      equal fp32 survival are then re-ranked exactly, so the order is the
//      exact one;
//   4. contiguity (only when some survival increases): a candidate can be kept
//      only if all shallower positions of its request are candidates placed
//      before it;
//   5. one wave walks the sorted candidates 64 at a time: tau is extended in
//      candidate order, lane by lane, then the 64 tests theta_{m+1} > theta_m
//      run at once; the walk stops at the block holding the first failure
//      (or at the budget), so it visits only about m* + 64 candidates;
//   6. lengths are tallied from the first m* candidates.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"
#include "sv_wave.h"

namespace sv {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kMaxCand = 4096;
constexpr int kRegSort = 1024;     // at most this many slots: one per thread, sorted in registers
constexpr int kPad = 0x7fffffff;

struct SchedSmem {
    double key[kMaxCand];      // survival (slot = b * G + k), then sorted survival
    int id[kMaxCand];          // k * B + b, or kPad for padding / non-candidates
    union {
        double conf[kMaxCand]; // the confidences (slot = b * G + k)
        int pos[kMaxCand];     // contiguity: sorted position of each candidate (slot b * G + k), or -1
        struct {
            uint64_t xq[2][kRegSort]; // register sort: exchange buffers for strides >= 64
            double fs[kRegSort];      // then the sorted exact survivals and ids (run fix-up)
            int fi[kRegSort];
        } reg;
    } u;
    int len[kMaxCand];         // per request kept length (B <= kMaxCand)
    float cost[kMaxCand + 1];  // cost[B + m] for m = 0..min(B*G, budget - B)
    int nvalid, mstar;
    double taustar;            // tau_{m*}
    double red[kMaxThreads / 64][kMaxRatios];   // ratio budgets: per-wave progress sums
    int wsum[kMaxThreads / 64];                 // per-wave totals of a block scan
};

// Order: larger survival first; equal survival -> smaller k, then smaller b
// (the id k * B + b compares in exactly that order; padding sorts last).
__device__ __forceinline__ bool before(double s1, int id1, double s2, int id2) {
    return s1 > s2 || (s1 == s2 && id1 < id2);
}
// Sorting-network key: the survival rounded to fp32 (larger first) above the
// id k * B + b; padding sorts last.  Rounding is monotone, so the key order
// equals the exact order except inside runs of equal fp32 survival, which the
// sort then re-ranks exactly.  One 64-bit unsigned compare per network step.
constexpr uint64_t kPadKey = ~0ull;
__device__ __forceinline__ uint64_t pack_key(double s, int id) {
    if (id == kPad) return kPadKey;
    const uint32_t u = __float_as_uint(float(s + 0.0));                 // -0 -> +0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);    // ascending with the value
    return (uint64_t(~ord) << 32) | uint32_t(id);
}
__device__ __forceinline__ uint32_t key_run(uint64_t k) { return uint32_t(k >> 32); }
__device__ __forceinline__ int key_id(uint64_t k) { return k == kPadKey ? kPad : int(uint32_t(k)); }

// Value of lane (lane ^ S) of the wave, S < 64.  (Every DPP pattern used
// reads an active lane inside its row, so no lane needs an old value.)
template <int S> __device__ __forceinline__ int xor_lane(int x, int lane) {
    if constexpr (S == 1) return dpp_i<0xB1>(x);               // quad_perm [1, 0, 3, 2]
    else if constexpr (S == 2) return dpp_i<0x4E>(x);          // quad_perm [2, 3, 0, 1]
    else if constexpr (S == 4) return dpp_i<0x1B>(dpp_i<0x141>(x));   // row_half_mirror (^7), then quad_perm [3, 2, 1, 0] (^3)
    else if constexpr (S == 8) return dpp_i<0x128>(x);         // row_ror:8
    else if constexpr (S == 16) {
        // Row swap: result 0 holds the even row's lanes, result 1 the odd row's.
        const auto r = __builtin_amdgcn_permlane16_swap(unsigned(x), unsigned(x), false, false);
        return int((lane & 16) ? r[0] : r[1]);
    } else {
        static_assert(S == 32, "in-wave stride");
        const auto r = __builtin_amdgcn_permlane32_swap(unsigned(x), unsigned(x), false, false);
        return int((lane & 32) ? r[0] : r[1]);
    }
}
__device__ __forceinline__ uint64_t join64(int lo, int hi) { return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo); }
template <int S> __device__ __forceinline__ uint64_t xor_lane_k(uint64_t x, int lane) {
    return join64(xor_lane<S>(int(uint32_t(x)), lane), xor_lane<S>(int(uint32_t(x >> 32)), lane));
}

// The key position pos keeps after the step (size, stride) of a pair whose
// keys are k1 at pos and k2 at its partner: the first in order when pos keeps
// "first" (its bit `stride` agrees with its bit `size`), else the second.
__device__ __forceinline__ uint64_t cx_keep(uint64_t k1, uint64_t k2, int pos, int size, int stride) {
    const bool keep_first = ((pos & stride) == 0) == ((pos & size) == 0);
    return (keep_first == (k1 < k2)) ? k1 : k2;
}
// The row-swap permutes leave every lane both members of its pair: result 0
// holds the lower lane's value, result 1 the upper one's.
template <int S> __device__ __forceinline__ void pair_of(int x, int &lo, int &hi) {
    if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(unsigned(x), unsigned(x), false, false);
        lo = int(r[0]);
        hi = int(r[1]);
    } else {
        static_assert(S == 32, "row-swap stride");
        const auto r = __builtin_amdgcn_permlane32_swap(unsigned(x), unsigned(x), false, false);
        lo = int(r[0]);
        hi = int(r[1]);
    }
}
template <int S>
__device__ __forceinline__ void cx_wave(uint64_t &k, int tid, int lane, int size) {
    if constexpr (S == 16 || S == 32) {
        int l0, h0, l1, h1;
        pair_of<S>(int(uint32_t(k)), l0, h0);
        pair_of<S>(int(uint32_t(k >> 32)), l1, h1);
        const uint64_t kl = join64(l0, l1), kh = join64(h0, h1);
        const bool keep_first = ((tid & S) == 0) == ((tid & size) == 0);
        k = (keep_first == (kl < kh)) ? kl : kh;
    } else {
        k = cx_keep(k, xor_lane_k<S>(k, lane), tid, size, S);
    }
}
// The in-wave strides of a merge stage of `size`, largest first.
__device__ __forceinline__ void cx_in_wave(uint64_t &k, int tid, int lane, int size, int top) {
    if (top >= 32) cx_wave<32>(k, tid, lane, size);
    if (top >= 16) cx_wave<16>(k, tid, lane, size);
    if (top >= 8) cx_wave<8>(k, tid, lane, size);
    if (top >= 4) cx_wave<4>(k, tid, lane, size);
    if (top >= 2) cx_wave<2>(k, tid, lane, size);
    cx_wave<1>(k, tid, lane, size);
}

// Calibrated confidence ("UraionSpec", Sequential Temperature Scaling):
// float32(c^(1/T)) formed as 2^(log2(c) / T) in double (0 -> 0, 1 -> 1).
__device__ __forceinline__ float calibrate(float c, float T) {
    return float(exp2(log2(double(c)) / double(T)));
}
__device__ __forceinline__ float conf_at(const float *conf, const Calib &cal, int i, int G) {
    const float c = conf[i];
    return cal.on ? calibrate(c, cal.temp[i % G]) : c;
}

// Sorting slot i: its survival when it is a candidate, else -inf padding.
// L = 0: slot i is draft i = b * G + k.  L > 0 (survival never rises along a
// request): request b owns the run of L slots from b * L, its drafts in order
// (reversed for odd b), padding after them, so every run is already sorted
// and consecutive runs alternate direction: the bitonic network can start at
// stage 2L.
__device__ __forceinline__ void slot_key(const SchedSmem &sh, int i, int N, int B, int G, int L, double eps,
                                         double &s, int &id) {
    s = -__builtin_inf();
    id = kPad;
    int b, k;
    if (L > 0) {
        b = i / L;
        const int j = i - b * L;
        k = (b & 1) ? L - 1 - j : j;
        if (b >= B || k >= G) return;
    } else {
        if (i >= N) return;
        b = i / G;
        k = i - b * G;
    }
    const double v = sh.key[b * G + k];
    if (v > eps) {
        s = v;
        id = k * B + b;
    }
}

// 2. Survival s[b, k] = ((c[b,0] * c[b,1]) * ...) * c[b,k] (confidences in
//    sh.u.conf), the sequential product, one thread per request (for G <= 16
//    its reads are issued together: clamped in bounds, the ones past G
//    unused).  Returns whether survival is non-increasing along every request.
__device__ __forceinline__ bool survivals(SchedSmem &sh, int B, int G, int tid, int nth) {
    const int N = B * G;
    bool mono = true;
    for (int b = tid; b < B; b += nth) {
        const double *c = sh.u.conf + b * G;
        double *sv = sh.key + b * G;
        double acc = 1.0;
        if (G > 0 && G <= 16) {
            double cv[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) cv[k] = sh.u.conf[min(b * G + k, N - 1)];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (k < G) {
                    const double nx = acc * cv[k];
                    if (k > 0 && !(nx <= acc)) mono = false;
                    acc = nx;
                    sv[k] = acc;
                }
            }
        } else {
            for (int k = 0; k < G; ++k) {
                const double nx = acc * c[k];
                if (k > 0 && !(nx <= acc)) mono = false;
                acc = nx;
                sv[k] = acc;
            }
        }
        sh.len[b] = 0;
    }
    return __syncthreads_and(mono);
}

// 3. Sort the candidates (survival in sh.key above eps) in the order (s desc,
//    k asc, b asc), padding last: sh.key / sh.id hold the sorted survivals and
//    ids k * B + b.  Returns the number of candidates.  presorted: survival
//    never rises along any request, so the run layout of slot_key applies when
//    it needs no more slots than the workgroup has threads.
__device__ __forceinline__ int sort_candidates(SchedSmem &sh, int B, int G, double eps, int tid, int lane, int nth,
                                               bool presorted = false) {
    const int N = B * G;
    int Np = 1;
    while (Np < N) Np <<= 1;
    int L = 0;
    if (presorted && G >= 2) {
        int l = 1;
        while (l < G) l <<= 1;
        int np = 1;
        while (np < B * l) np <<= 1;
        if (np <= nth && np <= kRegSort) {
            L = l;
            Np = np;
        }
    }
    int ncand;
    if (Np <= kRegSort) {
        // One slot per thread, bitonic network in registers on the packed
        // keys: partners in the wave by cross-lane reads (the in-wave strides
        // of a stage unrolled), farther ones through LDS (two buffers, so one
        // barrier per step).
        double s0;
        int id0;
        slot_key(sh, tid, N, B, G, L, eps, s0, id0);
        uint64_t k = pack_key(s0, id0);
        int buf = 0;
        for (int size = (L > 0) ? 2 * L : 2; size <= Np; size <<= 1) {
            int stride = size >> 1;
            while (stride >= 64) {
                sh.u.reg.xq[buf][tid] = k;
                __syncthreads();
                if (stride >= 128) {
                    // Two steps per barrier: strides (stride, h) over the four
                    // positions t, t^stride, t^h, t^stride^h.
                    const int h = stride >> 1;
                    const uint64_t ka = sh.u.reg.xq[buf][tid ^ stride], kb = sh.u.reg.xq[buf][tid ^ h],
                                   kc = sh.u.reg.xq[buf][tid ^ stride ^ h];
                    const uint64_t k1t = cx_keep(k, ka, tid, size, stride);
                    const uint64_t k1h = cx_keep(kb, kc, tid ^ h, size, stride);
                    k = cx_keep(k1t, k1h, tid, size, h);
                    stride >>= 2;
                } else {
                    k = cx_keep(k, sh.u.reg.xq[buf][tid ^ stride], tid, size, stride);
                    stride >>= 1;
                }
                buf ^= 1;
            }
            cx_in_wave(k, tid, lane, size, min(size >> 1, 32));
        }
        // Runs of equal key_run (equal fp32 survival) are in id order; rank
        // each element exactly inside its run (usually a run of one).
        const int id = key_id(k);
        double s = -__builtin_inf();
        if (id != kPad) {
            const int kk = id / B, b = id - kk * B;
            s = sh.key[b * G + kk];
        }
        __syncthreads();                           // the last exchange buffer is read
        sh.u.reg.xq[0][tid] = k;
        sh.u.reg.fs[tid] = s;
        sh.u.reg.fi[tid] = id;
        ncand = __syncthreads_count(tid < Np && id != kPad);
        int rank = tid;
        if (id != kPad) {
            const uint32_t run = key_run(k);
            int lo = tid, hi = tid;
            while (lo > 0 && key_run(sh.u.reg.xq[0][lo - 1]) == run) --lo;
            while (hi + 1 < Np && key_run(sh.u.reg.xq[0][hi + 1]) == run) ++hi;
            if (hi > lo) {
                rank = lo;
                for (int p = lo; p <= hi; ++p)
                    if (p != tid && before(sh.u.reg.fs[p], sh.u.reg.fi[p], s, id)) ++rank;
            }
        }
        if (tid < Np) { sh.key[rank] = s; sh.id[rank] = id; }
        __syncthreads();
    } else {
        for (int i = tid; i < Np; i += nth) {
            double v;
            int id;
            slot_key(sh, i, N, B, G, 0, eps, v, id);
            sh.key[i] = v;          // slot i is read only by its own thread here
            sh.id[i] = id;
        }
        __syncthreads();
        for (int size = 2; size <= Np; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = tid; t < Np / 2; t += nth) {
                    const int lo = 2 * t - (t & (stride - 1));
                    const int hi = lo + stride;
                    const bool up = ((lo & size) == 0);         // this block sorts "before" first
                    const double s1 = sh.key[lo], s2 = sh.key[hi];
                    const int i1 = sh.id[lo], i2 = sh.id[hi];
                    const bool swap = up ? before(s2, i2, s1, i1) : before(s1, i1, s2, i2);
                    if (swap) { sh.key[lo] = s2; sh.key[hi] = s1; sh.id[lo] = i2; sh.id[hi] = i1; }
                }
                __syncthreads();
            }
        }
        // Candidates (finite survival) sort before the -inf padding: count the prefix.
        if (tid == 0) {
            int lo = 0, hi = Np;                              // first padding slot
            while (lo < hi) { const int mid = (lo + hi) >> 1; if (sh.id[mid] != kPad) lo = mid + 1; else hi = mid; }
            sh.nvalid = lo;
        }
        __syncthreads();
        ncand = sh.nvalid;
        __syncthreads();
    }

    return ncand;
}

// One block of the grid; blockDim.x = max(64, Np) when Np <= kRegSort (the
// register sort), else kMaxThreads.
__global__ __launch_bounds__(kMaxThreads) void k_schedule(ScheduleArgs a) {
    __shared__ SchedSmem sh;
    const int tid = threadIdx.x, lane = tid & 63, nth = blockDim.x;
    const int B = a.B, G = a.G, N = B * G;
    const double eps = double(a.eps);
    const int mt_max = min(N, a.budget - B);          // kept drafts never exceed this

    // 1. every input the scan can read, in one round trip.
    for (int i = tid; i < N; i += nth) sh.u.conf[i] = double(conf_at(a.conf, a.cal, i, G));
    for (int i = tid; i <= mt_max; i += nth) sh.cost[i] = a.cost[B + i];
    __syncthreads();

    const bool nonincr = survivals(sh, B, G, tid, nth);
    int ncand = sort_candidates(sh, B, G, eps, tid, lane, nth, nonincr);

    // 4. contiguity: only when some survival increases along a request.
    if (!nonincr) {
        for (int i = tid; i < N; i += nth) sh.u.pos[i] = -1;
        __syncthreads();
        for (int p = tid; p < ncand; p += nth) {
            const int id = sh.id[p];
            const int k = id / B, b = id - k * B;
            sh.u.pos[b * G + k] = p;
        }
        __syncthreads();
        for (int p = tid; p < ncand; p += nth) {
            const int id = sh.id[p];
            const int k = id / B, b = id - k * B;
            bool valid = true;
            int prevp = -1;
            for (int kk = 0; kk <= k; ++kk) {
                const int pp = sh.u.pos[b * G + kk];
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
        ncand = sh.nvalid;
    }
    const int mt = min(ncand, mt_max);                // at most budget - B can be kept

    // 5. walk the sorted candidates; m* = first m with !(theta_{m+1} > theta_m).
    //    tau_m = B + s_(0) + ... + s_(m-1) in candidate order; theta_m = tau_m / cost[B + m].
    if (tid < 64) {
        double t = double(B);
        if (mt == 0 && lane == 0) { sh.mstar = 0; sh.taustar = t; }
        for (int base = 0; base < mt; base += 64) {
            const int m = base + lane;
            const double sm = (m < mt) ? sh.key[m] : 0.0;
            double tau0 = 0.0, tau1 = 0.0;
            const int cnt = min(64, mt - base);
            if (cnt == 64) {                      // a full block: no per-step bound
#pragma unroll
                for (int j = 0; j < 64; ++j) {
                    if (lane == j) tau0 = t;
                    t = t + lane_d(sm, j);
                    if (lane == j) tau1 = t;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 64; ++j) {
                    if (j < cnt) {
                        if (lane == j) tau0 = t;
                        t = t + lane_d(sm, j);
                        if (lane == j) tau1 = t;
                    }
                }
            }
            bool fail = false;
            if (m < mt) {
                const double th0 = tau0 / double(sh.cost[m]);
                const double th1 = tau1 / double(sh.cost[m + 1]);
                fail = !(th1 > th0);
            }
            const unsigned long long f = __ballot(fail);
            if (f) {
                const int first = __builtin_ctzll(f);
                if (lane == first) { sh.mstar = base + first; sh.taustar = tau0; }
                break;
            }
            if (base + 64 >= mt && lane == 0) { sh.mstar = mt; sh.taustar = t; }   // no failure up to mt
        }
    }
    __syncthreads();
    const int mstar = sh.mstar;

    // 6. lengths from the first m* candidates, tau_{m*} for the caller.
    for (int m = tid; m < mstar; m += nth) {
        const int id = sh.id[m];
        const int k = id / B, b = id - k * B;
        atomicMax(&sh.len[b], k + 1);
    }
    __syncthreads();
    for (int b = tid; b < B; b += nth) a.out_len[b] = sh.len[b];
    if (tid == 0) {
        a.out_T[0] = B + mstar;
        if (a.out_tau) a.out_tau[0] = float(sh.taustar);
    }
}

// Ratio-budgeted depth ("AngelSpec", section 4.2, Eq. 20-24): one block,
// blockDim.x as for k_schedule.  Every draft is ranked once (the sort above,
// with every draft a candidate); the budget of ratio r keeps the drafts of
// sorted position < keep[r] = K_r - B, which is a contiguous prefix of every
// request because survival never rises (confidences clamped into [0, 1]) and
// equal survivals rank shallower first.  Then, per ratio, the estimated
// progress U_r = sum_b (1 + kept survivals of b), the ratio with the largest
// U_r / C_r (the first on ties), its keep depths and the packed row offsets.
__global__ __launch_bounds__(kMaxThreads) void k_dcut(DcutArgs a) {
    __shared__ SchedSmem sh;
    const int tid = threadIdx.x, lane = tid & 63, nth = blockDim.x, wv = tid >> 6;
    const int B = a.B, G = a.G, N = B * G;

    for (int i = tid; i < N; i += nth) {
        const double c = double(conf_at(a.conf, a.cal, i, G));
        sh.u.conf[i] = (c > 0.0) ? fmin(c, 1.0) : 0.0;   // NaN -> 0
    }
    __syncthreads();
    survivals(sh, B, G, tid, nth);
    sort_candidates(sh, B, G, -__builtin_inf(), tid, lane, nth, true);   // clamped: survival never rises
    for (int p = tid; p < N; p += nth) {                  // sorted position of each draft
        const int id = sh.id[p];
        const int k = id / B, b = id - k * B;
        sh.u.pos[b * G + k] = p;
    }
    __syncthreads();

    // Progress of request b at each ratio's depth, in position order:
    // A_b = 1 + s_0 + ... + s_{n-1}, and the depth n itself; summed per
    // thread, then per wave (DPP), then over the waves that hold requests,
    // in order.
    const int R = a.R;
    double U[kMaxRatios];
    int nr[kMaxRatios];                                // depths of this thread's (last) request
#pragma unroll
    for (int r = 0; r < kMaxRatios; ++r) {
        U[r] = 0.0;
        nr[r] = 0;
    }
    for (int b = tid; b < B; b += nth) {
        double A = 1.0, Ab[kMaxRatios];
#pragma unroll
        for (int r = 0; r < kMaxRatios; ++r) {
            Ab[r] = 1.0;
            nr[r] = 0;
        }
        if (G > 0 && G <= 16) {
            // positions, then survivals, each batch issued together
            int pp[16];
            double sv[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) pp[k] = sh.u.pos[min(b * G + k, N - 1)];
#pragma unroll
            for (int k = 0; k < 16; ++k) sv[k] = sh.key[pp[k]];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (k < G) {
                    A = A + sv[k];
#pragma unroll
                    for (int r = 0; r < kMaxRatios; ++r)
                        if (pp[k] < a.keep[r]) {
                            Ab[r] = A;
                            nr[r] = k + 1;
                        }
                }
            }
        } else {
            for (int k = 0; k < G; ++k) {
                const int p = sh.u.pos[b * G + k];
                A = A + sh.key[p];
#pragma unroll
                for (int r = 0; r < kMaxRatios; ++r)
                    if (p < a.keep[r]) {
                        Ab[r] = A;
                        nr[r] = k + 1;
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < kMaxRatios; ++r) U[r] = U[r] + Ab[r];
    }
    const int nw = (min(B, nth) + 63) >> 6;            // waves holding requests
    if (wv < nw) {
#pragma unroll
        for (int r = 0; r < kMaxRatios; ++r) {
            if (r < R) {
                const double w = wave_sum_d(U[r]);
                if (lane == 0) sh.red[wv][r] = w;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        int best = 0;
        double bv = 0.0;
        for (int r = 0; r < R; ++r) {
            double u = 0.0;
            for (int v = 0; v < nw; ++v) u = u + sh.red[v][r];
            const double th = u / double(a.cost[r]);
            if (r == 0 || th > bv) {
                bv = th;
                best = r;
            }
            if (a.out_utility) a.out_utility[r] = u;
        }
        sh.nvalid = best;
        sh.mstar = a.keep[best];
        a.out_ratio[0] = best;
        a.out_rows[0] = B + a.keep[best];
    }
    __syncthreads();
    const int best = sh.nvalid, keep = sh.mstar;

    // Keep depths at the chosen ratio and the packed row offsets (exclusive
    // prefix of n_b + 1).
    if (B <= nth) {
        // One request per thread: the depth is in registers, and the prefix
        // is a DPP wave scan plus the totals of the waves before.
        int n = 0;
#pragma unroll
        for (int r = 0; r < kMaxRatios; ++r) n = (r == best) ? nr[r] : n;
        const int cnt = (tid < B) ? n + 1 : 0;
        const int incl = wave_scan_i(cnt);
        if (lane == 63) sh.wsum[wv] = incl;
        if (tid < B) a.out_len[tid] = n;
        __syncthreads();
        int o = incl - cnt;
        for (int v = 0; v < wv; ++v) o += sh.wsum[v];
        if (tid < B) a.out_off[tid] = o;
    } else {
        for (int b = tid; b < B; b += nth) {
            int n = 0;
            for (int k = 0; k < G; ++k) n += int(sh.u.pos[b * G + k] < keep);
            sh.len[b] = n;
            a.out_len[b] = n;
        }
        __syncthreads();
        // each thread a contiguous run of requests
        const int per = (B + nth - 1) / nth;
        const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
        int local = 0;
        for (int b = b0; b < b1; ++b) local += sh.len[b] + 1;
        const int incl = wave_scan_i(local);
        if (lane == 63) sh.wsum[wv] = incl;
        __syncthreads();
        int o = incl - local;
        for (int v = 0; v < wv; ++v) o += sh.wsum[v];
        for (int b = b0; b < b1; ++b) {
            a.out_off[b] = o;
            o += sh.len[b] + 1;
        }
    }
    if (tid == 0) a.out_off[B] = B + keep;
}

}  // namespace

int launch_schedule(const ScheduleArgs &a, void *stream) {
    int Np = 1;
    while (Np < a.B * a.G) Np <<= 1;
    const int threads = (Np <= kRegSort) ? (Np < 64 ? 64 : Np) : kMaxThreads;
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(threads), 0, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

// Static scheduler (one workgroup): each thread a contiguous run of
// requests; fixed length, or the leading (calibrated) confidences above tau;
// then the total and the packed row offsets by a block scan.
__global__ __launch_bounds__(kMaxThreads) void k_static(StaticArgs a) {
    __shared__ int wsum[kMaxThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nth = blockDim.x;
    const int B = a.B, G = a.G;
    const int per = (B + nth - 1) / nth;
    const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
    const int fixed = min(max(a.len, 0), G);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        int n = fixed;
        if (a.mode == 1) {
            // 16 confidences at a time, all loaded before any is tested
            n = 0;
            for (int k0 = 0; k0 < G && n == k0; k0 += 16) {
                float cv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) cv[i] = a.conf[size_t(b) * G + min(k0 + i, G - 1)];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int k = k0 + i;
                    const float c = a.cal.on ? calibrate(cv[i], a.cal.temp[min(k, G - 1)]) : cv[i];
                    if (n == k && k < G && c > a.tau) n = k + 1;
                }
            }
        }
        a.out_len[b] = n;
        local += n + 1;
    }
    const int incl = wave_scan_i(local);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int o = incl - local;
    for (int v = 0; v < wv; ++v) o += wsum[v];
    if (a.out_off) {
        for (int b = b0; b < b1; ++b) {
            a.out_off[b] = o;
            o += a.out_len[b] + 1;     // this thread's own store, read back
        }
    }
    if (tid == nth - 1) {
        int tot = 0;
        for (int v = 0; v < (nth >> 6); ++v) tot += wsum[v];
        if (a.out_T) a.out_T[0] = tot;
        if (a.out_off) a.out_off[B] = tot;
    }
}

int launch_static(const StaticArgs &a, void *stream) {
    hipLaunchKernelGGL(k_static, dim3(1), dim3(kMaxThreads), 0, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

int launch_dcut(const DcutArgs &a, void *stream) {
    int Np = 1;
    while (Np < a.B * a.G) Np <<= 1;
    const int threads = (Np <= kRegSort) ? (Np < 64 ? 64 : Np) : kMaxThreads;
    hipLaunchKernelGGL(k_dcut, dim3(1), dim3(threads), 0, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

}  // namespace sv
