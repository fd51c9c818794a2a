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
// only the independent parts (ranking, the theta comparisons, the length
// tally) run in parallel.  The work is a chain of dependent steps on one
// workgroup, so the design minimises round trips, barriers and the length of
// each thread's instruction stream:
//
//   1. every confidence and every cost entry the scan can reach is loaded into
//      LDS at once (one memory round trip);
//   2. one slot (b, k) per thread: its survival, the fp64 product of
//      c[b,0..k] in order, and whether it exceeds the one before;
//   3. the exact rank of every candidate without a sorting network: each
//      candidate counts into a bin of its fp32-rounded survival (8 bins per
//      octave, an LDS atomic that also numbers it inside the bin), a block
//      scan of the bins gives each bin's first rank, and a candidate's rank is
//      that plus the number of candidates of its own bin that precede it,
//      compared exactly.  A bin with many candidates (equal survivals) sends
//      the call to a bitonic network over packed (fp32 survival, id) keys with
//      an exact re-rank inside runs of equal fp32 survival;
//   4. contiguity (only when some survival increases): a candidate can be kept
//      only if all shallower positions of its request are candidates placed
//      before it;
//   5. one wave walks the ranked candidates 64 at a time: one lane extends
//      tau in candidate order and stores each step in LDS, then the 64 tests
//      theta_{m+1} > theta_m run at once; the walk stops at the block holding
//      the first failure (or at the budget), so it visits only about m* + 64
//      candidates;
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
constexpr int kEpt = kMaxCand / kMaxThreads;   // slots per thread
// Window bins: 1/64 octave of survival each, counted from the highest
// candidate's down, kWinPer per thread (the lowest also takes everything
// below the window).
constexpr int kWinShift = 17;      // fp32 order key >> kWinShift: the bin scale
constexpr int kWinPer = 4;
constexpr int kBins = kWinPer * kMaxThreads;
constexpr int kWinCap = 64;        // a bin ranked inside holds at most this many candidates, else the network sort
constexpr int kTopK = 256;         // k_schedule ranks the bins that start before this place
constexpr int kGrp = kTopK + kWinCap;

// Slots: draft (b, k) is slot k * B + b, which is also its id in the order
// (equal survivals: smaller k, then smaller b, first).
struct SchedSmem {
    double key[kMaxCand];      // survival by slot; after the network sort, sorted survival
    int id[kMaxCand];          // network sort: ids in order; bin ranking: ids grouped by bin (by place)
    union {
        double conf[kMaxCand]; // the confidences by slot; bin ranking: survivals grouped by bin (by place)
        int pos[kMaxCand];     // contiguity: sorted position of each candidate (by slot), or -1
        struct {
            uint64_t xq[2][kRegSort]; // register sort: exchange buffers for strides >= 64
            double fs[kRegSort];      // then the sorted exact survivals and ids (run fix-up)
            int fi[kRegSort];
        } reg;
    } u;
    int len[kMaxCand];         // per request kept length (B <= kMaxCand)
    float cost[kMaxCand + 1];  // cost[B + m] for m = 0..min(B*G, budget - B)
    int nvalid, mstar, nsel;
    double taustar;            // tau_{m*}
    double red[kMaxThreads / 64][kMaxRatios];   // ratio budgets: per-wave progress sums
    int wsum[kMaxThreads / 64];                 // per-wave totals of a block scan
    int wmax[kMaxThreads / 64];                 // per-wave maxima
    int wany[kMaxThreads / 64];                 // per-wave flags
    alignas(16) int hist[kBins];                // window bins: counts, then each bin's first place
    double rs[kGrp];           // k_schedule: the first places in order (survival, id)
    int ri[kGrp];
    uint8_t kept[kMaxCand];    // k_dcut: by slot, bit r set when ratio r keeps the draft
    double tau[9];             // the walk: tau before candidates 0, 8, ..., 56 of a block, and after the last
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
// L = 0: slot i.  L > 0 (survival never rises along a request): request b
// owns the run of L slots from b * L, its drafts in order (reversed for odd
// b), padding after them, so every run is already sorted and consecutive runs
// alternate direction: the bitonic network can start at stage 2L.
__device__ __forceinline__ void slot_key(const SchedSmem &sh, int i, int N, int B, int G, int L, double eps,
                                         double &s, int &id) {
    s = -__builtin_inf();
    id = kPad;
    int j;
    if (L > 0) {
        const int b = i / L, r = i - b * L;
        const int k = (b & 1) ? L - 1 - r : r;
        if (b >= B || k >= G) return;
        j = k * B + b;
    } else {
        if (i >= N) return;
        j = i;
    }
    const double v = sh.key[j];
    if (v > eps) {
        s = v;
        id = j;
    }
}

// Network sort of the candidates (survival in sh.key above eps) in the order
//    (s desc, k asc, b asc), padding last: sh.key / sh.id hold the sorted survivals and
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
        if (id != kPad) s = sh.key[id];
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

// 5. Walk the sorted candidates key[0..mt) (wave 0): m* = the first m with
//    !(theta_{m+1} > theta_m), or mt; tau_m = B + s_(0) + ... + s_(m-1) in
//    candidate order and theta_m = tau_m / cost[B + m].  Per block of 64: one
//    lane extends the running sum over the block and stores it before every
//    8th candidate; each lane then repeats the sum from its checkpoint to its
//    own candidate (the same additions in the same order, so the same tau),
//    and the 64 tests run at once, one per lane; the walk stops at the block
//    holding the first failure.  Sets sh.mstar and sh.taustar.
__device__ __forceinline__ void walk(SchedSmem &sh, const double *key, int mt, int B, int lane) {
    double t = double(B);
    if (mt == 0 && lane == 0) { sh.mstar = 0; sh.taustar = t; }
    for (int base = 0; base < mt; base += 64) {
        const int cnt = min(64, mt - base);
        const double *kb = key + base;
        if (lane == 0) {
            double u = t;
            if (cnt == 64) {                          // a full block: no per-step bound
#pragma unroll
                for (int j0 = 0; j0 < 64; j0 += 32) {
                    double v[32];
#pragma unroll
                    for (int j = 0; j < 32; ++j) v[j] = kb[j0 + j];
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        if (((j0 + j) & 7) == 0) sh.tau[(j0 + j) >> 3] = u;
                        u = u + v[j];
                    }
                }
            } else {
                for (int j = 0; j < cnt; ++j) {
                    if ((j & 7) == 0) sh.tau[j >> 3] = u;
                    u = u + kb[j];
                }
            }
            sh.tau[8] = u;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        bool fail = false;
        double tau0 = 0.0;
        if (lane < cnt) {
            const int m = base + lane, r = lane & 7;
            double v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = kb[min((lane & ~7) + q, cnt - 1)];   // those past r unused
            double u = sh.tau[lane >> 3];
#pragma unroll
            for (int q = 0; q < 7; ++q)
                if (q < r) u = u + v[q];
            tau0 = u;
            double sm = v[0];
#pragma unroll
            for (int q = 1; q < 8; ++q) sm = (q == r) ? v[q] : sm;
            const double tau1 = u + sm;
            const double th0 = tau0 / double(sh.cost[m]);
            const double th1 = tau1 / double(sh.cost[m + 1]);
            fail = !(th1 > th0);
        }
        t = sh.tau[8];
        const unsigned long long f = __ballot(fail);
        if (f) {
            const int first = __builtin_ctzll(f);
            if (lane == first) { sh.mstar = base + first; sh.taustar = tau0; }
            break;
        }
        if (base + 64 >= mt && lane == 0) { sh.mstar = mt; sh.taustar = t; }   // no failure up to mt
        __builtin_amdgcn_wave_barrier();                                       // tau[] is rewritten next
    }
}

// 6. Lengths from the first m* candidates (ids[0..m*)), tau_{m*} for the caller.
__device__ __forceinline__ void tally(SchedSmem &sh, const ScheduleArgs &a, const int *ids, int mstar, int tid,
                                      int nth) {
    const int B = a.B;
    for (int m = tid; m < mstar; m += nth) {
        const int id = ids[m];
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

// fp32 order key of a survival (ascending with the value; -0 as +0).
__device__ __forceinline__ uint32_t ord32(double s) {
    const uint32_t u = __float_as_uint(float(s + 0.0));
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 2. Survivals, one thread per request b: s[b,k] = the running product of
//    c[b,0..k] in order (sh.u.conf by slot) into sh.key.  Per thread: `up`,
//    some survival rises; `top`, the highest candidate's bin scale
//    (ord32 >> kWinShift; s[b,0] is a request's highest when none rises).
__device__ __forceinline__ void survivals(SchedSmem &sh, int B, int G, double eps, int tid, int nth, bool &up,
                                          int &top) {
    up = false;
    top = -1;
    for (int b = tid; b < B && G > 0; b += nth) {
        double acc = 1.0, s0;
        if (G <= 16) {
            // Branch-free: positions past G multiply by 1 (acc unchanged,
            // never a rise) and store the same value again at G - 1.
            double cv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const double x = sh.u.conf[min(t, G - 1) * B + b];
                cv[t] = (t < G) ? x : 1.0;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const double nx = acc * cv[t];
                up |= t > 0 && !(nx <= acc);
                acc = nx;
                if (t == 0) s0 = acc;
                sh.key[min(t, G - 1) * B + b] = acc;
            }
        } else {
            for (int t = 0; t < G; ++t) {
                const double nx = acc * sh.u.conf[t * B + b];
                if (t > 0 && !(nx <= acc)) up = true;
                acc = nx;
                sh.key[t * B + b] = acc;
            }
            s0 = sh.key[b];
        }
        if (s0 > eps) top = max(top, int(ord32(s0) >> kWinShift));
    }
}

// Block-wide OR of `up` and maximum of `top` (both per thread), with the one
// barrier the survivals need anyway.  Returns the maximum; `any` the OR.
__device__ __forceinline__ int reduce_survival_flags(SchedSmem &sh, bool up, int top, int lane, int wv, int nw,
                                                     bool &any) {
    const int tw = wave_scan_max_i(top + 1);
    const bool wu = __ballot(up) != 0ull;
    if (lane == 63) {
        sh.wmax[wv] = tw;
        sh.wany[wv] = wu ? 1 : 0;
    }
    __syncthreads();
    const int x = (lane < nw) ? sh.wmax[lane] : 0, f = (lane < nw) ? sh.wany[lane] : 0;
    any = __ballot(f != 0) != 0ull;
    return __builtin_amdgcn_readlane(wave_scan_max_i(x), 63) - 1;
}

// 3. Window bins (survival never rises; sh.key by slot; sh.hist[0, kWinPer *
//    nth) zero).  Every candidate slot goes to bin top - (ord32(s) >>
//    kWinShift), at most the last, and takes a number inside it (LDS atomic);
//    a block scan turns the counts into each bin's first place (bins ascend
//    as survival descends, and hold ordered ranges of it).  Per thread: its
//    slots' (survival, bin or -1, number) and its own bins' counts c4 and
//    first places s4; returns the number of candidates.  The caller's barrier
//    publishes the first places.
__device__ int window_bins(SchedSmem &sh, int N, double eps, int top, int tid, int lane, int nth,
                           double (&sv)[kEpt], int (&fb)[kEpt], int (&at)[kEpt], int4 &c4, int4 &s4) {
    const int wv = tid >> 6, nw = nth >> 6, nb = kWinPer * nth;
#pragma unroll
    for (int r = 0; r < kEpt; ++r) {
        const int i = tid + r * nth;
        fb[r] = -1;
        sv[r] = 0.0;
        at[r] = 0;
        if (i < N) {
            sv[r] = sh.key[i];
            if (sv[r] > eps) {
                fb[r] = min(max(top - int(ord32(sv[r]) >> kWinShift), 0), nb - 1);
                at[r] = atomicAdd(&sh.hist[fb[r]], 1);
            }
        }
    }
    __syncthreads();
    c4 = *reinterpret_cast<const int4 *>(&sh.hist[kWinPer * tid]);
    const int local = (c4.x + c4.y) + (c4.z + c4.w);
    const int incl = wave_scan_i(local);
    if (lane == 63) sh.wsum[wv] = incl;
    __syncthreads();
    const int wx = wave_scan_i((lane < nw) ? sh.wsum[lane] : 0);
    const int total = __builtin_amdgcn_readlane(wx, 63);
    const int w = __builtin_amdgcn_readfirstlane(wv);
    int cum = incl - local + ((w > 0) ? __builtin_amdgcn_readlane(wx, w - 1) : 0);
    s4.x = cum;
    cum += c4.x;
    s4.y = cum;
    cum += c4.y;
    s4.z = cum;
    cum += c4.z;
    s4.w = cum;
    *reinterpret_cast<int4 *>(&sh.hist[kWinPer * tid]) = s4;
    return total;
}

// Places inside a bin: candidates in bins marked by `rank_it` are grouped by
// place (survival in sh.u.conf, id in sh.id, at first place + number), then
// each one's place is its bin's first place plus the candidates of its bin
// that precede it (exact comparisons).  place[r] = -1 for the others.
// Bins end at the next bin's first place, the last at `total`.
template <class F>
__device__ void place_in_bins(SchedSmem &sh, int total, int tid, int nth, const double (&sv)[kEpt],
                              const int (&fb)[kEpt], const int (&at)[kEpt], int (&place)[kEpt], F rank_it) {
    const int nb = kWinPer * nth;
    int lo[kEpt], hi[kEpt];
#pragma unroll
    for (int r = 0; r < kEpt; ++r) {
        place[r] = -1;
        lo[r] = hi[r] = 0;
        if (fb[r] >= 0) {
            lo[r] = sh.hist[fb[r]];
            hi[r] = (fb[r] + 1 < nb) ? sh.hist[fb[r] + 1] : total;
            if (rank_it(lo[r], hi[r])) {
                sh.u.conf[lo[r] + at[r]] = sv[r];
                sh.id[lo[r] + at[r]] = tid + r * nth;
            } else {
                lo[r] = hi[r] = -1;                 // not ranked inside
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kEpt; ++r) {
        if (lo[r] >= 0 && fb[r] >= 0) {             // lo = -1: not ranked; fb = -1: not a candidate
            const int id = tid + r * nth;
            int p = lo[r];
            for (int q0 = lo[r]; q0 < hi[r]; q0 += 4) {     // four reads in flight
                double gs[4];
                int gi[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    gs[q] = sh.u.conf[min(q0 + q, hi[r] - 1)];
                    gi[q] = sh.id[min(q0 + q, hi[r] - 1)];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) p += (q0 + q < hi[r] && before(gs[q], gi[q], sv[r], id)) ? 1 : 0;
            }
            place[r] = p;
        }
    }
}

// One block of the grid; blockDim.x = max(64, Np) when Np <= kRegSort, else
// kMaxThreads.  When survival never rises (the usual case): window bins, the
// bins that start before kTopK ranked inside (they are the first S places of
// the order exactly), and the walk over them; the walk needs only about m* +
// 64 places, so it is decided there unless it passes S or a ranked bin is
// too full.  Otherwise (and then): the network sort of every candidate.
__global__ __launch_bounds__(kMaxThreads) void k_schedule(ScheduleArgs a) {
    __shared__ SchedSmem sh;
    const int tid = threadIdx.x, lane = tid & 63, nth = blockDim.x, wv = tid >> 6, nw = nth >> 6;
    const int B = a.B, G = a.G, N = B * G;
    const double eps = double(a.eps);
    const int mt_max = min(N, a.budget - B);          // kept drafts never exceed this

    // 1. every input the scan can read, in one round trip (confidences by
    //    slot); bins and lengths cleared.
    for (int j = tid; j < N; j += nth) {
        const int k = j / B, b = j - k * B;
        sh.u.conf[j] = double(conf_at(a.conf, a.cal, b * G + k, G));
    }
    for (int i = tid; i <= mt_max; i += nth) sh.cost[i] = a.cost[B + i];
    *reinterpret_cast<int4 *>(&sh.hist[kWinPer * tid]) = make_int4(0, 0, 0, 0);
    for (int b = tid; b < B; b += nth) sh.len[b] = 0;
    __syncthreads();

    bool up;
    int top;
    survivals(sh, B, G, eps, tid, nth, up, top);
    bool rises;
    const int topb = reduce_survival_flags(sh, up, top, lane, wv, nw, rises);

    if (!rises) {
        double sv[kEpt];
        int fb[kEpt], at[kEpt], place[kEpt];
        int4 c4, s4;
        const int total = window_bins(sh, N, eps, topb, tid, lane, nth, sv, fb, at, c4, s4);
        // S = the end of the bin holding place kTopK - 1 (one writer), or
        // every candidate when there are fewer; a ranked bin over kWinCap
        // sends the call to the network sort.
        const int cs[4] = {c4.x, c4.y, c4.z, c4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
        bool big = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (cs[q] > 0 && ss[q] < kTopK && ss[q] + cs[q] >= kTopK) sh.nsel = ss[q] + cs[q];
            big |= cs[q] > kWinCap && ss[q] < kTopK;
        }
        const bool wb = __ballot(big) != 0ull;
        if (lane == 63) sh.wany[wv] = wb ? 1 : 0;
        __syncthreads();
        if (__ballot(lane < nw && sh.wany[lane] != 0) == 0ull) {
            const int S = (total < kTopK) ? total : sh.nsel;
            place_in_bins(sh, total, tid, nth, sv, fb, at, place, [](int lo, int) { return lo < kTopK; });
#pragma unroll
            for (int r = 0; r < kEpt; ++r) {
                if (place[r] >= 0) {
                    sh.rs[place[r]] = sv[r];
                    sh.ri[place[r]] = tid + r * nth;
                }
            }
            __syncthreads();
            const int mt = min(total, mt_max);
            const int mtw = min(S, mt);
            if (tid < 64) walk(sh, sh.rs, mtw, B, lane);
            __syncthreads();
            const int mstar = sh.mstar;
            if (!(mstar == mtw && mtw < mt)) {        // decided inside the ranked places
                tally(sh, a, sh.ri, mstar, tid, nth);
                return;
            }
        }
        __syncthreads();
    }
    int ncand = sort_candidates(sh, B, G, eps, tid, lane, nth, !rises);

    // 4. contiguity: only when some survival increases along a request.
    if (rises) {
        for (int i = tid; i < N; i += nth) sh.u.pos[i] = -1;
        __syncthreads();
        for (int p = tid; p < ncand; p += nth) sh.u.pos[sh.id[p]] = p;
        __syncthreads();
        for (int p = tid; p < ncand; p += nth) {
            const int id = sh.id[p];
            const int k = id / B, b = id - k * B;
            bool valid = true;
            int prevp = -1;
            for (int kk = 0; kk <= k; ++kk) {
                const int pp = sh.u.pos[kk * B + b];
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
    if (tid < 64) walk(sh, sh.key, mt, B, lane);
    __syncthreads();
    tally(sh, a, sh.id, sh.mstar, tid, nth);
}

// Ratio-budgeted depth ("AngelSpec", section 4.2, Eq. 20-24): one block,
// blockDim.x as for k_schedule.  The budget of ratio r keeps the drafts of
// sorted position < keep[r] = K_r - B, which is a contiguous prefix of every
// request because survival never rises (confidences clamped into [0, 1]) and
// equal survivals rank shallower first.  Only which side of each keep[r] a
// draft falls on matters: with window bins, a bin that ends by keep[r] is
// kept whole and one that starts at or after it not at all; only the bins
// holding a keep[r] strictly inside are ranked inside (the network sort when
// one is too full).  Then, per ratio, the estimated progress U_r = sum_b
// (1 + kept survivals of b), the ratio with the largest U_r / C_r (the first
// on ties), its keep depths and the packed row offsets.
__global__ __launch_bounds__(kMaxThreads) void k_dcut(DcutArgs a) {
    __shared__ SchedSmem sh;
    const int tid = threadIdx.x, lane = tid & 63, nth = blockDim.x, wv = tid >> 6, nwt = nth >> 6;
    const int B = a.B, G = a.G, N = B * G, R = a.R;
    const double ninf = -__builtin_inf();

    for (int j = tid; j < N; j += nth) {
        const int k = j / B, b = j - k * B;
        const double c = double(conf_at(a.conf, a.cal, b * G + k, G));
        sh.u.conf[j] = (c > 0.0) ? fmin(c, 1.0) : 0.0;   // NaN -> 0
    }
    *reinterpret_cast<int4 *>(&sh.hist[kWinPer * tid]) = make_int4(0, 0, 0, 0);
    __syncthreads();
    bool up;
    int top;
    survivals(sh, B, G, ninf, tid, nth, up, top);
    bool rises;                                           // clamped: never
    const int topb = reduce_survival_flags(sh, up, top, lane, wv, nwt, rises);

    double sv[kEpt];
    int fb[kEpt], at[kEpt], place[kEpt];
    int4 c4, s4;
    const int total = window_bins(sh, N, ninf, topb, tid, lane, nth, sv, fb, at, c4, s4);
    // A bin holding some keep[r] strictly inside is ranked inside; too full: network sort.
    const auto straddles = [&](int lo, int hi) {
        bool x = false;
#pragma unroll
        for (int r = 0; r < kMaxRatios; ++r) x |= r < R && lo < a.keep[r] && a.keep[r] < hi;
        return x;
    };
    const int cs[4] = {c4.x, c4.y, c4.z, c4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
    bool big = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) big |= cs[q] > kWinCap && straddles(ss[q], ss[q] + cs[q]);
    const bool wb = __ballot(big) != 0ull;
    if (lane == 63) sh.wany[wv] = wb ? 1 : 0;
    __syncthreads();
    const double *surv = sh.key;                          // survival by slot
    if (__ballot(lane < nwt && sh.wany[lane] != 0) == 0ull) {
        place_in_bins(sh, total, tid, nth, sv, fb, at, place, straddles);
#pragma unroll
        for (int r = 0; r < kEpt; ++r) {
            const int i = tid + r * nth;
            if (i < N) {
                const int lo = sh.hist[fb[r]];
                const int hi = (fb[r] + 1 < kWinPer * nth) ? sh.hist[fb[r] + 1] : total;
                uint32_t m = 0;
#pragma unroll
                for (int q = 0; q < kMaxRatios; ++q) {
                    const int kp = a.keep[q];
                    const bool kept = hi <= kp || (lo < kp && place[r] >= 0 && place[r] < kp);
                    m |= (q < R && kept) ? (1u << q) : 0u;
                }
                sh.kept[i] = uint8_t(m);
            }
        }
        __syncthreads();
    } else {
        __syncthreads();
        sort_candidates(sh, B, G, ninf, tid, lane, nth, true);
        for (int p = tid; p < N; p += nth) {              // by slot: survival and kept bits
            const int id = sh.id[p];
            uint32_t m = 0;
#pragma unroll
            for (int q = 0; q < kMaxRatios; ++q) m |= (q < R && p < a.keep[q]) ? (1u << q) : 0u;
            sh.kept[id] = uint8_t(m);
            sh.u.conf[id] = sh.key[p];
        }
        __syncthreads();
        surv = sh.u.conf;
    }

    // Progress of request b at each ratio's depth, in position order:
    // A_b = 1 + s_0 + ... + s_{n-1}, and the depth n itself; summed per
    // thread, then per wave (DPP), then over the waves that hold requests,
    // in order.
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
            // kept bits, then survivals, each batch issued together
            uint32_t km[16];
            double s[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                km[k] = sh.kept[min(k, G - 1) * B + b];
                s[k] = surv[min(k, G - 1) * B + b];
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (k < G) {
                    A = A + s[k];
#pragma unroll
                    for (int r = 0; r < kMaxRatios; ++r)
                        if ((km[k] >> r) & 1u) {
                            Ab[r] = A;
                            nr[r] = k + 1;
                        }
                }
            }
        } else {
            for (int k = 0; k < G; ++k) {
                const uint32_t m = sh.kept[k * B + b];
                A = A + surv[k * B + b];
#pragma unroll
                for (int r = 0; r < kMaxRatios; ++r)
                    if ((m >> r) & 1u) {
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
            for (int k = 0; k < G; ++k) n += int((sh.kept[k * B + b] >> best) & 1u);
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
