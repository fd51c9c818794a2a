// Sequential Temperature Scaling fit on CDNA4 (gfx950).
//
// What is computed ("UraionSpec", section "Sequential Temperature Scaling"):
// positions k = 0..G-1 left to right; for each, over a grid of temperatures T,
// the expected calibration error (equal-width bins on [0, 1]) of the
// cumulative survival a_n(T) = prefix_n * c_{n,k}^(1/T) against the labels
// y_n = [acc_len_n > k]; T_k is the first grid point with the least error, and
// prefix_n then gains the factor c_{n,k}^(1/T_k).  Confidences are clamped
// into [0, 1] (NaN as 0).
//
// Three launches per position (the choice of T_k orders everything after it):
//   accumulate  a grid-stride pass over the samples: the sample's survival is
//               advanced by the previous position's fitted factor, then for
//               every grid temperature its bin gains the label and the
//               prediction in LDS (the prediction in 2^-40 fixed point, so the
//               sums do not depend on the order of the atomics).  Lane l visits the
//               temperatures starting at l, so the lanes of a wave update
//               different temperature rows at once instead of colliding on one.
//               Each workgroup writes its own slot of partial sums;
//   error       one workgroup per temperature adds the slots of its bins and
//               forms sum_bins |sum a - sum y| / N (bins in order);
//   choose      one workgroup takes the first minimum.
// The exponent is log2(c) times the double reciprocal of T.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"

namespace sv {
namespace {

__device__ __forceinline__ double clamp01(float c) { return (c > 0.0f) ? fmin(double(c), 1.0) : 0.0; }   // NaN -> 0

__global__ __launch_bounds__(kFitThreads) void k_fit_accumulate(FitArgs a) {
    extern __shared__ unsigned long long acc[];       // [nt][bins][2]: labels, fixed-point predictions
    __shared__ double rT[kFitMaxTemps];
    const int tid = threadIdx.x, lane = tid & 63;
    const int cells = a.nt * a.bins * 2;
    for (int i = tid; i < cells; i += kFitThreads) acc[i] = 0ull;
    for (int t = tid; t < a.nt; t += kFitThreads) rT[t] = 1.0 / double(a.temps[t]);
    __syncthreads();
    const int k = a.k, G = a.G;
    const double Tprev = (k > 0) ? double(a.out_temps[k - 1]) : 1.0;
    for (int n = int(blockIdx.x) * kFitThreads + tid; n < a.N; n += int(gridDim.x) * kFitThreads) {
        double pre = 1.0;
        if (k > 0) pre = a.prefix[n] * exp2(log2(clamp01(a.conf[size_t(n) * G + k - 1])) * (1.0 / Tprev));
        a.prefix[n] = pre;
        const double lc = log2(clamp01(a.conf[size_t(n) * G + k]));
        const unsigned long long y = (a.acc_len[n] > k) ? 1ull : 0ull;
        int t = lane % a.nt;
        for (int s = 0; s < a.nt; ++s, t = (t + 1 == a.nt) ? 0 : t + 1) {
            const double p = pre * exp2(lc * rT[t]);
            const int bin = min(int(floor(p * double(a.bins))), a.bins - 1);
            unsigned long long *cell = acc + (size_t(t) * a.bins + bin) * 2;
            if (y) atomicAdd(cell + 0, 1ull);
            atomicAdd(cell + 1, (unsigned long long)llrint(p * kFitScale));
        }
    }
    __syncthreads();
    int64_t *slot = a.part + size_t(blockIdx.x) * cells;
    for (int i = tid; i < cells; i += kFitThreads) slot[i] = int64_t(acc[i]);
}

// One workgroup per grid temperature: its bins' sums over the slots, then
// the error (bins in order).
__global__ __launch_bounds__(kFitThreads) void k_fit_error(FitArgs a) {
    __shared__ int64_t red[kFitThreads / 64][kFitMaxBins][2];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cells = a.nt * a.bins * 2;
    for (int b = 0; b < a.bins; ++b) {
        const int64_t *c0 = a.part + (size_t(t) * a.bins + b) * 2;
        int64_t lab = 0, pred = 0;
        for (int w = tid; w < a.nwg; w += kFitThreads) {
            lab += c0[size_t(w) * cells + 0];
            pred += c0[size_t(w) * cells + 1];
        }
        // integer sums: any order gives the same total
        for (int o = 32; o > 0; o >>= 1) {
            lab += __shfl_xor(lab, o);
            pred += __shfl_xor(pred, o);
        }
        if (lane == 0) {
            red[wv][b][0] = lab;
            red[wv][b][1] = pred;
        }
    }
    __syncthreads();
    if (tid == 0) {
        double e = 0.0;
        for (int b = 0; b < a.bins; ++b) {
            int64_t lab = 0, pred = 0;
            for (int v = 0; v < kFitThreads / 64; ++v) {
                lab += red[v][b][0];
                pred += red[v][b][1];
            }
            e = e + fabs(double(pred) / kFitScale - double(lab));
        }
        a.err[t] = e / double(a.N);
    }
}

// The errors are loaded together into LDS, then scanned in grid order.
__global__ __launch_bounds__(kFitMaxTemps) void k_fit_choose(FitArgs a) {
    __shared__ double e[kFitMaxTemps];
    if (int(threadIdx.x) < a.nt) e[threadIdx.x] = a.err[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 0) {
        int best = 0;
        for (int t = 1; t < a.nt; ++t)
            if (e[t] < e[best]) best = t;
        a.out_temps[a.k] = a.temps[best];
    }
}

}  // namespace

int launch_fit_accumulate(const FitArgs &a, void *stream) {
    const size_t lds = size_t(a.nt) * a.bins * 2 * sizeof(unsigned long long);
    hipLaunchKernelGGL(k_fit_accumulate, dim3(a.nwg), dim3(kFitThreads), lds, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

int launch_fit_choose(const FitArgs &a, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_fit_error, dim3(a.nt), dim3(kFitThreads), 0, st, a);
    hipLaunchKernelGGL(k_fit_choose, dim3(1), dim3(kFitMaxTemps), 0, st, a);
    return int(hipGetLastError());
}

}  // namespace sv
