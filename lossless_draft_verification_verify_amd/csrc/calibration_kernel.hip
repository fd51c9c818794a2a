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
// Two launches per position (the choice of T_k orders everything after it):
//   accumulate  a grid-stride pass over the samples: the sample's survival is
//               advanced by the previous position's fitted factor, then for
//               every grid temperature its bin is counted in LDS (count,
//               labels, prediction sum in 2^-40 fixed point, so the sums do
//               not depend on the order of the atomics); each workgroup writes
//               its own slot of partial sums;
//   choose      one workgroup adds the slots, forms each temperature's error
//               sum_bins |sum a - sum y| / N (bins in order) and takes the first
//               minimum.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.h"

namespace sv {
namespace {

__device__ __forceinline__ double clamp01(float c) { return (c > 0.0f) ? fmin(double(c), 1.0) : 0.0; }   // NaN -> 0
__device__ __forceinline__ double powT(double c, double T) { return exp2(log2(c) / T); }

__global__ __launch_bounds__(kFitThreads) void k_fit_accumulate(FitArgs a) {
    extern __shared__ unsigned long long acc[];       // [nt][bins][3]
    const int tid = threadIdx.x;
    const int cells = a.nt * a.bins * 3;
    for (int i = tid; i < cells; i += kFitThreads) acc[i] = 0ull;
    __syncthreads();
    const int k = a.k, G = a.G;
    const double Tprev = (k > 0) ? double(a.out_temps[k - 1]) : 1.0;
    for (int n = int(blockIdx.x) * kFitThreads + tid; n < a.N; n += int(gridDim.x) * kFitThreads) {
        double pre = 1.0;
        if (k > 0) pre = a.prefix[n] * powT(clamp01(a.conf[size_t(n) * G + k - 1]), Tprev);
        a.prefix[n] = pre;
        const double lc = log2(clamp01(a.conf[size_t(n) * G + k]));
        const unsigned long long y = (a.acc_len[n] > k) ? 1ull : 0ull;
        for (int t = 0; t < a.nt; ++t) {
            const double p = pre * exp2(lc / double(a.temps[t]));
            const int bin = min(int(floor(p * double(a.bins))), a.bins - 1);
            unsigned long long *cell = acc + (size_t(t) * a.bins + bin) * 3;
            atomicAdd(cell + 0, 1ull);
            if (y) atomicAdd(cell + 1, 1ull);
            atomicAdd(cell + 2, (unsigned long long)llrint(p * kFitScale));
        }
    }
    __syncthreads();
    int64_t *slot = a.part + size_t(blockIdx.x) * cells;
    for (int i = tid; i < cells; i += kFitThreads) slot[i] = int64_t(acc[i]);
}

__global__ __launch_bounds__(kFitThreads) void k_fit_choose(FitArgs a) {
    __shared__ double gap[kFitMaxTemps * kFitMaxBins];
    __shared__ double err[kFitMaxTemps];
    const int tid = threadIdx.x;
    const int pairs = a.nt * a.bins, cells = pairs * 3;
    for (int p = tid; p < pairs; p += kFitThreads) {
        int64_t lab = 0, pred = 0;
        for (int w = 0; w < a.nwg; ++w) {
            const int64_t *c = a.part + size_t(w) * cells + size_t(p) * 3;
            lab += c[1];
            pred += c[2];
        }
        gap[p] = fabs(double(pred) / kFitScale - double(lab));
    }
    __syncthreads();
    for (int t = tid; t < a.nt; t += kFitThreads) {
        double e = 0.0;
        for (int b = 0; b < a.bins; ++b) e = e + gap[t * a.bins + b];
        err[t] = e / double(a.N);
    }
    __syncthreads();
    if (tid == 0) {
        int best = 0;
        for (int t = 1; t < a.nt; ++t)
            if (err[t] < err[best]) best = t;
        a.out_temps[a.k] = a.temps[best];
    }
}

}  // namespace

int launch_fit_accumulate(const FitArgs &a, void *stream) {
    const size_t lds = size_t(a.nt) * a.bins * 3 * sizeof(unsigned long long);
    hipLaunchKernelGGL(k_fit_accumulate, dim3(a.nwg), dim3(kFitThreads), lds, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

int launch_fit_choose(const FitArgs &a, void *stream) {
    hipLaunchKernelGGL(k_fit_choose, dim3(1), dim3(kFitThreads), 0, static_cast<hipStream_t>(stream), a);
    return int(hipGetLastError());
}

}  // namespace sv
