// Wave-level DPP reductions and scans for CDNA4 (wave64), shared by the
// verification and scheduling kernels.  Device code only; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {
namespace {

// ---------------------------------------------------------- DPP reductions
//
// Inside a row of 16 lanes: exchange with lane ^ 1, lane ^ 2 (quad
// permutes), then the half-row and row mirrors.  Every step is own + partner
// with a commutative operation, so all 16 lanes end with bitwise the same
// value.  Across the wave the four row results are read with readlane.
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
constexpr int kWaveShr1 = 0x138;

// DPP move; lanes whose source is out of range, or whose row is masked off,
// read 0.
template <int C, int RM = 0xF> __device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, C, RM, 0xF, true);
}
template <int C> __device__ __forceinline__ float dpp_f(float x) { return __int_as_float(dpp_i<C>(__float_as_int(x))); }
template <int C, int RM = 0xF> __device__ __forceinline__ double dpp_d(double x) {
    const uint64_t v = uint64_t(__double_as_longlong(x));
    const uint32_t lo = uint32_t(dpp_i<C, RM>(int(uint32_t(v)))), hi = uint32_t(dpp_i<C, RM>(int(uint32_t(v >> 32))));
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_f(float x, int l) { return __int_as_float(lane_i(__float_as_int(x), l)); }
__device__ __forceinline__ double lane_d(double x, int l) {
    const uint64_t v = uint64_t(__double_as_longlong(x));
    const uint32_t lo = uint32_t(lane_i(int(uint32_t(v)), l)), hi = uint32_t(lane_i(int(uint32_t(v >> 32)), l));
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<kXor1>(x));
    x = fmaxf(x, dpp_f<kXor2>(x));
    x = fmaxf(x, dpp_f<kHalfMirror>(x));
    return fmaxf(x, dpp_f<kMirror>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x = x + dpp_f<kXor1>(x);
    x = x + dpp_f<kXor2>(x);
    x = x + dpp_f<kHalfMirror>(x);
    return x + dpp_f<kMirror>(x);
}
__device__ __forceinline__ double row16_sum_d(double x) {
    x = x + dpp_d<kXor1>(x);
    x = x + dpp_d<kXor2>(x);
    x = x + dpp_d<kHalfMirror>(x);
    return x + dpp_d<kMirror>(x);
}
__device__ __forceinline__ int row16_and(int x) {
    x = x & dpp_i<kXor1>(x);
    x = x & dpp_i<kXor2>(x);
    x = x & dpp_i<kHalfMirror>(x);
    return x & dpp_i<kMirror>(x);
}
__device__ __forceinline__ int row16_min_i(int x) {
    x = min(x, dpp_i<kXor1>(x));
    x = min(x, dpp_i<kXor2>(x));
    x = min(x, dpp_i<kHalfMirror>(x));
    return min(x, dpp_i<kMirror>(x));
}
// Whole-wave results, uniform across the wave.
__device__ __forceinline__ int wave_min_i(int x) {
    x = row16_min_i(x);
    return min(min(lane_i(x, 0), lane_i(x, 16)), min(lane_i(x, 32), lane_i(x, 48)));
}
__device__ __forceinline__ float wave_max(float x) {
    x = row16_max(x);
    return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}
// The butterfly sum; by commutativity it is bitwise the value wave_scan_d
// leaves in lane 63.
__device__ __forceinline__ double wave_sum_d(double x) {
    x = row16_sum_d(x);
    return (lane_d(x, 0) + lane_d(x, 16)) + (lane_d(x, 32) + lane_d(x, 48));
}
// Inclusive prefix across the wave: own + lane - d for d = 1, 2, 4, 8 inside
// each row of 16, then row 0's total into row 1 and row 2's into row 3, then
// the first two rows' total into rows 2 and 3.  (Adding a 0 where a lane has
// no partner leaves it unchanged.)  At lane 63 this is the same tree as
// wave_sum_d's: ((r3 + r2) + (r1 + r0)) with each row total t15 + t7-style.
__device__ __forceinline__ double wave_scan_d(double x) {
    x = x + dpp_d<kRowShr1>(x);
    x = x + dpp_d<kRowShr2>(x);
    x = x + dpp_d<kRowShr4>(x);
    x = x + dpp_d<kRowShr8>(x);
    x = x + dpp_d<kRowBcast15, 0xA>(x);
    x = x + dpp_d<kRowBcast31, 0xC>(x);
    return x;
}

// Inclusive prefix sum of an int over the wave (same DPP pattern).
__device__ __forceinline__ int wave_scan_i(int x) {
    x = x + dpp_i<kRowShr1>(x);
    x = x + dpp_i<kRowShr2>(x);
    x = x + dpp_i<kRowShr4>(x);
    x = x + dpp_i<kRowShr8>(x);
    x = x + dpp_i<kRowBcast15, 0xA>(x);
    x = x + dpp_i<kRowBcast31, 0xC>(x);
    return x;
}

// Inclusive prefix maximum of a non-negative int over the wave (lane 63
// holds the wave's maximum; lanes without a source read 0, the identity).
__device__ __forceinline__ int wave_scan_max_i(int x) {
    x = max(x, dpp_i<kRowShr1>(x));
    x = max(x, dpp_i<kRowShr2>(x));
    x = max(x, dpp_i<kRowShr4>(x));
    x = max(x, dpp_i<kRowShr8>(x));
    x = max(x, dpp_i<kRowBcast15, 0xA>(x));
    x = max(x, dpp_i<kRowBcast31, 0xC>(x));
    return x;
}

}  // namespace
}  // namespace sv
