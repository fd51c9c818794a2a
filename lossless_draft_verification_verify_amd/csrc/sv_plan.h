// Internal launch plan and workspace layout shared by the host API (capi.cpp)
// and the kernels (verify_kernels.hip, schedule_kernel.hip).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kWG = 256;            // threads per workgroup: 4 wave64s
constexpr int kVecPerThread = 8;    // 16-byte loads in flight per thread in the row pass
constexpr int kRun = 32;            // contiguous elements per thread in the final-draw pass
constexpr int kTile = kWG * kRun;   // elements per final-draw tile (8192)
constexpr int kNanIdx = -2;         // greedy partial: chunk holds a NaN

constexpr unsigned kFlagReady = 1;  // decision record valid
constexpr unsigned kFlagError = 2;  // request has a data error; outputs already written

// Elements per row-pass chunk: 256 threads x 8 loads x 16 bytes.
inline int chunk_elems(int esize) { return kWG * kVecPerThread * (16 / esize); }

// Workspace layout.  The first kCounterBytes hold one 16-byte slot of
// counters per request, {row-pass arrivals, decision flag, draw-pass
// arrivals, unused}, at the same offsets for every shape: these must start at
// zero and every completed call leaves them at zero, so one zero-filled
// workspace stays valid across calls of any shape.  Everything after them is
// written before it is read within a call.
constexpr int kMaxBatch = 65536;
constexpr size_t kSlotBytes = 16;
constexpr size_t kCounterBytes = size_t(kMaxBatch) * kSlotBytes;

struct Layout {
    size_t part;               // [B*(G+1)*nc1] 8 bytes: (max, sum) or (max, argmax)
    size_t dec;                // [B] Decision
    size_t mass;               // [B*ntiles] 2 doubles: (residual mass, target mass) per tile
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout make_layout(int64_t B, int64_t G, int64_t V, int esize) {
    const int64_t nc1 = (V + chunk_elems(esize) - 1) / chunk_elems(esize);
    const int64_t ntiles = (V + kTile - 1) / kTile;
    Layout L;
    size_t o = kCounterBytes;
    L.part = o; o += align256(size_t(B) * size_t(G + 1) * size_t(nc1) * 8);
    L.dec = o;  o += align256(size_t(B) * 32);
    L.mass = o; o += align256(size_t(B) * size_t(ntiles) * 16);
    L.total = o;
    return L;
}

// Per-request decision written by the workgroup that finishes the request's
// row pass, read by the final-draw workgroups.
struct Decision {
    int32_t j;        // accepted drafts
    int32_t row;      // target row of the final draw: always j (j = len when all accepted)
    int32_t resid;    // 1: draw from max(p_j - q_j, 0); 0: draw from p_row
    int32_t pad;
    float m;          // row maximum (logit units)
    float inv_s;      // 1 / S of that row, fp32
    double s;         // S of that row, fp64
};
static_assert(sizeof(Decision) == 32, "Decision is 32 bytes");

struct VerifyArgs {
    const void *logits;
    const float *q;
    const int32_t *x;
    const float *u;
    const int32_t *vlen;
    int32_t *out_acc;
    int32_t *out_tok;
    float *d_lse, *d_p, *d_q, *d_r;
    unsigned char *ws;
    Layout lay;
    int32_t B, G, V;
    float T;          // temperature
    float c32;        // log2(e) / T, the fp32 exponent scale of the row pass
    int32_t nc1, ch1; // row-pass chunks per row, elements per chunk
    int32_t ntiles;   // final-draw tiles per row
    int32_t nc2, tpw; // final-draw workgroups per request, tiles per workgroup
    int32_t lag;      // requests between a request's row pass and its draw items
    int32_t mode;     // 0: one fused launch; 1: row pass only; 2: draw pass only
    uint32_t spin_limit;
};

// Launchers (verify_kernels.hip).  Return a hipError_t as int.
int launch_verify_sampled(const VerifyArgs &a, bool aligned_z, bool aligned_q, int esize,
                          int grid, void *stream);
int launch_verify_greedy(const VerifyArgs &a, bool aligned_z, int esize, int grid, void *stream);
int verify_sampled_occupancy(bool aligned_z, bool aligned_q, int esize, int *blocks_per_cu);

struct ScheduleArgs {
    const float *conf;
    const float *cost;
    int32_t B, G, budget;
    float eps;
    int32_t *out_len;
    int32_t *out_T;
    float *out_tau;
};
int launch_schedule(const ScheduleArgs &a, void *stream);

}  // namespace sv
