// Internal launch plan and workspace layout shared by the host API (capi.cpp)
// and the kernels (verify_kernels.hip, schedule_kernel.hip).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kWG = 256;            // threads per workgroup: 4 wave64s
constexpr int kWaves = kWG / 64;    // waves per workgroup
constexpr int kRowVec = 4;          // 16-byte loads per lane of a row-pass chunk
constexpr int kSubPerThread = 8;    // contiguous elements per thread in a draw sub-tile
constexpr int kSub = kWG * kSubPerThread;   // elements per draw sub-tile (2048)
constexpr int kSubBatch = 2;        // sub-tiles loaded together by a draw workgroup
constexpr int kNanIdx = -2;         // greedy partial: chunk holds a NaN

// Elements per row-pass chunk, the unit of one wave: 64 lanes x 4 loads x 16
// bytes (2048 bf16 or 1024 fp32 values).
inline int chunk_elems(int esize) { return 64 * kRowVec * (16 / esize); }

// Workspace.  Between calls every byte the kernels use is zero: each word is
// reset by the last workgroup that reads it, and every word carries its own
// written mark (nothing is a counter), so one zero-filled workspace stays
// valid across calls of any shape.
//   zero     256 bytes never written: the draft row a bonus draw reads in
//            place of q (so the draw loads need no branch);
//   partd    [B*G*np1] u64 partials of the draft rows, same format (draft
//            logits only);
//   part     [B*(G+1)*np1] u64 partials, bit 63 set once written
//            one per row workgroup of kWaves chunks (np1 = ceil(nc1 / kWaves)
//            per row; the region is sized for nc1): sampled, low = max bits,
//            high = sum bits | 1<<31; greedy, low = max bits, high =
//            (argmax + 2) | 1<<31 (argmax -2: a NaN, -1: none);
//   mass     [B*nsub] 2 u64: fp64 (residual mass, target mass) per sub-tile,
//            bit 63 set once written;
//   gx       [B*G] u64: the row pass's gather of draft k (sampled only):
//            low = fp32 bits of z[b,k,x_k], high = bits of q[b,k,x_k] (with
//            draft logits: of d[b,k,x_k], stored by the draft row's pass;
//            in the one-launch verify, max(q, 0) with bit 63 set once written);
//   dec      [B] 4 u64: the one-launch verify's decision record of request b,
//            each word with bit 63 set once written: word 0 low = fp32 bits
//            of m_j, high = j | resid << 15 | ok << 16; word 1 low = fp32
//            bits of 1 / S_j; word 2 (written once every read row and gather
//            has been checked) bit 0 = no data error; word 3 unused.

constexpr int kMaxBatch = 65536;
constexpr uint32_t kValid = 0x80000000u;

struct Layout {
    size_t zero;
    size_t part;
    size_t partd;
    size_t mass;
    size_t gx;
    size_t dec;
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout make_layout(int64_t B, int64_t G, int64_t V, int esize) {
    const int64_t nc1 = (V + chunk_elems(esize) - 1) / chunk_elems(esize);
    const int64_t nsub = (V + kSub - 1) / kSub;
    Layout L;
    size_t o = 0;
    L.zero = o; o += 256;
    L.part = o; o += align256(size_t(B) * size_t(G + 1) * size_t(nc1) * 8);
    L.partd = o; o += align256(size_t(B) * size_t(G) * size_t(nc1) * 8);
    L.mass = o; o += align256(size_t(B) * size_t(nsub) * 16);
    L.gx = o; o += align256(size_t(B) * size_t(G) * 8);
    L.dec = o; o += align256(size_t(B) * 32);
    L.total = o;
    return L;
}

// The layout as the kernels take it: each region's offset in units of 256
// bytes (every region is 256-byte aligned), so that the kernel arguments stay
// small.
struct LayoutUnits {
    uint32_t zero, part, partd, mass, gx, dec;
};
inline LayoutUnits to_units(const Layout &L) {
    return {uint32_t(L.zero >> 8), uint32_t(L.part >> 8), uint32_t(L.partd >> 8), uint32_t(L.mass >> 8),
            uint32_t(L.gx >> 8), uint32_t(L.dec >> 8)};
}

struct VerifyArgs {
    const void *logits;
    const float *q;
    const void *dl;       // draft logits [B, G, V] of the target dtype (NULL: draft probabilities q)
    const int32_t *x;
    const float *u;
    const int32_t *vlen;
    const int32_t *roff;  // packed target rows: [B+1] row offsets (NULL: [B, G+1, V] rows)
    int32_t rows;         // rows of a packed target buffer
    int32_t *out_acc;
    int32_t *out_tok;
    float *d_lse, *d_p, *d_q, *d_r;
    unsigned char *ws;
    LayoutUnits lay;
    int32_t B, G, V;
    float T;          // temperature
    float c32;        // log2(e) / T, the fp32 exponent scale
    int32_t nc1, ch1; // row-pass chunks (waves) per row, elements per chunk
    int32_t np1;      // partials per row: ceil(nc1 / kWaves), one per row workgroup
    int32_t nsub;     // draw sub-tiles per row
    int32_t nc2, spw; // request workgroups per request, sub-tiles per workgroup
    int32_t mode;     // greedy kernel: 0 row items then request items; 1 row items only; 2 request items only
    const int32_t *tpar, *ttok;   // tree walk: [B, G+1] parents and tokens of the candidate nodes
    int32_t *out_path;            // tree walk: [B, G+1] accepted nodes, then -1
    uint32_t spin_limit;
    int32_t lag;                  // one-launch verify: requests between a request's rows and its decision workgroup
    int32_t vlrows;               // one-launch verify with verify lengths: its row workgroups (0: full grid)
};

// Launchers (verify_kernels.hip).  Return a hipError_t as int.
int launch_rows_sampled(const VerifyArgs &a, bool aligned_z, int esize, int grid, void *stream);
int launch_rows_sampled_vl(const VerifyArgs &a, bool aligned_z, int esize, int grid, void *stream);
int launch_requests_sampled(const VerifyArgs &a, bool aligned_z, bool aligned_q, int esize, int grid,
                            void *stream);   // draft logits when a.dl is set
// One launch: the row workgroups, a decision workgroup per request, then the
// request workgroups (draft probabilities only); a.vlrows > 0: the row
// workgroups are a.vlrows of the verify-length kind.
int launch_verify_sampled(const VerifyArgs &a, bool aligned_z, bool aligned_q, int esize, int grid, void *stream);
int launch_verify_greedy(const VerifyArgs &a, bool aligned_z, int esize, int grid, void *stream);
int greedy_occupancy(bool aligned_z, int esize, int *blocks_per_cu);
int launch_tree_walk(const VerifyArgs &a, int grid, void *stream);
// Tree verification in one launch: B * M * np1 row workgroups, then B walks.
int launch_tree_fused(const VerifyArgs &a, bool aligned_z, int esize, int grid, void *stream);

// Static scratch of spec_verify_noalloc (noalloc.hip): its size, this
// device's address of it (asked once per device), and a fill kernel that
// clears its first `bytes` (a multiple of 256) on `stream`.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
int noalloc_scratch(int dev, void **out);
int launch_zero(void *p, size_t bytes, void *stream);

constexpr int kMaxDrafts = 255;
// Sequential Temperature Scaling, applied as confidences are loaded:
// c~ = float32(2^(log2(c) / T_k)) in double, when calib is set.
struct Calib {
    int32_t on;
    float temp[kMaxDrafts];
};

struct ScheduleArgs {
    const float *conf;
    const float *cost;
    int32_t B, G, budget;
    float eps;
    Calib cal;
    int32_t *out_len;
    int32_t *out_T;
    float *out_tau;
};
int launch_schedule(const ScheduleArgs &a, void *stream);

constexpr int kMaxRatios = 8;
struct DcutArgs {
    const float *conf;
    int32_t B, G, R;
    Calib cal;
    float cost[kMaxRatios];   // profiled cost of each ratio at this batch size, in the caller's order
    int32_t keep[kMaxRatios]; // drafts kept by each ratio: K_rho - B
    int32_t *out_len;         // [B]
    int32_t *out_off;         // [B+1]
    int32_t *out_ratio;       // [1]
    int32_t *out_rows;        // [1]
    double *out_utility;      // [R] or NULL
};
int launch_dcut(const DcutArgs &a, void *stream);

// Static scheduler: fixed length (mode 0) or leading confidences above tau (mode 1).
struct StaticArgs {
    const float *conf;
    int32_t B, G, mode, len;
    float tau;
    Calib cal;
    int32_t *out_len;         // [B]
    int32_t *out_T;           // [1] sum of (len + 1), or NULL
    int32_t *out_off;         // [B+1] packed row offsets, or NULL
};
int launch_static(const StaticArgs &a, void *stream);

// Sequential Temperature Scaling fit, one position per pair of launches.
struct FitArgs {
    const float *conf;        // [N, G]
    const int32_t *acc_len;   // [N]
    float *out_temps;         // [G]
    double *prefix;           // workspace [N]: calibrated survival of the positions fitted so far
    int64_t *part;            // workspace [nwg][nt][bins][2]: labels, fixed-point predictions
    double *err;              // workspace [nt]: the calibration error of each grid point
    int32_t N, G, nt, bins, nwg, k;
    float temps[128];         // the grid
};
constexpr int kFitMaxTemps = 128, kFitMaxBins = 32, kFitThreads = 1024;
constexpr double kFitScale = 1099511627776.0;   // 2^40: fixed-point unit of the prediction sums
int launch_fit_accumulate(const FitArgs &a, void *stream);
int launch_fit_choose(const FitArgs &a, void *stream);   // two launches: per-temperature error, then the argmin

struct AcceptArgs {
    const void *z;            // [B, G+1, V] target logits
    const void *d;            // [B, G, V] draft probabilities (fp32) or draft logits (target dtype)
    const int32_t *vlen;      // [B] or NULL
    float *out;               // [B, G] alpha
    int32_t B, G, V;
    float c32;                // log2(e) / T
};
int launch_acceptance(const AcceptArgs &a, bool aligned, int esize, bool draft_logits, void *stream);

}  // namespace sv
