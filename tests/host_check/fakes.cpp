// Fake device side for the sanitizer build of capi.cpp: the HIP calls it makes
// and the kernel launchers it calls, each checking the launch plan it is given
// against the shape (grid sizes, workspace layout, required pointers) instead
// of launching anything.  Every launch is counted.
#include <cstdio>
#include <cstdlib>

#include "hip/hip_runtime.h"
#include "sv_plan.h"

int g_launches = 0;

#define CHECK(c)                                                                    \
    do {                                                                            \
        if (!(c)) {                                                                 \
            std::fprintf(stderr, "launch-plan check failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
            std::abort();                                                           \
        }                                                                           \
    } while (0)

hipError_t hipGetDevice(int *device) { *device = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t, int) { *value = 256; return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace sv {
namespace {
bool same_layout(const VerifyArgs &a, int es) {
    const LayoutUnits u = to_units(make_layout(a.B, a.G, a.V, es));
    return u.zero == a.lay.zero && u.part == a.lay.part && u.partd == a.lay.partd && u.mass == a.lay.mass &&
           u.gx == a.lay.gx && u.dec == a.lay.dec;
}
void common(const VerifyArgs &a, int es, int grid) {
    CHECK(grid > 0);
    CHECK(a.B >= 1 && a.G >= 0 && a.V >= 1);
    CHECK(a.ws != nullptr && (reinterpret_cast<uintptr_t>(a.ws) & 255) == 0);
    CHECK(same_layout(a, es));
    CHECK(a.logits && a.out_acc && a.out_tok);
    CHECK(a.nc1 == (a.V + a.ch1 - 1) / a.ch1 && a.ch1 == chunk_elems(es));
    CHECK(a.nsub == (a.V + kSub - 1) / kSub);
    ++g_launches;
}
}  // namespace

int launch_rows_sampled(const VerifyArgs &a, bool, int es, int grid, void *) {
    common(a, es, grid);
    CHECK(a.G == 0 || a.x);
    CHECK(long(grid) == long(a.B) * ((a.G + 1) + (a.dl ? a.G : 0)) * a.np1);
    return 0;
}
int launch_rows_sampled_vl(const VerifyArgs &a, bool, int es, int grid, void *) {
    common(a, es, grid);
    CHECK(a.B <= kWG && (a.vlen || a.roff));
    return 0;
}
int launch_requests_sampled(const VerifyArgs &a, bool, bool, int es, int grid, void *) {
    common(a, es, grid);
    CHECK(a.G == 0 || a.x);
    CHECK(a.u && (a.G == 0 || a.q || a.dl));
    CHECK(a.spw >= 1 && a.nc2 * a.spw >= a.nsub && (a.nc2 - 1) * a.spw < a.nsub);
    CHECK(long(grid) == long(a.B) * a.nc2);
    return 0;
}
int launch_verify_sampled(const VerifyArgs &a, bool, bool, int es, int grid, void *) {
    common(a, es, grid);
    CHECK(a.G == 0 || a.x);
    CHECK(!a.dl && a.u && (a.G == 0 || a.q));
    CHECK(a.spw >= 1 && a.nc2 * a.spw >= a.nsub && (a.nc2 - 1) * a.spw < a.nsub);
    if (a.vlrows == 0) {
        CHECK(long(grid) == long(a.B) * ((a.G + 1) * a.np1 + 1 + a.nc2));
    } else {                                        // verify lengths: at most one resident load of row workgroups
        CHECK(a.B <= kWG && (a.vlen || a.roff));
        CHECK(a.vlrows >= 1 && a.vlrows <= long(a.B) * (a.G + 1) * a.np1 && a.vlrows <= 8L * 256);
        CHECK(long(grid) == a.vlrows + long(a.B) * (1 + a.nc2));
    }
    return 0;
}
int launch_verify_greedy(const VerifyArgs &a, bool, int es, int grid, void *) {
    common(a, es, grid);
    const long rows = long(a.B) * (a.G + 1) * a.np1;
    CHECK(a.mode == 1 || a.G == 0 || a.x);          // the tree's row pass (mode 1) reads no draft ids
    CHECK((a.mode == 0 && grid == rows + a.B) || (a.mode == 1 && grid == rows) || (a.mode == 2 && grid == a.B));
    return 0;
}
int greedy_occupancy(bool, int, int *n) { *n = 8; return 0; }
int launch_tree_fused(const VerifyArgs &a, bool, int es, int grid, void *) {
    common(a, es, grid);
    CHECK(a.out_path && (a.G == 0 || (a.tpar && a.ttok)));
    CHECK(long(grid) == long(a.B) * (a.G + 1) * a.np1 + a.B);
    return 0;
}
int launch_tree_walk(const VerifyArgs &a, int grid, void *) {
    CHECK(grid == a.B && a.out_path && (a.G == 0 || (a.tpar && a.ttok)));
    ++g_launches;
    return 0;
}
int noalloc_scratch(int, void **out) {
    *out = reinterpret_cast<void *>(uintptr_t(1) << 40);   // a stand-in device address, never dereferenced
    return 0;
}
int launch_zero(void *p, size_t bytes, void *) {
    CHECK(p && bytes % 256 == 0 && bytes <= kNoAllocScratchBytes);
    ++g_launches;
    return 0;
}
int launch_schedule(const ScheduleArgs &a, void *) {
    CHECK(a.B >= 1 && a.G >= 0 && long(a.B) * a.G <= 4096 && a.budget >= a.B && a.cost && a.out_len && a.out_T);
    CHECK(!a.cal.on || a.G <= kMaxDrafts);
    ++g_launches;
    return 0;
}
int launch_dcut(const DcutArgs &a, void *) {
    CHECK(a.R >= 1 && a.R <= kMaxRatios && a.out_len && a.out_off && a.out_ratio && a.out_rows);
    for (int r = 0; r < a.R; ++r) CHECK(a.keep[r] >= 0 && a.keep[r] <= a.B * a.G && a.cost[r] > 0.0f);
    ++g_launches;
    return 0;
}
int launch_static(const StaticArgs &a, void *) {
    CHECK(a.B >= 1 && a.G >= 0 && a.out_len && (a.mode == 0 || a.mode == 1));
    ++g_launches;
    return 0;
}
int launch_fit_accumulate(const FitArgs &a, void *) {
    CHECK(a.N >= 1 && a.nt >= 1 && a.nt <= kFitMaxTemps && a.bins >= 1 && a.bins <= kFitMaxBins);
    CHECK(a.k >= 0 && a.k < a.G && a.nwg >= 1 && a.prefix && a.part && a.err);
    ++g_launches;
    return 0;
}
int launch_fit_choose(const FitArgs &a, void *) {
    CHECK(a.out_temps && a.k < a.G);
    ++g_launches;
    return 0;
}
int launch_acceptance(const AcceptArgs &a, bool, int, bool, void *) {
    CHECK(a.B >= 1 && a.G >= 1 && a.V >= 1 && a.z && a.d && a.out && a.c32 > 0.0f);
    ++g_launches;
    return 0;
}
}  // namespace sv
