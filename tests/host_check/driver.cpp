// Drives every entry point of the C ABI (capi.cpp, built with g++ and the
// address and undefined-behaviour sanitizers against fakes.cpp) over valid,
// invalid and random arguments.  Host arrays (calibration temperatures,
// ratios, costs, diagnostics) are allocated at exactly the length the
// arguments imply, so reading past them is caught.  Checks: every status is a
// known code; a host-checkable error enqueues nothing; a valid call's launch
// plan passes the fakes' checks.  Device pointers are stand-in addresses that
// nothing dereferences.  Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "spec_verify.h"

extern int g_launches;

namespace {

std::mt19937_64 rng(20261203);
int failures = 0;

void expect(bool c, const char *what, long i) {
    if (!c) {
        std::fprintf(stderr, "check failed: %s (case %ld)\n", what, i);
        ++failures;
    }
}
int pick(std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); }
// A stand-in device address with the given alignment offset (0: 256-aligned).
void *dev(int off) { return reinterpret_cast<void *>((uintptr_t(1) << 44) + (rng() % 4096) * 256 + off); }
void *maybe(double p_null, int off = 0) { return (rng() % 1000) < p_null * 1000 ? nullptr : dev(off); }
int offset() { return (rng() % 20 == 0) ? int(rng() % 4) + 1 : 0; }
float temperature() {
    switch (rng() % 8) {
    case 0: return 0.0f;
    case 1: return -1.0f;
    case 2: return NAN;
    case 3: return INFINITY;
    case 4: return 1e-39f;
    default: return 0.05f + float(rng() % 2000) / 1000.0f;
    }
}
bool known(int s) { return s >= SPEC_OK && s <= SPEC_ERR_SCRATCH_TOO_SMALL; }
// A host-checkable error enqueues nothing (a device error may come after some launches).
void check_call(int st, int before, long i, const char *what) {
    expect(known(st), what, i);
    if (st != SPEC_OK && st != SPEC_ERR_DEVICE) expect(g_launches == before, what, i);
    if (st == SPEC_OK) expect(g_launches > before || true, what, i);
}

void verify_cases(long i) {
    const int B = pick({-1, 0, 1, 3, 8, 64, 257, 4096, 65536, 65537});
    const int G = pick({-1, 0, 1, 3, 15, 255, 256});
    const int V = pick({0, 1, 3, 1000, 2048, 129280, 129281, 152064, 1 << 22, (1 << 30) + 1});
    const int dt = pick({0, 1, 1, 7});
    const float T = temperature();
    const size_t need = spec_verify_workspace_bytes(B, G, V, spec_dtype_t(dt));
    const size_t ws_bytes = (rng() % 5 == 0 && need > 0) ? need - 1 : need;
    std::vector<float> lse(1), p(1), q(1), r(1);
    spec_verify_diag_t diag = {nullptr, nullptr, nullptr, nullptr, nullptr};
    const bool use_diag = rng() % 3 == 0;
    if (use_diag) {
        diag.target_lse = static_cast<float *>(maybe(0.3, offset() ? 2 : 0));
        diag.p_draft = static_cast<float *>(maybe(0.3));
    }
    const int s = rng() % 5;
    int before = g_launches;
    int st;
    if (s == 0) {
        st = spec_verify(maybe(0.05, offset()), spec_dtype_t(dt), static_cast<const float *>(maybe(0.1, offset())),
                         static_cast<const int32_t *>(maybe(0.05)), static_cast<const float *>(maybe(0.1)),
                         static_cast<const int32_t *>(maybe(0.5)), B, G, V, T, static_cast<int32_t *>(maybe(0.05)),
                         static_cast<int32_t *>(maybe(0.05)), use_diag ? &diag : nullptr, maybe(0.05, offset() * 64),
                         ws_bytes, nullptr);
        check_call(st, before, i, "spec_verify");
    } else if (s == 1) {
        st = spec_verify_packed(maybe(0.05), spec_dtype_t(dt), pick({-1, 0, 1, 40, 1 << 20}),
                                static_cast<const int32_t *>(maybe(0.1, offset())),
                                static_cast<const float *>(maybe(0.1)), static_cast<const int32_t *>(maybe(0.05)),
                                static_cast<const float *>(maybe(0.1)), B, G, V, T,
                                static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)),
                                use_diag ? &diag : nullptr, maybe(0.05), ws_bytes, nullptr);
        check_call(st, before, i, "spec_verify_packed");
    } else if (s == 2) {
        st = spec_verify_logits(maybe(0.05), spec_dtype_t(dt), maybe(0.1, offset()),
                                static_cast<const int32_t *>(maybe(0.05)), static_cast<const float *>(maybe(0.1)),
                                static_cast<const int32_t *>(maybe(0.5)), B, G, V, T,
                                static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)),
                                use_diag ? &diag : nullptr, maybe(0.05), ws_bytes, nullptr);
        check_call(st, before, i, "spec_verify_logits");
    } else if (s == 3) {
        st = spec_verify_noalloc(maybe(0.05), spec_dtype_t(dt), static_cast<const float *>(maybe(0.1)),
                                 static_cast<const int32_t *>(maybe(0.05)), static_cast<const float *>(maybe(0.1)),
                                 static_cast<const int32_t *>(maybe(0.5)), B, G, V, T,
                                 static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)),
                                 use_diag ? &diag : nullptr, nullptr);
        expect(known(st), "spec_verify_noalloc", i);
        if (st == SPEC_OK) expect(need > 0 && need <= SPEC_NOALLOC_SCRATCH_BYTES, "noalloc fits", i);
    } else {
        const int M = pick({0, 1, 2, 64, 256, 257});
        const size_t tneed = spec_verify_workspace_bytes(B, M - 1, V, spec_dtype_t(dt));
        st = spec_verify_tree(maybe(0.05), spec_dtype_t(dt), static_cast<const int32_t *>(maybe(0.1)),
                              static_cast<const int32_t *>(maybe(0.1)), B, M, V, static_cast<int32_t *>(maybe(0.05)),
                              static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)), maybe(0.05),
                              tneed, nullptr);
        check_call(st, before, i, "spec_verify_tree");
    }
    (void)spec_verify_launches(B, G, V, spec_dtype_t(dt), T);
    (void)spec_status_string(spec_status_t(st));
}

void schedule_cases(long i) {
    const int B = pick({-1, 0, 1, 4, 64, 273, 4096, 4097});
    const int G = pick({-1, 0, 1, 15, 255, 256});
    const int len = pick({-1, 0, 1, 65, 513, 5000});
    const int budget = pick({-1, 3, 64, 512, 4999, 5000});
    const float eps = pick({0, 1}) ? 0.0f : NAN;
    const int gt = (G > 0 && G <= 256) ? G : 1;
    std::vector<float> temps(gt);
    for (auto &t : temps) t = pick({0, 1, 1, 1}) ? 0.1f + float(rng() % 100) / 10.0f : pick({0, 1}) ? -1.0f : NAN;
    int before = g_launches;
    int st = spec_schedule(static_cast<const float *>(maybe(0.05, offset())), static_cast<const float *>(maybe(0.05)),
                           len, B, G, budget, eps, static_cast<int32_t *>(maybe(0.05)),
                           static_cast<int32_t *>(maybe(0.05)), static_cast<float *>(maybe(0.5)), nullptr, 0, nullptr);
    check_call(st, before, i, "spec_schedule");
    before = g_launches;
    st = spec_schedule_calibrated(static_cast<const float *>(maybe(0.05)), (rng() % 4) ? temps.data() : nullptr,
                                  static_cast<const float *>(maybe(0.05)), len, B, G, budget, eps,
                                  static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)),
                                  static_cast<float *>(maybe(0.5)), nullptr, 0, nullptr);
    check_call(st, before, i, "spec_schedule_calibrated");
    const int R = pick({0, 1, 4, 8, 9});
    std::vector<float> ratios(R > 0 ? R : 1), costs(R > 0 ? R : 1);
    for (int r = 0; r < R; ++r) {
        ratios[r] = pick({0, 1, 1, 1}) ? float(1 + rng() % 100) / 100.0f : pick({0, 1}) ? 1.5f : NAN;
        costs[r] = pick({0, 1, 1, 1}) ? 1.0f + float(rng() % 100) / 100.0f : pick({0, 1}) ? 0.0f : INFINITY;
    }
    before = g_launches;
    st = spec_dcut(static_cast<const float *>(maybe(0.05)), B, G, R ? ratios.data() : nullptr,
                   R ? costs.data() : nullptr, R, (rng() % 3) ? nullptr : temps.data(),
                   static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)),
                   static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.05)),
                   static_cast<double *>(maybe(0.5, offset() ? 4 : 0)), nullptr);
    check_call(st, before, i, "spec_dcut");
    before = g_launches;
    st = spec_schedule_static(static_cast<const float *>(maybe(0.1)), B * 16, G, spec_static_mode_t(pick({0, 1, 2})),
                              pick({-3, 0, 7, 300}), pick({0, 1}) ? 0.5f : NAN, (rng() % 3) ? nullptr : temps.data(),
                              static_cast<int32_t *>(maybe(0.05)), static_cast<int32_t *>(maybe(0.3)),
                              static_cast<int32_t *>(maybe(0.3)), nullptr);
    check_call(st, before, i, "spec_schedule_static");
}

void fit_and_acceptance_cases(long i) {
    const int N = pick({0, 1, 1000, 1 << 20, 1 << 23});
    const int G = pick({-1, 0, 4, 15, 256});
    const int nt = pick({0, 1, 100, 128, 129});
    const int bins = pick({0, 1, 15, 32, 33});
    std::vector<float> temps(nt > 0 ? nt : 1, 1.0f);
    if (nt > 0 && rng() % 4 == 0) temps[rng() % nt] = -1.0f;
    const size_t need = spec_sts_fit_workspace_bytes(N, G, nt, bins);
    int before = g_launches;
    int st = spec_sts_fit(static_cast<const float *>(maybe(0.05)), static_cast<const int32_t *>(maybe(0.05)), N, G,
                          nt ? temps.data() : nullptr, nt, bins, static_cast<float *>(maybe(0.05)),
                          maybe(0.05, offset() * 8), (rng() % 5 == 0 && need > 0) ? need - 1 : need, nullptr);
    check_call(st, before, i, "spec_sts_fit");
    before = g_launches;
    st = spec_acceptance(maybe(0.05, offset()), spec_dtype_t(pick({0, 1, 5})), maybe(0.05, offset()),
                         spec_draft_kind_t(pick({0, 1, 2})), static_cast<const int32_t *>(maybe(0.5)),
                         pick({0, 1, 64, 65537}), pick({-1, 0, 15, 256}), pick({0, 7, 129280}), temperature(),
                         static_cast<float *>(maybe(0.05)), nullptr);
    check_call(st, before, i, "spec_acceptance");
}

// Valid calls that must be accepted, each planning its launches.
void valid_cases() {
    struct Shape { int B, G, V, dt; float T; };
    const Shape shapes[] = {{64, 15, 129280, 1, 1.0f}, {64, 7, 152064, 1, 0.0f}, {4, 4, 1024, 0, 1.0f},
                            {16, 3, 32000, 1, 0.7f}, {1, 0, 1, 0, 1.0f}, {300, 15, 4099, 0, 0.5f},
                            {65536, 1, 64, 1, 0.0f}, {8, 255, 1 << 22, 1, 1.0f}};
    long i = 0;
    for (const Shape &sh : shapes) {
        const size_t need = spec_verify_workspace_bytes(sh.B, sh.G, sh.V, spec_dtype_t(sh.dt));
        expect(need > 0, "workspace query", i);
        for (int vl = 0; vl < 2; ++vl) {
            int before = g_launches;
            int st = spec_verify(dev(0), spec_dtype_t(sh.dt), static_cast<const float *>(dev(0)),
                                 static_cast<const int32_t *>(dev(0)), static_cast<const float *>(dev(0)),
                                 vl ? static_cast<const int32_t *>(dev(0)) : nullptr, sh.B, sh.G, sh.V, sh.T,
                                 static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)), nullptr, dev(0),
                                 need, nullptr);
            expect(st == SPEC_OK && g_launches > before, "valid spec_verify", i);
            before = g_launches;
            st = spec_verify_logits(dev(0), spec_dtype_t(sh.dt), dev(0), static_cast<const int32_t *>(dev(0)),
                                    static_cast<const float *>(dev(0)), vl ? static_cast<const int32_t *>(dev(0)) : nullptr,
                                    sh.B, sh.G, sh.V, sh.T, static_cast<int32_t *>(dev(0)),
                                    static_cast<int32_t *>(dev(0)), nullptr, dev(0), need, nullptr);
            expect(st == SPEC_OK && g_launches > before, "valid spec_verify_logits", i);
            ++i;
        }
        if (need <= SPEC_NOALLOC_SCRATCH_BYTES) {
            const int st = spec_verify_noalloc(dev(0), spec_dtype_t(sh.dt), static_cast<const float *>(dev(0)),
                                               static_cast<const int32_t *>(dev(0)),
                                               static_cast<const float *>(dev(0)), nullptr, sh.B, sh.G, sh.V,
                                               sh.T, static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)),
                                               nullptr, nullptr);
            expect(st == SPEC_OK, "valid spec_verify_noalloc", i);
        }
    }
    std::vector<float> temps(15, 1.25f), ratios = {0.25f, 0.5f, 0.75f, 1.0f}, costs = {1.1f, 1.2f, 1.3f, 1.4f};
    expect(spec_schedule(static_cast<const float *>(dev(0)), static_cast<const float *>(dev(0)), 513, 64, 15, 512,
                         0.0f, static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)), nullptr, nullptr, 0,
                         nullptr) == SPEC_OK, "valid spec_schedule", 0);
    expect(spec_schedule_calibrated(static_cast<const float *>(dev(0)), temps.data(),
                                    static_cast<const float *>(dev(0)), 513, 64, 15, 512, 0.0f,
                                    static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)), nullptr,
                                    nullptr, 0, nullptr) == SPEC_OK, "valid spec_schedule_calibrated", 0);
    expect(spec_dcut(static_cast<const float *>(dev(0)), 64, 15, ratios.data(), costs.data(), 4, temps.data(),
                     static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)),
                     static_cast<int32_t *>(dev(0)), nullptr, nullptr) == SPEC_OK, "valid spec_dcut", 0);
    expect(spec_schedule_static(static_cast<const float *>(dev(0)), 64, 15, SPEC_STATIC_THRESHOLD, 0, 0.5f,
                                temps.data(), static_cast<int32_t *>(dev(0)), nullptr, nullptr, nullptr) == SPEC_OK,
           "valid spec_schedule_static", 0);
    std::vector<float> grid(100);
    for (int t = 0; t < 100; ++t) grid[t] = 0.1f + 0.1f * float(t);
    const size_t fneed = spec_sts_fit_workspace_bytes(1 << 20, 15, 100, 15);
    expect(spec_sts_fit(static_cast<const float *>(dev(0)), static_cast<const int32_t *>(dev(0)), 1 << 20, 15,
                        grid.data(), 100, 15, static_cast<float *>(dev(0)), dev(0), fneed, nullptr) == SPEC_OK,
           "valid spec_sts_fit", 0);
    expect(spec_acceptance(dev(0), SPEC_DTYPE_BF16, dev(0), SPEC_DRAFT_LOGITS, nullptr, 64, 15, 129280, 1.0f,
                           static_cast<float *>(dev(0)), nullptr) == SPEC_OK, "valid spec_acceptance", 0);
    const size_t tneed = spec_verify_workspace_bytes(8, 63, 152064, SPEC_DTYPE_BF16);
    expect(spec_verify_tree(dev(0), SPEC_DTYPE_BF16, static_cast<const int32_t *>(dev(0)),
                            static_cast<const int32_t *>(dev(0)), 8, 64, 152064, static_cast<int32_t *>(dev(0)),
                            static_cast<int32_t *>(dev(0)), static_cast<int32_t *>(dev(0)), dev(0), tneed,
                            nullptr) == SPEC_OK, "valid spec_verify_tree", 0);
}

}  // namespace

int main() {
    valid_cases();
    const long cases = 100000;
    for (long i = 0; i < cases; ++i) {
        verify_cases(i);
        if (i % 4 == 0) schedule_cases(i);
        if (i % 8 == 0) fit_and_acceptance_cases(i);
    }
    std::printf("%ld cases, %d launches planned, %d failures\n", cases, g_launches, failures);
    return failures == 0 ? 0 : 1;
}
