// Host side of the C ABI: argument validation (before any HIP call), launch
// planning from the device's resident capacity, and kernel launches.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "spec_verify.h"
#include "sv_plan.h"

static_assert(SPEC_MAX_BATCH == sv::kMaxBatch, "one batch limit for the header and the kernels");
static_assert(SPEC_MAX_RATIOS == sv::kMaxRatios, "one ratio limit for the header and the kernels");
static_assert(SPEC_NOALLOC_SCRATCH_BYTES == sv::kNoAllocScratchBytes, "one scratch size for the header and the library");

namespace {

using sv::Layout;

int esize_of(int dt) {
    if (dt == SPEC_DTYPE_F32) return 4;
    if (dt == SPEC_DTYPE_BF16) return 2;
    return 0;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape limits of the verify launch: grid size and 32-bit element offsets
// inside a row stay representable.
spec_status_t check_verify_shape(int64_t B, int64_t G, int64_t V, int es) {
    if (B < 1 || G < 0 || V < 1) return SPEC_ERR_BAD_SHAPE;
    if (B > SPEC_MAX_BATCH || G > SPEC_MAX_DRAFTS || V > SPEC_MAX_VOCAB) return SPEC_ERR_UNSUPPORTED;
    const int64_t nc1 = (V + sv::chunk_elems(es) - 1) / sv::chunk_elems(es);
    const int64_t nsub = (V + sv::kSub - 1) / sv::kSub;
    const int64_t items = B * ((2 * G + 1) * nc1 + nsub + 1);   // row groups (target, draft rows) + decision + request workgroups
    if (items >= (int64_t(1) << 31)) return SPEC_ERR_UNSUPPORTED;
    if (B * (G + 1) > (int64_t(1) << 40) / V) return SPEC_ERR_UNSUPPORTED;
    return SPEC_OK;
}

struct DeviceInfo {
    bool ready = false;
    int cus = 0;
    int occ[2][2] = {};   // [esize==2][aligned_z] greedy-kernel blocks per CU, 0 = unknown
};
std::mutex g_mu;
DeviceInfo g_dev[128];

// Resident workgroups of the greedy verify kernel on this device; -1 on error.
long resident_capacity(int dev, bool az, int es) {
    if (dev < 0 || dev >= 128) return -1;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.ready) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return -1;
        d.cus = cus;
        d.ready = true;
    }
    int &o = d.occ[es == 2][az];
    if (o == 0) {
        int n = 0;
        if (sv::greedy_occupancy(az, es, &n) != 0 || n <= 0) return -1;
        o = n;
    }
    return long(o) * d.cus;
}

// Host-validated STS temperatures (NULL: none) into the kernel arguments.
spec_status_t set_calib(sv::Calib &cal, const float *temps, int32_t G) {
    cal.on = 0;
    if (!temps) return SPEC_OK;
    if (G > sv::kMaxDrafts) return SPEC_ERR_UNSUPPORTED;
    for (int k = 0; k < G; ++k) {
        if (!std::isfinite(temps[k]) || !(temps[k] > 0.0f)) return SPEC_ERR_BAD_SHAPE;
        cal.temp[k] = temps[k];
    }
    cal.on = 1;
    return SPEC_OK;
}

// Greedy launch plan: whether the per-request workgroups share the row
// launch (they wait for their rows, so they stay below half the resident
// capacity).  -1 on a device query failure.
int greedy_one_launch(int dev, bool az, int es, long B) {
    const long cap = resident_capacity(dev, az, es);
    if (cap <= 0) return -1;
    return B <= cap / 2;
}

}  // namespace

extern "C" {

const char *spec_status_string(spec_status_t s) {
    switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SPEC_ERR_BAD_SHAPE: return "shape, table, budget, eps, ratio or cost out of range";
    case SPEC_ERR_BAD_TEMPERATURE: return "temperature must be 0 or a finite value >= 2^-126";
    case SPEC_ERR_BAD_DTYPE: return "unknown dtype";
    case SPEC_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the workspace-size query";
    case SPEC_ERR_UNSUPPORTED: return "shape beyond this build's limits";
    case SPEC_ERR_DEVICE: return "HIP error while querying the device or launching";
    case SPEC_ERR_MISALIGNED: return "pointer misaligned for its element type (workspace: 256 bytes)";
    case SPEC_ERR_SCRATCH_TOO_SMALL:
        return "spec_verify_noalloc: the shape needs more workspace than the static scratch holds "
               "(SPEC_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

size_t spec_verify_workspace_bytes(int32_t B, int32_t G, int32_t V, spec_dtype_t dt) {
    const int es = esize_of(int(dt));
    if (es == 0 || check_verify_shape(B, G, V, es) != SPEC_OK) return 0;
    return sv::make_layout(B, G, V, es).total;
}

}  // extern "C"

namespace {

// spec_verify and spec_verify_packed: the target rows are [B, G+1, V]
// (row_offsets NULL) or `rows` packed rows addressed through row_offsets.
spec_status_t verify_impl(const void *target_logits, spec_dtype_t target_dtype, const int32_t *row_offsets,
                          int32_t rows, const float *draft_probs, const void *draft_logits,
                          const int32_t *draft_tokens,
                          const float *uniforms, const int32_t *verify_len, int32_t B, int32_t G, int32_t V,
                          float temperature, int32_t *out_accepted, int32_t *out_tokens,
                          const spec_verify_diag_t *diag, void *workspace, size_t workspace_bytes,
                          spec_stream_t stream, bool noalloc = false) {
    // ---- host-checkable errors, before anything touches the device
    const int es = esize_of(int(target_dtype));
    if (es == 0) return SPEC_ERR_BAD_DTYPE;
    const spec_status_t sh = check_verify_shape(B, G, V, es);
    if (sh != SPEC_OK) return sh;
    if (row_offsets) {
        if (rows < 1) return SPEC_ERR_BAD_SHAPE;
        if (int64_t(rows) > (int64_t(1) << 40) / V) return SPEC_ERR_UNSUPPORTED;
        if (!aligned(row_offsets, 4)) return SPEC_ERR_MISALIGNED;
    }
    const float T = temperature;
    if (!std::isfinite(T) || T < 0.0f || (T > 0.0f && T < 1.17549435e-38f)) return SPEC_ERR_BAD_TEMPERATURE;
    const bool sampled = T > 0.0f;
    if (!target_logits || !out_accepted || !out_tokens) return SPEC_ERR_NULL_POINTER;
    if (G > 0 && !draft_tokens) return SPEC_ERR_NULL_POINTER;
    if (sampled && G > 0 && !draft_probs && !draft_logits) return SPEC_ERR_NULL_POINTER;
    if (!aligned(draft_logits, es)) return SPEC_ERR_MISALIGNED;
    if (sampled && !uniforms) return SPEC_ERR_NULL_POINTER;
    if (!aligned(target_logits, es) || !aligned(draft_probs, 4) || !aligned(draft_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(verify_len, 4) || !aligned(out_accepted, 4) ||
        !aligned(out_tokens, 4))
        return SPEC_ERR_MISALIGNED;
    spec_verify_diag_t dg = {nullptr, nullptr, nullptr, nullptr, nullptr};
    hipEvent_t row_event = diag ? static_cast<hipEvent_t>(diag->row_pass_event) : nullptr;
    if (diag && sampled) dg = *diag;
    if (!aligned(dg.target_lse, 4) || !aligned(dg.p_draft, 4) || !aligned(dg.q_draft, 4) ||
        !aligned(dg.resid_mass, 4))
        return SPEC_ERR_MISALIGNED;
    const Layout lay = sv::make_layout(B, G, V, es);
    if (noalloc) {
        // the static scratch stands in for the workspace
        if (lay.total > sv::kNoAllocScratchBytes) return SPEC_ERR_SCRATCH_TOO_SMALL;
    } else {
        if (!workspace) return SPEC_ERR_NULL_POINTER;
        if (!aligned(workspace, 256)) return SPEC_ERR_MISALIGNED;
        if (workspace_bytes < lay.total) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_ERR_DEVICE;
    if (noalloc) {
        // this device's address of the scratch, then clear what the call uses
        if (sv::noalloc_scratch(dev, &workspace) != 0) return SPEC_ERR_DEVICE;
        if (sv::launch_zero(workspace, lay.total, stream) != 0) return SPEC_ERR_DEVICE;
    }

    // ---- launch plan
    sv::VerifyArgs a = {};
    a.logits = target_logits;
    a.q = draft_probs;
    a.dl = (sampled && G > 0) ? draft_logits : nullptr;   // the greedy limit never reads the draft
    a.x = draft_tokens;
    a.u = uniforms;
    a.vlen = verify_len;
    a.roff = row_offsets;
    a.rows = rows;
    a.out_acc = out_accepted;
    a.out_tok = out_tokens;
    a.d_lse = dg.target_lse;
    a.d_p = dg.p_draft;
    a.d_q = dg.q_draft;
    a.d_r = dg.resid_mass;
    a.ws = static_cast<unsigned char *>(workspace);
    a.lay = sv::to_units(lay);
    a.B = B;
    a.G = G;
    a.V = V;
    a.T = T;
    a.c32 = sampled ? float(1.4426950408889634 / double(T)) : 0.0f;
    a.ch1 = sv::chunk_elems(es);
    a.nc1 = (V + a.ch1 - 1) / a.ch1;
    a.nsub = (V + sv::kSub - 1) / sv::kSub;
    a.spin_limit = 1u << 20;
    const bool az = aligned(target_logits, 16) && (size_t(V) * es) % 16 == 0;
    const bool aq = a.dl ? aligned(a.dl, 16) && (size_t(V) * es) % 16 == 0 : aligned(draft_probs, 16) && V % 4 == 0;

    if (sampled) {
        // Row pass, then request pass (the kernel boundary orders every row
        // partial before the per-request work, across all XCDs).  One row
        // workgroup per (request, row, group of kWaves chunks).
        a.np1 = (a.nc1 + sv::kWaves - 1) / sv::kWaves;
        const long row_groups = long(B) * ((G + 1) + (a.dl ? G : 0)) * a.np1;   // target rows, draft rows
        // Sub-tiles per draw workgroup: about 1024 draw workgroups in all (each
        // one repeats the request's decision, so fewer and longer ones keep
        // that traffic from queueing behind the draw streams).
        {
            const long want = (long(B) * a.nsub + 1023) / 1024;
            int spw = 1;
            while (spw < want && spw < 8) spw <<= 1;
            a.spw = spw;
        }
        a.nc2 = (a.nsub + a.spw - 1) / a.spw;
        const bool vl_pass = (verify_len || row_offsets) && B <= sv::kWG;
        if (!a.dl) {
            // One launch (draft probabilities): the row
            // workgroups, one decision workgroup per request (in grid order one
            // request after its rows), then the request workgroups, which only
            // poll the request's decision record: about 2048 of them in all
            // (B = 64: 2048 at 51.4 us per call, against 1024 at 52.7 and 4096
            // at 52.1).  Each waits only on workgroups before it in grid order.
            const long want = (long(B) * a.nsub + 2047) / 2048;
            int spw = 1;
            while (spw < want && spw < 8) spw <<= 1;
            a.spw = spw;
            a.nc2 = (a.nsub + a.spw - 1) / a.spw;
            a.lag = 1;
            long rows = row_groups;
            if (vl_pass) {
                // Verify lengths leave rows unread: at most one resident load
                // of row workgroups that visit only the read row groups.
                const long cap = resident_capacity(dev, az, es);
                if (cap <= 0) return SPEC_ERR_DEVICE;
                rows = std::min(row_groups, cap);
                a.vlrows = int32_t(rows);
            }
            if (sv::launch_verify_sampled(a, az, aq, es, int(rows + long(B) * (1 + a.nc2)), stream) != 0)
                return SPEC_ERR_DEVICE;
            if (row_event && hipEventRecord(row_event, static_cast<hipStream_t>(stream)) != hipSuccess)
                return SPEC_ERR_DEVICE;
            return SPEC_OK;
        }
        if (vl_pass) {
            // Draft logits with verify lengths: a grid of two resident loads of
            // workgroups (no workgroup waits on another) whose workgroups visit
            // only the read row groups.  Two loads measured best: one leaves
            // the last jobs of a busy workgroup queued behind its earlier ones
            // (static, B = 64: 49.3 against 47.2 us per call), four add more
            // length prefixes than they save (48.3 us).
            const long cap = resident_capacity(dev, az, es);
            if (cap <= 0) return SPEC_ERR_DEVICE;
            if (sv::launch_rows_sampled_vl(a, az, es, int(std::min(row_groups, 2 * cap)), stream) != 0)
                return SPEC_ERR_DEVICE;
        } else if (sv::launch_rows_sampled(a, az, es, int(row_groups), stream) != 0) {
            return SPEC_ERR_DEVICE;
        }
        if (row_event && hipEventRecord(row_event, static_cast<hipStream_t>(stream)) != hipSuccess)
            return SPEC_ERR_DEVICE;
        return sv::launch_requests_sampled(a, az, aq, es, int(long(B) * a.nc2), stream) == 0 ? SPEC_OK
                                                                                            : SPEC_ERR_DEVICE;
    }
    // Greedy: the per-request items are cheap and wait for their rows, so they
    // share the row launch while they stay below half the resident capacity.
    const int one = greedy_one_launch(dev, az, es, B);
    if (one < 0) return SPEC_ERR_DEVICE;
    // One row workgroup per (request, row, group of kWaves chunks).
    a.np1 = (a.nc1 + sv::kWaves - 1) / sv::kWaves;
    const long row_wgs = long(B) * (G + 1) * a.np1;
    a.nc2 = 1;
    if (one) {
        a.mode = 0;
        if (sv::launch_verify_greedy(a, az, es, int(row_wgs + B), stream) != 0) return SPEC_ERR_DEVICE;
        if (row_event && hipEventRecord(row_event, static_cast<hipStream_t>(stream)) != hipSuccess)
            return SPEC_ERR_DEVICE;
        return SPEC_OK;
    }
    a.mode = 1;
    if (sv::launch_verify_greedy(a, az, es, int(row_wgs), stream) != 0) return SPEC_ERR_DEVICE;
    if (row_event && hipEventRecord(row_event, static_cast<hipStream_t>(stream)) != hipSuccess)
        return SPEC_ERR_DEVICE;
    a.mode = 2;
    return sv::launch_verify_greedy(a, az, es, B, stream) == 0 ? SPEC_OK : SPEC_ERR_DEVICE;
}

}  // namespace

extern "C" {

spec_status_t spec_verify(const void *target_logits, spec_dtype_t target_dtype, const float *draft_probs,
                          const int32_t *draft_tokens, const float *uniforms, const int32_t *verify_len,
                          int32_t B, int32_t G, int32_t V, float temperature, int32_t *out_accepted,
                          int32_t *out_tokens, const spec_verify_diag_t *diag, void *workspace,
                          size_t workspace_bytes, spec_stream_t stream) {
    return verify_impl(target_logits, target_dtype, nullptr, 0, draft_probs, nullptr, draft_tokens, uniforms,
                       verify_len, B, G, V, temperature, out_accepted, out_tokens, diag, workspace, workspace_bytes,
                       stream);
}

spec_status_t spec_verify_noalloc(const void *target_logits, spec_dtype_t target_dtype, const float *draft_probs,
                                  const int32_t *draft_tokens, const float *uniforms, const int32_t *verify_len,
                                  int32_t B, int32_t G, int32_t V, float temperature, int32_t *out_accepted,
                                  int32_t *out_tokens, const spec_verify_diag_t *diag, spec_stream_t stream) {
    return verify_impl(target_logits, target_dtype, nullptr, 0, draft_probs, nullptr, draft_tokens, uniforms,
                       verify_len, B, G, V, temperature, out_accepted, out_tokens, diag, nullptr, 0, stream,
                       /*noalloc=*/true);
}

spec_status_t spec_verify_logits(const void *target_logits, spec_dtype_t target_dtype, const void *draft_logits,
                                 const int32_t *draft_tokens, const float *uniforms, const int32_t *verify_len,
                                 int32_t B, int32_t G, int32_t V, float temperature, int32_t *out_accepted,
                                 int32_t *out_tokens, const spec_verify_diag_t *diag, void *workspace,
                                 size_t workspace_bytes, spec_stream_t stream) {
    if (G > 0 && temperature > 0.0f && !draft_logits) return SPEC_ERR_NULL_POINTER;
    return verify_impl(target_logits, target_dtype, nullptr, 0, nullptr, draft_logits, draft_tokens, uniforms,
                       verify_len, B, G, V, temperature, out_accepted, out_tokens, diag, workspace, workspace_bytes,
                       stream);
}

spec_status_t spec_verify_packed(const void *target_logits, spec_dtype_t target_dtype, int32_t rows,
                                 const int32_t *row_offsets, const float *draft_probs,
                                 const int32_t *draft_tokens, const float *uniforms, int32_t B, int32_t G,
                                 int32_t V, float temperature, int32_t *out_accepted, int32_t *out_tokens,
                                 const spec_verify_diag_t *diag, void *workspace, size_t workspace_bytes,
                                 spec_stream_t stream) {
    if (!row_offsets) return SPEC_ERR_NULL_POINTER;
    return verify_impl(target_logits, target_dtype, row_offsets, rows, draft_probs, nullptr, draft_tokens, uniforms,
                       nullptr, B, G, V, temperature, out_accepted, out_tokens, diag, workspace,
                       workspace_bytes, stream);
}

spec_status_t spec_verify_tree(const void *target_logits, spec_dtype_t target_dtype, const int32_t *parents,
                               const int32_t *node_tokens, int32_t B, int32_t M, int32_t V, int32_t *out_accepted,
                               int32_t *out_tokens, int32_t *out_path, void *workspace, size_t workspace_bytes,
                               spec_stream_t stream) {
    const int es = esize_of(int(target_dtype));
    if (es == 0) return SPEC_ERR_BAD_DTYPE;
    if (M < 1) return SPEC_ERR_BAD_SHAPE;
    if (M > SPEC_MAX_DRAFTS + 1) return SPEC_ERR_UNSUPPORTED;
    const int32_t G = M - 1;
    const spec_status_t sh = check_verify_shape(B, G, V, es);
    if (sh != SPEC_OK) return sh;
    if (!target_logits || !out_accepted || !out_tokens || !out_path || !workspace) return SPEC_ERR_NULL_POINTER;
    if (M > 1 && (!parents || !node_tokens)) return SPEC_ERR_NULL_POINTER;
    if (!aligned(target_logits, es) || !aligned(parents, 4) || !aligned(node_tokens, 4) ||
        !aligned(out_accepted, 4) || !aligned(out_tokens, 4) || !aligned(out_path, 4) || !aligned(workspace, 256))
        return SPEC_ERR_MISALIGNED;
    const Layout lay = sv::make_layout(B, G, V, es);
    if (workspace_bytes < lay.total) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    sv::VerifyArgs a = {};
    a.logits = target_logits;
    a.out_acc = out_accepted;
    a.out_tok = out_tokens;
    a.out_path = out_path;
    a.tpar = parents;
    a.ttok = node_tokens;
    a.ws = static_cast<unsigned char *>(workspace);
    a.lay = sv::to_units(lay);
    a.B = B;
    a.G = G;
    a.V = V;
    a.ch1 = sv::chunk_elems(es);
    a.nc1 = (V + a.ch1 - 1) / a.ch1;
    a.np1 = (a.nc1 + sv::kWaves - 1) / sv::kWaves;
    a.nsub = (V + sv::kSub - 1) / sv::kSub;
    a.nc2 = 1;
    a.spin_limit = 1u << 20;
    const bool az = aligned(target_logits, 16) && (size_t(V) * es) % 16 == 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_ERR_DEVICE;
    // One launch (rows, then one walk workgroup per request that polls its
    // rows) while the walk workgroups stay below half the resident capacity,
    // as for the greedy verify; else the row launch, then the walks.
    const int one = greedy_one_launch(dev, az, es, B);
    if (one < 0) return SPEC_ERR_DEVICE;
    const long row_wgs = long(B) * M * a.np1;
    if (one) return sv::launch_tree_fused(a, az, es, int(row_wgs + B), stream) == 0 ? SPEC_OK : SPEC_ERR_DEVICE;
    a.mode = 1;                                        // the greedy row workgroups only: every node row
    if (sv::launch_verify_greedy(a, az, es, int(row_wgs), stream) != 0) return SPEC_ERR_DEVICE;
    return sv::launch_tree_walk(a, B, stream) == 0 ? SPEC_OK : SPEC_ERR_DEVICE;
}

int32_t spec_verify_launches(int32_t B, int32_t G, int32_t V, spec_dtype_t dt, float temperature) {
    const int es = esize_of(int(dt));
    if (es == 0 || check_verify_shape(B, G, V, es) != SPEC_OK) return -1;
    if (!std::isfinite(temperature) || temperature < 0.0f) return -1;
    if (temperature > 0.0f) return 1;                 // one launch (verify_len NULL: the full-grid row layout)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    const int one = greedy_one_launch(dev, (size_t(V) * es) % 16 == 0, es, B);
    return one < 0 ? -1 : (one ? 1 : 2);
}

size_t spec_schedule_workspace_bytes(int32_t, int32_t) { return 0; }

}  // extern "C"

namespace {

// spec_schedule and spec_schedule_calibrated (calib_temps NULL: as given).
spec_status_t schedule_impl(const float *confidence, const float *calib_temps, const float *cost_table,
                            int32_t table_len, int32_t B, int32_t G, int32_t token_budget, float eps,
                            int32_t *out_verify_len, int32_t *out_total_tokens, float *out_expected_tokens,
                            spec_stream_t stream) {
    if (B < 1 || G < 0 || table_len < 1) return SPEC_ERR_BAD_SHAPE;
    if (int64_t(B) * G > SPEC_MAX_SCHEDULE_CANDIDATES || B > SPEC_MAX_SCHEDULE_CANDIDATES)
        return SPEC_ERR_UNSUPPORTED;
    if (token_budget < B || token_budget >= table_len) return SPEC_ERR_BAD_SHAPE;
    if (!std::isfinite(eps)) return SPEC_ERR_BAD_SHAPE;
    if ((G > 0 && !confidence) || !cost_table || !out_verify_len || !out_total_tokens) return SPEC_ERR_NULL_POINTER;
    if (!aligned(confidence, 4) || !aligned(cost_table, 4) || !aligned(out_verify_len, 4) ||
        !aligned(out_total_tokens, 4) || !aligned(out_expected_tokens, 4))
        return SPEC_ERR_MISALIGNED;
    sv::ScheduleArgs a = {};
    if (const spec_status_t cs = set_calib(a.cal, calib_temps, G); cs != SPEC_OK) return cs;
    a.conf = confidence;
    a.cost = cost_table;
    a.B = B;
    a.G = G;
    a.budget = token_budget;
    a.eps = eps;
    a.out_len = out_verify_len;
    a.out_T = out_total_tokens;
    a.out_tau = out_expected_tokens;
    return sv::launch_schedule(a, stream) == 0 ? SPEC_OK : SPEC_ERR_DEVICE;
}

}  // namespace

extern "C" {

spec_status_t spec_schedule(const float *confidence, const float *cost_table, int32_t table_len, int32_t B,
                            int32_t G, int32_t token_budget, float eps, int32_t *out_verify_len,
                            int32_t *out_total_tokens, float *out_expected_tokens, void *workspace,
                            size_t workspace_bytes, spec_stream_t stream) {
    (void)workspace;            // spec_schedule_workspace_bytes is 0: the scheduler works in LDS
    (void)workspace_bytes;
    return schedule_impl(confidence, nullptr, cost_table, table_len, B, G, token_budget, eps, out_verify_len,
                         out_total_tokens, out_expected_tokens, stream);
}

spec_status_t spec_schedule_calibrated(const float *confidence, const float *calib_temps, const float *cost_table,
                                       int32_t table_len, int32_t B, int32_t G, int32_t token_budget, float eps,
                                       int32_t *out_verify_len, int32_t *out_total_tokens,
                                       float *out_expected_tokens, void *workspace, size_t workspace_bytes,
                                       spec_stream_t stream) {
    (void)workspace;
    (void)workspace_bytes;
    return schedule_impl(confidence, calib_temps, cost_table, table_len, B, G, token_budget, eps, out_verify_len,
                         out_total_tokens, out_expected_tokens, stream);
}

spec_status_t spec_schedule_static(const float *confidence, int32_t B, int32_t G, spec_static_mode_t mode,
                                   int32_t fixed_len, float threshold, const float *calib_temps,
                                   int32_t *out_verify_len, int32_t *out_total_tokens,
                                   int32_t *out_row_offsets, spec_stream_t stream) {
    if (B < 1 || G < 0) return SPEC_ERR_BAD_SHAPE;
    if (B > SPEC_MAX_BATCH || G > SPEC_MAX_DRAFTS) return SPEC_ERR_UNSUPPORTED;
    if (mode != SPEC_STATIC_FIXED && mode != SPEC_STATIC_THRESHOLD) return SPEC_ERR_BAD_SHAPE;
    if (mode == SPEC_STATIC_THRESHOLD && std::isnan(threshold)) return SPEC_ERR_BAD_SHAPE;
    if (!out_verify_len || (mode == SPEC_STATIC_THRESHOLD && G > 0 && !confidence)) return SPEC_ERR_NULL_POINTER;
    if (!aligned(confidence, 4) || !aligned(out_verify_len, 4) || !aligned(out_total_tokens, 4) ||
        !aligned(out_row_offsets, 4))
        return SPEC_ERR_MISALIGNED;
    sv::StaticArgs a = {};
    if (const spec_status_t cs = set_calib(a.cal, calib_temps, G); cs != SPEC_OK) return cs;
    a.conf = confidence;
    a.B = B;
    a.G = G;
    a.mode = int32_t(mode);
    a.len = fixed_len;
    a.tau = threshold;
    a.out_len = out_verify_len;
    a.out_T = out_total_tokens;
    a.out_off = out_row_offsets;
    return sv::launch_static(a, stream) == 0 ? SPEC_OK : SPEC_ERR_DEVICE;
}

namespace {
int fit_groups(int32_t N) { return int(std::min<int64_t>(256, (int64_t(N) + sv::kFitThreads - 1) / sv::kFitThreads)); }
bool fit_shape_ok(int32_t N, int32_t G, int32_t nt, int32_t bins) {
    return N >= 1 && N < (1 << 23) && G >= 0 && G <= SPEC_MAX_DRAFTS && nt >= 1 && nt <= sv::kFitMaxTemps &&
           bins >= 1 && bins <= sv::kFitMaxBins && size_t(nt) * bins * 2 * 8 <= 65536;
}
}  // namespace

size_t spec_sts_fit_workspace_bytes(int32_t N, int32_t G, int32_t num_temps, int32_t bins) {
    if (!fit_shape_ok(N, G, num_temps, bins)) return 0;
    return sv::align256(size_t(N) * 8) + sv::align256(size_t(num_temps) * 8) +
           size_t(fit_groups(N)) * num_temps * bins * 2 * 8;
}

spec_status_t spec_sts_fit(const float *confidence, const int32_t *acc_len, int32_t N, int32_t G,
                           const float *temps, int32_t num_temps, int32_t bins, float *out_temps, void *workspace,
                           size_t workspace_bytes, spec_stream_t stream) {
    if (!fit_shape_ok(N, G, num_temps, bins)) {
        if (N >= (1 << 23) || G > SPEC_MAX_DRAFTS) return SPEC_ERR_UNSUPPORTED;
        return SPEC_ERR_BAD_SHAPE;
    }
    if (!temps) return SPEC_ERR_NULL_POINTER;
    sv::FitArgs a = {};
    for (int t = 0; t < num_temps; ++t) {
        if (!std::isfinite(temps[t]) || !(temps[t] > 0.0f)) return SPEC_ERR_BAD_SHAPE;
        a.temps[t] = temps[t];
    }
    if (G == 0) return SPEC_OK;
    if (!confidence || !acc_len || !out_temps || !workspace) return SPEC_ERR_NULL_POINTER;
    if (!aligned(confidence, 4) || !aligned(acc_len, 4) || !aligned(out_temps, 4) || !aligned(workspace, 256))
        return SPEC_ERR_MISALIGNED;
    if (workspace_bytes < spec_sts_fit_workspace_bytes(N, G, num_temps, bins)) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    a.conf = confidence;
    a.acc_len = acc_len;
    a.out_temps = out_temps;
    a.prefix = static_cast<double *>(workspace);
    a.err = reinterpret_cast<double *>(static_cast<unsigned char *>(workspace) + sv::align256(size_t(N) * 8));
    a.part = reinterpret_cast<int64_t *>(static_cast<unsigned char *>(workspace) + sv::align256(size_t(N) * 8) +
                                         sv::align256(size_t(num_temps) * 8));
    a.N = N;
    a.G = G;
    a.nt = num_temps;
    a.bins = bins;
    a.nwg = fit_groups(N);
    for (int k = 0; k < G; ++k) {
        a.k = k;
        if (sv::launch_fit_accumulate(a, stream) != 0 || sv::launch_fit_choose(a, stream) != 0) return SPEC_ERR_DEVICE;
    }
    return SPEC_OK;
}

spec_status_t spec_acceptance(const void *target_logits, spec_dtype_t target_dtype, const void *draft,
                              spec_draft_kind_t draft_kind, const int32_t *verify_len, int32_t B, int32_t G,
                              int32_t V, float temperature, float *out_alpha, spec_stream_t stream) {
    const int es = esize_of(int(target_dtype));
    if (es == 0) return SPEC_ERR_BAD_DTYPE;
    if (draft_kind != SPEC_DRAFT_PROBS && draft_kind != SPEC_DRAFT_LOGITS) return SPEC_ERR_BAD_DTYPE;
    const spec_status_t sh = check_verify_shape(B, G, V, es);
    if (sh != SPEC_OK) return sh;
    if (int64_t(B) * G >= (int64_t(1) << 31)) return SPEC_ERR_UNSUPPORTED;
    const float T = temperature;
    if (!std::isfinite(T) || !(T >= 1.17549435e-38f)) return SPEC_ERR_BAD_TEMPERATURE;
    if (!target_logits || (G > 0 && (!draft || !out_alpha))) return SPEC_ERR_NULL_POINTER;
    const int ds = draft_kind == SPEC_DRAFT_LOGITS ? es : 4;
    if (!aligned(target_logits, es) || !aligned(draft, ds) || !aligned(verify_len, 4) || !aligned(out_alpha, 4))
        return SPEC_ERR_MISALIGNED;
    if (G == 0) return SPEC_OK;
    sv::AcceptArgs a = {};
    a.z = target_logits;
    a.d = draft;
    a.vlen = verify_len;
    a.out = out_alpha;
    a.B = B;
    a.G = G;
    a.V = V;
    a.c32 = float(1.4426950408889634 / double(T));
    const bool al = aligned(target_logits, 16) && aligned(draft, 16) && (size_t(V) * es) % 16 == 0 &&
                    (size_t(V) * ds) % 16 == 0;
    return sv::launch_acceptance(a, al, es, draft_kind == SPEC_DRAFT_LOGITS, stream) == 0 ? SPEC_OK
                                                                                        : SPEC_ERR_DEVICE;
}

spec_status_t spec_dcut(const float *confidence, int32_t B, int32_t G, const float *ratios,
                        const float *ratio_cost, int32_t num_ratios, const float *calib_temps,
                        int32_t *out_verify_len,
                        int32_t *out_row_offsets, int32_t *out_ratio_index, int32_t *out_total_rows,
                        double *out_utility, spec_stream_t stream) {
    if (B < 1 || G < 0) return SPEC_ERR_BAD_SHAPE;
    if (int64_t(B) * G > SPEC_MAX_SCHEDULE_CANDIDATES || B > SPEC_MAX_SCHEDULE_CANDIDATES)
        return SPEC_ERR_UNSUPPORTED;
    if (num_ratios < 1 || num_ratios > SPEC_MAX_RATIOS) return SPEC_ERR_BAD_SHAPE;
    if (!ratios || !ratio_cost) return SPEC_ERR_NULL_POINTER;
    sv::DcutArgs a = {};
    if (const spec_status_t cs = set_calib(a.cal, calib_temps, G); cs != SPEC_OK) return cs;
    for (int r = 0; r < num_ratios; ++r) {
        const float rho = ratios[r], c = ratio_cost[r];
        if (!std::isfinite(rho) || !(rho > 0.0f) || rho > 1.0f) return SPEC_ERR_BAD_SHAPE;
        if (!std::isfinite(c) || !(c > 0.0f)) return SPEC_ERR_BAD_SHAPE;
        // K_rho = max(B, ceil(rho * B * (G + 1))); the product is exact in double.
        const int64_t K = std::max<int64_t>(B, int64_t(std::ceil(double(rho) * double(int64_t(B) * (G + 1)))));
        a.keep[r] = int32_t(K - B);
        a.cost[r] = c;
    }
    if ((G > 0 && !confidence) || !out_verify_len || !out_row_offsets || !out_ratio_index || !out_total_rows)
        return SPEC_ERR_NULL_POINTER;
    if (!aligned(confidence, 4) || !aligned(out_verify_len, 4) || !aligned(out_row_offsets, 4) ||
        !aligned(out_ratio_index, 4) || !aligned(out_total_rows, 4) || !aligned(out_utility, 8))
        return SPEC_ERR_MISALIGNED;
    a.conf = confidence;
    a.B = B;
    a.G = G;
    a.R = num_ratios;
    a.out_len = out_verify_len;
    a.out_off = out_row_offsets;
    a.out_ratio = out_ratio_index;
    a.out_rows = out_total_rows;
    a.out_utility = out_utility;
    return sv::launch_dcut(a, stream) == 0 ? SPEC_OK : SPEC_ERR_DEVICE;
}

}  // extern "C"
