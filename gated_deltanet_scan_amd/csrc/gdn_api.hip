// C ABI of the frame-wise GDN forward scan: argument checks, launch planning
// and kernel launches.  Declarations and the contract are in include/gdn.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_kernels.hpp"

namespace {

using gdn::ScanArgs;

constexpr int kVersion = 10000;  // 1.0.0

enum KernelKind { K_GRAM = 0, K_STATE = 1, K_OUTPUT = 2, K_COPY = 3, K_STEP = 4 };
const char* const kKernelNames[GDN_NUM_KERNELS] = {"frame_gram", "state_scan", "frame_output",
                                                   "state_copy", "frame_step"};

// The one-frame path sizes its workspace for this many CUs (MI355X has 256;
// a device with fewer uses fewer token ranges).
constexpr int kSizingCUs = 256;

// ---------------------------------------------------------------- profiling
struct Profiler {
    bool on = false;
    std::vector<hipEvent_t> pool;   // created lazily, reused across sessions
    std::vector<int> kind;          // kernel kind of each recorded pair
    size_t used = 0;                // pairs used in this session
};
Profiler g_prof;
std::mutex g_prof_mu;

struct ProfScope {
    hipEvent_t end = nullptr;
    hipStream_t stream;
    ProfScope(KernelKind k, hipStream_t s) : stream(s) {
        if (!g_prof.on) return;
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (g_prof.used >= GDN_PROFILE_MAX_LAUNCHES) return;
        const size_t i = g_prof.used;
        while (g_prof.pool.size() < 2 * (i + 1)) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return;
            g_prof.pool.push_back(e);
        }
        if (g_prof.kind.size() < i + 1) g_prof.kind.resize(i + 1);
        g_prof.kind[i] = k;
        g_prof.used = i + 1;
        (void)hipEventRecord(g_prof.pool[2 * i], s);
        end = g_prof.pool[2 * i + 1];
    }
    ~ProfScope() {
        if (end) (void)hipEventRecord(end, stream);
    }
};

// ---------------------------------------------------------------- device checks
struct DevInfo {
    bool known = false;
    bool ok = false;
    int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

gdn_status check_device(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_NO_DEVICE;
    if (dev >= 64) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo& di = g_dev[dev];
    if (!di.known) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return GDN_ERR_NO_DEVICE;
        di.ok = strncmp(p.gcnArchName, "gfx950", 6) == 0;
        di.cus = p.multiProcessorCount;
        di.known = true;
    }
    if (cus) *cus = di.cus;
    return di.ok ? GDN_OK : GDN_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------- planning
struct Plan {
    int D = 0;
    int esz = 0;             // bytes per q/k/v/o element
    int64_t units = 0;       // B*H
    int Fc = 0;              // frames per launch chunk
    size_t item_bytes = 0;   // workspace per (b, h, frame)
    size_t carry_off = 0;    // fp32 [B][H][Dv][Dk] state carried between launches
    // one-frame path (F == 1): fp32 partial G and U per (b, h, token range),
    // then a copy of S_in
    int parts_max = 0;
    size_t scopy_off = 0;
    size_t ws_bytes = 0;
};

// Token ranges of frame_gram on the one-frame path: enough (b, h, range) items
// to give every CU one, each range a whole number of frame_gram stages.
int gram_stage_tokens(int esz, int D) { return 16384 / (D * esz); }   // GramCfg::TS
void step_ranges(int64_t units, int N, int ts, int cus, int* parts, int* tpart) {
    if (N <= 0 || units <= 0) {
        *parts = 1;
        *tpart = N > 0 ? N : 0;
        return;
    }
    const int stages = (N + ts - 1) / ts;
    int64_t want = ((int64_t)cus + units - 1) / units;
    int p = (int)(want < stages ? want : stages);
    if (p < 1) p = 1;
    const int per = ((N + p - 1) / p + ts - 1) / ts * ts;
    *tpart = per;
    *parts = (N + per - 1) / per;
}

bool dim_ok(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }

gdn_status check_desc(const gdn_desc* d, bool step, Plan* p) {
    if (!d) return GDN_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->F < 0 || d->N < 0) return GDN_ERR_INVALID_ARG;
    if (d->io_dtype != GDN_BF16 && d->io_dtype != GDN_F32) return GDN_ERR_INVALID_ARG;
    if ((d->flags & ~GDN_FLAG_GATES_ARE_LOGITS) != 0) return GDN_ERR_INVALID_ARG;
    if (!(d->eps > 0.0f) || !isfinite(d->eps)) return GDN_ERR_INVALID_ARG;
    if (step && d->F != 1) return GDN_ERR_INVALID_ARG;
    if (d->Dk < 1 || d->Dv < 1) return GDN_ERR_INVALID_ARG;
    if (d->Dk != d->Dv || !dim_ok(d->Dk)) return GDN_ERR_UNSUPPORTED;
    // element counts must fit comfortably in 64-bit byte offsets, and one
    // frame of one tensor in the 32-bit offsets of a buffer resource
    const double tok = (double)d->B * d->F * d->N * d->H * d->Dk;
    if (tok > 1e15) return GDN_ERR_INVALID_ARG;
    const double esz = d->io_dtype == GDN_BF16 ? 2.0 : 4.0;
    if (((double)d->N + 1024.0) * d->H * d->Dk * esz >= 2147483648.0) return GDN_ERR_UNSUPPORTED;
    p->D = d->Dk;
    p->esz = d->io_dtype == GDN_BF16 ? 2 : 4;
    p->units = (int64_t)d->B * d->H;
    // frames per launch chunk (state_scan stages the chunk's gates in LDS)
    p->Fc = d->F < gdn::kMaxChunkFrames ? d->F : gdn::kMaxChunkFrames;
    p->item_bytes = gdn::ws_item_bytes(p->esz, p->D);
    if (d->F == 1) {
        int tpart = 0;
        step_ranges(p->units, d->N, gram_stage_tokens(p->esz, p->D), kSizingCUs, &p->parts_max, &tpart);
        p->scopy_off = ((size_t)p->units * p->parts_max * gdn::part_bytes(p->D) + 255) / 256 * 256;
        p->ws_bytes = p->units > 0 ? p->scopy_off + (size_t)p->units * p->D * p->D * sizeof(float) : 0;
        return GDN_OK;
    }
    p->carry_off = ((size_t)p->units * p->Fc * p->item_bytes + 255) / 256 * 256;
    p->ws_bytes = (p->units > 0 && d->F > 0)
                      ? p->carry_off + (size_t)p->units * p->D * p->D * sizeof(float)
                      : 0;
    return GDN_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range rng(const void* ptr, size_t bytes) {
    const uintptr_t b = (uintptr_t)ptr;
    return Range{b, b + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
bool aligned(const void* p, uintptr_t al) { return ((uintptr_t)p & (al - 1)) == 0; }

template <typename T, int D>
gdn_status launch_state(ScanArgs a, hipStream_t stream) {
    using SC = gdn::StateCfg<T, D>;
    const int units = a.B * a.H;
    const int grid = 8 * ((units + 7) / 8) * SC::RG;
    ProfScope ps(K_STATE, stream);
    hipLaunchKernelGGL((gdn::state_scan_kernel<T, D>), dim3(grid), dim3(SC::NW * 64), 0, stream, a);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename T, int D>
gdn_status launch_output(ScanArgs a, hipStream_t stream, int cus) {
    if (a.N <= 0 || a.Fc <= 0) return GDN_OK;
    const int items = a.B * a.H * a.Fc;
    // token ranges per frame: only as many as it takes to give every CU a
    // workgroup (each range reads its frame's state planes again; at B1 H16
    // F21 N880 d128, 336 frames: one range 100.5 us per scan, two 106, four
    // 114)
    const int want = cus > 0 ? cus : 256;
    int tsplit = (want + items - 1) / items;
    const int maxsplit = (a.N + 63) / 64;
    if (tsplit > maxsplit) tsplit = maxsplit;
    if (tsplit < 1) tsplit = 1;
    int tchunk = (a.N + tsplit - 1) / tsplit;
    tchunk = (tchunk + 15) / 16 * 16;
    tsplit = (a.N + tchunk - 1) / tchunk;
    a.tsplit = tsplit;
    a.tchunk = tchunk;
    // the last quarter of the workgroups, at most one per CU, run as halves
    const int units = items * tsplit, c = cus > 0 ? cus : 256;
    a.ntail = units / 4 < c ? units / 4 : c;
    ProfScope ps(K_OUTPUT, stream);
    hipLaunchKernelGGL((gdn::frame_output_kernel<T, D>), dim3(units + a.ntail), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// Launch order, per chunk of up to kMaxChunkFrames frames, all on the caller's
// stream: frame_gram, then the recurrence (whose state is carried in `carry`:
// S_final, or the workspace's carry region), then the output pass.
// (Running the recurrence on a second stream in sub-chunks, overlapped with
// the output pass, measured slower.)
template <typename T, int D>
gdn_status launch_all(const Plan& p, ScanArgs a, hipStream_t stream, int cus, float* carry) {
    const int units = (int)p.units;
    gdn_status st = GDN_OK;
    for (int f0 = 0; f0 < a.F; f0 += p.Fc) {
        a.f0 = f0;
        a.Fc = a.F - f0 < p.Fc ? a.F - f0 : p.Fc;
        const int items = units * a.Fc;
        {
            ProfScope ps(K_GRAM, stream);
            // persistent: one workgroup per CU, each streaming its share of the items
            const int grid = items < cus ? items : (cus > 0 ? cus : 256);
            hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false>), dim3(grid), dim3(1024), 0, stream, a);
        }
        if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
        ScanArgs s = a;
        s.S_out = carry;
        if ((st = launch_state<T, D>(s, stream)) != GDN_OK) return st;
        a.S_in = carry;
        if ((st = launch_output<T, D>(a, stream, cus)) != GDN_OK) return st;
    }
    return GDN_OK;
}

// Output token ranges of a one-frame launch: about `want` workgroups over all
// (b, h) units, whole 16-token blocks, at least 64 tokens each.
inline void step_out_ranges(ScanArgs& s, int units, int want) {
    int tsplit = (want + units - 1) / units;
    const int maxsplit = s.N > 0 ? (s.N + 63) / 64 : 1;
    if (tsplit > maxsplit) tsplit = maxsplit;
    if (tsplit < 1) tsplit = 1;
    int tchunk = s.N > 0 ? (s.N + tsplit - 1) / tsplit : 0;
    tchunk = (tchunk + 15) / 16 * 16;
    if (s.N > 0) tsplit = (s.N + tchunk - 1) / tchunk;
    s.tsplit = tsplit;
    s.tchunk = tchunk;
}

// One frame (F == 1).  bf16 with D <= 64 and a state that is not updated in
// place: frame_step alone, every workgroup forming the frame's whole G and U
// (measured at B4 H32 d64 N880: 23.8 against 26.7 us per step for the two
// launches below).  Otherwise frame_gram over (b, h, token range) items,
// writing fp32 partials and copying S_in, then frame_step (state update and
// output pass).
template <typename T, int D>
gdn_status launch_step(const Plan& p, ScanArgs a, hipStream_t stream, int cus) {
    const int units = (int)p.units;
    a.f0 = 0;
    a.Fc = 1;
    const int want = cus > 0 ? cus : 256;
    if constexpr (sizeof(T) == 2 && D <= 64) {
        if (a.S_in == nullptr || a.S_in != a.S_out) {
            ScanArgs s = a;
            step_out_ranges(s, units, want);
            ProfScope ps(K_STEP, stream);
            const int grid = 8 * ((units + 7) / 8) * s.tsplit;
            hipLaunchKernelGGL((gdn::frame_step_kernel<T, D, true>), dim3(grid), dim3(gdn::StepCfg<T, D>::NTH), 0,
                               stream, s);
            return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
        }
    }
    int parts = 1, tpart = 0;
    step_ranges(p.units, a.N, gdn::GramCfg<T, D>::TS, cus < kSizingCUs ? cus : kSizingCUs, &parts, &tpart);
    if (parts > p.parts_max) return GDN_ERR_LAUNCH;   // cannot happen: sized for kSizingCUs
    a.parts = parts;
    a.tpart = tpart;
    unsigned char* ws = a.ws;
    a.spart = reinterpret_cast<float*>(ws);
    float* scopy = reinterpret_cast<float*>(ws + p.scopy_off);
    a.scopy = a.S_in ? scopy : nullptr;
    a.ncopy = units * D * D;
    {
        ProfScope ps(K_GRAM, stream);
        const int items = units * parts;
        const int grid = items < cus ? items : (cus > 0 ? cus : 256);
        hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, true>), dim3(grid), dim3(1024), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    ScanArgs s = a;
    s.S_in = a.S_in ? scopy : nullptr;
    // output ranges: about one workgroup per CU (measured at B4 H32 d64 N880:
    // 26.6 us per step with two ranges per (b, h), 27.0 with four, 29.6 with
    // eight)
    step_out_ranges(s, units, want);
    {
        ProfScope ps(K_STEP, stream);
        const int grid = 8 * ((units + 7) / 8) * s.tsplit;
        hipLaunchKernelGGL((gdn::frame_step_kernel<T, D, false>), dim3(grid), dim3(gdn::StepCfg<T, D>::NTH), 0,
                           stream, s);
    }
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename T>
gdn_status dispatch_d(const Plan& p, const ScanArgs& a, hipStream_t s, int cus, float* carry) {
    if (a.F == 1) {
        switch (p.D) {
            case 16: return launch_step<T, 16>(p, a, s, cus);
            case 32: return launch_step<T, 32>(p, a, s, cus);
            case 64: return launch_step<T, 64>(p, a, s, cus);
            case 128: return launch_step<T, 128>(p, a, s, cus);
            default: return GDN_ERR_UNSUPPORTED;
        }
    }
    switch (p.D) {
        case 16: return launch_all<T, 16>(p, a, s, cus, carry);
        case 32: return launch_all<T, 32>(p, a, s, cus, carry);
        case 64: return launch_all<T, 64>(p, a, s, cus, carry);
        case 128: return launch_all<T, 128>(p, a, s, cus, carry);
        default: return GDN_ERR_UNSUPPORTED;
    }
}

gdn_status run(const gdn_desc* d, bool step, const void* q, const void* k, const void* v,
               const float* beta, const float* alpha, const float* S0, void* o, float* S_final,
               void* workspace, size_t workspace_bytes, void* stream_v) {
    Plan p;
    gdn_status st = check_desc(d, step, &p);
    if (st != GDN_OK) return st;

    const size_t ntok = (size_t)d->B * d->F * d->N * d->H;
    const size_t tok_bytes = ntok * (size_t)p.D * p.esz;
    const size_t beta_bytes = ntok * sizeof(float);
    const size_t alpha_bytes = (size_t)d->B * d->F * d->H * sizeof(float);
    const size_t state_bytes = (size_t)p.units * p.D * p.D * sizeof(float);

    // required pointers
    if (ntok > 0 && (!q || !k || !v || !beta || !o)) return GDN_ERR_INVALID_ARG;
    if (alpha_bytes > 0 && !alpha) return GDN_ERR_INVALID_ARG;
    // alignment
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return GDN_ERR_ALIGNMENT;
    if (!aligned(beta, 4) || !aligned(alpha, 4)) return GDN_ERR_ALIGNMENT;
    if (!aligned(S0, 16) || !aligned(S_final, 16)) return GDN_ERR_ALIGNMENT;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return GDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return GDN_ERR_ALIGNMENT;
    }
    // aliasing: outputs must not overlap inputs, each other or the workspace
    const Range rq = rng(q, q ? tok_bytes : 0), rk = rng(k, k ? tok_bytes : 0),
                rv = rng(v, v ? tok_bytes : 0), rb = rng(beta, beta ? beta_bytes : 0),
                ra = rng(alpha, alpha ? alpha_bytes : 0), rs0 = rng(S0, S0 ? state_bytes : 0),
                ro = rng(o, o ? tok_bytes : 0), rsf = rng(S_final, S_final ? state_bytes : 0),
                rw = rng(workspace, workspace ? p.ws_bytes : 0);
    const Range ins[] = {rq, rk, rv, rb, ra, rs0};
    for (const Range& x : ins) {
        if (overlap(ro, x)) return GDN_ERR_ALIAS;
        if (overlap(rw, x)) return GDN_ERR_ALIAS;
    }
    for (int i = 0; i < 5; ++i)
        if (overlap(rsf, ins[i])) return GDN_ERR_ALIAS;
    if (overlap(rsf, rs0) && S_final != S0) return GDN_ERR_ALIAS;
    if (overlap(ro, rsf) || overlap(ro, rw) || overlap(rsf, rw)) return GDN_ERR_ALIAS;

    // nothing to compute
    if (p.units == 0) return GDN_OK;
    if (d->F == 0 && !S_final) return GDN_OK;

    int cus = 0;
    st = check_device(&cus);
    if (st != GDN_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);

    if (d->F == 0) {  // S_final <- S0 (or zeros)
        if (S_final == S0) return GDN_OK;
        const size_t n = (size_t)p.units * p.D * p.D;
        ProfScope ps(K_COPY, stream);
        hipLaunchKernelGGL(gdn::state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, S0, S_final, n);
        return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
    }

    ScanArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.alpha = alpha;
    a.S_in = S0;
    a.o = o;
    a.S_out = S_final;
    a.ws = static_cast<unsigned char*>(workspace);
    a.B = d->B;
    a.H = d->H;
    a.F = d->F;
    a.N = d->N;
    a.logits = (d->flags & GDN_FLAG_GATES_ARE_LOGITS) ? 1 : 0;
    a.eps = d->eps;
    a.tsplit = 1;
    a.tchunk = 16;
    a.ntail = 0;
    a.parts = 1;
    a.tpart = d->N;
    a.spart = nullptr;
    a.scopy = nullptr;
    a.ncopy = 0;
    // the state between launches lives in S_final, or in the workspace's carry region
    float* carry = (S_final || d->F == 1)
                       ? S_final
                       : reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + p.carry_off);
    return d->io_dtype == GDN_BF16 ? dispatch_d<uint16_t>(p, a, stream, cus, carry)
                                   : dispatch_d<float>(p, a, stream, cus, carry);
}

}  // namespace

extern "C" {

size_t gdn_workspace_size(const gdn_desc* d) {
    Plan p;
    if (check_desc(d, false, &p) != GDN_OK) return 0;
    return p.ws_bytes;
}

gdn_status gdn_frame_scan_fwd(const gdn_desc* d, const void* q, const void* k, const void* v,
                              const float* beta, const float* alpha, const float* S0, void* o,
                              float* S_final, void* workspace, size_t workspace_bytes, void* stream) {
    return run(d, false, q, k, v, beta, alpha, S0, o, S_final, workspace, workspace_bytes, stream);
}

gdn_status gdn_frame_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                          const float* beta, const float* alpha, const float* S_in, void* o,
                          float* S_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (!S_out) return GDN_ERR_INVALID_ARG;
    return run(d, true, q, k, v, beta, alpha, S_in, o, S_out, workspace, workspace_bytes, stream);
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_ALIGNMENT: return "misaligned pointer";
        case GDN_ERR_ALIAS: return "output aliases another buffer";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
        case GDN_ERR_NO_DEVICE: return "no HIP device";
    }
    return "unknown status";
}

int32_t gdn_version(void) { return kVersion; }

gdn_status gdn_profile_begin(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.used = 0;
    g_prof.on = true;
    return GDN_OK;
}

gdn_status gdn_profile_end(double* total_ms, int64_t* launches) {
    std::vector<hipEvent_t> ev;
    std::vector<int> kinds;
    size_t used;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof.on = false;
        used = g_prof.used;
        ev = g_prof.pool;
        kinds = g_prof.kind;
    }
    for (int k = 0; k < GDN_NUM_KERNELS; ++k) {
        if (total_ms) total_ms[k] = 0.0;
        if (launches) launches[k] = 0;
    }
    for (size_t i = 0; i < used; ++i) {
        if (hipEventSynchronize(ev[2 * i + 1]) != hipSuccess) return GDN_ERR_LAUNCH;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) != hipSuccess) return GDN_ERR_LAUNCH;
        if (total_ms) total_ms[kinds[i]] += ms;
        if (launches) launches[kinds[i]] += 1;
    }
    return GDN_OK;
}

const char* gdn_kernel_name(int32_t k) {
    return (k >= 0 && k < GDN_NUM_KERNELS) ? kKernelNames[k] : nullptr;
}

}  // extern "C"
