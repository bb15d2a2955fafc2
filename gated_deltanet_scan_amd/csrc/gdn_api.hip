// C ABI of the frame-wise GDN scan (forward and backward): argument checks,
// launch planning and kernel launches.  Declarations and the contract are in
// include/gdn.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_kernels.hpp"
#include "gdn_bwd.hpp"

namespace {

using gdn::ScanArgs;

constexpr int kVersion = 10000;  // 1.0.0

enum KernelKind {
    K_GRAM = 0, K_STATE = 1, K_OUTPUT = 2, K_COPY = 3, K_STEP = 4,
    K_WGRAM = 5, K_ADJOINT = 6, K_DQ = 7, K_DKV = 8
};
const char* const kKernelNames[GDN_NUM_KERNELS] = {"frame_gram", "state_scan", "frame_output", "state_copy",
                                                   "frame_step", "w_gram",     "adjoint_scan", "frame_dq",
                                                   "frame_dkv"};

// The one-frame path sizes its workspace for this many CUs (MI355X has 256;
// a device with fewer uses fewer token ranges).
constexpr int kSizingCUs = 256;

// ---------------------------------------------------------------- profiling
struct Profiler {
    std::atomic<bool> on{false};
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
    bool lp = false;         // forward scan: U and the state planes in bf16 (see check_desc)
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

// fc_cap bounds the frames per launch chunk (the static-scratch entry point
// sizes its chunks to fit the scratch array).
gdn_status check_desc(const gdn_desc* d, bool step, Plan* p, int fc_cap = gdn::kMaxChunkFrames) {
    if (!d) return GDN_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->F < 0 || d->N < 0) return GDN_ERR_INVALID_ARG;
    const bool mx = d->io_dtype == GDN_FP8_E4M3 || d->io_dtype == GDN_FP4_E2M1;   // block-scaled inputs
    if (d->io_dtype != GDN_BF16 && d->io_dtype != GDN_F32 && !mx) return GDN_ERR_INVALID_ARG;
    if ((d->flags & ~(GDN_FLAG_GATES_ARE_LOGITS | GDN_FLAG_NO_KEY_NORM | GDN_FLAG_REVERSE)) != 0)
        return GDN_ERR_INVALID_ARG;
    if (!(d->eps > 0.0f) || !isfinite(d->eps)) return GDN_ERR_INVALID_ARG;
    if (step && d->F != 1) return GDN_ERR_INVALID_ARG;
    if (d->Dk < 1 || d->Dv < 1) return GDN_ERR_INVALID_ARG;
    if (d->Dk != d->Dv || !dim_ok(d->Dk)) return GDN_ERR_UNSUPPORTED;
    if (mx && d->Dk < gdn::kMxBlock) return GDN_ERR_UNSUPPORTED;   // one scale block
    // element counts must fit comfortably in 64-bit byte offsets, and one
    // frame of one tensor in the 32-bit offsets of a buffer resource
    const double tok = (double)d->B * d->F * d->N * d->H * d->Dk;
    if (tok > 1e15) return GDN_ERR_INVALID_ARG;
    const double esz = d->io_dtype == GDN_F32 ? 4.0 : 2.0;
    if (((double)d->N + 1024.0) * d->H * d->Dk * esz >= 2147483648.0) return GDN_ERR_UNSUPPORTED;
    p->D = d->Dk;
    p->esz = d->io_dtype == GDN_F32 ? 4 : 2;    // the block-scaled mode computes in bf16
    p->units = (int64_t)d->B * d->H;
    // frames per launch chunk (state_scan stages the chunk's gates in LDS)
    p->Fc = d->F < fc_cap ? d->F : fc_cap;
    p->item_bytes = gdn::ws_item_bytes(p->esz, p->D);
    if (d->F == 1 && !mx) {   // (block-scaled inputs take the scan path)
        int tpart = 0;
        step_ranges(p->units, d->N, gram_stage_tokens(p->esz, p->D), kSizingCUs, &p->parts_max, &tpart);
        p->scopy_off = ((size_t)p->units * p->parts_max * gdn::part_bytes(p->D) + 255) / 256 * 256;
        p->ws_bytes = p->units > 0 ? p->scopy_off + (size_t)p->units * p->D * p->D * sizeof(float) : 0;
        return GDN_OK;
    }
    // The forward scan's intermediates at larger shapes: U (frame_gram to the
    // recurrence) and the state planes (recurrence to the output pass) are
    // stored in bf16 instead of fp32 and bf16 plus remainder codes: a third
    // fewer workspace bytes touched.  Each adds about one bf16 rounding (2^-9
    // relative) to a value the products already carry at that precision; at
    // d >= 64 with at least 128 tokens per frame the error stays well inside
    // the tolerance (measured against the fp64 reference at the full-minute
    // shape: O 3.3e-3, S_F 2.3e-3 relative, every (b, h) within 3.4e-3; the
    // budget 5e-3).  Tiny frames keep the finer forms: there one token's
    // rounding is not averaged with others.
    p->lp = d->io_dtype != GDN_F32 && d->Dk >= 64 && d->N >= 128;
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

template <typename T, int D, bool BWD = false, bool LP = false>
gdn_status launch_state(ScanArgs a, hipStream_t stream) {
    using SC = gdn::StateCfg<T, D>;
    const int units = a.B * a.H;
    // one workgroup per (b, h, row slab); the slabs of a unit share an XCD
    const int grid = 8 * ((units + 7) / 8) * SC::ET;
    ProfScope ps(BWD ? K_ADJOINT : K_STATE, stream);
    hipLaunchKernelGGL((gdn::state_scan_kernel<T, D, BWD, LP>), dim3(grid), dim3(SC::NTH), 0, stream, a);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename T, int D, bool TRS = false, bool LP = false>
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
    // the last half of the (frame, range) items run as two workgroups of half
    // the tokens each (full-minute scan, one process A/B: 417.6 us with half,
    // 421.4 with a quarter capped at two per CU, 422.8 with a quarter capped
    // at one per CU, 425 with none)
    const int units = items * tsplit;
    a.ntail = units / 2;
    ProfScope ps(TRS ? K_DQ : K_OUTPUT, stream);
    hipLaunchKernelGGL((gdn::frame_output_kernel<T, D, TRS, LP>), dim3(units + a.ntail), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// Launch order, per chunk of up to p.Fc frames, all on the caller's stream:
// frame_gram, then the recurrence (whose state is carried in `carry`:
// S_final, or the workspace's carry region), then the output pass.  The
// reverse direction visits the chunks from the last to the first.
// (Running the recurrence on a second stream in sub-chunks, overlapped with
// the output pass, measured slower: the two passes slow each other down
// where they share compute units.)  LP: U and the state planes in bf16.
template <typename T, int D, bool LP>
gdn_status launch_chunks(const Plan& p, ScanArgs a, hipStream_t stream, int cus, float* carry) {
    const int units = (int)p.units;
    gdn_status st = GDN_OK;
    const int nchunks = (a.F + p.Fc - 1) / p.Fc;
    for (int ci = 0; ci < nchunks; ++ci) {
        const int f0 = (a.reverse ? nchunks - 1 - ci : ci) * p.Fc;
        a.f0 = f0;
        a.Fc = a.F - f0 < p.Fc ? a.F - f0 : p.Fc;
        const int items = units * a.Fc;
        {
            ProfScope ps(K_GRAM, stream);
            // persistent: one workgroup per CU, each streaming its share of the items
            const int grid = items < cus ? items : (cus > 0 ? cus : 256);
            hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false, false, false, LP>), dim3(grid), dim3(1024), 0,
                               stream, a);
        }
        if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
        ScanArgs s = a;
        s.S_out = carry;
        if ((st = launch_state<typename gdn::Elem<T>::C, D, false, LP>(s, stream)) != GDN_OK) return st;
        a.S_in = carry;
        if ((st = launch_output<T, D, false, LP>(a, stream, cus)) != GDN_OK) return st;
    }
    return GDN_OK;
}

template <typename T, int D>
gdn_status launch_all(const Plan& p, const ScanArgs& a, hipStream_t stream, int cus, float* carry) {
    if constexpr (sizeof(typename gdn::Elem<T>::C) == 2 && D >= 64) {
        if (p.lp) return launch_chunks<T, D, true>(p, a, stream, cus, carry);
    }
    return launch_chunks<T, D, false>(p, a, stream, cus, carry);
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

// ---------------------------------------------------------------- static scratch
// The allocation-free entry point's workspace: one array per device, held
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code it is only a stand-in for the device symbol); it
// passes the device address that hipGetSymbolAddress returns, looked up once
// per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

gdn_status scratch_for_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_NO_DEVICE;
    if (dev >= 64) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GDN_ERR_NO_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

// Frames per chunk that fit the static scratch: every chunk's items plus the
// carried state (0 when not even one frame fits).
int scratch_chunk_cap(const gdn_desc* d) {
    Plan p;
    if (check_desc(d, false, &p) != GDN_OK || p.units <= 0) return gdn::kMaxChunkFrames;
    const size_t carry = (size_t)p.units * p.D * p.D * sizeof(float) + 256;
    if (carry >= kScratchBytes) return 0;
    const size_t per_frame = (size_t)p.units * p.item_bytes;
    const size_t cap = (kScratchBytes - carry) / per_frame;
    return cap < (size_t)gdn::kMaxChunkFrames ? (int)cap : gdn::kMaxChunkFrames;
}

gdn_status run(const gdn_desc* d, bool step, const void* q, const void* k, const void* v,
               const float* beta, const float* alpha, const float* S0, void* o, float* S_final,
               void* workspace, size_t workspace_bytes, void* stream_v, bool static_ws = false) {
    Plan p;
    int fc_cap = gdn::kMaxChunkFrames;
    if (static_ws) {
        fc_cap = scratch_chunk_cap(d);
        if (fc_cap < 1 && d && d->F > 1) return GDN_ERR_WORKSPACE;   // one frame does not fit
        if (fc_cap < 1) fc_cap = 1;
    }
    gdn_status st = check_desc(d, step, &p, fc_cap);
    if (st != GDN_OK) return st;
    if (d->io_dtype == GDN_FP8_E4M3 || d->io_dtype == GDN_FP4_E2M1)
        return GDN_ERR_INVALID_ARG;   // needs the scales: gdn_frame_scan_fwd_fp8 / _fp4
    if (static_ws) {
        if (p.ws_bytes > kScratchBytes) return GDN_ERR_WORKSPACE;
        workspace = nullptr;
        workspace_bytes = 0;
        if (p.ws_bytes > 0 && p.units > 0) {
            if ((st = scratch_for_device(&workspace)) != GDN_OK) return st;
            workspace_bytes = kScratchBytes;
        }
    }

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
    a.raw_keys = (d->flags & GDN_FLAG_NO_KEY_NORM) ? 1 : 0;
    a.reverse = (d->flags & GDN_FLAG_REVERSE) ? 1 : 0;
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

// ---------------------------------------------------------------- block-scaled inputs
template <typename TIN>
gdn_status launch_mx(const Plan& p, const ScanArgs& a, hipStream_t s, int cus, float* carry) {
    switch (p.D) {
        case 32: return launch_all<TIN, 32>(p, a, s, cus, carry);
        case 64: return launch_all<TIN, 64>(p, a, s, cus, carry);
        case 128: return launch_all<TIN, 128>(p, a, s, cus, carry);
        default: return GDN_ERR_UNSUPPORTED;
    }
}

// Block-scaled inputs: want is GDN_FP8_E4M3 or GDN_FP4_E2M1 (the entry point's format).
gdn_status run_mx(int want, const gdn_desc* d, const void* q, const uint8_t* qs, const void* k, const uint8_t* ks,
                  const void* v, const uint8_t* vs, const float* beta, const float* alpha, const float* S0, void* o,
                  float* S_final, void* workspace, size_t workspace_bytes, void* stream_v) {
    Plan p;
    gdn_status st = check_desc(d, false, &p);
    if (st != GDN_OK) return st;
    if (d->io_dtype != want) return GDN_ERR_INVALID_ARG;
    const size_t ntok = (size_t)d->B * d->F * d->N * d->H;
    const size_t in_bytes = want == GDN_FP8_E4M3 ? ntok * (size_t)p.D : ntok * (size_t)p.D / 2;   // 8 or 4 bits
    const size_t sc_bytes = ntok * (size_t)(p.D / gdn::kMxBlock);     // one E8M0 byte per 32 values
    const size_t o_bytes = ntok * (size_t)p.D * 2;                    // bf16
    const size_t beta_bytes = ntok * sizeof(float);
    const size_t alpha_bytes = (size_t)d->B * d->F * d->H * sizeof(float);
    const size_t state_bytes = (size_t)p.units * p.D * p.D * sizeof(float);
    if (ntok > 0 && (!q || !qs || !k || !ks || !v || !vs || !beta || !o)) return GDN_ERR_INVALID_ARG;
    if (alpha_bytes > 0 && !alpha) return GDN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GDN_ERR_ALIGNMENT;
    if (!aligned(beta, 4) || !aligned(alpha, 4)) return GDN_ERR_ALIGNMENT;
    if (!aligned(S0, 16) || !aligned(S_final, 16)) return GDN_ERR_ALIGNMENT;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return GDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return GDN_ERR_ALIGNMENT;
    }
    auto R = [](const void* ptr, size_t n) { return rng(ptr, ptr ? n : 0); };
    const Range ins[] = {R(q, in_bytes), R(qs, sc_bytes), R(k, in_bytes), R(ks, sc_bytes), R(v, in_bytes),
                         R(vs, sc_bytes), R(beta, beta_bytes), R(alpha, alpha_bytes), R(S0, state_bytes)};
    const Range ro = R(o, o_bytes), rsf = R(S_final, state_bytes), rw = R(workspace, workspace ? p.ws_bytes : 0);
    for (const Range& x : ins) {
        if (overlap(ro, x) || overlap(rw, x)) return GDN_ERR_ALIAS;
        if (overlap(rsf, x) && !(x.lo == rsf.lo && S_final == S0)) return GDN_ERR_ALIAS;
    }
    if (overlap(rsf, R(S0, state_bytes)) && S_final != S0) return GDN_ERR_ALIAS;
    if (overlap(ro, rsf) || overlap(ro, rw) || overlap(rsf, rw)) return GDN_ERR_ALIAS;

    if (p.units == 0) return GDN_OK;
    if (d->F == 0 && !S_final) return GDN_OK;
    int cus = 0;
    st = check_device(&cus);
    if (st != GDN_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    if (d->F == 0) {
        if (S_final == S0) return GDN_OK;
        const size_t n = (size_t)p.units * p.D * p.D;
        ProfScope ps(K_COPY, stream);
        hipLaunchKernelGGL(gdn::state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, S0,
                           S_final, n);
        return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
    }
    ScanArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.qs = qs;
    a.ks = ks;
    a.vs = vs;
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
    a.raw_keys = (d->flags & GDN_FLAG_NO_KEY_NORM) ? 1 : 0;
    a.reverse = (d->flags & GDN_FLAG_REVERSE) ? 1 : 0;
    a.eps = d->eps;
    a.tsplit = 1;
    a.tchunk = 16;
    a.parts = 1;
    a.tpart = d->N;
    float* carry = S_final ? S_final : reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + p.carry_off);
    return want == GDN_FP8_E4M3 ? launch_mx<gdn::fp8e4m3>(p, a, stream, cus, carry)
                                : launch_mx<gdn::fp4e2m1>(p, a, stream, cus, carry);
}

// ---------------------------------------------------------------- backward pass
// Workspace of gdn_frame_scan_bwd: per chunk of up to Fc frames the forward
// items (Gm, U, S planes) and the backward items (W, X planes); the states
// entering chunks 1.. of the forward walk; the state gradient carried between
// chunks; every token's key scale (fp32 [B][F][N][H]).
//
// With saved states (gdn_frame_scan_fwd_save), the forward items of every
// chunk, the states entering the chunks and the key scales live in the
// caller's `saved` buffer instead: one item set per chunk (in the order the
// walk visits them), then one state per chunk (the state entering it: S0 or
// zeros for the first), then the key scales.  The backward workspace then
// holds only the backward items and the carried state gradient.
struct BwdPlan {
    Plan p;
    int nchunks = 0;
    size_t set = 0;          // one item set (every (b, h) unit, Fc frames)
    size_t ws2_off = 0, enter_off = 0, state_bytes = 0, dcarry_off = 0, rho_off = 0, ws_bytes = 0;
    // saved-state layout
    size_t sv_enter_off = 0, sv_rho_off = 0, sv_bytes = 0;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

gdn_status check_bwd(const gdn_desc* d, BwdPlan* bp, bool saved = false) {
    Plan& p = bp->p;
    gdn_status st = check_desc(d, false, &p);
    if (st != GDN_OK) return st;
    if (d->io_dtype == GDN_FP8_E4M3 || d->io_dtype == GDN_FP4_E2M1) return GDN_ERR_UNSUPPORTED;
    bp->nchunks = d->F > 0 ? (d->F + p.Fc - 1) / p.Fc : 0;
    const size_t set = round256((size_t)p.units * p.Fc * p.item_bytes);
    bp->set = set;
    bp->state_bytes = round256((size_t)p.units * p.D * p.D * sizeof(float));
    const size_t rho_bytes = round256((size_t)d->B * d->F * d->N * d->H * sizeof(float));
    const bool any = p.units > 0 && d->F > 0;
    bp->sv_enter_off = (size_t)bp->nchunks * set;
    bp->sv_rho_off = bp->sv_enter_off + (size_t)bp->nchunks * bp->state_bytes;
    bp->sv_bytes = any ? bp->sv_rho_off + rho_bytes : 0;
    if (saved) {
        bp->ws2_off = 0;
        bp->dcarry_off = set;
        bp->ws_bytes = any ? set + bp->state_bytes : 0;
        return GDN_OK;
    }
    bp->ws2_off = set;
    bp->enter_off = 2 * set;
    bp->dcarry_off = bp->enter_off + (size_t)(bp->nchunks > 1 ? bp->nchunks - 1 : 0) * bp->state_bytes;
    bp->rho_off = bp->dcarry_off + bp->state_bytes;
    bp->ws_bytes = any ? bp->rho_off + rho_bytes : 0;
    return GDN_OK;
}

struct BwdIO {
    const void* dO;
    const float* dS_final;
    void* dq;
    void* dk;
    void* dv;
    float* dbeta;
    float* dalpha;
    float* dS0;
};

// Launch order, all on the caller's stream.  With more than one chunk, a first
// forward walk (frame_gram, state_scan) leaves the state entering every chunk.
// Then per chunk, from the last visited to the first: frame_gram and
// state_scan recompute the chunk's Gm, U and S planes; frame_gram's W pass
// forms W_f = dO_f^T Q_f; the adjoint state_scan walks the frames the other
// way and leaves X_f (the state gradient carried in dS0 or the workspace);
// frame_output in its transposed role forms dq; frame_dkv forms dk, dv, dbeta
// and dalpha.
//
// With `saved` (not NULL) the forward items, the states entering the chunks
// and the key scales come from the buffer gdn_frame_scan_fwd_save filled, and
// the recomputation (the first walk and each chunk's frame_gram and
// state_scan) is skipped.
template <typename T, int D>
gdn_status launch_bwd(const BwdPlan& bp, ScanArgs a, const BwdIO& g, hipStream_t stream, int cus,
                      const unsigned char* saved = nullptr) {
    const Plan& p = bp.p;
    const int units = (int)p.units;
    unsigned char* ws = a.ws;
    unsigned char* ws2 = ws + bp.ws2_off;
    float* dcarry = reinterpret_cast<float*>(ws + bp.dcarry_off);
    const float* S0 = a.S_in;
    unsigned char* sv = const_cast<unsigned char*>(saved);
    auto enter = [&](int v) -> float* {
        if (sv) return reinterpret_cast<float*>(sv + bp.sv_enter_off + (size_t)v * bp.state_bytes);
        return v == 0 ? const_cast<float*>(S0) : reinterpret_cast<float*>(ws + bp.enter_off + (size_t)(v - 1) * bp.state_bytes);
    };
    auto chunk = [&](int v, ScanArgs& s) {
        const int ci = a.reverse ? bp.nchunks - 1 - v : v;
        s.f0 = ci * p.Fc;
        s.Fc = a.F - s.f0 < p.Fc ? a.F - s.f0 : p.Fc;
    };
    // mode 0: G and U; 1: also every token's key scale; 2: the W pass
    auto gram = [&](const ScanArgs& s, int mode) {
        const int items = units * s.Fc;
        const int grid = items < cus ? items : (cus > 0 ? cus : 256);
        ProfScope ps(mode == 2 ? K_WGRAM : K_GRAM, stream);
        if (mode == 2)
            hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false, true>), dim3(grid), dim3(1024), 0, stream, s);
        else if (mode == 1)
            hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false, false, true>), dim3(grid), dim3(1024), 0, stream, s);
        else
            hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false>), dim3(grid), dim3(1024), 0, stream, s);
        return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
    };
    gdn_status st = GDN_OK;
    for (int v = 0; !sv && v + 1 < bp.nchunks; ++v) {   // states entering chunks 1..
        ScanArgs s = a;
        chunk(v, s);
        s.S_in = enter(v);
        s.S_out = enter(v + 1);
        if ((st = gram(s, 0)) != GDN_OK) return st;
        if ((st = launch_state<T, D>(s, stream)) != GDN_OK) return st;
    }
    for (int v = bp.nchunks - 1; v >= 0; --v) {
        ScanArgs s = a;
        chunk(v, s);
        s.S_in = enter(v);
        s.S_out = nullptr;
        if (sv) {                                    // the forward call's items and key scales
            s.ws = sv + (size_t)v * bp.set;
            s.rho = reinterpret_cast<float*>(sv + bp.sv_rho_off);
        } else {                                     // recompute them
            s.rho = reinterpret_cast<float*>(ws + bp.rho_off);   // unused with keys as given
            if ((st = gram(s, a.raw_keys ? 0 : 1)) != GDN_OK) return st;
            if ((st = launch_state<T, D>(s, stream)) != GDN_OK) return st;
        }
        ScanArgs w = s;                              // W_f = dO_f^T Q_f into the backward items
        w.k = a.q;
        w.v = g.dO;
        w.ws = ws2;
        if ((st = gram(w, 2)) != GDN_OK) return st;
        ScanArgs adj = s;                            // X_f, and the gradient entering the chunk
        adj.ws2 = ws2;
        adj.reverse = !a.reverse;
        adj.S_in = v == bp.nchunks - 1 ? g.dS_final : dcarry;
        adj.S_out = v == 0 ? g.dS0 : dcarry;
        if ((st = launch_state<T, D, true>(adj, stream)) != GDN_OK) return st;
        ScanArgs dqa = s;                            // dq = S_f^T do
        dqa.q = g.dO;
        dqa.o = g.dq;
        if ((st = launch_output<T, D, true>(dqa, stream, cus)) != GDN_OK) return st;
        {
            // dk, dv, dbeta, dalpha (with no tokens only dalpha = <X_f, S_{f-1}>)
            gdn::DkvArgs da;
            da.s = s;
            da.s.ws2 = ws2;
            da.dk = g.dk;
            da.dv = g.dv;
            da.dbeta = g.dbeta;
            da.dalpha = g.dalpha;
            ProfScope ps(K_DKV, stream);
            hipLaunchKernelGGL((gdn::frame_dkv_kernel<T, D>), dim3(units * s.Fc), dim3(gdn::DkvCfg<T, D>::NTH), 0,
                               stream, da);
            if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
        }
    }
    return GDN_OK;
}

template <typename T>
gdn_status dispatch_bwd(const BwdPlan& bp, const ScanArgs& a, const BwdIO& g, hipStream_t s, int cus,
                        const unsigned char* saved) {
    switch (bp.p.D) {
        case 16: return launch_bwd<T, 16>(bp, a, g, s, cus, saved);
        case 32: return launch_bwd<T, 32>(bp, a, g, s, cus, saved);
        case 64: return launch_bwd<T, 64>(bp, a, g, s, cus, saved);
        case 128: return launch_bwd<T, 128>(bp, a, g, s, cus, saved);
        default: return GDN_ERR_UNSUPPORTED;
    }
}

// saved_mode: gdn_frame_scan_bwd_saved (S0 is not an argument; `saved` holds
// what the forward call left)
gdn_status run_bwd(const gdn_desc* d, const void* q, const void* k, const void* v, const float* beta,
                   const float* alpha, const float* S0, const BwdIO& g, void* workspace, size_t workspace_bytes,
                   void* stream_v, bool saved_mode = false, const void* saved = nullptr, size_t saved_bytes = 0) {
    BwdPlan bp;
    gdn_status st = check_bwd(d, &bp, saved_mode);
    if (st != GDN_OK) return st;
    const Plan& p = bp.p;
    const size_t ntok = (size_t)d->B * d->F * d->N * d->H;
    const size_t tok_bytes = ntok * (size_t)p.D * p.esz;
    const size_t beta_bytes = ntok * sizeof(float);
    const size_t alpha_bytes = (size_t)d->B * d->F * d->H * sizeof(float);
    const size_t state_bytes = (size_t)p.units * p.D * p.D * sizeof(float);

    if (ntok > 0 && (!q || !k || !v || !beta || !g.dO || !g.dq || !g.dk || !g.dv || !g.dbeta))
        return GDN_ERR_INVALID_ARG;
    if (alpha_bytes > 0 && (!alpha || !g.dalpha)) return GDN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g.dO, 16) || !aligned(g.dq, 16) ||
        !aligned(g.dk, 16) || !aligned(g.dv, 16))
        return GDN_ERR_ALIGNMENT;
    if (!aligned(beta, 4) || !aligned(alpha, 4) || !aligned(g.dbeta, 4) || !aligned(g.dalpha, 4))
        return GDN_ERR_ALIGNMENT;
    if (!aligned(S0, 16) || !aligned(g.dS_final, 16) || !aligned(g.dS0, 16)) return GDN_ERR_ALIGNMENT;
    if (bp.ws_bytes > 0) {
        if (!workspace || workspace_bytes < bp.ws_bytes) return GDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return GDN_ERR_ALIGNMENT;
    }
    if (saved_mode && bp.sv_bytes > 0) {
        if (!saved || saved_bytes < bp.sv_bytes) return GDN_ERR_WORKSPACE;
        if (!aligned(saved, 256)) return GDN_ERR_ALIGNMENT;
    }
    // aliasing: outputs overlap no input, no other output and not the workspace
    // (dS0 == dS_final exactly is allowed); `saved` is an input
    auto R = [](const void* ptr, size_t n) { return rng(ptr, ptr ? n : 0); };
    const Range ins[] = {R(q, tok_bytes),      R(k, tok_bytes),     R(v, tok_bytes),
                         R(beta, beta_bytes),  R(alpha, alpha_bytes), R(S0, state_bytes),
                         R(g.dO, tok_bytes),   R(g.dS_final, state_bytes),
                         R(saved_mode ? saved : nullptr, bp.sv_bytes)};
    const Range outs[] = {R(g.dq, tok_bytes),        R(g.dk, tok_bytes),         R(g.dv, tok_bytes),
                          R(g.dbeta, beta_bytes),    R(g.dalpha, alpha_bytes),   R(g.dS0, state_bytes),
                          R(workspace, workspace ? bp.ws_bytes : 0)};
    const int nout = sizeof(outs) / sizeof(outs[0]), nin = sizeof(ins) / sizeof(ins[0]);
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j) {
            const bool inplace = i == 5 && j == 7 && g.dS0 == g.dS_final;
            if (!inplace && overlap(outs[i], ins[j])) return GDN_ERR_ALIAS;
        }
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
    }

    if (p.units == 0) return GDN_OK;
    if (d->F == 0 && !g.dS0) return GDN_OK;
    int cus = 0;
    st = check_device(&cus);
    if (st != GDN_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    if (d->F == 0) {  // dS0 <- dS_final (or zeros)
        if (g.dS0 == g.dS_final) return GDN_OK;
        const size_t n = (size_t)p.units * p.D * p.D;
        ProfScope ps(K_COPY, stream);
        hipLaunchKernelGGL(gdn::state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, g.dS_final,
                           g.dS0, n);
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
    a.ws = static_cast<unsigned char*>(workspace);
    a.B = d->B;
    a.H = d->H;
    a.F = d->F;
    a.N = d->N;
    a.logits = (d->flags & GDN_FLAG_GATES_ARE_LOGITS) ? 1 : 0;
    a.raw_keys = (d->flags & GDN_FLAG_NO_KEY_NORM) ? 1 : 0;
    a.reverse = (d->flags & GDN_FLAG_REVERSE) ? 1 : 0;
    a.eps = d->eps;
    a.tsplit = 1;
    a.tchunk = 16;
    a.parts = 1;
    a.tpart = d->N;
    const unsigned char* sv = saved_mode ? static_cast<const unsigned char*>(saved) : nullptr;
    return d->io_dtype == GDN_BF16 ? dispatch_bwd<uint16_t>(bp, a, g, stream, cus, sv)
                                   : dispatch_bwd<float>(bp, a, g, stream, cus, sv);
}

// ---------------------------------------------------------------- forward with saved states
// gdn_frame_scan_fwd's launches with the saved buffer as the workspace: chunk
// v (in visit order) builds its items in item set v, reads the state entering
// it from slot v and leaves the state after it in slot v + 1 (S_final after
// the last chunk); frame_gram also writes the key scales.  Slot 0 first
// receives S0 (or zeros), so the backward call needs no S0 even when S_final
// overwrote it.
template <typename T, int D>
gdn_status launch_save(const BwdPlan& bp, ScanArgs a, unsigned char* sv, hipStream_t stream, int cus) {
    const Plan& p = bp.p;
    const int units = (int)p.units;
    auto slot = [&](int v) { return reinterpret_cast<float*>(sv + bp.sv_enter_off + (size_t)v * bp.state_bytes); };
    {
        const size_t n = (size_t)units * D * D;
        ProfScope ps(K_COPY, stream);
        hipLaunchKernelGGL(gdn::state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.S_in,
                           slot(0), n);
        if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    }
    float* const S_final = a.S_out;
    gdn_status st = GDN_OK;
    for (int v = 0; v < bp.nchunks; ++v) {
        ScanArgs s = a;
        const int ci = a.reverse ? bp.nchunks - 1 - v : v;
        s.f0 = ci * p.Fc;
        s.Fc = a.F - s.f0 < p.Fc ? a.F - s.f0 : p.Fc;
        s.ws = sv + (size_t)v * bp.set;
        s.S_in = slot(v);
        s.S_out = v + 1 < bp.nchunks ? slot(v + 1) : S_final;
        s.rho = reinterpret_cast<float*>(sv + bp.sv_rho_off);
        {
            const int items = units * s.Fc;
            const int grid = items < cus ? items : (cus > 0 ? cus : 256);
            ProfScope ps(K_GRAM, stream);
            if (a.raw_keys)
                hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false>), dim3(grid), dim3(1024), 0, stream, s);
            else
                hipLaunchKernelGGL((gdn::frame_gram_kernel<T, D, false, false, true>), dim3(grid), dim3(1024), 0,
                                   stream, s);
            if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
        }
        if ((st = launch_state<T, D>(s, stream)) != GDN_OK) return st;
        if ((st = launch_output<T, D>(s, stream, cus)) != GDN_OK) return st;
    }
    return GDN_OK;
}

template <typename T>
gdn_status dispatch_save(const BwdPlan& bp, const ScanArgs& a, unsigned char* sv, hipStream_t s, int cus) {
    switch (bp.p.D) {
        case 16: return launch_save<T, 16>(bp, a, sv, s, cus);
        case 32: return launch_save<T, 32>(bp, a, sv, s, cus);
        case 64: return launch_save<T, 64>(bp, a, sv, s, cus);
        case 128: return launch_save<T, 128>(bp, a, sv, s, cus);
        default: return GDN_ERR_UNSUPPORTED;
    }
}

gdn_status run_save(const gdn_desc* d, const void* q, const void* k, const void* v, const float* beta,
                    const float* alpha, const float* S0, void* o, float* S_final, void* saved, size_t saved_bytes,
                    void* stream_v) {
    BwdPlan bp;
    gdn_status st = check_bwd(d, &bp, true);
    if (st != GDN_OK) return st;
    const Plan& p = bp.p;
    const size_t ntok = (size_t)d->B * d->F * d->N * d->H;
    const size_t tok_bytes = ntok * (size_t)p.D * p.esz;
    const size_t beta_bytes = ntok * sizeof(float);
    const size_t alpha_bytes = (size_t)d->B * d->F * d->H * sizeof(float);
    const size_t state_bytes = (size_t)p.units * p.D * p.D * sizeof(float);
    if (ntok > 0 && (!q || !k || !v || !beta || !o)) return GDN_ERR_INVALID_ARG;
    if (alpha_bytes > 0 && !alpha) return GDN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GDN_ERR_ALIGNMENT;
    if (!aligned(beta, 4) || !aligned(alpha, 4)) return GDN_ERR_ALIGNMENT;
    if (!aligned(S0, 16) || !aligned(S_final, 16)) return GDN_ERR_ALIGNMENT;
    if (bp.sv_bytes > 0) {
        if (!saved || saved_bytes < bp.sv_bytes) return GDN_ERR_WORKSPACE;
        if (!aligned(saved, 256)) return GDN_ERR_ALIGNMENT;
    }
    auto R = [](const void* ptr, size_t n) { return rng(ptr, ptr ? n : 0); };
    const Range ins[] = {R(q, tok_bytes), R(k, tok_bytes), R(v, tok_bytes), R(beta, beta_bytes), R(alpha, alpha_bytes),
                         R(S0, state_bytes)};
    const Range ro = R(o, tok_bytes), rsf = R(S_final, state_bytes), rs = R(saved, bp.sv_bytes);
    for (int i = 0; i < 6; ++i) {
        if (overlap(ro, ins[i]) || overlap(rs, ins[i])) return GDN_ERR_ALIAS;
        if (i < 5 && overlap(rsf, ins[i])) return GDN_ERR_ALIAS;
    }
    if (overlap(rsf, ins[5]) && S_final != S0) return GDN_ERR_ALIAS;
    if (overlap(ro, rsf) || overlap(ro, rs) || overlap(rsf, rs)) return GDN_ERR_ALIAS;

    if (p.units == 0) return GDN_OK;
    if (d->F == 0 && !S_final) return GDN_OK;
    int cus = 0;
    if ((st = check_device(&cus)) != GDN_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    if (d->F == 0) {  // S_final <- S0 (or zeros); nothing to save
        if (S_final == S0) return GDN_OK;
        const size_t n = (size_t)p.units * p.D * p.D;
        ProfScope ps(K_COPY, stream);
        hipLaunchKernelGGL(gdn::state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, S0,
                           S_final, n);
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
    a.B = d->B;
    a.H = d->H;
    a.F = d->F;
    a.N = d->N;
    a.logits = (d->flags & GDN_FLAG_GATES_ARE_LOGITS) ? 1 : 0;
    a.raw_keys = (d->flags & GDN_FLAG_NO_KEY_NORM) ? 1 : 0;
    a.reverse = (d->flags & GDN_FLAG_REVERSE) ? 1 : 0;
    a.eps = d->eps;
    a.tsplit = 1;
    a.tchunk = 16;
    a.parts = 1;
    a.tpart = d->N;
    unsigned char* sv = static_cast<unsigned char*>(saved);
    return d->io_dtype == GDN_BF16 ? dispatch_save<uint16_t>(bp, a, sv, stream, cus)
                                   : dispatch_save<float>(bp, a, sv, stream, cus);
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

gdn_status gdn_frame_scan_fwd_static(const gdn_desc* d, const void* q, const void* k, const void* v,
                                     const float* beta, const float* alpha, const float* S0, void* o,
                                     float* S_final, void* stream) {
    return run(d, false, q, k, v, beta, alpha, S0, o, S_final, nullptr, 0, stream, true);
}

size_t gdn_static_scratch_bytes(void) { return kScratchBytes; }

gdn_status gdn_frame_scan_fwd_fp8(const gdn_desc* d, const void* q, const uint8_t* q_scale, const void* k,
                                  const uint8_t* k_scale, const void* v, const uint8_t* v_scale, const float* beta,
                                  const float* alpha, const float* S0, void* o, float* S_final, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return run_mx(GDN_FP8_E4M3, d, q, q_scale, k, k_scale, v, v_scale, beta, alpha, S0, o, S_final, workspace,
                  workspace_bytes, stream);
}

gdn_status gdn_frame_scan_fwd_fp4(const gdn_desc* d, const void* q, const uint8_t* q_scale, const void* k,
                                  const uint8_t* k_scale, const void* v, const uint8_t* v_scale, const float* beta,
                                  const float* alpha, const float* S0, void* o, float* S_final, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return run_mx(GDN_FP4_E2M1, d, q, q_scale, k, k_scale, v, v_scale, beta, alpha, S0, o, S_final, workspace,
                  workspace_bytes, stream);
}

gdn_status gdn_frame_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                          const float* beta, const float* alpha, const float* S_in, void* o,
                          float* S_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (!S_out) return GDN_ERR_INVALID_ARG;
    return run(d, true, q, k, v, beta, alpha, S_in, o, S_out, workspace, workspace_bytes, stream);
}

size_t gdn_workspace_size_bwd(const gdn_desc* d) {
    BwdPlan bp;
    if (check_bwd(d, &bp) != GDN_OK) return 0;
    return bp.ws_bytes;
}

gdn_status gdn_frame_scan_bwd(const gdn_desc* d, const void* q, const void* k, const void* v,
                              const float* beta, const float* alpha, const float* S0, const void* dO,
                              const float* dS_final, void* dq, void* dk, void* dv, float* dbeta,
                              float* dalpha, float* dS0, void* workspace, size_t workspace_bytes,
                              void* stream) {
    const BwdIO g{dO, dS_final, dq, dk, dv, dbeta, dalpha, dS0};
    return run_bwd(d, q, k, v, beta, alpha, S0, g, workspace, workspace_bytes, stream);
}

size_t gdn_saved_size(const gdn_desc* d) {
    BwdPlan bp;
    if (check_bwd(d, &bp, true) != GDN_OK) return 0;
    return bp.sv_bytes;
}

size_t gdn_workspace_size_bwd_saved(const gdn_desc* d) {
    BwdPlan bp;
    if (check_bwd(d, &bp, true) != GDN_OK) return 0;
    return bp.ws_bytes;
}

gdn_status gdn_frame_scan_fwd_save(const gdn_desc* d, const void* q, const void* k, const void* v,
                                   const float* beta, const float* alpha, const float* S0, void* o, float* S_final,
                                   void* saved, size_t saved_bytes, void* stream) {
    return run_save(d, q, k, v, beta, alpha, S0, o, S_final, saved, saved_bytes, stream);
}

gdn_status gdn_frame_scan_bwd_saved(const gdn_desc* d, const void* q, const void* k, const void* v,
                                    const float* beta, const float* alpha, const void* dO, const float* dS_final,
                                    void* dq, void* dk, void* dv, float* dbeta, float* dalpha, float* dS0,
                                    const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    const BwdIO g{dO, dS_final, dq, dk, dv, dbeta, dalpha, dS0};
    return run_bwd(d, q, k, v, beta, alpha, nullptr, g, workspace, workspace_bytes, stream, true, saved, saved_bytes);
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
