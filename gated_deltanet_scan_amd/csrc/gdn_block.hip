// Projections either side of the scan inside a GDN block: the C ABI of
// gdn_block_in_proj / gdn_block_out_proj (declared in include/gdn.h).
//
// The GEMMs are plain bf16 products with fp32 accumulation and go to
// hipBLASLt; the two steps that are not GEMMs (splitting the gate logits and
// averaging the decay logits over a frame's tokens) are kernels of this file.
// Row-major products Y[M][N] = X[M][K] W[K][N] are issued as their
// column-major transposes Y^T = W^T X^T, which read the same memory.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/gdn.h"

namespace {

constexpr size_t kLtWorkspace = (size_t)32 << 20;   // hipBLASLt's share of the workspace

std::mutex g_lt_mu;
hipblasLtHandle_t g_lt[64];

gdn_status lt_handle(hipblasLtHandle_t* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_NO_DEVICE;
    if (dev >= 64) return GDN_ERR_UNSUPPORTED;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return GDN_ERR_NO_DEVICE;
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_lt_mu);
    if (!g_lt[dev] && hipblasLtCreate(&g_lt[dev]) != HIPBLAS_STATUS_SUCCESS) return GDN_ERR_LAUNCH;
    *out = g_lt[dev];
    return GDN_OK;
}

// Y[M][N] (row stride ldy, type yt) = X[M][K] (row stride ldx) W[K][N] (row
// stride ldw), X and W bf16, fp32 accumulation.
gdn_status gemm(hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, const void* W,
                int64_t ldw, void* Y, int64_t ldy, hipDataType yt, void* lt_ws, hipStream_t stream) {
    if (M == 0 || N == 0) return GDN_OK;
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    gdn_status st = GDN_ERR_LAUNCH;
    do {
        if (hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) break;
        const hipblasOperation_t nt = HIPBLAS_OP_N;
        hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &nt, sizeof(nt));
        hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &nt, sizeof(nt));
        // column-major: A = W^T (N x K, ld ldw), B = X^T (K x M, ld ldx), D = Y^T (N x M, ld ldy)
        if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, N, K, ldw) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, K, M, ldx) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatrixLayoutCreate(&lc, yt, N, M, ldy) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) break;
        const uint64_t wsb = kLtWorkspace;
        hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
        hipblasLtMatmulHeuristicResult_t res[1];
        int nres = 0;
        if (hipblasLtMatmulAlgoGetHeuristic(h, op, la, lb, lc, lc, pref, 1, res, &nres) != HIPBLAS_STATUS_SUCCESS ||
            nres < 1)
            break;
        const float one = 1.0f, zero = 0.0f;
        if (hipblasLtMatmul(h, op, &one, W, la, X, lb, &zero, Y, lc, Y, lc, &res[0].algo, lt_ws, kLtWorkspace,
                            stream) != HIPBLAS_STATUS_SUCCESS)
            break;
        st = GDN_OK;
    } while (false);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (lc) hipblasLtMatrixLayoutDestroy(lc);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (op) hipblasLtMatmulDescDestroy(op);
    return st;
}

// Gate logits from the fused gate product Z[token][2H] (columns 0..H-1: the
// beta logits, H..2H-1: per-token alpha terms): beta_logit[token][h] = Z[token][h],
// alpha_logit[b][f][h] = the mean over the frame's N tokens of Z[token][H + h].
// One workgroup per (b, f); thread h sums its column in token order.
__global__ void gate_split_kernel(const float* __restrict__ Z, float* __restrict__ beta_logit,
                                  float* __restrict__ alpha_logit, int N, int H) {
    const int bf = blockIdx.x;
    const size_t tok0 = (size_t)bf * N;
    const float inv_n = N > 0 ? 1.0f / (float)N : 0.0f;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float s = 0.0f;
        for (int n = 0; n < N; ++n) {
            const float* z = Z + (tok0 + n) * 2 * H;
            beta_logit[(tok0 + n) * H + h] = z[h];
            s += z[H + h];
        }
        alpha_logit[(size_t)bf * H + h] = s * inv_n;
    }
}

struct Range {
    uintptr_t lo, hi;
};
Range rng(const void* p, size_t n) { return Range{(uintptr_t)p, (uintptr_t)p + (p ? n : 0)}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
bool aligned(const void* p, uintptr_t al) { return ((uintptr_t)p & (al - 1)) == 0; }

gdn_status check_block(const gdn_desc* d, int32_t C) {
    if (!d) return GDN_ERR_INVALID_ARG;
    if (d->B < 0 || d->F < 0 || d->N < 0 || d->H < 1 || d->Dk < 1 || C < 1) return GDN_ERR_INVALID_ARG;
    if (d->io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (d->Dk != d->Dv) return GDN_ERR_UNSUPPORTED;
    if (C % 8 != 0 || ((int64_t)d->H * d->Dk) % 8 != 0) return GDN_ERR_UNSUPPORTED;   // 16-byte rows
    return GDN_OK;
}

size_t gate_bytes(const gdn_desc* d) {
    return ((size_t)d->B * d->F * d->N * 2 * d->H * sizeof(float) + 255) / 256 * 256;
}

}  // namespace

extern "C" {

size_t gdn_block_workspace_size(const gdn_desc* d, int32_t C) {
    if (check_block(d, C) != GDN_OK) return 0;
    return kLtWorkspace + gate_bytes(d);
}

gdn_status gdn_block_in_proj(const gdn_desc* d, int32_t C, const void* x, const void* w_qkv, const void* w_gate,
                             void* q, void* k, void* v, float* beta_logit, float* alpha_logit, void* workspace,
                             size_t workspace_bytes, void* stream_v) {
    gdn_status st = check_block(d, C);
    if (st != GDN_OK) return st;
    const int64_t M = (int64_t)d->B * d->F * d->N, HD = (int64_t)d->H * d->Dk;
    const size_t xb = (size_t)M * C * 2, wb = (size_t)C * 3 * HD * 2, gb = (size_t)C * 2 * d->H * 2;
    const size_t tb = (size_t)M * HD * 2, bb = (size_t)M * d->H * 4, ab = (size_t)d->B * d->F * d->H * 4;
    if (M > 0 && C > 0 && (!x || !w_qkv || !w_gate)) return GDN_ERR_INVALID_ARG;
    if (M > 0 && HD > 0 && (!q || !k || !v)) return GDN_ERR_INVALID_ARG;
    if (M > 0 && d->H > 0 && !beta_logit) return GDN_ERR_INVALID_ARG;
    if ((size_t)d->B * d->F * d->H > 0 && !alpha_logit) return GDN_ERR_INVALID_ARG;
    for (const void* p : {x, w_qkv, w_gate, (const void*)q, (const void*)k, (const void*)v})
        if (!aligned(p, 16)) return GDN_ERR_ALIGNMENT;
    if (!aligned(beta_logit, 4) || !aligned(alpha_logit, 4)) return GDN_ERR_ALIGNMENT;
    const size_t need = gdn_block_workspace_size(d, C);
    if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GDN_ERR_ALIGNMENT;
    const Range ins[] = {rng(x, xb), rng(w_qkv, wb), rng(w_gate, gb)};
    const Range outs[] = {rng(q, tb), rng(k, tb), rng(v, tb), rng(beta_logit, bb), rng(alpha_logit, ab),
                          rng(workspace, need)};
    for (int i = 0; i < 6; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return GDN_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
    }
    if (M == 0 && (size_t)d->B * d->F * d->H == 0) return GDN_OK;
    hipblasLtHandle_t h;
    if ((st = lt_handle(&h)) != GDN_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* Z = reinterpret_cast<float*>(ws + kLtWorkspace);
    // q, k, v: the three column blocks of w_qkv [C][3][H][D]
    const unsigned char* w = static_cast<const unsigned char*>(w_qkv);
    void* outs_qkv[3] = {q, k, v};
    for (int j = 0; j < 3; ++j)
        if ((st = gemm(h, M, HD, C, x, C, w + (size_t)j * HD * 2, 3 * HD, outs_qkv[j], HD, HIP_R_16BF, ws, stream)) !=
            GDN_OK)
            return st;
    // gate logits: Z = x w_gate ([C][2][H]: beta, then alpha), then the split and the frame means
    if ((st = gemm(h, M, 2 * (int64_t)d->H, C, x, C, w_gate, 2 * d->H, Z, 2 * d->H, HIP_R_32F, ws, stream)) != GDN_OK)
        return st;
    if ((size_t)d->B * d->F > 0 && d->H > 0) {
        hipLaunchKernelGGL(gate_split_kernel, dim3((unsigned)(d->B * d->F)), dim3(64), 0, stream, Z, beta_logit,
                           alpha_logit, d->N, d->H);
        if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    }
    return GDN_OK;
}

gdn_status gdn_block_out_proj(const gdn_desc* d, int32_t C, const void* o, const void* w_out, void* y,
                              void* workspace, size_t workspace_bytes, void* stream_v) {
    gdn_status st = check_block(d, C);
    if (st != GDN_OK) return st;
    const int64_t M = (int64_t)d->B * d->F * d->N, HD = (int64_t)d->H * d->Dk;
    const size_t ob = (size_t)M * HD * 2, wb = (size_t)HD * C * 2, yb = (size_t)M * C * 2;
    if (M > 0 && C > 0 && (!o || !w_out || !y)) return GDN_ERR_INVALID_ARG;
    if (!aligned(o, 16) || !aligned(w_out, 16) || !aligned(y, 16)) return GDN_ERR_ALIGNMENT;
    const size_t need = gdn_block_workspace_size(d, C);
    if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GDN_ERR_ALIGNMENT;
    const Range ry = rng(y, yb), rw = rng(workspace, need);
    if (overlap(ry, rng(o, ob)) || overlap(ry, rng(w_out, wb)) || overlap(ry, rw) || overlap(rw, rng(o, ob)) ||
        overlap(rw, rng(w_out, wb)))
        return GDN_ERR_ALIAS;
    if (M == 0 || C == 0) return GDN_OK;
    hipblasLtHandle_t h;
    if ((st = lt_handle(&h)) != GDN_OK) return st;
    return gemm(h, M, C, HD, o, HD, w_out, C, y, C, HIP_R_16BF, workspace, reinterpret_cast<hipStream_t>(stream_v));
}

}  // extern "C"
