// Projections either side of the scan inside a GDN block: the C ABI of
// gdn_block_in_proj / gdn_block_out_proj (declared in include/gdn.h).
//
// The q, k, v and output products are plain bf16 GEMMs with fp32 accumulation
// and go to hipBLASLt; the gate logits (2H outputs per token, with a mean over
// each frame's tokens) are kernels of this file.  Weights are stored
// output-major, one row of inputs per output.  Row-major products
// Y[M][N] = X[M][K] W^T are issued as their column-major transposes
// Y^T = W X^T, which read the same memory.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/gdn.h"

namespace {

constexpr size_t kLtWorkspace = (size_t)32 << 20;   // hipBLASLt's share of the workspace
constexpr int kMaxWidth = 1 << 20;                   // C and H*D (32-bit offsets within 64 rows)

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

// Y[M][N] (row stride ldy, type yt) = X[M][K] (row stride ldx) W^T, with the
// weights W stored output-major ([N][K], row stride ldw); X and W bf16, fp32
// accumulation.
gdn_status gemm(hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, const void* W,
                int64_t ldw, void* Y, int64_t ldy, hipDataType yt, void* lt_ws, hipStream_t stream) {
    if (M == 0 || N == 0) return GDN_OK;
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    gdn_status st = GDN_ERR_LAUNCH;
    do {
        if (hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) break;
        const hipblasOperation_t tr = HIPBLAS_OP_T, nt = HIPBLAS_OP_N;
        hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &tr, sizeof(tr));
        hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &nt, sizeof(nt));
        // column-major view: Y^T (N x M) = op(A) B with A = W^T stored K x N (ld ldw)
        // and transposed, B = X^T stored K x M (ld ldx)
        if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, K, N, ldw) != HIPBLAS_STATUS_SUCCESS) break;
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

// ------------------------------------------------------------------ gate logits
// The gate rows of the input projection have only 2H outputs per token, so a
// library GEMM would stream the hidden states at a fraction of HBM speed and
// leave the frame mean to another pass.  gate_proj_kernel reads each hidden
// state once, forms the 2H logits of 64 tokens with MFMA, writes the beta
// logits and one partial sum of the alpha terms per 64-token chunk;
// alpha_mean_kernel adds the chunks of a frame in order and divides by N.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kGateTok = 64;    // tokens per workgroup: four 16-token MFMA tiles
constexpr int kGateWaves = 4;   // waves per workgroup; they split the contraction
constexpr int kGateThreads = 64 * kGateWaves;

// Raw buffer resource over [p, p + bytes): loads past the end return zeros,
// which masks the rows past the last token and the outputs past 2H.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                   0, 0, 0);
}

// Grid (B*F*ceil(N/64) chunks, the chunk index fastest; 1; slabs of 16*OT gate rows).  MFMA operands: A = gate
// weights (16 rows = outputs), B = hidden states (16 columns = tokens); lane
// l = 16g + r holds row/column r and eight contraction indices.  In 128-wide
// steps lane group g reads 32 consecutive inputs at 128s + 32g (64 bytes per
// row, so four lanes cover 256 contiguous bytes), and the j-th MFMA of the
// step takes the eight at offset 8j: both operands use this same order, so the
// sum covers every input exactly once.  Waves take every fourth step; their
// partial tiles are added in wave order through LDS.
template <int OT>
__global__ __launch_bounds__(kGateThreads) void gate_proj_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wg,
                                                                 float* __restrict__ beta_logit,
                                                                 float* __restrict__ part, int N, int C, int H,
                                                                 int nchunk) {
    constexpr int MW = 16 * OT;     // gate rows per workgroup
    constexpr int ZS = MW + 4;      // padded row stride of the logit tile in LDS (floats)
    __shared__ f32x4 red[kGateWaves][OT * 4][64];
    __shared__ float zt[kGateTok * ZS];
    const int c = (int)(blockIdx.x % (unsigned)nchunk), bf = (int)(blockIdx.x / (unsigned)nchunk);
    const int m0 = blockIdx.z * MW;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int n0 = c * kGateTok;
    const int rows = min(kGateTok, N - n0);
    const int mrows = min(MW, 2 * H - m0);
    const uint32_t rowb = (uint32_t)C * 2;
    const rsrc_t rx = make_rsrc(x + ((size_t)bf * N + n0) * C, (uint32_t)rows * rowb);
    const rsrc_t rw = make_rsrc(wg + (size_t)m0 * C, (uint32_t)mrows * rowb);
    f32x4 acc[OT][4];
#pragma unroll
    for (int o = 0; o < OT; ++o)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[o][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsup = C / 128;
    for (int s = wave; s < nsup; s += kGateWaves) {
        const uint32_t kb = (uint32_t)(128 * s + 32 * g) * 2;
        u32x4 xa[4][4], wa[OT][4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) xa[t][j] = bload16(rx, (16 * t + r) * rowb + kb + 16 * j);
#pragma unroll
        for (int o = 0; o < OT; ++o)
#pragma unroll
            for (int j = 0; j < 4; ++j) wa[o][j] = bload16(rw, (16 * o + r) * rowb + kb + 16 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int o = 0; o < OT; ++o)
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[o][t] = mma(wa[o][j], xa[t][j], acc[o][t]);
    }
    // inputs past the last whole 128-wide step: 32-wide steps, lane group g
    // taking the eight at k0 + 8g (zeros past C; C is a multiple of 8)
    for (int k0 = nsup * 128 + 32 * wave; k0 < C; k0 += 32 * kGateWaves) {
        const int k = k0 + 8 * g;
        u32x4 xa[4], wa[OT];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            xa[t] = k < C ? bload16(rx, (16 * t + r) * rowb + (uint32_t)k * 2) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int o = 0; o < OT; ++o)
            wa[o] = k < C ? bload16(rw, (16 * o + r) * rowb + (uint32_t)k * 2) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int o = 0; o < OT; ++o)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[o][t] = mma(wa[o], xa[t], acc[o][t]);
    }

#pragma unroll
    for (int o = 0; o < OT; ++o)
#pragma unroll
        for (int t = 0; t < 4; ++t) red[wave][o * 4 + t][lane] = acc[o][t];
    __syncthreads();
    // tile q = 4o + t of lane l: gate rows 16o + 4g .. +3 of token 16t + r
#pragma unroll
    for (int i = 0; i < OT; ++i) {
        const int q = wave + kGateWaves * i;
        f32x4 z = red[0][q][lane];
#pragma unroll
        for (int w = 1; w < kGateWaves; ++w) z += red[w][q][lane];
        const int o = q >> 2, t = q & 3;
        *reinterpret_cast<f32x4*>(&zt[(16 * t + r) * ZS + 16 * o + 4 * g]) = z;
    }
    __syncthreads();
    // beta logits: token-major rows of H, this slab's beta columns contiguous
    const size_t tok0 = (size_t)bf * N + n0;
    for (int idx = tid; idx < kGateTok * MW; idx += kGateThreads) {
        const int n = idx / MW, m = idx % MW, mg = m0 + m;
        if (n < rows && mg < H) beta_logit[(tok0 + n) * H + mg] = zt[n * ZS + m];
    }
    // alpha terms: one partial sum per chunk, tokens in order
    if (tid < MW) {
        const int mg = m0 + tid;
        if (mg >= H && mg < 2 * H) {
            float sum = 0.f;
            for (int n = 0; n < rows; ++n) sum += zt[n * ZS + tid];
            part[((size_t)bf * nchunk + c) * H + (mg - H)] = sum;
        }
    }
}

// alpha_logit[bf][h] = (sum over the frame's chunks, in order, of the partial
// sums) / N; one workgroup per (b, f).  With N == 0 there are no chunks and the
// logit is 0.
__global__ void alpha_mean_kernel(const float* __restrict__ part, float* __restrict__ alpha_logit, int nchunk,
                                  int H, float inv_n) {
    const int bf = blockIdx.x;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float s = 0.f;
        for (int c = 0; c < nchunk; ++c) s += part[((size_t)bf * nchunk + c) * H + h];
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
    if (C > kMaxWidth || (int64_t)d->H * d->Dk > kMaxWidth) return GDN_ERR_UNSUPPORTED;
    // one gate workgroup per (b, f, 64-token chunk) in a one-dimensional grid
    if ((int64_t)d->B * d->F * ((d->N + 63) / 64) > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

int gate_chunks(const gdn_desc* d) { return (d->N + kGateTok - 1) / kGateTok; }

// fp32 partial sums of the alpha terms, [B*F][chunks][H]
size_t gate_bytes(const gdn_desc* d) {
    return ((size_t)d->B * d->F * gate_chunks(d) * d->H * sizeof(float) + 255) / 256 * 256;
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
    float* part = reinterpret_cast<float*>(ws + kLtWorkspace);
    // q, k, v: the three row blocks of w_qkv [3][H][D][C]
    const unsigned char* w = static_cast<const unsigned char*>(w_qkv);
    void* outs_qkv[3] = {q, k, v};
    for (int j = 0; j < 3; ++j)
        if ((st = gemm(h, M, HD, C, x, C, w + (size_t)j * HD * C * 2, C, outs_qkv[j], HD, HIP_R_16BF, ws, stream)) !=
            GDN_OK)
            return st;
    // gate logits and the frame means of the alpha terms
    const int nchunk = gate_chunks(d);
    const int BF = d->B * d->F;
    if (nchunk > 0 && BF > 0) {
        const int H2 = 2 * d->H;
        const unsigned slabs = (unsigned)((H2 + 63) / 64);
        const dim3 grid((unsigned)((int64_t)nchunk * BF), 1u, H2 <= 32 ? 1u : slabs);
        const uint16_t* xx = static_cast<const uint16_t*>(x);
        const uint16_t* wg = static_cast<const uint16_t*>(w_gate);
        if (H2 <= 16)
            hipLaunchKernelGGL(gate_proj_kernel<1>, grid, dim3(kGateThreads), 0, stream, xx, wg, beta_logit, part,
                               d->N, C, d->H, nchunk);
        else if (H2 <= 32)
            hipLaunchKernelGGL(gate_proj_kernel<2>, grid, dim3(kGateThreads), 0, stream, xx, wg, beta_logit, part,
                               d->N, C, d->H, nchunk);
        else
            hipLaunchKernelGGL(gate_proj_kernel<4>, grid, dim3(kGateThreads), 0, stream, xx, wg, beta_logit, part,
                               d->N, C, d->H, nchunk);
        if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    }
    if (BF > 0) {
        hipLaunchKernelGGL(alpha_mean_kernel, dim3((unsigned)BF), dim3(64), 0, stream, part, alpha_logit, nchunk,
                           d->H, d->N > 0 ? 1.0f / (float)d->N : 0.0f);
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
    return gemm(h, M, C, HD, o, HD, w_out, HD, y, C, HIP_R_16BF, workspace, reinterpret_cast<hipStream_t>(stream_v));
}

}  // extern "C"
