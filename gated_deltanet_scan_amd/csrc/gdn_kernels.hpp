// HIP kernels of the frame-wise GDN forward scan for gfx950 (CDNA4).
//
// The scan is split into three kernels so that the two passes over the large
// token tensors run with every frame in parallel and only a small d x d
// recurrence stays sequential:
//
//   frame_gram    one workgroup per (b, h, f): streams K_f and V_f once,
//                 normalises keys, and forms  Gm_f = -alpha_f * G_f  and U_f
//                 with MFMA (fp32 accumulate).  Writes them to the workspace in
//                 the exact operand layouts state_scan loads.
//   state_scan    one workgroup per (b, h, 16-row tile of S): keeps its rows of
//                 S resident across the sequential frame loop and applies
//                 S <- alpha S + S Gm_f + U_f.  Rows of S evolve independently,
//                 so tiles never communicate.  Emits S_f for every frame.
//   frame_output  one workgroup per (b, h, f, token range): O_f = Q_f S_f^T.
//
// G and U contract over tokens, so frame_gram transposes K and V through LDS;
// Q.S^T and S.Gm contract over the feature dimension, which is contiguous in
// memory, so their operands load straight from global memory.
//
// MFMA fragment convention (v_mfma_f32_16x16x32_bf16): lane l = 16*g + r holds,
// for operand A (16 x 32), row r and contraction indices 8g..8g+7; for operand
// B (32 x 16), column r and the same 8 contraction indices.  A and B always use
// the same contraction order, so the product is exact whatever order the
// hardware assigns inside a lane.  The 16x16 fp32 result sits in lane l as rows
// 4g..4g+3 of column r.  The fp32 I/O mode keeps the same 8-value fragments and
// issues eight v_mfma_f32_16x16x4_f32, one per fragment element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- scalar helpers
__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 b = (__bf16)x;  // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------- I/O type traits
// Storage type of q/k/v/o: uint16_t holds bfloat16 bits; float is the fp32 mode.
template <typename T> struct IO;

template <> struct IO<uint16_t> {
    using frag = u32x4;  // 8 bf16 contraction values (16 bytes)
    static constexpr int bytes = 2;
    __device__ static __forceinline__ frag zero() { return frag{0u, 0u, 0u, 0u}; }
    __device__ static __forceinline__ frag load(const uint16_t* p) {
        return *reinterpret_cast<const u32x4*>(p);
    }
    __device__ static __forceinline__ void mma(f32x4& acc, const frag& x, const frag& y) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                      __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ float get(const frag& x, int e) {
        const uint32_t w = x[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static __forceinline__ uint32_t bits(float x) { return f2bf(x); }
};

template <> struct IO<float> {
    using frag = f32x8;  // 8 fp32 contraction values (32 bytes)
    static constexpr int bytes = 4;
    __device__ static __forceinline__ frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ static __forceinline__ frag load(const float* p) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
        return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    __device__ static __forceinline__ void mma(f32x4& acc, const frag& x, const frag& y) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], y[s], acc, 0, 0, 0);
    }
    __device__ static __forceinline__ float get(const frag& x, int e) { return x[e]; }
    __device__ static __forceinline__ uint32_t bits(float x) { return __float_as_uint(x); }
};

// Workspace: per (b, h, local frame) item, a block of 12*D*D bytes:
//   [0, 4D^2)     Gm^T  (bf16 mode: hi plane then lo plane; fp32 mode: fp32)
//   [4D^2, 8D^2)  U^T   fp32
//   [8D^2, 12D^2) S_f   (bf16 mode: hi plane then lo plane; fp32 mode: fp32), [a][e]
// with Gm^T[e][c] = -alpha G[c][e] and U^T[e][a] = U[a][e]: the transposes make
// state_scan's operand and accumulator loads contiguous 16-byte runs.
template <int D> struct WS {
    static constexpr size_t item_bytes = (size_t)12 * D * D;
    static constexpr size_t gm_off = 0;
    static constexpr size_t ut_off = (size_t)4 * D * D;
    static constexpr size_t sp_off = (size_t)8 * D * D;
};

struct ScanArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* alpha;
    const float* S_in;    // state entering frame f0 (NULL: zeros)
    void* o;
    float* S_out;         // state after the last frame of the launch (may equal S_in)
    float* S_out2;        // optional second copy of that state (NULL: none)
    unsigned char* ws;
    int B, H, F, N;
    int f0, Fc;           // frames [f0, f0 + Fc) of this launch
    int tsplit;           // token ranges per frame in frame_output
    int tchunk;           // tokens per range (multiple of 16)
    int logits;
    float eps;
};

// XCD-aware placement: workgroups are dispatched round-robin over the 8 XCDs,
// so id % 8 is the XCD.  Map ids so that groups of `per` consecutive logical
// ids (the tiles that share one head's data) land on the same XCD and hence
// share its L2.  Returns -1 for padding ids.
__device__ __forceinline__ int xcd_remap(int id, int per, int total) {
    const int xcd = id & 7, slot = id >> 3;
    const int group = (slot / per) * 8 + xcd;
    const int logical = group * per + slot % per;
    return logical < total ? logical : -1;
}

// ================================================================== frame_gram
template <typename T, int D> struct GramCfg {
    static constexpr int SZ = IO<T>::bytes;
    static constexpr int SL = D / 8;                                // 8-value slices per token
    static constexpr int TS0 = SZ == 2 ? 128 : 64;
    static constexpr int TS = (TS0 * SL >= 256) ? TS0 : 256 / SL;  // tokens per LDS stage
    static constexpr int TPT = TS * SL / 256;                       // tokens per thread per stage
    static constexpr int ROWB = TS * SZ;                            // bytes per LDS row
    static constexpr int CHUNKS = ROWB / 16;                        // 16-byte chunks per row
    static constexpr int ARR = D * ROWB;                            // bytes per transposed array
    static constexpr int LDS = 3 * ARR;
    static constexpr int RB = D / 16;                               // 16-row blocks per matrix
    static constexpr int NRW = (2 * RB + 3) / 4;                    // row blocks per wave
    static constexpr int KST = TS / 32;                             // 32-token steps per stage
    static constexpr int TPC = 16 / SZ;                             // tokens per 16-byte chunk
    static_assert(TPT >= 1 && TPT * SZ <= 16 && TPC % TPT == 0, "stage shape");
    static_assert(CHUNKS >= 8 && (CHUNKS & (CHUNKS - 1)) == 0, "swizzle needs >= 8 chunks");
};

// Byte offset of 16-byte chunk c of LDS row `row`.  The XOR swizzle spreads
// both the transposing writes (rows 8 apart) and the fragment reads (16
// consecutive rows) over the banks.
template <int ROWB>
__device__ __forceinline__ int lds_chunk(int row, int c) {
    return row * ROWB + ((c ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// Pack TPT consecutive tokens of one feature (bits already in storage width)
// into one LDS store of TPT*SZ bytes.
template <int TPT, int SZ>
__device__ __forceinline__ void lds_store_tokens(unsigned char* p, const uint32_t (&v)[TPT]) {
    if constexpr (SZ == 2) {
        if constexpr (TPT == 8) {
            *reinterpret_cast<u32x4*>(p) = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16),
                                                 v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
        } else if constexpr (TPT == 4) {
            *reinterpret_cast<u32x2*>(p) = u32x2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
        } else if constexpr (TPT == 2) {
            *reinterpret_cast<uint32_t*>(p) = v[0] | (v[1] << 16);
        } else {
            *reinterpret_cast<uint16_t*>(p) = (uint16_t)v[0];
        }
    } else {
        if constexpr (TPT == 4) {
            *reinterpret_cast<u32x4*>(p) = u32x4{v[0], v[1], v[2], v[3]};
        } else if constexpr (TPT == 2) {
            *reinterpret_cast<u32x2*>(p) = u32x2{v[0], v[1]};
        } else {
            *reinterpret_cast<uint32_t*>(p) = v[0];
        }
    }
}

// Fragment (8 contraction values) of LDS row `row`, tokens 8g..8g+7 of 32-token step ks.
template <typename T, int ROWB>
__device__ __forceinline__ typename IO<T>::frag lds_frag(const unsigned char* base, int row, int ks,
                                                         int g) {
    if constexpr (sizeof(T) == 2) {
        return *reinterpret_cast<const u32x4*>(base + lds_chunk<ROWB>(row, ks * 4 + g));
    } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(base + lds_chunk<ROWB>(row, ks * 8 + 2 * g));
        const f32x4 hi =
            *reinterpret_cast<const f32x4*>(base + lds_chunk<ROWB>(row, ks * 8 + 2 * g + 1));
        return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void frame_gram_kernel(ScanArgs a) {
    using C = GramCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
    unsigned char* const sKT = smem;                // raw keys          [feature][token]
    unsigned char* const sWK = smem + C::ARR;       // beta*rho^2 * k    [feature][token]
    unsigned char* const sUV = smem + 2 * C::ARR;   // beta*rho   * v    [feature][token]

    const int item = blockIdx.x;                    // (b*H + h)*Fc + fl
    const int fl = item % a.Fc;
    const int bh = item / a.Fc;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int f = a.f0 + fl;
    const int N = a.N, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;

    const size_t rowstride = (size_t)H * D;                     // elements between tokens
    const size_t tok0 = ((size_t)b * a.F + f) * (size_t)N;      // first token of the frame
    const T* kb = static_cast<const T*>(a.k) + tok0 * rowstride + (size_t)h * D;
    const T* vb = static_cast<const T*>(a.v) + tok0 * rowstride + (size_t)h * D;
    const float* bb = a.beta + tok0 * H + h;

    // loader role: 8-feature slice s of tokens tl*TPT + j
    const int s = tid % C::SL;
    const int tl = tid / C::SL;

    frag kr[C::TPT], vr[C::TPT];
    float br[C::TPT];
    auto load_stage = [&](int st) {
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) {
            const int n = st * C::TS + tl * C::TPT + j;
            if (n < N) {
                kr[j] = io::load(kb + (size_t)n * rowstride + s * 8);
                vr[j] = io::load(vb + (size_t)n * rowstride + s * 8);
                br[j] = bb[(size_t)n * H];
            } else {
                kr[j] = io::zero();
                vr[j] = io::zero();
                br[j] = 0.0f;
            }
        }
    };

    f32x4 acc[C::NRW][C::RB];
#pragma unroll
    for (int i = 0; i < C::NRW; ++i)
#pragma unroll
        for (int j = 0; j < C::RB; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

    const int nst = (N + C::TS - 1) / C::TS;
    const float inv_n = N > 0 ? 1.0f / (float)N : 0.0f;
    if (nst > 0) load_stage(0);

    for (int st = 0; st < nst; ++st) {
        // ---- key norms (wavefront reduction over the SL lanes of a token) and
        //      per-token scales; the previous stage's fragment reads finished
        //      at the barrier that closed the last iteration
        float wsc[C::TPT], usc[C::TPT];
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = io::get(kr[j], e);
                ss = fmaf(x, x, ss);
            }
#pragma unroll
            for (int m = 1; m < C::SL; m <<= 1) ss += __shfl_xor(ss, m, 64);
            float bt = br[j];
            if (a.logits) bt = (st * C::TS + tl * C::TPT + j < N) ? sigmoid_f(bt) * inv_n : 0.0f;
            const float rho = 1.0f / fmaxf(sqrtf(ss), a.eps);
            wsc[j] = bt * rho * rho;   // G = sum_i w_i k_i k_i^T
            usc[j] = bt * rho;         // U = sum_i u_i v_i k_i^T
        }
        // ---- transposed write: one LDS store per (feature, array) packs this
        //      thread's TPT consecutive tokens
        {
            const int t0 = tl * C::TPT;
            const int cbase = t0 / C::TPC, within = (t0 % C::TPC) * C::SZ;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int off = lds_chunk<C::ROWB>(s * 8 + e, cbase) + within;
                uint32_t raw[C::TPT], wk[C::TPT], uv[C::TPT];
#pragma unroll
                for (int j = 0; j < C::TPT; ++j) {
                    const float x = io::get(kr[j], e);
                    if constexpr (sizeof(T) == 2) {
                        raw[j] = __float_as_uint(x) >> 16;
                    } else {
                        raw[j] = __float_as_uint(x);
                    }
                    wk[j] = io::bits(wsc[j] * x);
                    uv[j] = io::bits(usc[j] * io::get(vr[j], e));
                }
                lds_store_tokens<C::TPT, C::SZ>(sKT + off, raw);
                lds_store_tokens<C::TPT, C::SZ>(sWK + off, wk);
                lds_store_tokens<C::TPT, C::SZ>(sUV + off, uv);
            }
        }
        __syncthreads();
        if (st + 1 < nst) load_stage(st + 1);     // in flight during the MFMAs

        // ---- G += (wK)^T K,  U += (uV)^T K  over the stage's tokens
#pragma unroll
        for (int ks = 0; ks < C::KST; ++ks) {
            frag bk[C::RB];
#pragma unroll
            for (int j = 0; j < C::RB; ++j) bk[j] = lds_frag<T, C::ROWB>(sKT, j * 16 + r, ks, g);
#pragma unroll
            for (int i = 0; i < C::NRW; ++i) {
                const int gb = wave + 4 * i;      // row block over [G rows ; U rows]
                if (gb < 2 * C::RB) {
                    const unsigned char* src = gb < C::RB ? sWK : sUV;
                    const int rowb = gb < C::RB ? gb : gb - C::RB;
                    const frag ak = lds_frag<T, C::ROWB>(src, rowb * 16 + r, ks, g);
#pragma unroll
                    for (int j = 0; j < C::RB; ++j) io::mma(acc[i][j], ak, bk[j]);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: Gm^T = -alpha G^T (hi/lo planes or fp32) and U^T (fp32)
    float al = a.alpha[((size_t)b * a.F + f) * H + h];
    if (a.logits) al = sigmoid_f(al);
    unsigned char* wsi = a.ws + (size_t)item * WS<D>::item_bytes;
#pragma unroll
    for (int i = 0; i < C::NRW; ++i) {
        const int gb = wave + 4 * i;
        if (gb >= 2 * C::RB) continue;
#pragma unroll
        for (int j = 0; j < C::RB; ++j) {
            const f32x4 x = acc[i][j];
            const int col = j * 16 + r;                    // e
            if (gb < C::RB) {
                const int row0 = gb * 16 + 4 * g;           // c
                const size_t idx = (size_t)col * D + row0;  // Gm^T[e][c..c+3]
                const f32x4 m = x * (-al);
                if constexpr (sizeof(T) == 2) {
                    uint16_t* hi = reinterpret_cast<uint16_t*>(wsi + WS<D>::gm_off);
                    uint16_t* lo = hi + (size_t)D * D;
                    uint32_t hb[4], lb[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        hb[t] = f2bf(m[t]);
                        lb[t] = f2bf(m[t] - bf2f((uint16_t)hb[t]));
                    }
                    *reinterpret_cast<u32x2*>(hi + idx) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
                    *reinterpret_cast<u32x2*>(lo + idx) = u32x2{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
                } else {
                    float* gm = reinterpret_cast<float*>(wsi + WS<D>::gm_off);
                    *reinterpret_cast<f32x4*>(gm + idx) = m;
                }
            } else {
                const int row0 = (gb - C::RB) * 16 + 4 * g;  // a
                float* ut = reinterpret_cast<float*>(wsi + WS<D>::ut_off);
                *reinterpret_cast<f32x4*>(ut + (size_t)col * D + row0) = x;
            }
        }
    }
}

// ================================================================== state_scan
template <typename T, int D> struct StateCfg {
    static constexpr int CT = D >= 32 ? 2 : 1;       // 16-column tiles per wave
    static constexpr int NW = D / (16 * CT);         // waves per workgroup
    static constexpr int KS = (D + 31) / 32;         // 32-wide contraction steps
    static constexpr int RT = D / 16;                // row tiles per (b, h)
    static constexpr int PADB = 16;                  // LDS row padding (bytes)
    static constexpr int ROWB = D * IO<T>::bytes + PADB;
    static constexpr int NPL = sizeof(T) == 2 ? 2 : 1;  // planes (hi, lo) of S in LDS
};

// One workgroup owns rows [16*rt, 16*rt+16) of one (b, h) state; wave w owns
// columns [32w, 32w+32) (16 wide for D = 16).  Per frame:
//   acc = alpha*S + U_f ;  acc += S_hi Gm_hi + S_lo Gm_hi + S_hi Gm_lo  (bf16)
//   (fp32 mode: acc += S Gm with fp32 MFMA)
// S is kept in fp32 registers; its bf16 hi/lo split lives in LDS as the A
// operand and is copied to the workspace for frame_output.
template <typename T, int D>
__global__ __launch_bounds__(D >= 32 ? 2 * D : 64) void state_scan_kernel(ScanArgs a) {  // NW*64
    using C = StateCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    __shared__ __attribute__((aligned(16))) unsigned char sS[C::NPL][16 * C::ROWB];

    const int units = a.B * a.H;
    const int id = xcd_remap(blockIdx.x, C::RT, units * C::RT);
    if (id < 0) return;
    const int rt = id % C::RT;
    const int bh = id / C::RT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int a0 = rt * 16;                          // first state row of this tile
    const int h = bh % a.H, b = bh / a.H;

    // ---- initial state: registers (accumulator layout) and LDS (operand layout)
    f32x4 S[C::CT];
    const float* sin = a.S_in ? a.S_in + (size_t)bh * D * D : nullptr;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
        const int col = (wave * C::CT + ct) * 16 + r;
#pragma unroll
        for (int t = 0; t < 4; ++t) S[ct][t] = sin ? sin[(size_t)(a0 + 4 * g + t) * D + col] : 0.0f;
    }
    auto put_lds = [&]() {
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
            const int col = (wave * C::CT + ct) * 16 + r;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int off = (4 * g + t) * C::ROWB + col * io::bytes;
                if constexpr (sizeof(T) == 2) {
                    const uint16_t hi = f2bf(S[ct][t]);
                    *reinterpret_cast<uint16_t*>(&sS[0][off]) = hi;
                    *reinterpret_cast<uint16_t*>(&sS[1][off]) = f2bf(S[ct][t] - bf2f(hi));
                } else {
                    *reinterpret_cast<float*>(&sS[0][off]) = S[ct][t];
                }
            }
        }
    };
    put_lds();
    __syncthreads();

    // ---- per-frame operands, prefetched one frame ahead
    struct Ops {
        frag bh_[C::CT][C::KS];   // Gm hi (fp32 mode: Gm)
        frag bl_[C::CT][C::KS];   // Gm lo (unused in fp32 mode)
        f32x4 u[C::CT];           // U rows of this tile, accumulator layout
    };
    const size_t item0 = (size_t)bh * a.Fc;
    auto load_ops = [&](int fl, Ops& o) {
        const unsigned char* wsi = a.ws + (item0 + fl) * WS<D>::item_bytes;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
            const int col = (wave * C::CT + ct) * 16 + r;   // e
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int c0 = ks * 32 + 8 * g;
                if (c0 < D) {
                    const T* gm = reinterpret_cast<const T*>(wsi + WS<D>::gm_off);
                    o.bh_[ct][ks] = io::load(gm + (size_t)col * D + c0);
                    if constexpr (sizeof(T) == 2)
                        o.bl_[ct][ks] = io::load(gm + (size_t)D * D + (size_t)col * D + c0);
                } else {
                    o.bh_[ct][ks] = io::zero();
                    o.bl_[ct][ks] = io::zero();
                }
            }
            const float* ut = reinterpret_cast<const float*>(wsi + WS<D>::ut_off);
            o.u[ct] = *reinterpret_cast<const f32x4*>(ut + (size_t)col * D + a0 + 4 * g);
        }
    };

    Ops cur, nxt;
    if (a.Fc > 0) load_ops(0, cur);
    for (int fl = 0; fl < a.Fc; ++fl) {
        if (fl + 1 < a.Fc) load_ops(fl + 1, nxt);
        const int f = a.f0 + fl;
        float al = a.alpha[((size_t)b * a.F + f) * a.H + h];
        if (a.logits) al = sigmoid_f(al);

        f32x4 acc[C::CT];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) acc[ct] = S[ct] * al + cur.u[ct];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int c0 = ks * 32 + 8 * g;
            frag ahi = io::zero(), alo = io::zero();
            if (c0 < D) {
                if constexpr (sizeof(T) == 2) {
                    ahi = *reinterpret_cast<const u32x4*>(&sS[0][r * C::ROWB + c0 * 2]);
                    alo = *reinterpret_cast<const u32x4*>(&sS[1][r * C::ROWB + c0 * 2]);
                } else {
                    ahi = io::load(reinterpret_cast<const float*>(&sS[0][r * C::ROWB + c0 * 4]));
                }
            }
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                io::mma(acc[ct], ahi, cur.bh_[ct][ks]);
                if constexpr (sizeof(T) == 2) {
                    io::mma(acc[ct], alo, cur.bh_[ct][ks]);
                    io::mma(acc[ct], ahi, cur.bl_[ct][ks]);
                }
            }
        }
        __syncthreads();                 // every wave has read S_{f-1} from LDS
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) S[ct] = acc[ct];
        put_lds();
        __syncthreads();                 // S_f visible in LDS

        // S_f (operand planes) to the workspace for frame_output: 16 rows x D
        unsigned char* sp = a.ws + (item0 + fl) * WS<D>::item_bytes + WS<D>::sp_off;
        constexpr int rowbytes = D * io::bytes;
        constexpr int chunks = 16 * rowbytes / 16;   // per plane
        for (int x = tid; x < C::NPL * chunks; x += C::NW * 64) {
            const int pl = x / chunks, cc = x % chunks;
            const int row = cc / (rowbytes / 16), col16 = cc % (rowbytes / 16);
            const u32x4 val = *reinterpret_cast<const u32x4*>(&sS[pl][row * C::ROWB + col16 * 16]);
            *reinterpret_cast<u32x4*>(sp + (size_t)pl * D * D * io::bytes +
                                      (size_t)(a0 + row) * rowbytes + col16 * 16) = val;
        }
        cur = nxt;
    }

    // ---- final state (fp32, row-major [a][e])
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
        const int col = (wave * C::CT + ct) * 16 + r;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const size_t idx = (size_t)bh * D * D + (size_t)(a0 + 4 * g + t) * D + col;
            if (a.S_out) a.S_out[idx] = S[ct][t];
            if (a.S_out2) a.S_out2[idx] = S[ct][t];
        }
    }
}

// ================================================================== frame_output
template <typename T, int D> struct OutCfg {
    static constexpr int RT = D / 16;               // 16-row tiles of S (output features)
    static constexpr int NWR = RT < 4 ? RT : 4;     // waves splitting the rows
    static constexpr int RPW = RT / NWR;            // row tiles per wave
    static constexpr int TG = 4 / NWR;              // waves splitting the tokens
    static constexpr int KS = (D + 31) / 32;
};

// o_i = S_f q_i computed as O^T = S Q^T: A = S (rows a, contraction e) held in
// registers for the whole token loop, B = Q^T whose fragments are 8 contiguous
// features of one token, loaded straight from global memory.
template <typename T, int D>
__global__ __launch_bounds__(256) void frame_output_kernel(ScanArgs a) {
    using C = OutCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;

    const int item = blockIdx.x / a.tsplit;       // (b*H + h)*Fc + fl
    const int part = blockIdx.x % a.tsplit;
    const int fl = item % a.Fc;
    const int bh = item / a.Fc;
    const int h = bh % a.H, b = bh / a.H;
    const int f = a.f0 + fl;
    const int N = a.N, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wr = wave % C::NWR, wt = wave / C::NWR;

    const int nbeg = part * a.tchunk;
    const int nend = min(N, nbeg + a.tchunk);
    if (nbeg >= nend) return;

    // ---- S_f rows of this wave as A fragments
    const unsigned char* sp = a.ws + (size_t)item * WS<D>::item_bytes + WS<D>::sp_off;
    const T* s_hi = reinterpret_cast<const T*>(sp);
    const T* s_lo = s_hi + (size_t)D * D;         // bf16 mode only
    frag ah[C::RPW][C::KS], alw[C::RPW][C::KS];
#pragma unroll
    for (int i = 0; i < C::RPW; ++i) {
        const int row = (wr * C::RPW + i) * 16 + r;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int c0 = ks * 32 + 8 * g;
            if (c0 < D) {
                ah[i][ks] = io::load(s_hi + (size_t)row * D + c0);
                if constexpr (sizeof(T) == 2) alw[i][ks] = io::load(s_lo + (size_t)row * D + c0);
            } else {
                ah[i][ks] = io::zero();
                alw[i][ks] = io::zero();
            }
        }
    }

    const size_t rowstride = (size_t)H * D;
    const size_t tok0 = ((size_t)b * a.F + f) * (size_t)N;
    const T* qb = static_cast<const T*>(a.q) + tok0 * rowstride + (size_t)h * D;
    T* ob = static_cast<T*>(a.o) + tok0 * rowstride + (size_t)h * D;

    auto load_q = [&](int t0, frag (&bq)[C::KS]) {
        const int n = t0 + r;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int c0 = ks * 32 + 8 * g;
            bq[ks] = (n < nend && c0 < D) ? io::load(qb + (size_t)n * rowstride + c0) : io::zero();
        }
    };

    const int step = 16 * C::TG;
    int t0 = nbeg + 16 * wt;
    frag cq[C::KS], nq[C::KS];
    if (t0 < nend) load_q(t0, cq);
    for (; t0 < nend; t0 += step) {
        if (t0 + step < nend) load_q(t0 + step, nq);
        f32x4 acc[C::RPW];
#pragma unroll
        for (int i = 0; i < C::RPW; ++i) {
            acc[i] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                io::mma(acc[i], ah[i][ks], cq[ks]);
                if constexpr (sizeof(T) == 2) io::mma(acc[i], alw[i][ks], cq[ks]);
            }
        }
        const int n = t0 + r;
        if (n < nend) {
#pragma unroll
            for (int i = 0; i < C::RPW; ++i) {
                const int col0 = (wr * C::RPW + i) * 16 + 4 * g;   // output features a..a+3
                T* dst = ob + (size_t)n * rowstride + col0;
                if constexpr (sizeof(T) == 2) {
                    const uint32_t x0 = f2bf(acc[i][0]), x1 = f2bf(acc[i][1]);
                    const uint32_t x2 = f2bf(acc[i][2]), x3 = f2bf(acc[i][3]);
                    *reinterpret_cast<u32x2*>(dst) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
                } else {
                    *reinterpret_cast<f32x4*>(dst) = acc[i];
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) cq[ks] = nq[ks];
    }
}

// ================================================================== state_copy
// S_final <- S0 (or zeros) for an empty scan (F == 0).  A plain kernel rather
// than a memset/memcpy node so the call stays capturable in a graph.
__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace gdn
