// HIP kernel of the backward pass's per-token gradients for gfx950 (CDNA4).
//
// The backward pass of the frame scan runs as the forward kernels in other
// roles (see gdn_kernels.hpp: frame_gram recomputes G and U and, as the
// W pass, W_f = dO_f^T Q_f; state_scan recomputes the states S_f and, as the
// adjoint recurrence, the state gradients X_f; frame_output forms
// dq_i = S_f^T do_i), plus frame_dkv below.  With X = X_f, Sp = S_{f-1} (the
// state entering frame f in the forward walk), M = Sp^T X and Ms = M + M^T,
// per token i of frame f (k^ = rho k, rho = 1 / max(|k|, eps)):
//     y_i   = X k^_i          z_i = Ms k^_i          w_i = X^T v_i
//     dv_i  = beta_i y_i
//     dk^_i = beta_i (w_i - alpha_f z_i)
//     s_i   = k^_i . z_i      p_i = v_i . y_i  (= k^_i . w_i)
//     dk_i  = rho (dk^_i - k^_i (k^_i . dk^_i)),  k^_i . dk^_i = beta_i (p_i - alpha_f s_i)
//             (dk^_i / eps where |k_i| <= eps; dk^_i itself with unnormalised keys)
//     dbeta_i  = p_i - alpha_f s_i / 2
//     dalpha_f = <X, Sp> - (1/2) sum_i beta_i s_i
// (then the sigmoid chain for gate logits).  This is the chain rule of
// S_f = alpha_f Sp (I - G_f) + U_f and o_i = S_f q_i, the frame recurrence of
// "NVIDIA's New 2.6B World Model Generates Minute-Scale 720p Video on a Single
// GPU" (section "The Architecture: Replacing Softmax Attention at Scale"); its
// gradient is what training on minute-long sequences needs ("SANA-WM:
// democratizing Minute-Scale World Modeling with Hybrid Linear DiT", section
// "Problem & Motivation").
#pragma once

#include "gdn_kernels.hpp"

namespace gdn {

struct DkvArgs {
    ScanArgs s;         // k, v, beta, alpha, S_in (the state entering the launch's
                        // chunk, NULL: zeros), ws (forward items: S planes), ws2
                        // (backward items: X planes), shapes, chunk, flags
    void* dk;
    void* dv;
    float* dbeta;
    float* dalpha;
};

template <typename T, int D> struct DkvCfg {
    static constexpr bool B16 = sizeof(T) == 2;
    static constexpr int SZ = IO<T>::bytes;
    static constexpr int NW = 8, NTH = 64 * NW;
    static constexpr int RT = D / 16;               // 16-feature tiles of the products
    static constexpr int TG = NW / RT;              // waves per tile: token groups
    static constexpr int KS = (D + 31) / 32;
    // LDS token row, padded by 16 bytes.  Within each 32-feature window the
    // 4-feature pieces are stored in the order 0,4,1,5,2,6,3,7, so that the
    // split-order fragment of lane group g (pieces g and 4+g) is contiguous
    // (at D = 16 the window is 16 features and keeps its order).
    static constexpr int ROWB = D * SZ + 16;
    static constexpr int PIECE = 4 * SZ;            // bytes of 4 features
    __device__ static constexpr int pos(int q) { return D >= 32 ? (q < 4 ? 2 * q : 2 * (q - 4) + 1) : q; }
    // byte offset in a row of the piece holding features 4p .. 4p+3
    __device__ static constexpr int piece_off(int p) { return (p >> 3) * 8 * PIECE + pos(p & 7) * PIECE; }
    static constexpr int LPR = D * SZ / 16;         // 16-byte loads per token row
    static constexpr int RPP = NTH / LPR;           // token rows per load pass
    static constexpr int BT0 = B16 ? 64 : 32;       // (fp32: half the tokens, half the LDS)
    static constexpr int BT = RPP > BT0 ? RPP : BT0;   // tokens per block
    static constexpr int NLD = BT / RPP;            // loads per thread, tensor and block
    static constexpr int NSB = BT / 16;             // 16-token sub-blocks per block
    static constexpr int MSB = NSB / TG;            // sub-blocks per wave and block
    static constexpr int PD = 2;                    // blocks in flight (register ring)
    static constexpr int TBUF = BT * ROWB;          // one tensor's tile of a block
    static constexpr int TOK = 2 * 2 * TBUF;        // K and V tiles, double-buffered
    static constexpr int PREP = 2 * TState<T, D>::BYTES;   // X^T and Sp^T staging
    // what a wave keeps of each sub-block between its two halves: dk^ (fp32 x4),
    // k (bf16 x4 or fp32 x4), rho and beta
    static constexpr int KQB = B16 ? 8 : 16;
    static constexpr int KEEP = NW * MSB * 64 * (16 + KQB + 8);
    static constexpr int BIG = TOK + KEEP > PREP ? TOK + KEEP : PREP;
    static constexpr int RED = 2 * RT * BT * 8;     // per-token (s, p) partials, double-buffered
    static constexpr int BETA = 2 * 2 * BT * 4;     // the blocks' betas and key scales
    static constexpr int LDS = BIG + RED + BETA + 2 * NW * 4;
    static_assert(MSB >= 1 && NSB % TG == 0 && NLD >= 1 && BT % RPP == 0 && BT % 16 == 0 && PD % 2 == 0 &&
                      2 * BT <= NTH,
                  "block shape");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float wave_sum(float x) {
    x = group_sum<16>(x);
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}
// Sum over the four lanes 16g + r (g = 0..3) that hold one token: a swap of
// rows 0,2 with rows 1,3, then of rows 0,1 with rows 2,3 (v_permlane16_swap
// and v_permlane32_swap); after each swap the two registers hold a lane's own
// value and its partner's, in some order, so their sum is the pair's sum.
__device__ __forceinline__ float token_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// acc += (ah + al)(bh + bl) without the al*bl term (bf16 mode); fp32 mode
// has no low parts.
template <typename T>
__device__ __forceinline__ void mma_hl(f32x4& acc, const typename IO<T>::frag& ah, const typename IO<T>::frag& al,
                                       const typename IO<T>::frag& bh, const typename IO<T>::frag& bl) {
    IO<T>::mma(acc, ah, bh);
    if constexpr (sizeof(T) == 2) {
        IO<T>::mma(acc, ah, bl);
        IO<T>::mma(acc, al, bh);
    }
}

// One workgroup of 8 waves per (b, h, f) item.  Prologue: X_f and Sp are
// staged transposed in LDS; wave (tile wr, token group wt) keeps, for its 16
// features, the operand fragments of X (rows of X), X^T and Ms as high and
// low bf16 parts in registers.  Ms's column block wr is formed as
// Sp^T X + X^T Sp over all row blocks; Ms is symmetric, so those result blocks
// are exactly the wave's row fragments of Ms in the split contraction order.
// Token loop: 64-token blocks of K and V stream from HBM two blocks ahead into
// registers and through a double-buffered LDS tile (split-order fragments, as
// in frame_output); per 16 tokens a wave forms its 16 features of y, z and w
// with MFMA, writes dv, and leaves its partial sums of s and p in LDS.  After
// the next block's barrier every wave adds the tiles' partials in a fixed
// order and finishes dk; the waves of tile 0 write dbeta and sum the dalpha
// term.  Every reduction has a fixed order: results are bitwise reproducible.
template <typename T, int D>
__global__ __launch_bounds__(512, 1) void frame_dkv_kernel(DkvArgs da) {
    using C = DkvCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    using W = WS<T, D>;
    using TSt = TState<T, D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
    const ScanArgs& a = da.s;

    // items in frame-major order, head fastest, heads rotated by the rest of
    // the index so that the XCDs see every head
    const int x = blockIdx.x;
    const int h = (x % a.H + x / a.H) % a.H;
    const int fl = (x / a.H) % a.Fc;
    const int b = x / (a.H * a.Fc);
    const int bh = b * a.H + h;
    const int f = a.f0 + fl;
    const int N = a.N, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int wr = wave % C::RT, wt = wave / C::RT;

    float al = a.alpha[((size_t)b * a.F + f) * H + h];
    float dal_chain = 1.0f;
    if (a.logits) {
        al = sigmoid_f(al);
        dal_chain = al * (1.0f - al);
    }
    const float inv_n = N > 0 ? 1.0f / (float)N : 0.0f;
    const float inv_eps = 1.0f / a.eps;
    const bool raw = a.raw_keys != 0;

    // this head's rows of the frame through buffer resources (rows past N
    // read as zeros, stores to them are dropped)
    const size_t rowstride = (size_t)H * D;
    const size_t tok0 = ((size_t)b * a.F + f) * (size_t)N;
    const uint32_t rbytes = N > 0 ? (uint32_t)(((size_t)(N - 1) * rowstride + D) * C::SZ) : 0u;
    const rsrc_t rk = make_rsrc(static_cast<const T*>(a.k) + tok0 * rowstride + (size_t)h * D, rbytes);
    const rsrc_t rv = make_rsrc(static_cast<const T*>(a.v) + tok0 * rowstride + (size_t)h * D, rbytes);
    const rsrc_t rdk = make_rsrc(static_cast<T*>(da.dk) + tok0 * rowstride + (size_t)h * D, rbytes);
    const rsrc_t rdv = make_rsrc(static_cast<T*>(da.dv) + tok0 * rowstride + (size_t)h * D, rbytes);
    const uint32_t bbytes = N > 0 ? (uint32_t)(((N - 1) * H + 1) * 4) : 0u;
    const rsrc_t rb = make_rsrc(a.beta + tok0 * H + h, bbytes);
    const rsrc_t rrho = make_rsrc(raw ? nullptr : a.rho + tok0 * H + h, raw ? 0u : bbytes);   // raw: scale 1
    const rsrc_t rdb = make_rsrc(da.dbeta + tok0 * H + h, bbytes);
    const uint32_t row_bytes = (uint32_t)(H * D * C::SZ);
    const int nblk = (N + C::BT - 1) / C::BT;

    unsigned char* const tx = smem;                              // X^T staging
    unsigned char* const tsp = smem + TSt::BYTES;                // Sp^T staging
    float* const red = reinterpret_cast<float*>(smem + C::BIG);  // [2][RT][BT] x (s, p)
    float* const sbeta = red + 2 * C::RT * C::BT * 2;            // [2][BT] betas, then [2][BT] key scales
    float* const wsum = sbeta + 4 * C::BT;                       // [2][NW]

    // ---- token blocks: loader role (row lr of each pass, 16-byte column lc)
    const int lc = tid % C::LPR, lr = tid / C::LPR;
    struct TStage {
        u32x4 k[C::NLD], v[C::NLD];
        float bt;           // threads < BT: beta of token tid; BT..2BT-1: its key scale
    };
    const int sbt = tid % (2 * C::BT);
    auto load_blk = [&](int blk, TStage& R) {
        const uint32_t base = (uint32_t)(blk * C::BT + lr) * row_bytes + (uint32_t)(lc * 16);
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            R.k[i] = bload16_nt(rk, base + (uint32_t)(i * C::RPP) * row_bytes);
            R.v[i] = bload16_nt(rv, base + (uint32_t)(i * C::RPP) * row_bytes);
        }
        const uint32_t boff = (uint32_t)((blk * C::BT + (sbt % C::BT)) * H * 4);
        R.bt = sbt < C::BT ? bload4f(rb, boff) : bload4f(rrho, boff);
    };
    auto put_blk = [&](const TStage& R, unsigned char* buf, float* sb) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int row = lr + i * C::RPP;
            unsigned char* kr = buf + row * C::ROWB;
            unsigned char* vr = kr + C::TBUF;
            if constexpr (C::B16) {                              // a 16-byte chunk is pieces 2lc, 2lc+1
                *reinterpret_cast<u32x2*>(kr + C::piece_off(2 * lc)) = u32x2{R.k[i][0], R.k[i][1]};
                *reinterpret_cast<u32x2*>(kr + C::piece_off(2 * lc + 1)) = u32x2{R.k[i][2], R.k[i][3]};
                *reinterpret_cast<u32x2*>(vr + C::piece_off(2 * lc)) = u32x2{R.v[i][0], R.v[i][1]};
                *reinterpret_cast<u32x2*>(vr + C::piece_off(2 * lc + 1)) = u32x2{R.v[i][2], R.v[i][3]};
            } else {                                             // a 16-byte chunk is piece lc
                *reinterpret_cast<u32x4*>(kr + C::piece_off(lc)) = R.k[i];
                *reinterpret_cast<u32x4*>(vr + C::piece_off(lc)) = R.v[i];
            }
        }
        if (tid < 2 * C::BT) sb[tid < C::BT ? tid : C::BT + tid] = R.bt;
    };
    TStage ring[C::PD];
#pragma unroll
    for (int j = 0; j < C::PD; ++j) load_blk(j, ring[j]);

    // ---- prologue: stage X^T and Sp^T, keep this wave's operand fragments
    const unsigned char* xp = a.ws2 + ((size_t)bh * a.Fc + fl) * W::item_bytes + W::sp_off;
    const bool first = a.reverse ? (fl == a.Fc - 1) : (fl == 0);    // Sp enters the chunk
    const int flp = a.reverse ? fl + 1 : fl - 1;
    const unsigned char* spp = first ? nullptr : a.ws + ((size_t)bh * a.Fc + flp) * W::item_bytes + W::sp_off;
    const float* srm = (first && a.S_in) ? a.S_in + (size_t)bh * D * D : nullptr;
    // Every global load of the prologue is issued before the first LDS write
    // (a store between them would keep the compiler from hoisting the loads):
    // this wave's rows of X (tile wr, every step), and of Sp the steps it
    // stages.  Wave (wr, wt) stages the fragments (wr, kk) of X and Sp with
    // kk = wt mod TG, so every fragment is staged exactly once.
    // (The source of Sp is chosen once, outside the loops: a choice per load
    // made the compiler wait for each load before issuing the next.)
    auto staged = [&](int kk) { return C::TG == 1 || kk % C::TG == wt; };
    frag xd_h[C::KS], xd_l[C::KS];                               // rows 16wr.. of X
    frag sp_h[C::KS], sp_l[C::KS];
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) state_frag<T, D>(xp, nullptr, wr, kk, lane, xd_h[kk], xd_l[kk]);
    if (spp) {
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk)
            if (staged(kk)) state_frag<T, D>(spp, nullptr, wr, kk, lane, sp_h[kk], sp_l[kk]);
    } else {
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk)
            if (staged(kk)) state_frag<T, D>(nullptr, srm, wr, kk, lane, sp_h[kk], sp_l[kk]);
    }
    float dot = 0.0f;                                            // <X, Sp>, this thread's share
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
        if (staged(kk)) {
            put_transposed<T, D>(tx, wr, kk, lane, xd_h[kk], xd_l[kk]);
            put_transposed<T, D>(tsp, wr, kk, lane, sp_h[kk], sp_l[kk]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dot += (io::get(xd_h[kk], e) + io::get(xd_l[kk], e)) * (io::get(sp_h[kk], e) + io::get(sp_l[kk], e));
        }
    }
    dot = wave_sum(dot);
    if (lane == 0) wsum[wave] = dot;
    __syncthreads();

    frag xt_h[C::KS], xt_l[C::KS], ms_h[C::KS], ms_l[C::KS];
    {
        frag st_h[C::KS], st_l[C::KS];
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
            get_transposed<T, D>(tx, wr, kk, lane, xt_h[kk], xt_l[kk]);
            get_transposed<T, D>(tsp, wr, kk, lane, st_h[kk], st_l[kk]);
        }
        // column block wr of Ms: block i = (Sp^T)_i X_wr + (X^T)_i Sp_wr, contracted over rows
        // (steps outermost, so that consecutive products go to different blocks)
        f32x4 m[C::RT];
#pragma unroll
        for (int i = 0; i < C::RT; ++i) m[i] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
#pragma unroll
            for (int i = 0; i < C::RT; ++i) {
                frag ah, alo;
                get_transposed<T, D>(tsp, i, kk, lane, ah, alo);
                mma_hl<T>(m[i], ah, alo, xt_h[kk], xt_l[kk]);
                get_transposed<T, D>(tx, i, kk, lane, ah, alo);
                mma_hl<T>(m[i], ah, alo, st_h[kk], st_l[kk]);
            }
        }
        // lane 16g+r of block i holds Ms[16i + 4g + t][16wr + r] = Ms[16wr + r][16i + 4g + t]:
        // blocks 2kk and 2kk+1 are the two halves of the split-order fragment kk
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
            const f32x4 u0 = m[2 * kk < C::RT ? 2 * kk : 0];
            const f32x4 u1 = 2 * kk + 1 < C::RT ? m[2 * kk + 1 < C::RT ? 2 * kk + 1 : 0] : f32x4{0, 0, 0, 0};
            if constexpr (C::B16) {
                const u32x4 hh{pack_bf16x2(u0[0], u0[1]), pack_bf16x2(u0[2], u0[3]), pack_bf16x2(u1[0], u1[1]),
                               pack_bf16x2(u1[2], u1[3])};
                ms_h[kk] = hh;
                ms_l[kk] = u32x4{pack_bf16x2(u0[0] - io::get(hh, 0), u0[1] - io::get(hh, 1)),
                                 pack_bf16x2(u0[2] - io::get(hh, 2), u0[3] - io::get(hh, 3)),
                                 pack_bf16x2(u1[0] - io::get(hh, 4), u1[1] - io::get(hh, 5)),
                                 pack_bf16x2(u1[2] - io::get(hh, 6), u1[3] - io::get(hh, 7))};
            } else {
                ms_h[kk] = f32x8{u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                ms_l[kk] = io::zero();
            }
        }
    }
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {                         // formed before the barrier, not after it
        hold(xt_h[kk]);
        hold(xt_l[kk]);
        hold(ms_h[kk]);
        hold(ms_l[kk]);
    }
    __syncthreads();                                             // staging read before the token tiles reuse it

    // ---- token loop
    // per sub-block this wave keeps in LDS, for its finish after the next
    // barrier: dk^ at the lane's four features, k there, rho (negative where
    // dk has no projection term: dk = |rho| dk^ - (rho > 0 ? rho^2 : 0) (k^ . dk^) k)
    // and beta
    unsigned char* const keep = smem + C::TOK + wave * (C::MSB * 64 * (16 + C::KQB + 8));
    auto keep_dkh = [&](int m) { return reinterpret_cast<f32x4*>(keep + (m * 64 + lane) * 16); };
    auto keep_kq = [&](int m) { return keep + C::MSB * 64 * 16 + (m * 64 + lane) * C::KQB; };
    auto keep_rb = [&](int m) { return reinterpret_cast<f32x2*>(keep + C::MSB * 64 * (16 + C::KQB) + (m * 64 + lane) * 8); };
    float bsum = 0.0f;                                           // sum of beta_i s_i (waves of tile 0)
    const int fcol = (16 * wr + 4 * g) * C::SZ;                  // byte offset of this lane's features

    auto unpack4 = [](u32x2 w2) {
        return f32x4{__uint_as_float(w2[0] << 16), __uint_as_float(w2[0] & 0xffff0000u), __uint_as_float(w2[1] << 16),
                     __uint_as_float(w2[1] & 0xffff0000u)};
    };
    // this lane's four features of token row `row` of a tile (raw bits in bf16 mode)
    const int own_off = C::piece_off(4 * wr + g);                // piece of features 16wr + 4g ..
    auto own_raw = [&](const unsigned char* tile, int row) {
        if constexpr (C::B16)
            return *reinterpret_cast<const u32x2*>(tile + row * C::ROWB + own_off);
        else
            return *reinterpret_cast<const f32x4*>(tile + row * C::ROWB + own_off);
    };
    // split-order fragment of step kk of token row `row`
    auto split_frag = [&](const unsigned char* tile, int row, int kk) {
        // pieces g and 4+g of window kk: contiguous (D = 16: piece g, no second half)
        const unsigned char* p0 = tile + row * C::ROWB + kk * 8 * C::PIECE + 2 * g * C::PIECE;
        if constexpr (C::B16) {
            if constexpr (D >= 32) {
                return *reinterpret_cast<const frag*>(p0);
            } else {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(tile + row * C::ROWB + g * C::PIECE);
                return frag{lo[0], lo[1], 0u, 0u};
            }
        } else {
            if constexpr (D >= 32) {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(p0);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(p0 + 16);
                return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(tile + row * C::ROWB + g * C::PIECE);
                return frag{lo[0], lo[1], lo[2], lo[3], 0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };
    auto store4 = [&](rsrc_t rs, int n, f32x4 val) {
        const uint32_t off = (uint32_t)n * row_bytes + (uint32_t)fcol;
        if constexpr (C::B16)
            bstore8(rs, off, u32x2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])});
        else
            bstore16(rs, off, __builtin_bit_cast(u32x4, val));
    };

    // (sub-blocks unrolled: 621 against 638 us at the full-minute shape; the
    // finishing pass stays a loop, unrolling it or merging it into this one
    // measured no better)
    auto compute = [&](const unsigned char* buf, const float* sb, float* rd, int blk) {
#pragma unroll
        for (int m = 0; m < C::MSB; ++m) {
            const int tl = (wt + C::TG * m) * 16 + r;            // token of the block
            const int n = blk * C::BT + tl;
            const unsigned char* kt = buf;
            const unsigned char* vt = buf + C::TBUF;
            // high and low parts accumulate separately: six independent MFMA chains
            f32x4 yh = f32x4{0, 0, 0, 0}, zh = yh, wh = yh, yl = yh, zl = yh, wl = yh;
#pragma unroll
            for (int kk = 0; kk < C::KS; ++kk) {
                const frag kb = split_frag(kt, tl, kk), vb = split_frag(vt, tl, kk);
                io::mma(yh, xd_h[kk], kb);
                io::mma(zh, ms_h[kk], kb);
                io::mma(wh, xt_h[kk], vb);
                if constexpr (C::B16) {
                    io::mma(yl, xd_l[kk], kb);
                    io::mma(zl, ms_l[kk], kb);
                    io::mma(wl, xt_l[kk], vb);
                }
            }
            const f32x4 y = yh + yl, z = zh + zl, w = wh + wl;
            const float rho = raw ? 1.0f : sb[2 * C::BT + tl];   // 1 / max(|k|, eps), from the recomputation
            const bool proj = !raw && rho < inv_eps;             // |k| > eps: dk has the projection term
            u32x2 kraw = u32x2{0u, 0u};
            f32x4 kq, vq;
            if constexpr (C::B16) {
                kraw = own_raw(kt, tl);
                kq = unpack4(kraw);
                vq = unpack4(own_raw(vt, tl));
            } else {
                kq = own_raw(kt, tl);
                vq = own_raw(vt, tl);
            }
            // y and z here are X k and Ms k; the key scale enters as scalars
            float sp = 0.0f, pp = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sp = fmaf(kq[j], z[j], sp);
                pp = fmaf(vq[j], y[j], pp);
            }
            sp = token_sum(sp * (rho * rho));                    // k^ . Ms k^ over this tile's features
            pp = token_sum(pp * rho);                            // v . X k^
            if (g == 0) *reinterpret_cast<f32x2*>(rd + 2 * (wr * C::BT + tl)) = f32x2{sp, pp};
            float bt = sb[tl];
            if (a.logits) bt = sigmoid_f(bt) * inv_n;
            if (n >= N) bt = 0.0f;
            const float br = bt * rho;
            store4(rdv, n, y * br);                              // dv = beta X k^
            *keep_dkh(m) = w * bt - z * (al * br);               // dk^ = beta (X^T v - alpha Ms k^)
            if constexpr (C::B16)
                *reinterpret_cast<u32x2*>(keep_kq(m)) = kraw;
            else
                *reinterpret_cast<f32x4*>(keep_kq(m)) = kq;
            *keep_rb(m) = f32x2{proj ? rho : -rho, bt};
        }
    };
    auto finish = [&](const float* rd, int blk) {
#pragma unroll 1
        for (int m = 0; m < C::MSB; ++m) {
            const int tl = (wt + C::TG * m) * 16 + r;
            const int n = blk * C::BT + tl;
            float s = 0.0f, p = 0.0f;
#pragma unroll
            for (int t = 0; t < C::RT; ++t) {
                const f32x2 v2 = *reinterpret_cast<const f32x2*>(rd + 2 * (t * C::BT + tl));
                s += v2[0];
                p += v2[1];
            }
            const f32x2 rb2 = *keep_rb(m);
            const float rh = rb2[0], bt = rb2[1];
            const float cdot = bt * (p - al * s);                // k^ . dk^
            f32x4 kq;
            if constexpr (C::B16)
                kq = unpack4(*reinterpret_cast<const u32x2*>(keep_kq(m)));
            else
                kq = *reinterpret_cast<const f32x4*>(keep_kq(m));
            store4(rdk, n, *keep_dkh(m) * fabsf(rh) - kq * ((rh > 0.0f ? rh * rh : 0.0f) * cdot));
            if (wr == 0 && g == 0) {
                // logits: d beta / d logit = sigma (1 - sigma) / N = beta (1 - N beta)
                const float chain = a.logits ? bt * (1.0f - (float)N * bt) : 1.0f;
                if (n < N) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((p - 0.5f * al * s) * chain), rdb,
                                                                 (uint32_t)(n * H * 4), 0, 0);
                bsum = fmaf(bt, s, bsum);
            }
        }
    };

    unsigned char* const tok = smem;
    const int nfull = nblk / C::PD;
    for (int gi = 0; gi < nfull; ++gi) {
#pragma unroll
        for (int j = 0; j < C::PD; ++j) {
            const int blk = gi * C::PD + j;
            unsigned char* buf = tok + (j & 1) * 2 * C::TBUF;
            put_blk(ring[j], buf, sbeta + (j & 1) * C::BT);
            __syncthreads();
            if (blk > 0) finish(red + ((j + 1) & 1) * C::RT * C::BT * 2, blk - 1);
            load_blk(blk + C::PD, ring[j]);                      // past the frame: zeros, no traffic
            compute(buf, sbeta + (j & 1) * C::BT, red + (j & 1) * C::RT * C::BT * 2, blk);
        }
    }
    const int rem = nblk - nfull * C::PD;
#pragma unroll
    for (int j = 0; j < C::PD; ++j) {
        if (j < rem) {
            const int blk = nfull * C::PD + j;
            unsigned char* buf = tok + (j & 1) * 2 * C::TBUF;
            put_blk(ring[j], buf, sbeta + (j & 1) * C::BT);
            __syncthreads();
            if (blk > 0) finish(red + ((j + 1) & 1) * C::RT * C::BT * 2, blk - 1);
            compute(buf, sbeta + (j & 1) * C::BT, red + (j & 1) * C::RT * C::BT * 2, blk);
        }
    }
    __syncthreads();
    if (nblk > 0) finish(red + ((nblk - 1) & 1) * C::RT * C::BT * 2, nblk - 1);

    // ---- dalpha: <X, Sp> - (1/2) sum beta_i s_i, partial sums in a fixed order
    bsum = wave_sum(bsum);
    if (lane == 0) wsum[C::NW + wave] = wr == 0 ? bsum : 0.0f;
    __syncthreads();
    if (tid == 0) {
        float dsum = 0.0f, bs = 0.0f;
        for (int i = 0; i < C::NW; ++i) {
            dsum += wsum[i];
            bs += wsum[C::NW + i];
        }
        da.dalpha[((size_t)b * a.F + f) * H + h] = (dsum - 0.5f * bs) * dal_chain;
    }
}

}  // namespace gdn
