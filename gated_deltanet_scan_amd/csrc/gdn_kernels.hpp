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
//   state_scan    one wave per (b, h, 16-row slab of S): keeps its rows of S
//                 in registers across the sequential frame loop and applies
//                 S <- alpha S + S Gm_f + U_f.  Rows of S evolve independently,
//                 so slabs never communicate.  Emits S_f for every frame.
//   frame_output  one workgroup per (b, h, f, token range): O_f = Q_f S_f^T.
//
// G and U contract over tokens, so frame_gram transposes K and V through LDS;
// Q.S^T and S.Gm contract over the feature dimension, which is contiguous in
// memory, so their operands load straight from global memory.
//
// MFMA fragment convention (v_mfma_f32_16x16x32_bf16): lane l = 16*g + r holds,
// for operand A (16 x 32), row r and eight contraction indices; for operand B
// (32 x 16), column r and the same eight.  A and B always use the same
// contraction order, so the product is exact whatever order the hardware
// assigns inside a lane.  The 16x16 fp32 result sits in lane l as rows
// 4g..4g+3 of column r.  The fp32 I/O mode keeps the same 8-value fragments and
// issues eight v_mfma_f32_16x16x4_f32, one per fragment element.
//
// Two contraction orders are used.  Natural: lane group g takes indices
// 8g..8g+7 of a 32-wide step.  Split: lane group g takes 4g..4g+3 and
// 16+4g..16+4g+3, i.e. the four values a lane holds in each of two adjacent
// 16x16 results.  The state products (S Gm in the recurrence, Q S^T in the
// output pass) contract over the columns of S in the split order, so that a
// lane's own two result blocks of S are already its operand fragment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- scalar helpers
__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 b = (__bf16)x;  // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }
// Sum over aligned groups of L consecutive lanes (L = 1, 2, 4, 8, 16), result
// in every lane of the group, using DPP lane swaps inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L <= 16, "group larger than a DPP row");
    if constexpr (L >= 2) x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (L >= 4) x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (L >= 8) x += dpp_f<0x141>(x);   // row_half_mirror
    if constexpr (L >= 16) x += dpp_f<0x140>(x);  // row_mirror
    return x;
}
// Two floats to two bf16 (round to nearest even) in one dword, x in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}
// Hold a value read from LDS in registers at this point.  hipcc sinks LDS
// reads whose first use lies past a later __syncthreads() below that barrier
// (nothing in the barrier's lowering stops it), where other waves may already
// be overwriting the memory; an empty asm statement that consumes the value
// keeps the read (and its wait) above the barrier.
template <typename V>
__device__ __forceinline__ void hold(const V& x) {
    static_assert(sizeof(V) % 4 == 0, "whole dwords");
    const auto d = __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(sizeof(V) / 4))), x);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(V) / 4); ++i) asm volatile("" ::"v"(d[i]));
}
// Remainder code of x against its bf16 rounding h (bits in the low half of
// hb): x - h is at most half a bf16 ulp, 2^(E-134) for h's biased exponent E;
// the code counts it in 1/256 ulps, rounded to nearest and clamped to int8.
// h plus rem_value(code) carries x to about 2^-16 relative, in 3 bytes.
__device__ __forceinline__ int rem_code(float x, uint32_t hb) {
    const int e = (int)((hb >> 7) & 0xffu);
    const float t = __builtin_rintf(__builtin_amdgcn_ldexpf(x - bf2f((uint16_t)hb), 142 - e));
    return (int)__builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
}
__device__ __forceinline__ float rem_value(int code, uint32_t hb) {
    return __builtin_amdgcn_ldexpf((float)code, (int)((hb >> 7) & 0xffu) - 142);
}
// byte i (signed) of a dword of codes
__device__ __forceinline__ int code_at(uint32_t w, int i) { return (int)(w << (24 - 8 * i)) >> 24; }
__device__ __forceinline__ uint32_t pack_codes(int c0, int c1, int c2, int c3) {
    return (uint32_t)(c0 & 0xff) | (uint32_t)(c1 & 0xff) << 8 | (uint32_t)(c2 & 0xff) << 16 | (uint32_t)c3 << 24;
}
// The remainders of an 8-value bf16 fragment as a bf16 fragment (exact: a
// code times a power of two has at most 8 significant bits).
__device__ __forceinline__ u32x4 rem_frag(u32x4 h, u32x2 c) {
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = c[j >> 1];
        out[j] = pack_bf16x2(rem_value(code_at(w, 2 * (j & 1)), h[j] & 0xffffu),
                             rem_value(code_at(w, 2 * (j & 1) + 1), h[j] >> 16));
    }
    return out;
}
// Codes of four fp32 values against their bf16 pair dwords h01, h23.
__device__ __forceinline__ uint32_t codes4(f32x4 x, uint32_t h01, uint32_t h23) {
    return pack_codes(rem_code(x[0], h01 & 0xffffu), rem_code(x[1], h01 >> 16), rem_code(x[2], h23 & 0xffffu),
                      rem_code(x[3], h23 >> 16));
}
// Frames per state_scan launch (alpha values are staged in LDS).
constexpr int kMaxChunkFrames = 256;

// ---------------------------------------------------------------- buffer resources
// Token tensors are read and written through raw buffer resources whose range
// ends at the last valid row: the hardware returns zeros for loads past it and
// drops stores past it.  Ragged tails therefore need no branches, and every
// prefetch is issued unconditionally, which keeps the compiler's wait counts
// exact (a conditional load forces a full drain at the next use).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9-family config word

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Streams read exactly once (K, V, Q): the non-temporal policy bit keeps them
// from displacing reused lines; measured about 12% faster for this pattern.
constexpr int kNonTemporal = 2;
// Stores of the recurrence's per-frame state planes: non-temporal with device
// scope (nt | sc1).  With the default policy their write-back backed up the
// shared vector-memory counter and stalled the next frames' operand loads
// once about half the frames were written (state_scan 124 -> 91 us).
constexpr int kStreamStore = 2 | 16;
// Stores of frame_gram's Gm and U: device scope (sc1).  Measured 6% faster
// for frame_gram than the default policy, with no cost to the recurrence that
// reads them; the non-temporal bit instead slowed those reads by half.
constexpr int kWorkspaceStore = 16;
// Buffer stores, each followed by a pad of wait states during which its data
// registers stay unchanged.  A VALU write to a buffer store's data registers
// in the cycles right after the store issues can change the stored value on
// gfx950, and the compiler pads that case only for stores without a scalar
// offset register (every store here has one).  Seen before this pad: one or
// two corrupted values per ~30 M stored when the instruction after the
// state planes' 16-byte store rewrote its first data register.  The asm
// consumes the data after the store, so the registers cannot be reused
// before the pad ends.
template <int AUX>
__device__ __forceinline__ void store_b128(u32x4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, AUX);
    asm volatile("s_nop 2" ::"v"(v));
}
template <int AUX>
__device__ __forceinline__ void store_b64(u32x2 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, AUX);
    asm volatile("s_nop 2" ::"v"(v));
}
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
}
__device__ __forceinline__ float bload4f(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
    store_b64<0>(v, r, off, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, u32x4 v) {
    store_b128<0>(v, r, off, 0);
}

// ---------------------------------------------------------------- I/O type traits
// Storage type of q/k/v/o: uint16_t holds bfloat16 bits; float is the fp32 mode.
// fp8e4m3 is the block-scaled input mode: q, k and v hold OCP FP8 E4M3 bytes,
// each run of 32 consecutive features of a token row shares an E8M0 scale
// 2^(e - 127) (the OCP microscaling "MXFP8" layout), and the kernels turn
// them into bf16 on load (exact: an E4M3 value times a power of two fits
// bf16), so everything after the load, the output included, is the bf16 mode.
// fp4e2m1 is the same layout with OCP FP4 E2M1 values, two per byte (the
// lower four bits hold the feature of even index): the "MXFP4" layout.
struct fp8e4m3 {
    uint8_t bits;
};
struct fp4e2m1 {
    uint8_t bits;                                      // two values
};
template <typename T> struct Elem {
    using C = T;                                       // compute (and output) type
    static constexpr int G2 = 2 * (int)sizeof(T);      // half-bytes per input element in HBM
};
template <> struct Elem<fp8e4m3> {
    using C = uint16_t;
    static constexpr int G2 = 2;
};
template <> struct Elem<fp4e2m1> {
    using C = uint16_t;
    static constexpr int G2 = 1;
};
// Bytes of n input elements (n even) and the address of element n of a tensor.
template <typename TIN>
__device__ __forceinline__ constexpr size_t elem_bytes(size_t n) {
    return n * Elem<TIN>::G2 / 2;
}
template <typename TIN>
__device__ __forceinline__ const unsigned char* elem_ptr(const void* p, size_t n) {
    return static_cast<const unsigned char*>(p) + elem_bytes<TIN>(n);
}
constexpr int kMxBlock = 32;                           // features per E8M0 scale
// Eight E4M3 values (two dwords) times 2^(e - 127), as eight bf16 values.
__device__ __forceinline__ u32x4 mx_to_bf16(u32x2 raw, uint32_t e) {
    const float sc = __builtin_amdgcn_ldexpf(1.0f, (int)e - 127);
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], sc, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], sc, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], sc, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], sc, true))};
}
// Eight E2M1 values (one dword, byte j holding features 2j and 2j+1) times
// 2^(e - 127), as eight bf16 values (exact: two significant bits).
__device__ __forceinline__ u32x4 mx_to_bf16(uint32_t raw, uint32_t e) {
    const float sc = __builtin_amdgcn_ldexpf(1.0f, (int)e - 127);
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, sc, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, sc, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, sc, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, sc, 3))};
}

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
    __device__ static __forceinline__ frag bload(rsrc_t r, uint32_t off) { return bload16(r, off); }
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
    __device__ static __forceinline__ frag bload(rsrc_t r, uint32_t off) {
        const u32x4 lo = bload16(r, off), hi = bload16(r, off + 16);
        return f32x8{__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]),
                     __uint_as_float(lo[3]), __uint_as_float(hi[0]), __uint_as_float(hi[1]),
                     __uint_as_float(hi[2]), __uint_as_float(hi[3])};
    }
    __device__ static __forceinline__ float get(const frag& x, int e) { return x[e]; }
    __device__ static __forceinline__ uint32_t bits(float x) { return __float_as_uint(x); }
};

// Workspace: per (b, h, local frame) item, three D x D matrices stored
// fragment-major.  An MFMA fragment (64 lanes x 8 contraction values) is kept
// as 64 consecutive 16-byte lane slots (bf16: one 1 KiB block; fp32: two
// 1 KiB blocks with values 0-3 and 4-7 of every lane), so that every 64-lane
// load or store of it touches one contiguous KiB.
//   Gm^T   operand A of state_scan: fragment (e-tile j, step kk), lane 16g+r:
//          Gm^T[16j + r][c] for the split order's c of step kk, where
//          Gm^T[e][c] = -alpha G[c][e] (bf16, rounded to nearest even, or
//          fp32).  At D = 16 the second half of each slot is never written.
//   U      tiles in the state's register layout in state_scan: block (e-tile,
//          a-tile) holds, in lane 16g+r, U[16a_t + r][16e_t + 4g + t] for
//          t = 0..3 (fp32)
//   S_f    operand A of frame_output: fragment (a-tile, step kk), lane 16g+r:
//          S_f[16a_t + r][c] in the split order (bf16 mode: the bf16 plane,
//          then its remainder codes (rem_code), 8 bytes per lane slot: three
//          bytes per value at about 2^-16 relative precision; fp32 mode: one
//          fp32 plane)
template <typename T, int D> struct WS {
    static constexpr bool B16 = sizeof(T) == 2;
    static constexpr int KS = (D + 31) / 32;                  // contraction fragments per tile
    static constexpr int RT = D / 16;                         // 16-row tiles
    static constexpr size_t FRAG = B16 ? 1024 : 2048;
    static constexpr size_t OPND = (size_t)RT * KS * FRAG;    // one operand plane
    static constexpr size_t gm_off = 0;
    static constexpr size_t ut_off = OPND;
    static constexpr size_t sp_off = ut_off + (size_t)RT * RT * 1024;
    static constexpr size_t sc_rel = OPND;                    // S codes, after the S plane (bf16)
    // bf16: the codes take half a plane; the item keeps a whole one (round
    // item strides measured faster for the recurrence's stores)
    static constexpr size_t item_bytes = sp_off + (B16 ? 2 : 1) * OPND;
    // byte offset of lane `lane`'s slot in operand fragment (tile, kt), half h (fp32)
    __device__ static __forceinline__ uint32_t frag_off(int tile, int kt, int h, int lane) {
        return (uint32_t)((tile * KS + kt) * FRAG) + (uint32_t)(h * 1024 + lane * 16);
    }
    // bf16 U (the forward scan at larger shapes): block pair (e blocks 2ep and
    // 2ep + 1, a block ga), lane 16g + r: the four values of each block as above,
    // rounded to bf16, in one 16-byte slot; the pairs fill the first half of
    // the U region
    __device__ static __forceinline__ size_t up_off(int ep, int ga) {
        return ut_off + (size_t)(ep * RT + ga) * 1024;
    }
    // the same slot's 8 remainder codes in the code plane of S_f (bf16)
    __device__ static __forceinline__ uint32_t code_off(int tile, int kt, int lane) {
        return (uint32_t)((tile * KS + kt) * 512) + (uint32_t)(lane * 8);
    }
};

// Host-side copy of the per-item workspace size (must match WS<T, D>).
constexpr size_t ws_item_bytes(int esz, int D) {
    const size_t KS = (size_t)(D + 31) / 32, RT = (size_t)D / 16;
    const size_t opnd = RT * KS * (esz == 2 ? 1024 : 2048);
    return (esz == 2 ? 3 : 2) * opnd + RT * RT * 1024;
}
static_assert(ws_item_bytes(2, 16) == WS<uint16_t, 16>::item_bytes && ws_item_bytes(2, 128) == WS<uint16_t, 128>::item_bytes &&
                  ws_item_bytes(4, 16) == WS<float, 16>::item_bytes && ws_item_bytes(4, 64) == WS<float, 64>::item_bytes,
              "host and device workspace layouts disagree");

struct ScanArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* alpha;
    const float* S_in;    // state entering frame f0 (NULL: zeros)
    void* o;
    float* S_out;         // state after the last frame of the launch (may equal S_in)
    unsigned char* ws;
    unsigned char* ws2;   // backward pass: the second item set (W_f and the adjoint
                          // state planes), same layout as ws
    int B, H, F, N;
    int f0, Fc;           // frames [f0, f0 + Fc) of this launch; the workspace holds
                          // Fc frames per (b, h): item (b, h, fl) is (b*H + h)*Fc + fl
    int tsplit;           // token ranges per frame in frame_output
    int tchunk;           // tokens per range (multiple of 16)
    int ntail;            // frame_output: the last ntail (frame, range) items run
                          // as two workgroups of half the tokens each
    int logits;
    int raw_keys;         // keys used as given (no L2 normalisation)
    int reverse;          // the recurrence walks the frames from last to first
    float eps;
    // One-frame path (see frame_step_kernel): frame_gram splits each (b, h)
    // into `parts` token ranges of `tpart` tokens (a multiple of its stage)
    // and, when parts > 1, writes unscaled fp32 partial G and U per range to
    // `spart`; it also copies `S_in` (ncopy floats) to `scopy` when that is
    // not NULL.  The scan path uses parts = 1, tpart = N.
    int parts;
    int tpart;
    float* spart;
    float* scopy;
    int ncopy;
    // Backward pass: the recomputing frame_gram also writes every token's key
    // scale rho = 1 / max(|k|, eps) here, fp32 [B][F][N][H].
    float* rho;
    // Block-scaled inputs: the E8M0 scales of q, k and v, [B][F][N][H][D/32].
    const uint8_t* qs;
    const uint8_t* ks;
    const uint8_t* vs;
};

// Partial G and U of one token range (one-frame path), both fp32: G in the
// fragment-major layout of the fp32 workspace (unscaled), then U as in the
// workspace.
template <int D> struct PartLayout {
    static constexpr int KS = (D + 31) / 32, RT = D / 16;
    static constexpr size_t g_off = 0;
    static constexpr size_t u_off = (size_t)RT * KS * 2048;
    static constexpr size_t bytes = u_off + (size_t)RT * RT * 1024;
    // byte offset of lane `lane`'s slot in G fragment (tile, kt), half h
    __device__ static __forceinline__ uint32_t frag_off(int tile, int kt, int h, int lane) {
        return (uint32_t)((tile * KS + kt) * 2048) + (uint32_t)(h * 1024 + lane * 16);
    }
};
constexpr size_t part_bytes(int D) { return (size_t)(D / 16) * ((D + 31) / 32) * 2048 + (size_t)(D / 16) * (D / 16) * 1024; }
static_assert(part_bytes(64) == PartLayout<64>::bytes && part_bytes(16) == PartLayout<16>::bytes, "partial layout");

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

// ---------------------------------------------------------------- LDS transpose reads
// gfx950's ds_read_b64_tr_b16 works on groups of 16 lanes: lane s of a group
// reads four 16-bit values w[s][0..3] (8 bytes at its own address), and lane
// i of the group receives w[i/4][i%4], w[4 + i/4][i%4], w[8 + i/4][i%4],
// w[12 + i/4][i%4] (layout checked on the device).  So if lane s points at
// row kb + s/4, columns c0 + 4(s%4) .. +3 of a row-major 16-bit array, lane i
// receives column c0 + i of rows kb .. kb+3: a column slice, i.e. the MFMA
// operand fragment of the transposed array, read from its natural layout.
// Token-major tiles (one row per token, D features of 2 bytes, 16-byte
// chunks XOR-permuted by (2 row) mod 8, which spreads the four rows one group
// reads over distinct chunk positions and keeps each row's eight chunks apart
// for the 16-byte writes; the counters still show more bank-conflict cycles
// than the transposing writes had) give the fragment for features f0 + r,
// tokens kb .. kb + 7 of a 32-token step as two such reads.
template <int ROWT>
__device__ __forceinline__ int tok_off(int row, int f) {      // byte offset of feature f of token `row`
    return row * ROWT + ((((f >> 3) ^ (2 * row)) & 7) << 4) + ((f & 7) << 1);
}
template <int ROWT>
__device__ __forceinline__ u32x4 tr_frag(const unsigned char* arr, int f0, int kb, int r) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int f = f0 + 4 * (r & 3);
    const lds_i16x4* p0 = (const lds_i16x4*)(arr + tok_off<ROWT>(kb + (r >> 2), f));
    const lds_i16x4* p1 = (const lds_i16x4*)(arr + tok_off<ROWT>(kb + 4 + (r >> 2), f));
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p0)));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p1)));
    return u32x4{a[0], a[1], b[0], b[1]};
}

// ================================================================== frame_gram
template <typename T, int D> struct GramCfg {
    static constexpr int SZ = IO<T>::bytes;
    static constexpr int FPT = 16 / SZ;                 // features per producer thread: one
                                                        // 16-byte load per token
    static constexpr int SL = D / FPT;                  // producer lanes sharing one token
    static constexpr int NP = 512;                      // producer threads (waves 8-15)
    static constexpr int TPT = 2;                       // tokens per producer thread: one
                                                        // 2-token transposed LDS write per feature
    static constexpr int TS = NP * TPT / SL;            // tokens per stage
    static constexpr int ROWB = TS * SZ;                // bytes per LDS row (one feature)
    static constexpr int CHUNKS = ROWB / 16;            // 16-byte chunks per row
    static constexpr int ARR = D * ROWB;                // one transposed array: 16 KiB
    static constexpr int BUF = 3 * ARR;                 // one stage: rho K, V, beta rho K
    static constexpr int LDS = 2 * BUF;                 // double buffer
    static constexpr int RB = D / 16;                   // 16-row blocks per matrix
    static constexpr int TR = RB >= 2 ? RB / 2 : 1;     // row blocks per consumer tile
    static constexpr int TC = RB >= 2 ? RB / 2 : 1;     // column blocks per consumer tile
    static constexpr int NCT = RB / TC;                 // column tiles
    static constexpr int NT = (2 * RB / TR) * NCT;      // tiles = busy consumer waves
    static constexpr int KST = TS / 32;                 // 32-token steps per stage
    static_assert(ARR == 16384 && NT <= 8 && TS % 32 == 0, "stage shape");
    static_assert(CHUNKS >= 8 && CHUNKS % 8 == 0, "the swizzle permutes groups of 8 chunks");
    static_assert(SL >= 2 && SL <= 32, "token lanes");
};

// Byte offset of 16-byte chunk c of LDS row `row`.  The XOR swizzle was
// chosen by measuring candidates on gfx950: with it the fragment reads (16
// consecutive rows, four chunks) run conflict-free at one KiB per 5 clocks,
// and the transposing 8-byte writes at the 8 clocks per wave that every
// candidate needed; (row ^ row >> 3) made the reads 2-way.
template <int ROWB>
__device__ __forceinline__ int lds_chunk(int row, int c) {
    return row * ROWB + ((c ^ ((row ^ (row >> 4)) & 7)) << 4);
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

// The 16 bytes of consecutive features of one token a producer thread loads.
template <typename T> struct Quad;
template <> struct Quad<uint16_t> {
    using type = u32x4;
    __device__ static __forceinline__ type load(rsrc_t r, uint32_t off) { return bload16_nt(r, off); }
    __device__ static __forceinline__ float get(const type& x, int e) {
        const uint32_t w = x[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static __forceinline__ uint32_t bits(const type& x, int e) {
        return (e & 1) ? (x[e >> 1] >> 16) : (x[e >> 1] & 0xffffu);
    }
};
template <> struct Quad<fp8e4m3> {                     // the same eight features as one byte each
    using type = u32x2;
    __device__ static __forceinline__ type load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
    }
};
template <> struct Quad<fp4e2m1> {                     // ... and as half a byte each
    using type = uint32_t;
    __device__ static __forceinline__ type load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNonTemporal);
    }
};
template <> struct Quad<float> {
    using type = u32x4;
    __device__ static __forceinline__ type load(rsrc_t r, uint32_t off) { return bload16_nt(r, off); }
    __device__ static __forceinline__ float get(const type& x, int e) { return __uint_as_float(x[e]); }
    __device__ static __forceinline__ uint32_t bits(const type& x, int e) { return x[e]; }
};

// Sum over aligned groups of L lanes (L <= 32); the step across the two rows
// of a 32-lane group (fp32 at D = 128) uses ds_swizzle (lane ^ 16).
template <int L>
__device__ __forceinline__ float lane_group_sum(float x) {
    if constexpr (L <= 16) {
        return group_sum<L>(x);
    } else {
        static_assert(L == 32, "group of 32 lanes at most");
        x = group_sum<16>(x);
        return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    }
}

// Persistent workgroups of 16 waves walking the (b, h, f) items in
// frame-major order (head fastest), round by round, so the heads of one frame
// together read each contiguous token row of [B,F,N,H,D].
// Waves 8-15 produce: each thread streams 16 bytes of features of two tokens
// of K_f and V_f (and their betas) through registers, four stages ahead, reduces the
// key norms over the lanes of each token, scales, and writes the stage
// transposed ([feature][token]) into one half of a double-buffered LDS.
// Waves 0-7 consume the other half with MFMA, one 64x64 tile of the stacked
// [G ; U] each:
//     G += (rho K)^T (beta rho K),    U += V^T (beta rho K)
// so both products share the scaled B operand and V is only transposed; after
// an item's last stage they write Gm = -alpha G and U to the workspace.  Two
// waves of each role per SIMD let one issue while the other waits: a single
// wave issues VALU work far below the SIMD's rate.
// PART selects the one-frame path's variant (token ranges, fp32 partials,
// state copy); the scan path's instantiation carries none of it.  WPASS is the
// backward pass's use of the same product with unit betas and keys as given:
// with k := Q and v := dO its U is W_f = dO_f^T Q_f, and only the U tiles run.
// RHO (the backward pass's recomputation) also writes each token's key scale
// to a.rho.  TIN is the input element type (fp8e4m3: block-scaled bytes,
// turned into bf16 as each stage is written to LDS; everything else is the
// bf16 mode).
template <typename TIN, int D, bool PART, bool WPASS = false, bool RHO = false, bool LP = false>
__global__ __launch_bounds__(1024, 1) void frame_gram_kernel(ScanArgs a) {
    using T = typename Elem<TIN>::C;
    constexpr bool MX = !__is_same(T, TIN);
    static_assert(!LP || (sizeof(T) == 2 && !PART && !WPASS && !RHO && D >= 64), "bf16 U: the scan path only");
    constexpr int GB2 = Elem<TIN>::G2;              // input half-bytes per element
    using C = GramCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    using Q = Quad<T>;                              // the stage's values (bf16 bits or fp32)
    using QL = Quad<TIN>;                           // what the loads return
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

    const int N = a.N, H = a.H;
    const int parts = PART ? a.parts : 1, tpart = PART ? a.tpart : N;
    const int items = a.B * a.H * a.Fc * parts;
    // Round k of the persistent loop covers items [k*G, (k+1)*G) (G = grid),
    // so the heads of a frame are read together; within a round, workgroup b
    // takes item k*G + slot(k).  The slot rotates with k, which walks every
    // workgroup through all heads: a head's 256-byte rows sit at one fixed
    // offset of every token row, and with a fixed head per workgroup the
    // workgroups of the slower heads (measured up to 15% slower) set the
    // kernel's time.  When a round's items per XCD (G/8; workgroup b runs on
    // XCD b mod 8) hold whole frames, the XCD of workgroup b takes slots
    // [G/8 * (b mod 8), G/8 * (b mod 8 + 1)), so every frame's heads share one
    // L2: their betas interleave in the same lines ([.., token, head]), and
    // with a frame's heads spread over all eight XCDs each XCD fetched those
    // lines again (54 MB of the full-minute scan's 58 MB of beta traffic).
    const int G = (int)gridDim.x, rounds = items / G;
    const int per = G / 8;
    const bool xcd_frames = !PART && G % 8 == 0 && per % H == 0;
    auto slot = [&](int k) {
        const int bx = (int)blockIdx.x;
        return xcd_frames ? per * (bx & 7) + ((bx >> 3) + k) % per : (bx + k) % G;
    };
    const int nmine = rounds + (slot(rounds) < items - rounds * G ? 1 : 0);
    const int nst = (tpart + C::TS - 1) / C::TS;    // stages per item (token range)
    const int total = nmine * nst;                  // stages of this workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches and offsets
    const int r = lane & 15, g = lane >> 4;
    const bool producer = wave >= 8;

    struct Item {
        int b, h, f, p, ws;                         // batch, head, frame, token range,
                                                    // workspace (or partial) slot
    };
    // item x: head fastest, then token range, frame, batch
    auto item_of = [&](int k) {
        const int x = k * G + slot(k);
        Item it;
        it.h = x % H;
        const int y = x / H;
        it.p = y % parts;
        const int fl = (y / parts) % a.Fc;
        it.b = y / (parts * a.Fc);
        it.f = a.f0 + fl;
        it.ws = ((it.b * H + it.h) * a.Fc + fl) * parts + it.p;
        return it;
    };
    // tokens of item `it`'s range (the host makes every range non-empty)
    auto range_tokens = [&](const Item& it) { return PART ? min(tpart, N - it.p * tpart) : N; };

    // ---- producer state (32-bit offsets: the host bounds a frame below 2 GiB)
    const int ptid = tid & (C::NP - 1);
    const int s = ptid % C::SL;                     // features s*FPT .. s*FPT+3
    const int tl = ptid / C::SL;                    // tokens tl*TPT .. tl*TPT+TPT-1
    const size_t rowstride = (size_t)H * D;         // elements between tokens
    const uint32_t row_bytes = (uint32_t)(H * D * GB2 / 2);
    const uint32_t kv_off0 = (uint32_t)(tl * C::TPT) * row_bytes + (uint32_t)(s * C::FPT * GB2 / 2);
    // block-scaled inputs: each token row has D/32 scale bytes; this thread's
    // eight features lie in block s*FPT/32
    constexpr int NB = D / kMxBlock;
    const uint32_t srow = (uint32_t)(H * NB);
    const uint32_t sc_off0 = (uint32_t)(tl * C::TPT) * srow + (uint32_t)(s * C::FPT / kMxBlock);
    // betas of this thread's tokens (the lanes of a token load the same value:
    // an exchange through ds_bpermute instead waited on LDS latency)
    const uint32_t b_off0 = (uint32_t)(tl * C::TPT * H * 4);
    const float inv_n = N > 0 ? 1.0f / (float)N : 0.0f;
    const float inv_eps = 1.0f / a.eps;
    // this thread's LDS write offsets (feature e, its TPT tokens), fixed for every stage
    int woff[C::FPT];
#pragma unroll
    for (int e = 0; e < C::FPT; ++e) {
        const int t0b = tl * C::TPT * C::SZ;        // byte position of the first token in a row
        woff[e] = lds_chunk<C::ROWB>(s * C::FPT + e, t0b >> 4) + (t0b & 15);
    }

    struct Stage {
        typename QL::type k[C::TPT], v[C::TPT];
        float bt[C::TPT];
        uint32_t ks[C::TPT], vs[C::TPT];            // E8M0 scales (block-scaled inputs)
    };
    // The producers' load stream walks this workgroup's stages in order, one
    // per call; the item's buffer resources are rebuilt only when an item
    // ends, so the per-stage cost is the loads and one offset add.  Stages past
    // the end stay on the last item past its last token: the buffer range
    // check returns zeros for them.
    struct Loader {
        rsrc_t rk, rv, rb, rks, rvs;
        uint32_t kvo, bo, so;                       // offsets of the next stage
        int kk, st;                                 // its item and stage within the item
    };
    auto loader_item = [&](Loader& L, int kk) {
        const Item it = item_of(kk);
        const size_t tok0 = ((size_t)it.b * a.F + it.f) * (size_t)N + (size_t)it.p * tpart;
        const int nt = range_tokens(it);
        const uint32_t kv_bytes = nt > 0 ? (uint32_t)elem_bytes<TIN>((size_t)(nt - 1) * H * D + D) : 0u;
        const uint32_t beta_bytes = nt > 0 ? (uint32_t)(((nt - 1) * H + 1) * 4) : 0u;
        L.rk = make_rsrc(elem_ptr<TIN>(a.k, tok0 * rowstride + (size_t)it.h * D), kv_bytes);
        L.rv = make_rsrc(elem_ptr<TIN>(a.v, tok0 * rowstride + (size_t)it.h * D), kv_bytes);
        if constexpr (MX) {
            const uint32_t sc_bytes = nt > 0 ? (uint32_t)((nt - 1) * H * NB + NB) : 0u;
            L.rks = make_rsrc(a.ks + tok0 * H * NB + (size_t)it.h * NB, sc_bytes);
            L.rvs = make_rsrc(a.vs + tok0 * H * NB + (size_t)it.h * NB, sc_bytes);
            L.so = sc_off0;
        }
        L.rb = make_rsrc(a.beta + tok0 * H + it.h, beta_bytes);
        L.kvo = kv_off0;
        L.bo = b_off0;
        L.kk = kk;
        L.st = 0;
    };
    auto load_stage = [&](Loader& L, Stage& R) {
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) {
            R.k[j] = QL::load(L.rk, L.kvo + (uint32_t)j * row_bytes);
            R.v[j] = QL::load(L.rv, L.kvo + (uint32_t)j * row_bytes);
        }
        if constexpr (MX) {
#pragma unroll
            for (int j = 0; j < C::TPT; ++j) {
                R.ks[j] = __builtin_amdgcn_raw_buffer_load_b8(L.rks, L.so + (uint32_t)j * srow, 0, 0);
                R.vs[j] = __builtin_amdgcn_raw_buffer_load_b8(L.rvs, L.so + (uint32_t)j * srow, 0, 0);
            }
            L.so += (uint32_t)C::TS * srow;
        }
        if constexpr (!WPASS) {
#pragma unroll
            for (int j = 0; j < C::TPT; ++j) R.bt[j] = bload4f(L.rb, L.bo + (uint32_t)(j * H * 4));
        }
        L.kvo += (uint32_t)C::TS * row_bytes;
        L.bo += (uint32_t)(C::TS * H * 4);
        if (++L.st == nst && L.kk + 1 < nmine) loader_item(L, L.kk + 1);
    };
    // Norms, scales and the transposed LDS write of stage gs.
    auto write_stage = [&](int gs, const Stage& R, unsigned char* buf) {
        // the stage's values (block-scaled inputs: converted to bf16 here)
        typename Q::type Rk[C::TPT], Rv[C::TPT];
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) {
            if constexpr (MX) {
                Rk[j] = mx_to_bf16(R.k[j], R.ks[j]);
                Rv[j] = mx_to_bf16(R.v[j], R.vs[j]);
            } else {
                Rk[j] = R.k[j];
                Rv[j] = R.v[j];
            }
        }
        // the tokens' sums of squares as independent chains (two per token),
        // then their lane reductions side by side, then the gates: a branch
        // inside the per-token loop kept the compiler from interleaving them
        float ssa[C::TPT], ssb[C::TPT], bt[C::TPT], rho[C::TPT], xs[C::TPT];
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) {
            ssa[j] = 0.0f;
            ssb[j] = 0.0f;
#pragma unroll
            for (int e = 0; e < C::FPT; e += 2) {
                const float k0 = Q::get(Rk[j], e), k1 = Q::get(Rk[j], e + 1);
                ssa[j] = fmaf(k0, k0, ssa[j]);
                ssb[j] = fmaf(k1, k1, ssb[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) ssa[j] = lane_group_sum<C::SL>(ssa[j] + ssb[j]);
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) bt[j] = WPASS ? 1.0f : R.bt[j];
        if (!WPASS && a.logits) {
            const int t0 = (gs % nst) * C::TS + tl * C::TPT, nt = range_tokens(item_of(gs / nst));
#pragma unroll
            for (int j = 0; j < C::TPT; ++j) bt[j] = (t0 + j < nt) ? sigmoid_f(bt[j]) * inv_n : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < C::TPT; ++j) {
            rho[j] = (WPASS || a.raw_keys) ? 1.0f : fminf(__builtin_amdgcn_rsqf(ssa[j]), inv_eps);   // 1 / max(|k|, eps)
            xs[j] = bt[j] * rho[j];
        }
        if constexpr (RHO) {
            if (s == 0) {                           // one lane of each token
                const Item it = item_of(gs / nst);
                const int t0 = (gs % nst) * C::TS + tl * C::TPT, nt = range_tokens(it);
#pragma unroll
                for (int j = 0; j < C::TPT; ++j)
                    if (t0 + j < nt) a.rho[(((size_t)it.b * a.F + it.f) * N + t0 + j) * H + it.h] = rho[j];
            }
        }
        unsigned char* sKH = buf;                   // rho k         (A of G)
        unsigned char* sVT = buf + C::ARR;          // v             (A of U)
        unsigned char* sXB = buf + 2 * C::ARR;      // beta rho k    (B of both)
#pragma unroll
        for (int e = 0; e < C::FPT; ++e) {
            const float k0 = Q::get(Rk[0], e), k1 = Q::get(Rk[1], e);
            if constexpr (sizeof(T) == 2) {         // the two tokens' bf16 values in one dword
                if constexpr (!WPASS)
                    *reinterpret_cast<uint32_t*>(sKH + woff[e]) = pack_bf16x2(rho[0] * k0, rho[1] * k1);
                *reinterpret_cast<uint32_t*>(sXB + woff[e]) = pack_bf16x2(xs[0] * k0, xs[1] * k1);
                *reinterpret_cast<uint32_t*>(sVT + woff[e]) = Q::bits(Rv[0], e) | (Q::bits(Rv[1], e) << 16);
            } else {
                if constexpr (!WPASS) *reinterpret_cast<f32x2*>(sKH + woff[e]) = f32x2{rho[0] * k0, rho[1] * k1};
                *reinterpret_cast<f32x2*>(sXB + woff[e]) = f32x2{xs[0] * k0, xs[1] * k1};
                *reinterpret_cast<f32x2*>(sVT + woff[e]) = f32x2{Q::get(Rv[0], e), Q::get(Rv[1], e)};
            }
        }
    };

    // ---- consumer state: wave `wave` owns row blocks rt*TR.. and column blocks ct*TC..
    const int rt = wave / C::NCT, ct = wave % C::NCT;
    f32x4 acc[C::TR][C::TC];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < C::TR; ++i)
#pragma unroll
            for (int j = 0; j < C::TC; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    };
    // G tiles: operand A from rho K (rows c), B from beta rho K (columns e).
    // U tiles are formed transposed, U^T = (beta rho K)^T V: A from beta rho K
    // (rows e), B from V (columns a), which leaves each lane four consecutive
    // columns of one row of U, the register layout of the state in state_scan.
    // Tiles are square in blocks (TR == TC), so a U tile's row blocks are its
    // e blocks and its column blocks its a blocks; the choice only moves the
    // (wave-uniform) LDS bases and rows.
    static_assert(C::TR == C::TC, "square tiles");
    const bool utile = rt * C::TR >= C::RB;         // this wave's tile lies in the U rows
    const bool cbusy = wave < C::NT && (!WPASS || utile);
    const int a_arr = utile ? 2 : (rt * C::TR < C::RB ? 0 : 1);      // LDS array of operand A
    const int b_arr = utile ? 1 : 2;                                   // LDS array of operand B
    const int a_row0 = utile ? ct * C::TC : (rt * C::TR) % C::RB;      // first block of A
    const int b_row0 = utile ? rt * C::TR - C::RB : ct * C::TC;        // first block of B
    // `fresh` (first stage of an item) clears the accumulators here, after
    // the stage's first fragment loads are issued rather than right after the
    // previous item's epilogue: the accumulators are the data of its stores,
    // and rewriting them makes the wave wait for those stores to complete.
    auto mfma_stage = [&](const unsigned char* buf, bool fresh) {
        const unsigned char* sA = buf + a_arr * C::ARR;
        const unsigned char* sB = buf + b_arr * C::ARR;
#pragma unroll 1
        for (int ks = 0; ks < C::KST; ++ks) {
            frag A[C::TR], Bf[C::TC];
#pragma unroll
            for (int i = 0; i < C::TR; ++i) A[i] = lds_frag<T, C::ROWB>(sA, (a_row0 + i) * 16 + r, ks, g);
#pragma unroll
            for (int j = 0; j < C::TC; ++j) Bf[j] = lds_frag<T, C::ROWB>(sB, (b_row0 + j) * 16 + r, ks, g);
            if constexpr (sizeof(T) == 2) {     // fp32 tiles have no registers to spare for this
                if (ks == 0 && fresh) {
                    __builtin_amdgcn_sched_barrier(0);
                    zero_acc();
                }
            }
#pragma unroll
            for (int i = 0; i < C::TR; ++i)
#pragma unroll
                for (int j = 0; j < C::TC; ++j) io::mma(acc[i][j], A[i], Bf[j]);
        }
    };
    // Gm^T = -alpha G^T (bf16 or fp32) and U^T (fp32) of item k, in the
    // fragment-major layout state_scan loads.  Stores go through a buffer
    // resource: each block's offset splits into a compile-time part (scalar
    // soffset) and one per-lane part, so no per-block addresses stay live.
    using W = WS<T, D>;
    const uint32_t u_lane = (uint32_t)(lane * 16);
    // alpha of item k, loaded one item ahead of its epilogue
    auto load_alpha = [&](int k) {
        const Item it = item_of(k);
        return a.alpha[((size_t)it.b * a.F + it.f) * H + it.h];
    };
    auto epilogue = [&](int k, float al) {
        const Item it = item_of(k);
        if constexpr (PART) {                        // one-frame path: fp32 partials
            using PL = PartLayout<D>;
            const rsrc_t rp = make_rsrc(reinterpret_cast<unsigned char*>(a.spart) + (size_t)it.ws * PL::bytes,
                                        (uint32_t)PL::bytes);
            const uint32_t g32_lane = (uint32_t)(1024 * (g & 1) + 256 * (g >> 1) + 16 * r);
            if (!utile) {
#pragma unroll
                for (int i = 0; i < C::TR; ++i)
#pragma unroll
                    for (int j = 0; j < C::TC; ++j) {
                        const int gb = a_row0 + i, jb = b_row0 + j;
                        const uint32_t blk = (uint32_t)(PL::g_off + (size_t)(jb * PL::KS + (gb >> 1)) * 2048 + 512 * (gb & 1));
                        store_b128<kWorkspaceStore>(__builtin_bit_cast(u32x4, acc[i][j]), rp, g32_lane, blk);
                    }
            } else {
#pragma unroll
                for (int i = 0; i < C::TR; ++i)
#pragma unroll
                    for (int j = 0; j < C::TC; ++j) {
                        const int eb = a_row0 + i, ga = b_row0 + j;
                        const uint32_t blk = (uint32_t)(PL::u_off + (size_t)(eb * PL::RT + ga) * 1024);
                        store_b128<kWorkspaceStore>(__builtin_bit_cast(u32x4, acc[i][j]), rp, u_lane, blk);
                    }
            }
            return;
        }
        if (a.logits) al = sigmoid_f(al);
        const rsrc_t rw = make_rsrc(a.ws + (size_t)it.ws * W::item_bytes, (uint32_t)W::item_bytes);
        // a wave's tile is all G or all U: two straight store sequences (a
        // per-block branch made the compiler wait for each store to complete)
        if (!utile) {
            // lane (r, g) of block (gb, jb) holds G[16gb + 4g + t][16jb + r] = Gm^T[e][c] with
            // e = 16jb + r and c = 32(gb/2) + 16(gb%2) + 4g + t: in the split order that is
            // fragment (e-tile jb, step gb/2), this lane's own slot, half gb%2.  With two
            // or more row blocks per wave the two halves of a slot (row blocks 2i, 2i+1)
            // belong to this wave and each slot is stored whole (bf16: one 16-byte store; a
            // half-slot store leaves every line it touches half written, and the cache then
            // reads the line from memory to complete it)
            constexpr int RSTEP = C::TR >= 2 ? 2 : 1;
            static_assert(C::TR == 1 || C::TR % 2 == 0, "row blocks pair up into slots");
#pragma unroll
            for (int i = 0; i < C::TR; i += RSTEP) {
                const int gb = a_row0 + i;
#pragma unroll
                for (int j = 0; j < C::TC; ++j) {
                    const int jb = b_row0 + j;
                    const f32x4 m = acc[i][j] * (-al);
                    const uint32_t blk = (uint32_t)(W::gm_off + (size_t)(jb * W::KS + (gb >> 1)) * W::FRAG);
                    if constexpr (RSTEP == 2) {
                        const f32x4 m1 = acc[i + RSTEP - 1][j] * (-al);
                        if constexpr (sizeof(T) == 2) {
                            store_b128<kWorkspaceStore>(
                                u32x4{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]), pack_bf16x2(m1[0], m1[1]),
                                      pack_bf16x2(m1[2], m1[3])},
                                rw, u_lane, blk);
                        } else {
                            store_b128<kWorkspaceStore>(__builtin_bit_cast(u32x4, m), rw, u_lane, blk);
                            store_b128<kWorkspaceStore>(__builtin_bit_cast(u32x4, m1), rw, u_lane,
                                                                   blk + 1024);
                        }
                    } else if constexpr (sizeof(T) == 2) {
                        store_b64<kWorkspaceStore>(u32x2{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])},
                                                              rw, u_lane, blk + 8 * (gb & 1));
                    } else {
                        store_b128<kWorkspaceStore>(__builtin_bit_cast(u32x4, m), rw, u_lane,
                                                               blk + 1024 * (gb & 1));
                    }
                }
            }
        } else if constexpr (LP) {
            // U in bf16: the blocks of e blocks eb and eb + 1 (eb even, rows 2i and
            // 2i + 1 of this wave's tile) share one 16-byte lane slot, the layout
            // the recurrence loads (WS::up_off)
#pragma unroll
            for (int i = 0; i < C::TR; i += 2)
#pragma unroll
                for (int j = 0; j < C::TC; ++j) {
                    const int eb = a_row0 + i, ga = b_row0 + j;
                    const f32x4 x = acc[i][j], y = acc[i + 1][j];
                    store_b128<kWorkspaceStore>(
                        u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
                              pack_bf16x2(y[2], y[3])},
                        rw, u_lane, (uint32_t)W::up_off(eb >> 1, ga));
                }
        } else {
#pragma unroll
            for (int i = 0; i < C::TR; ++i)
#pragma unroll
                for (int j = 0; j < C::TC; ++j) {
                    // U tile (transposed): acc[i][j] is block (e block a_row0 + i, a block
                    // b_row0 + j); lane (r, g) holds U[16ga + r][16eb + 4g + t], slot 16g + r
                    const int eb = a_row0 + i, ga = b_row0 + j;
                    const uint32_t blk = (uint32_t)(W::ut_off + (size_t)(eb * W::RT + ga) * 1024);
                    store_b128<kWorkspaceStore>(__builtin_bit_cast(u32x4, acc[i][j]), rw, u_lane, blk);
                }
        }
    };

    if (nst == 0) {                                  // no tokens: G = U = 0
        if constexpr (PART) {
            if (producer && a.scopy)
                for (int i = ((int)blockIdx.x * C::NP + ptid) * 4; i < a.ncopy; i += (int)gridDim.x * C::NP * 4)
                    *reinterpret_cast<f32x4*>(a.scopy + i) = *reinterpret_cast<const f32x4*>(a.S_in + i);
        }
        if (!producer && cbusy) {
            zero_acc();
            for (int k = 0; k < nmine; ++k) epilogue(k, load_alpha(k));
        }
        return;
    }

    // ---- pipeline: period p produces stage p into LDS buffer p&1 while the
    //      consumers multiply stage p-1 from buffer (p-1)&1.  The producers keep
    //      four register stages in flight (ring slot p&3).  The two roles run
    //      separate loops with the same number of barriers, so their registers
    //      (load stages vs accumulators) are never live together, and every
    //      load is unconditional so wait counts stay exact.
    unsigned char* const buf0 = smem;
    unsigned char* const buf1 = smem + C::BUF;
    const int nquad = (total + 1 + 3) / 4;          // periods 0..total, in groups of 4
    if (producer) {
        // The fences keep the prologue's loads in stage order: were stage 0
        // issued last, its wait at the loop head would drain the whole ring.
        Stage R0, R1, R2, R3;
        Loader L;
        loader_item(L, 0);
        load_stage(L, R0);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(L, R1);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(L, R2);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(L, R3);
        __builtin_amdgcn_sched_barrier(0);
        for (int q = 0; q < nquad; ++q) {
            const int p = 4 * q;
            if (p < total) write_stage(p, R0, buf0);
            load_stage(L, R0);
            __syncthreads();
            if (p + 1 < total) write_stage(p + 1, R1, buf1);
            load_stage(L, R1);
            __syncthreads();
            if (p + 2 < total) write_stage(p + 2, R2, buf0);
            load_stage(L, R2);
            __syncthreads();
            if (p + 3 < total) write_stage(p + 3, R3, buf1);
            load_stage(L, R3);
            __syncthreads();
        }
        return;
    }
    // one-frame path: copy S_in to the workspace (the state update reads the
    // copy, so S_out may alias S_in).  Each consumer thread loads its first
    // 16-byte piece before the pipeline and stores it after, so nothing waits
    // on the load (at D = 128 the accumulators leave no register for it, and
    // the whole copy follows the pipeline); further pieces (many (b, h) units
    // of large D) are copied after the pipeline.
    constexpr bool kCopyAhead = PART && D < 128;
    const int cbase = ((int)blockIdx.x * 512 + tid) * 4, cstride = (int)gridDim.x * 512 * 4;
    f32x4 cp0 = f32x4{0, 0, 0, 0};
    if constexpr (kCopyAhead) {
        if (a.scopy && cbase < a.ncopy) cp0 = *reinterpret_cast<const f32x4*>(a.S_in + cbase);
    }
    float al_next = load_alpha(0);
    bool fresh = true;
    if constexpr (sizeof(T) != 2) zero_acc();
    for (int p = 0; p < 4 * nquad; ++p) {
        if (cbusy && p >= 1 && p <= total) {
            mfma_stage((p & 1) ? buf0 : buf1, fresh);   // stage p-1 sits in buffer (p-1)&1
            fresh = false;
            if ((p - 1) % nst == nst - 1) {
                const int k = (p - 1) / nst;
                epilogue(k, al_next);
                fresh = true;
                if constexpr (sizeof(T) != 2) zero_acc();
                al_next = load_alpha(k + 1 < nmine ? k + 1 : k);
            }
        }
        __syncthreads();
    }
    if constexpr (PART) {
        if (a.scopy) {
            int i0 = cbase;
            if constexpr (kCopyAhead) {
                if (cbase < a.ncopy) *reinterpret_cast<f32x4*>(a.scopy + cbase) = cp0;
                i0 += cstride;
            }
            for (int i = i0; i < a.ncopy; i += cstride)
                *reinterpret_cast<f32x4*>(a.scopy + i) = *reinterpret_cast<const f32x4*>(a.S_in + i);
        }
    }
}

// ================================================================== state_scan
template <typename T, int D> struct StateCfg {
    static constexpr bool B16 = sizeof(T) == 2;
    static constexpr int ET = D / 16;                   // 16-column blocks of a slab (and slabs per state)
    static constexpr int KS = (D + 31) / 32;            // 32-wide contraction steps
    static constexpr int NC = ET >= 2 ? ET / 2 : 1;     // waves; wave c owns blocks 2c, 2c+1
    static constexpr int BPW = ET / NC;                 // blocks per wave (2, or 1 at D = 16)
    static constexpr int FRAGB = B16 ? 1 : 2;           // 16-byte loads per Gm fragment and lane
    static constexpr int LOADS = BPW * KS * FRAGB + BPW;    // per wave and frame: Gm^T rows, U blocks
    static constexpr int STORES = 2;                    // per wave and frame: its half-fragments of S_f
    // frames of operands in flight: the 6-bit vector-memory counter (63) and
    // ~256 registers bound the ring
    static constexpr int PD0 = 60 / (LOADS + STORES);
    static constexpr int PDR = 256 / (LOADS * 4);
    static constexpr int PD = (PD0 < PDR ? PD0 : PDR) > 8 ? 8 : (PD0 < PDR ? PD0 : PDR);
    static constexpr int NTH = 64 * NC;
    static_assert(PD >= 2, "ring too shallow");
};

// One workgroup per slab of 16 rows of one (b, h) state, S[16 at + r][*].
// Its NC waves split the slab's columns: wave c holds blocks 2c and 2c+1 as
// fp32 result blocks in registers (lane 16g+r of block j: columns 16j + 4g ..
// +3 of row 16 at + r) and per frame applies
//     S_f = alpha S + U_f + bf16(S) Gm        (Gm = -alpha G, bf16 MFMA)
// to them, formed transposed, (S Gm)^T = Gm^T S^T: operand A a Gm^T fragment
// of its rows, operand B a bf16 fragment of S in the split contraction order
// (blocks 2kk and 2kk+1 for step kk: wave c's own two blocks form fragment c,
// so S never needs re-laying out).  Each wave then writes its fragment of the
// new S to a double-buffered LDS exchange and reads the others' after the
// frame's one barrier.  Gm and S enter the product rounded to bf16 once: that
// relative error (2^-9 of S Gm, itself small next to alpha S) is of the size
// G already carries from its bf16 operands and far below the error of U, so a
// low part of Gm or of S in this product buys no accuracy.  (fp32 mode: fp32
// MFMA and fp32 fragments.)  Every wave also stores its blocks of S_f as an
// fp32 plane for frame_output.
// Each wave loads its own operands (its rows of Gm_f^T and its blocks of U_f)
// PD frames ahead into a register ring; splitting a slab over several waves
// is what keeps enough loads in flight, one wave's counter holding little more
// than one frame.  Rows of S evolve independently, so the workgroups of a
// state never communicate; the slabs of a head share an XCD (workgroup index
// mod 8), so its Gm^T rows come from one L2.
//
// BWD is the backward pass's adjoint recurrence, which has the same form.
// With X_f the loss gradient of S_f (its direct part W_f = dO_f^T Q_f plus
// what flows back from later frames) and the frames walked in the opposite
// order, the state entering step f is X_f and the step makes
//     alpha_f X_f + bf16(X_f) Gm_f + W_next,
// W_next being W of the frame the walk visits next (none after the last):
// that is X of the next frame, or after the last step the gradient of the
// initial state.  Gm_f is read from the forward items (ws); W and the stored
// planes of X_f live in the second item set (ws2): W_f where frame_gram's U
// would be, the planes of X_f, stored at the step that enters with it, where
// S_f would be.
// LP: the forward scan's lighter intermediates at larger shapes: U arrives in
// bf16 (frame_gram's packed block pairs) and S_f is stored as its bf16 plane
// alone (no remainder codes).
template <typename T, int D, bool BWD = false, bool LP = false>
__global__ __launch_bounds__(256, 1) void state_scan_kernel(ScanArgs a) {   // NTH <= 256 threads
    using C = StateCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    using W = WS<T, D>;
    static_assert(C::NTH <= 256, "block size");
    static_assert(!LP || (!BWD && C::B16 && C::BPW == 2), "bf16 U and planes: the forward scan, D >= 64");
    __shared__ __attribute__((aligned(16))) unsigned char sX[2][C::KS][64 * sizeof(frag)];
    __shared__ float sAlpha[kMaxChunkFrames];

    const int units = a.B * a.H;
    const int id = xcd_remap(blockIdx.x, C::ET, units * C::ET);
    if (id < 0) return;
    const int at = id % C::ET;                          // row slab
    const int bh = id / C::ET;
    const int tid = threadIdx.x, lane = tid & 63;
    const int c = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's fragment
    const int r = lane & 15, g = lane >> 4;
    const int h = bh % a.H, b = bh / a.H;
    const int Fc = a.Fc;
    const int row = 16 * at + r;
    const uint32_t lo16 = (uint32_t)(lane * 16);

    // step fl of the recurrence takes local frame phys(fl): the frames in
    // order, or from the last to the first in the reverse direction
    const int rev = a.reverse;
    auto phys = [&](int fl) { return rev ? Fc - 1 - fl : fl; };
    for (int i = tid; i < Fc; i += C::NTH) {
        const float x = a.alpha[((size_t)b * a.F + a.f0 + phys(i)) * a.H + h];
        sAlpha[i] = a.logits ? sigmoid_f(x) : x;
    }
    // this unit's workspace items through one buffer resource
    const size_t item0 = (size_t)bh * Fc;
    const rsrc_t rws = make_rsrc(a.ws + item0 * W::item_bytes, (uint32_t)(Fc * W::item_bytes));
    // the item set holding U (W) and the stored planes
    const rsrc_t rout = BWD ? make_rsrc(a.ws2 + item0 * W::item_bytes, (uint32_t)(Fc * W::item_bytes)) : rws;

    // this wave's blocks of S (fp32) and the fragment they form
    f32x4 S[C::BPW];
    const float* sin = a.S_in ? a.S_in + (size_t)bh * D * D + (size_t)row * D : nullptr;
#pragma unroll
    for (int q = 0; q < C::BPW; ++q) {
        const int jb = c * C::BPW + q;
        S[q] = sin ? *reinterpret_cast<const f32x4*>(sin + 16 * jb + 4 * g) : f32x4{0, 0, 0, 0};
        if constexpr (BWD)      // X of the first frame: the carried gradient plus its W
            S[q] += __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rout, lo16, (uint32_t)phys(0) * (uint32_t)W::item_bytes +
                                           (uint32_t)(W::ut_off + (size_t)(jb * W::RT + at) * 1024), 0));
    }
    auto own_frag = [&]() {
        const f32x4 x = S[0];
        const f32x4 y = C::BPW > 1 ? S[C::BPW - 1] : f32x4{0, 0, 0, 0};
        if constexpr (C::B16)
            return frag{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        else
            return frag{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    };
    auto put_x = [&](int buf, const frag& f) { *reinterpret_cast<frag*>(&sX[buf][c][lane * sizeof(frag)]) = f; };
    auto get_x = [&](int buf, int kk) { return *reinterpret_cast<const frag*>(&sX[buf][kk][lane * sizeof(frag)]); };
    put_x(0, own_frag());

    struct Ops {
        frag gm[C::KS][C::BPW];
        f32x4 u[C::BPW];
        u32x4 up;                                       // LP: this wave's two U blocks in bf16
    };
    // loads [j0, j1) of a frame's operands, in the order Gm^T fragments
    // (kk, q), then U blocks q: the recurrence issues them in three groups
    // spread over a step
    constexpr int NOPS = C::KS * C::BPW + C::BPW;
    auto load_ops = [&](int fl, Ops& o, int j0, int j1) {   // fl is always a valid step
        const uint32_t base = (uint32_t)phys(fl) * (uint32_t)W::item_bytes;
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
            for (int q = 0; q < C::BPW; ++q) {
                if (kk * C::BPW + q < j0 || kk * C::BPW + q >= j1) continue;
                const int jb = c * C::BPW + q;
                const uint32_t off = base + (uint32_t)(W::gm_off + (size_t)(jb * C::KS + kk) * W::FRAG);
                if constexpr (C::B16) {
                    o.gm[kk][q] = __builtin_amdgcn_raw_buffer_load_b128(rws, lo16, off, 0);
                } else {
                    const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rws, lo16, off, 0));
                    const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rws, lo16, off + 1024, 0));
                    o.gm[kk][q] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            }
        // BWD: W of the frame visited next; after the last frame an offset past
        // the resource, which loads zeros
        const uint32_t ubase = !BWD ? base : (fl + 1 < Fc ? (uint32_t)phys(fl + 1) * (uint32_t)W::item_bytes : 0x80000000u);
        if constexpr (LP) {
            if (C::KS * C::BPW >= j0 && C::KS * C::BPW < j1)
                o.up = __builtin_amdgcn_raw_buffer_load_b128(rout, lo16, ubase + (uint32_t)W::up_off(c, at), 0);
            return;
        }
#pragma unroll
        for (int q = 0; q < C::BPW; ++q) {
            if (C::KS * C::BPW + q < j0 || C::KS * C::BPW + q >= j1) continue;
            const int jb = c * C::BPW + q;
            o.u[q] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rout, lo16, ubase + (uint32_t)(W::ut_off + (size_t)(jb * W::RT + at) * 1024), 0));
        }
    };
    // this wave's fragment (at, c) of S_fl for frame_output (zeros past the
    // slab at D = 16): bf16 mode the high plane (the fragment just exchanged)
    // and the remainder codes, fp32 mode the two halves of the fp32 plane.
    // Frame -1 maps past the resource (at most 256 frames of at most 192 KiB)
    // and is dropped, so the first call needs no branch.
    auto encode = [&](const frag& hi, const f32x4& x, const f32x4& y) {
        if constexpr (C::B16 && !LP)
            return u32x2{codes4(x, hi[0], hi[1]), C::BPW > 1 ? codes4(y, hi[2], hi[3]) : 0u};
        else
            return u32x2{0u, 0u};
    };
    auto store_state = [&](int fl, const frag& hi, const f32x4& x, const f32x4& y, const u32x2& codes) {
        const uint32_t base = fl >= 0 ? (uint32_t)phys(fl) * (uint32_t)W::item_bytes + (uint32_t)W::sp_off : 0x80000000u;
        if constexpr (C::B16) {
            store_b128<kStreamStore>(hi, rout, lo16, base + (uint32_t)((at * C::KS + c) * 1024));
            if constexpr (!LP)
                store_b64<kStreamStore>(codes, rout, (uint32_t)(lane * 8),
                                                      base + (uint32_t)(W::sc_rel + (at * C::KS + c) * 512));
        } else {
            const uint32_t off = base + (uint32_t)((at * C::KS + c) * 2048);
            store_b128<kStreamStore>(__builtin_bit_cast(u32x4, x), rout, lo16, off);
            store_b128<kStreamStore>(__builtin_bit_cast(u32x4, y), rout, lo16, off + 1024);
        }
    };
    // One frame.  Every fragment of S_{fl-1}, this wave's own included, is read
    // from the exchange buffer written before the previous barrier (register
    // arrays are only ever indexed by compile-time constants: an index
    // depending on the wave would put them in scratch memory).
    auto step = [&](int fl, Ops& o, Ops& prev, int nx, bool reload) {
        const int xb = fl & 1;                          // exchange buffer holding S_{fl-1}
        frag bs[C::KS];
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) bs[kk] = get_x(xb, kk);
        // the slot frame fl-1 used takes frame nx, in three groups of loads
        // (at the start, after the encoding, after the products): issued
        // together, the four waves' loads back up the CU's memory pipeline
        // and stall the step's critical path at issue (78.0 against 83.4 us
        // at the full-minute shape; a group just before the barrier delays
        // the barrier instead)
        if (reload) load_ops(nx, prev, 0, NOPS / 3);
        // the state entering step fl, its bf16 fragment (the one exchanged:
        // bs[c]) and remainder codes, encoded while the exchange reads are in
        // flight and stored after the products are issued (measured 81.9
        // against 89.4 us at the full-minute shape when the encoding sat
        // between the exchange reads and the products)
        const f32x4 e0 = S[0], e1 = C::BPW > 1 ? S[C::BPW - 1] : f32x4{0, 0, 0, 0};
        const frag ehi = own_frag();
        const u32x2 ecodes = encode(ehi, e0, e1);
        __builtin_amdgcn_sched_barrier(0);
        if (reload) load_ops(nx, prev, NOPS / 3, 2 * NOPS / 3);
        __builtin_amdgcn_sched_barrier(0);
        const float al = sAlpha[fl];
        f32x4 acc[C::BPW];
#pragma unroll
        for (int q = 0; q < C::BPW; ++q) {
            if constexpr (LP) {                         // bf16 pair: block q in words 2q, 2q + 1
                const uint32_t w0 = o.up[2 * q], w1 = o.up[2 * q + 1];
                const f32x4 u{__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u),
                              __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u)};
                acc[q] = S[q] * al + u;
            } else {
                acc[q] = S[q] * al + o.u[q];
            }
        }
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
            for (int q = 0; q < C::BPW; ++q) {
                frag ga = o.gm[kk][q];
                if constexpr (D < 32) {                 // the unwritten second half of each slot
                    if constexpr (C::B16) {
                        ga[2] = 0u;
                        ga[3] = 0u;
                    } else {
                        ga[4] = ga[5] = ga[6] = ga[7] = 0.0f;
                    }
                }
                io::mma(acc[q], ga, bs[kk]);            // (S Gm)^T += Gm^T S^T
            }
        if (reload) load_ops(nx, prev, 2 * NOPS / 3, NOPS);
        store_state(BWD ? fl : fl - 1, ehi, e0, e1, ecodes);
#pragma unroll
        for (int q = 0; q < C::BPW; ++q) S[q] = acc[q];
        put_x(xb ^ 1, own_frag());
        __syncthreads();                                // fragments of S_fl visible
    };

    // ring slot j holds frame fl with fl % PD == j; at the start of frame fl
    // the slot of frame fl-1 is free and takes frame fl-1+PD
    Ops ring[C::PD];
#pragma unroll
    for (int j = 0; j < C::PD - 1; ++j) {
        load_ops(j < Fc ? j : Fc - 1, ring[j], 0, NOPS);
        __builtin_amdgcn_sched_barrier(0);              // keep the frames in issue order
    }
    __syncthreads();                                    // alphas and S_0 fragments staged
    const int nfull = Fc / C::PD;
    for (int gi = 0; gi < nfull; ++gi) {
#pragma unroll
        for (int j = 0; j < C::PD; ++j) {
            const int fl = gi * C::PD + j;
            const int nx = fl - 1 + C::PD;
            step(fl, ring[j], ring[(j + C::PD - 1) % C::PD], nx < Fc ? nx : Fc - 1, true);
        }
    }
    const int rem = Fc - nfull * C::PD;
#pragma unroll
    for (int j = 0; j < C::PD; ++j) {
        if (j < rem) {
            const int fl = nfull * C::PD + j, nx = fl - 1 + C::PD;
            step(fl, ring[j], ring[(j + C::PD - 1) % C::PD], nx < Fc ? nx : Fc - 1, true);
        }
    }
    if constexpr (!BWD) {
        const f32x4 e1 = C::BPW > 1 ? S[C::BPW - 1] : f32x4{0, 0, 0, 0};
        const frag ehi = own_frag();
        store_state(Fc - 1, ehi, S[0], e1, encode(ehi, S[0], e1));
    }

    // ---- final state (fp32, row-major [a][e])
    if (a.S_out) {
        float* so = a.S_out + (size_t)bh * D * D + (size_t)row * D;
#pragma unroll
        for (int q = 0; q < C::BPW; ++q) *reinterpret_cast<f32x4*>(so + 16 * (c * C::BPW + q) + 4 * g) = S[q];
    }
}

// ================================================================== transposed state
// The backward products contract a state over its row index, which the
// planes spread across lanes.  A state is staged transposed in LDS: row c of
// the staged array holds column c of the matrix, bf16 mode as two bf16 arrays
// (high parts, then low parts: value = hi + lo to about 2^-16 relative), fp32
// mode as one fp32 array.
template <typename T, int D> struct TState {
    static constexpr bool B16 = sizeof(T) == 2;
    static constexpr int SZ = IO<T>::bytes;
    static constexpr int KS = (D + 31) / 32, RT = D / 16;
    static constexpr int ROWB = D * SZ;               // one row
    static constexpr int ARR = D * ROWB;              // one array
    static constexpr int BYTES = (B16 ? 2 : 1) * ARR;
};

// Byte offset of byte `b` of row `row` in an LDS tile of ROWB-byte rows whose
// 16-byte chunks are XOR-swizzled by the row: the split-order fragment reads
// (16 consecutive rows, 8 or 16 bytes at the same column) then fall on
// distinct banks.
template <int ROWB>
__device__ __forceinline__ int swz(int row, int b) {
    constexpr int CPR = ROWB / 16;                    // chunks per row
    constexpr int M = (CPR < 16 ? CPR : 16) - 1;
    return row * ROWB + ((((b >> 4) ^ (row & M))) << 4) + (b & 15);
}

// Fragment (row tile t, step kk) of a state in the planes' layout (lane 16g+r:
// row 16t + r, the split order's columns of step kk) as high and low parts
// (fp32 mode: lo is not used).  The state comes from the planes at `sp` (an
// item's S region), else from the fp32 row-major matrix `rm`, else it is zero.
template <typename T, int D>
__device__ __forceinline__ void state_frag(const unsigned char* sp, const float* rm, int t, int kk, int lane,
                                           typename IO<T>::frag& hi, typename IO<T>::frag& lo) {
    using W = WS<T, D>;
    const int r = lane & 15, g = lane >> 4;
    if constexpr (sizeof(T) == 2) {
        if (sp) {
            hi = *reinterpret_cast<const u32x4*>(sp + W::frag_off(t, kk, 0, lane));
            lo = rem_frag(hi, *reinterpret_cast<const u32x2*>(sp + W::sc_rel + W::code_off(t, kk, lane)));
            return;
        }
    } else {
        if (sp) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(sp + W::frag_off(t, kk, 0, lane));
            const f32x4 y = *reinterpret_cast<const f32x4*>(sp + W::frag_off(t, kk, 1, lane));
            hi = f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            lo = IO<T>::zero();
            return;
        }
    }
    f32x4 x = f32x4{0, 0, 0, 0}, y = f32x4{0, 0, 0, 0};
    if (rm) {
        const float* row = rm + (size_t)(16 * t + r) * D + 32 * kk + 4 * g;
        x = *reinterpret_cast<const f32x4*>(row);
        if constexpr (D >= 32) y = *reinterpret_cast<const f32x4*>(row + 16);
    }
    if constexpr (sizeof(T) == 2) {
        hi = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        lo = u32x4{pack_bf16x2(x[0] - IO<T>::get(hi, 0), x[1] - IO<T>::get(hi, 1)),
                   pack_bf16x2(x[2] - IO<T>::get(hi, 2), x[3] - IO<T>::get(hi, 3)),
                   pack_bf16x2(y[0] - IO<T>::get(hi, 4), y[1] - IO<T>::get(hi, 5)),
                   pack_bf16x2(y[2] - IO<T>::get(hi, 6), y[3] - IO<T>::get(hi, 7))};
    } else {
        hi = f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        lo = IO<T>::zero();
    }
}

// Writes fragment (t, kk) of lane `lane` transposed into the staged arrays at
// `arr` (element (row, col) of the matrix goes to row col, position row).
template <typename T, int D>
__device__ __forceinline__ void put_transposed(unsigned char* arr, int t, int kk, int lane, const typename IO<T>::frag& hi,
                                               const typename IO<T>::frag& lo) {
    using TS = TState<T, D>;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < (D >= 32 ? 8 : 4); ++j) {
        const int col = 32 * kk + 16 * (j >> 2) + 4 * g + (j & 3);
        unsigned char* p = arr + swz<TS::ROWB>(col, (16 * t + r) * TS::SZ);
        if constexpr (sizeof(T) == 2) {
            const uint32_t wh = hi[j >> 1], wl = lo[j >> 1];
            *reinterpret_cast<uint16_t*>(p) = (uint16_t)((j & 1) ? (wh >> 16) : wh);
            *reinterpret_cast<uint16_t*>(p + TS::ARR) = (uint16_t)((j & 1) ? (wl >> 16) : wl);
        } else {
            *reinterpret_cast<float*>(p) = hi[j];
        }
    }
}

// Operand fragment (row tile t, step kk) of the transposed matrix from the
// staged arrays: lane 16g+r gets row 16t + r of M^T, i.e. column 16t + r of M,
// in the split order of step kk.
template <typename T, int D>
__device__ __forceinline__ void get_transposed(const unsigned char* arr, int t, int kk, int lane,
                                               typename IO<T>::frag& hi, typename IO<T>::frag& lo) {
    using TS = TState<T, D>;
    const int r = lane & 15, g = lane >> 4;
    const int row = 16 * t + r, b0 = (32 * kk + 4 * g) * TS::SZ;
    const unsigned char* p0 = arr + swz<TS::ROWB>(row, b0);
    const unsigned char* p1 = arr + swz<TS::ROWB>(row, b0 + 16 * TS::SZ);
    if constexpr (sizeof(T) == 2) {
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(p0);
        const u32x2 a1 = D >= 32 ? *reinterpret_cast<const u32x2*>(p1) : u32x2{0u, 0u};
        hi = u32x4{a0[0], a0[1], a1[0], a1[1]};
        const u32x2 c0 = *reinterpret_cast<const u32x2*>(p0 + TS::ARR);
        const u32x2 c1 = D >= 32 ? *reinterpret_cast<const u32x2*>(p1 + TS::ARR) : u32x2{0u, 0u};
        lo = u32x4{c0[0], c0[1], c1[0], c1[1]};
    } else {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(p0);
        const f32x4 a1 = D >= 32 ? *reinterpret_cast<const f32x4*>(p1) : f32x4{0, 0, 0, 0};
        hi = f32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        lo = IO<T>::zero();
    }
}

// ================================================================== frame_output
template <typename T, int D> struct OutCfg {
    static constexpr int SZ = IO<T>::bytes;
    static constexpr int RT = D / 16;               // 16-row tiles of S (output features)
    static constexpr int NWR = RT < 4 ? RT : 4;     // waves splitting the rows
    static constexpr int RPW = RT / NWR;            // row tiles per wave
    static constexpr int TG = 4 / NWR;              // waves splitting the tokens
    static constexpr int KS = (D + 31) / 32;
    static constexpr int ROWB = D * SZ + 16;        // padded LDS row (one token)
    static constexpr int LPR = D * SZ / 16;         // 16-byte loads per token row
    static constexpr int RPP = 256 / LPR;           // token rows per load pass
    static constexpr int BT = RPP > 64 ? RPP : 64;  // tokens per LDS block
    static constexpr int NLD = BT / RPP;            // loads per thread per block
    static constexpr int PD = SZ == 2 ? 4 : 2;      // blocks of Q in flight
    static constexpr int QBUF = BT * ROWB;          // one LDS block of Q
    static constexpr int ROWO = D * SZ + 16;        // padded LDS row of O (one token)
    static constexpr int OBUF = BT * ROWO;          // one LDS block of O
    static constexpr int NST = BT * LPR / 256;      // 16-byte O stores per thread per block
    static constexpr int LDS = 2 * QBUF + 2 * OBUF;
    static_assert(BT % RPP == 0 && RPP >= 1 && NST * 256 == BT * LPR, "block shape");
};

// o_i = S_f q_i computed as O^T = S Q^T: A = S (rows a, contraction e) held in
// registers for the whole token range, B = Q^T.  O goes back through LDS too:
// every wave drops its accumulators into a double-buffered O tile, and one
// block later all threads store whole token rows (16 lanes x 16 bytes per row),
// which measured 5.5 TB/s against 3.8 TB/s for the accumulators' own 32-byte
// pieces.  Q is staged once per
// workgroup: 64-token blocks stream from HBM PD blocks ahead into registers,
// then into a double-buffered LDS tile from which every wave reads its B
// fragments (a token row of Q is 8 contiguous features per lane).
// TRS is the backward pass's dq_i = S_f^T do_i: the same kernel with q := dO,
// o := dQ and the transposed state, staged through LDS before the pipeline.
// TIN is q's element type (fp8e4m3: block-scaled bytes, turned into bf16 as
// each block is written to LDS; o is then bf16).
// LP: the state planes are bf16 alone (see state_scan_kernel), one product
// per fragment.
template <typename TIN, int D, bool TRS = false, bool LP = false>
__global__ __launch_bounds__(256, 2) void frame_output_kernel(ScanArgs a) {
    using T = typename Elem<TIN>::C;
    static_assert(!LP || (!TRS && sizeof(T) == 2), "bf16 state planes: the forward scan");
    constexpr bool MX = !__is_same(T, TIN);
    constexpr int GB2 = Elem<TIN>::G2;
    using C = OutCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

    // frame-major order, head fastest: x = ((b*Fc + fl)*tsplit + part)*H + hs,
    // with the head rotated by the rest of the index, h = (hs + x/H) mod H:
    // workgroups are dealt to the XCDs round-robin, and without the rotation
    // each XCD would only ever get the same two heads (whose rows sit at
    // fixed offsets of every token row)
    // The last ntail items are split in two halves of their tokens, dispatched
    // last: the final, partial round of workgroups then holds half-size work.
    int x = blockIdx.x, half = -1;
    const int nwhole = a.B * a.Fc * a.H * a.tsplit - a.ntail;
    if (x >= nwhole) {
        half = (x - nwhole) & 1;
        x = nwhole + ((x - nwhole) >> 1);
    }
    const int h = (x % a.H + x / a.H) % a.H;
    const int part = (x / a.H) % a.tsplit;
    const int fl = (x / (a.H * a.tsplit)) % a.Fc;
    const int b = x / (a.H * a.tsplit * a.Fc);
    const int item = (b * a.H + h) * a.Fc + fl;    // workspace item
    const int f = a.f0 + fl;
    const int N = a.N, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wr = wave % C::NWR, wt = wave / C::NWR;

    int nbeg = part * a.tchunk;
    int nend = min(N, nbeg + a.tchunk);
    if (half >= 0) {
        const int mid = nbeg + ((nend - nbeg + 1) / 2 + 15) / 16 * 16;
        if (half == 0)
            nend = min(nend, mid);
        else
            nbeg = mid;
    }
    if (nbeg >= nend) return;

    // token range [nbeg, nend) of this head through buffer resources: rows past
    // nend read as zeros and their stores are dropped
    const size_t rowstride = (size_t)H * D;
    const size_t tok0 = ((size_t)b * a.F + f) * (size_t)N + nbeg;
    const uint32_t rbytes = (uint32_t)(((size_t)(nend - nbeg - 1) * rowstride + D) * C::SZ);
    const uint32_t qbytes = (uint32_t)elem_bytes<TIN>((size_t)(nend - nbeg - 1) * rowstride + D);
    const rsrc_t rq = make_rsrc(elem_ptr<TIN>(a.q, tok0 * rowstride + (size_t)h * D), qbytes);
    const rsrc_t ro = make_rsrc(static_cast<T*>(a.o) + tok0 * rowstride + (size_t)h * D, rbytes);
    const uint32_t row_bytes = (uint32_t)(H * D * C::SZ);     // o (and q unless block-scaled)
    const uint32_t qrow_bytes = (uint32_t)(H * D * GB2 / 2);
    const int nloc = nend - nbeg;
    const int nblk = (nloc + C::BT - 1) / C::BT;
    // block-scaled q: D/32 scale bytes per token row
    constexpr int NB = D / kMxBlock;
    rsrc_t rqs;
    if constexpr (MX)
        rqs = make_rsrc(a.qs + tok0 * H * NB + (size_t)h * NB, (uint32_t)((nend - nbeg - 1) * H * NB + NB));

    // loader role: row lr of each pass, 16-byte column lc (of the bf16 row:
    // eight features; block-scaled q loads their eight bytes and their scale)
    const int lc = tid % C::LPR, lr = tid / C::LPR;
    struct QStage {
        typename Quad<TIN>::type v[C::NLD];
        uint32_t e[MX ? C::NLD : 1];
    };
    auto load_blk = [&](int blk, QStage& R) {
        constexpr int FPC = 16 / C::SZ;             // features per 16-byte chunk of the LDS row
        const uint32_t base = (uint32_t)(blk * C::BT + lr) * qrow_bytes + (uint32_t)(lc * FPC * GB2 / 2);
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) R.v[i] = Quad<TIN>::load(rq, base + (uint32_t)(i * C::RPP) * qrow_bytes);
        if constexpr (MX) {
            const uint32_t sb = (uint32_t)(blk * C::BT + lr) * (uint32_t)(H * NB) + (uint32_t)(lc * FPC / kMxBlock);
#pragma unroll
            for (int i = 0; i < C::NLD; ++i)
                R.e[i] = __builtin_amdgcn_raw_buffer_load_b8(rqs, sb + (uint32_t)(i * C::RPP * H * NB), 0, 0);
        }
    };
    auto put_blk = [&](const QStage& R, unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            u32x4 val;
            if constexpr (MX)
                val = mx_to_bf16(R.v[i], R.e[i]);
            else
                val = R.v[i];
            *reinterpret_cast<u32x4*>(buf + (lr + i * C::RPP) * C::ROWB + lc * 16) = val;
        }
    };

    // ---- S_f rows of this wave as A fragments (fragment-major workspace)
    using W = WS<T, D>;
    const unsigned char* sp = a.ws + (size_t)item * W::item_bytes + W::sp_off;
    frag ah[C::RPW][C::KS], alw[C::RPW][C::KS];
    if constexpr (TRS) {
        static_assert(TState<T, D>::BYTES <= C::LDS, "the staged state fits in the Q and O tiles");
        for (int fi = wave; fi < C::RT * C::KS; fi += 4) {
            frag hi, lo;
            state_frag<T, D>(sp, nullptr, fi / C::KS, fi % C::KS, lane, hi, lo);
            put_transposed<T, D>(smem, fi / C::KS, fi % C::KS, lane, hi, lo);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < C::RPW; ++i)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                get_transposed<T, D>(smem, wr * C::RPW + i, ks, lane, ah[i][ks], alw[i][ks]);
                hold(ah[i][ks]);                        // read before the barrier, not after it
                hold(alw[i][ks]);
            }
        __syncthreads();                                // before the Q tiles overwrite the staging
    }
#pragma unroll
    for (int i = 0; i < C::RPW && !TRS; ++i) {
        const int rt = wr * C::RPW + i;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            if constexpr (LP) {                         // the bf16 plane alone
                ah[i][ks] = *reinterpret_cast<const u32x4*>(sp + W::frag_off(rt, ks, 0, lane));
            } else if constexpr (sizeof(T) == 2) {      // high plane and the low part from the codes
                ah[i][ks] = *reinterpret_cast<const u32x4*>(sp + W::frag_off(rt, ks, 0, lane));
                alw[i][ks] = rem_frag(ah[i][ks], *reinterpret_cast<const u32x2*>(sp + W::sc_rel + W::code_off(rt, ks, lane)));
            } else {
                const f32x4 x = *reinterpret_cast<const f32x4*>(sp + W::frag_off(rt, ks, 0, lane));
                const f32x4 y = *reinterpret_cast<const f32x4*>(sp + W::frag_off(rt, ks, 1, lane));
                ah[i][ks] = f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            }
        }
    }

    auto compute_blk = [&](const unsigned char* buf, unsigned char* obuf) {
#pragma unroll 1
        for (int sb = wt; sb < C::BT / 16; sb += C::TG) {       // 16-token sub-blocks
            frag bq[C::KS];
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                // split order: features 32ks + 4g.. and 32ks + 16 + 4g.. (none at D = 16)
                const unsigned char* src = buf + (sb * 16 + r) * C::ROWB + (ks * 32 + 4 * g) * C::SZ;
                if constexpr (sizeof(T) == 2) {
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
                    const u32x2 hi = D >= 32 ? *reinterpret_cast<const u32x2*>(src + 32) : u32x2{0u, 0u};
                    bq[ks] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                    const f32x4 hi = D >= 32 ? *reinterpret_cast<const f32x4*>(src + 64) : f32x4{0, 0, 0, 0};
                    bq[ks] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            }
            f32x4 acc[C::RPW];
#pragma unroll
            for (int i = 0; i < C::RPW; ++i) {
                acc[i] = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    io::mma(acc[i], ah[i][ks], bq[ks]);
                    if constexpr (sizeof(T) == 2 && !LP) io::mma(acc[i], alw[i][ks], bq[ks]);
                }
            }
            unsigned char* orow = obuf + (sb * 16 + r) * C::ROWO;          // token sb*16 + r of the block
#pragma unroll
            for (int i = 0; i < C::RPW; ++i) {
                const int col0 = (wr * C::RPW + i) * 16 + 4 * g;             // features col0..col0+3
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<u32x2*>(orow + col0 * 2) =
                        u32x2{pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3])};
                } else {
                    *reinterpret_cast<f32x4*>(orow + col0 * 4) = acc[i];
                }
            }
        }
    };
    // Whole rows of the O block `blk` from its LDS tile to HBM; block -1 (the
    // call before the first block) maps past the resource and is dropped.
    auto store_blk = [&](int blk, const unsigned char* obuf) {
        const uint32_t base = blk >= 0 ? (uint32_t)(blk * C::BT) * row_bytes : 0x80000000u;
#pragma unroll
        for (int i = 0; i < C::NST; ++i) {
            const int c = tid + 256 * i, n = c / C::LPR, part = c % C::LPR;
            const u32x4 val = *reinterpret_cast<const u32x4*>(obuf + n * C::ROWO + part * 16);
            bstore16(ro, base + (uint32_t)n * row_bytes + (uint32_t)(part * 16), val);
        }
    };

    // ---- pipeline over 64-token blocks: ring slot blk % PD, LDS buffer blk & 1.
    // One barrier per block: a wave at the barrier of block blk has finished
    // computing block blk-1, whose buffer block blk+1 overwrites.
    // Full groups of PD blocks run without conditions (exact wait counts); the
    // remainder consumes the blocks already in the ring.
    // The barrier of block blk also publishes the O tile of block blk-1, which
    // is stored right after it (its buffer is next written by block blk+1,
    // behind the next barrier).
    static_assert(C::PD % 2 == 0, "ring slot parity must match the LDS buffer parity");
    unsigned char* const obase = smem + 2 * C::QBUF;
    QStage ring[C::PD];
#pragma unroll
    for (int j = 0; j < C::PD; ++j) load_blk(j, ring[j]);
    const int nfull = nblk / C::PD;
    for (int gi = 0; gi < nfull; ++gi) {
#pragma unroll
        for (int j = 0; j < C::PD; ++j) {
            const int blk = gi * C::PD + j;
            unsigned char* buf = smem + (j & 1) * C::QBUF;
            put_blk(ring[j], buf);
            __syncthreads();
            store_blk(blk - 1, obase + ((j + 1) & 1) * C::OBUF);
            load_blk(blk + C::PD, ring[j]);       // past the range: zeros, no traffic
            compute_blk(buf, obase + (j & 1) * C::OBUF);
        }
    }
    const int rem = nblk - nfull * C::PD;
#pragma unroll
    for (int j = 0; j < C::PD; ++j) {
        if (j < rem) {
            const int blk = nfull * C::PD + j;
            unsigned char* buf = smem + (j & 1) * C::QBUF;
            put_blk(ring[j], buf);
            __syncthreads();
            store_blk(blk - 1, obase + ((j + 1) & 1) * C::OBUF);
            compute_blk(buf, obase + (j & 1) * C::OBUF);
        }
    }
    __syncthreads();
    store_blk(nblk - 1, obase + ((nblk - 1) & 1) * C::OBUF);
}

// ================================================================== frame_step
template <typename T, int D> struct StepCfg {
    static constexpr int SZ = IO<T>::bytes;
    static constexpr int NW = D / 16;               // waves: one 16-row tile of S each
    static constexpr int NTH = 64 * NW;
    static constexpr int KS = (D + 31) / 32;
    static constexpr int ET = D / 16;               // 16-column tiles of S
    static constexpr int ROWB = D * SZ + 16;        // padded LDS row (a token, or a row of S)
    static constexpr int LPR = D * SZ / 16;         // 16-byte loads per token row
    static constexpr int RPP = NTH / LPR;           // token rows per load pass
    static constexpr int BT = RPP > 64 ? RPP : 64;  // tokens per LDS block
    static constexpr int NLD = BT / RPP;            // loads per thread per block
    static constexpr int PD = SZ == 2 ? 4 : 2;      // blocks of Q in flight
    static constexpr int QBUF = BT * ROWB;          // one LDS block of Q (and of O)
    static constexpr int NST = BT * LPR / NTH;      // 16-byte O stores per thread per block
    static constexpr int NPL = SZ == 2 ? 2 : 1;     // planes of S_1 (bf16 hi, lo)
    static constexpr int PLANE = D * ROWB;          // one plane of a D x D state
    static constexpr int LDS_S = (1 + NPL) * PLANE; // S_0 (B operand), then the planes of S_1
    static constexpr int LDS_O = 4 * QBUF;
    static constexpr int LDS = LDS_S > LDS_O ? LDS_S : LDS_O;
    static constexpr int PD0 = D * D / (4 * NTH);   // f32x4 loads per thread to stage S_0
    static constexpr int PP = D >= 128 ? 1 : 2;     // partials loaded per batch (registers)
    static_assert(RPP >= 1 && BT % RPP == 0 && NST * NTH == BT * LPR, "block shape");
};

// One frame for streaming use, after frame_gram has written the fp32 partial
// G and U of every token range of every (b, h).  Each workgroup owns one
// (b, h) and one range of output tokens, and first forms the new state itself,
//     S_1 = alpha S_0 + U + bf16(S_0) Gm,   Gm = -alpha sum_p G_p,  U = sum_p U_p
// (the same arithmetic as the recurrence, with the partials summed in fp32 in
// range order), so the one-frame step needs no recurrence launch: the update
// is 2*D^3 flops, small next to the output's 2*N*D^2.  As in the recurrence,
// wave w owns columns [16w, 16w+16) of S_1 and needs only its slice of Gm and
// U; S_0 is staged once in LDS as the shared operand.  Then O = S_1 Q^T for
// its tokens as in the output pass, wave w now owning output features
// [16w, 16w+16) (S_1 as bf16 hi and lo planes, S_1 - hi rounded to bf16,
// through LDS into A fragments).  The ranges of a unit share blockIdx mod 8 (one XCD), so
// their reads of S_0 and the partials hit one L2; the first range writes S_1
// to S_out.  S_0 is read from frame_gram's copy of S_in, so S_out may be S_in.
//
// FUSED (bf16, D <= 64): the whole step in this one launch.  Each workgroup
// first forms the frame's entire G and U itself (phase A): K, V and beta of
// all N tokens of its (b, h) stream through registers, two tokens per thread
// and PDA 64-token blocks ahead, and are written transposed ([feature][token],
// rho k, beta rho k and v in bf16) into a double-buffered LDS tile, from which
// wave w forms the G tiles of columns [16w, 16w+16) and the U^T tiles of rows
// [16w, 16w+16) with MFMA.  The G tile of rows c lands in each lane as four
// consecutive c (4g..4g+3) of one column e: so the fragment of Gm^T for a
// 32-wide step holds c = 4g+t and 16+4g+t, and the S_0 fragment that meets it
// in the update takes the same columns (a fixed permutation of the
// contraction, the same on both operands); U^T lands already in the state's
// register layout.  The ranges of a (b, h) share one XCD, so their reads of
// K and V are served by one L2.  Nothing is written between launches, and S_0
// is read straight from S_in: the host takes this path only when S_out does
// not alias S_in.
template <typename T, int D, bool FUSED>
__global__ __launch_bounds__(64 * (D / 16), 2) void frame_step_kernel(ScanArgs a) {
    using C = StepCfg<T, D>;
    using io = IO<T>;
    using frag = typename io::frag;
    using PL = PartLayout<D>;
    static_assert(!FUSED || (sizeof(T) == 2 && D <= 64), "the one-launch step is bf16, D <= 64");
    constexpr int BTA = 64;                          // phase A: tokens per block
    // D = 64: K, V tiles token-major, operand fragments through transpose
    // reads (tr_frag); smaller D: feature-major tiles written transposed
    constexpr bool TRK = FUSED && D == 64;
    constexpr int ROWT = D * 2;                      //   token-major: bytes per LDS row (one token)
    static_assert(!TRK || BTA * ROWT == D * BTA * 2, "the token-major tile fills the same array");
    constexpr int ROWA = BTA * 2;                    //   bytes per LDS row (one feature)
    constexpr int ARRA = D * ROWA;                   //   one transposed array
    constexpr int LDSA = FUSED ? 2 * 3 * ARRA : 0;   //   rho K, beta rho K, V; double-buffered
    constexpr int LDSF = C::LDS > LDSA ? C::LDS : LDSA;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDSF];

    const int units = a.B * a.H;
    const int x = (int)blockIdx.x, slot = x >> 3;
    const int part = slot % a.tsplit;
    const int bh = (slot / a.tsplit) * 8 + (x & 7);
    if (bh >= units) return;
    const int h = bh % a.H, b = bh / a.H;
    const int N = a.N, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const bool kvalid = 8 * g < D || D >= 32;      // D = 16: lanes g >= 2 carry zeros

    // ---- tokens [nbeg, nend) of this unit's frame
    // Q streams in during the state update (it needs none of Q), issued just
    // after the first partials so that those come back first; an empty range
    // gets an empty buffer resource, whose loads return zeros
    const int nbeg = part * a.tchunk;
    const int nend = min(N, nbeg + a.tchunk);
    const size_t rowstride = (size_t)H * D;
    const size_t tok0 = (size_t)b * a.F * N + (nbeg < nend ? nbeg : 0);
    const uint32_t rbytes = nbeg < nend ? (uint32_t)(((size_t)(nend - nbeg - 1) * rowstride + D) * C::SZ) : 0u;
    const rsrc_t rq = make_rsrc(static_cast<const T*>(a.q) + tok0 * rowstride + (size_t)h * D, rbytes);
    const rsrc_t ro = make_rsrc(static_cast<T*>(a.o) + tok0 * rowstride + (size_t)h * D, rbytes);
    const uint32_t row_bytes = (uint32_t)(H * D * C::SZ);
    const int nblk = (nend - nbeg + C::BT - 1) / C::BT;
    const int lc = tid % C::LPR, lr = tid / C::LPR;
    struct QStage {
        u32x4 v[C::NLD];
    };
    auto load_blk = [&](int blk, QStage& R) {
        const uint32_t base = (uint32_t)(blk * C::BT + lr) * row_bytes + (uint32_t)(lc * 16);
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) R.v[i] = bload16_nt(rq, base + (uint32_t)(i * C::RPP) * row_bytes);
    };
    auto put_blk = [&](const QStage& R, unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i)
            *reinterpret_cast<u32x4*>(buf + (lr + i * C::RPP) * C::ROWB + lc * 16) = R.v[i];
    };
    static_assert(C::PD % 2 == 0, "ring slot parity must match the LDS buffer parity");
    QStage ring[C::PD];

    // ---- stage S_0 in LDS as bf16 rows (operand B of the update), and load
    //      this wave's slices of U and Gm: one batch of independent loads per
    //      partial
    float al = a.alpha[(size_t)b * a.F * H + h];
    if (a.logits) al = sigmoid_f(al);
    const float* s0 = a.S_in ? a.S_in + (size_t)bh * D * D : nullptr;
    unsigned char* const sS0 = smem;
    unsigned char* const sS1 = smem + C::PLANE;     // hi plane, then lo plane
    // every load first (S_0 for LDS, S_0 and U in this wave's slice, this
    // wave's Gm^T fragments), so that one round trip covers them: partials
    // come PP at a time through a buffer resource that ends at the last one,
    // so those of a batch past the end read zeros
    f32x4 glo[C::KS], ghi[C::KS], su[C::ET];        // sums: this wave's Gm^T fragments, U slice
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        glo[ks] = f32x4{0, 0, 0, 0};
        ghi[ks] = f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::ET; ++i) su[i] = f32x4{0, 0, 0, 0};
    f32x4 st0[C::PD0];
    f32x4 sn[C::ET];                                // lane (r, g) of row tile i: S_1[16 i + r][16 wave + 4 g ..]
    const int col0 = wave * 16 + 4 * g;
    auto load_s0 = [&]() {
#pragma unroll
        for (int i = 0; i < C::PD0; ++i)
            st0[i] = s0 ? *reinterpret_cast<const f32x4*>(s0 + (tid + i * C::NTH) * 4) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < C::ET; ++i)
            sn[i] = s0 ? *reinterpret_cast<const f32x4*>(s0 + (size_t)(16 * i + r) * D + col0) : f32x4{0, 0, 0, 0};
    };
    // the one-launch step loads S_0 after its K/V phase: held through that
    // phase its 32 registers cost more than the exposed load (23.3 against
    // 24.1 us per streaming step, bitwise the same result)
    if constexpr (!FUSED) load_s0();
    if constexpr (!FUSED) {
        const rsrc_t rp = make_rsrc(reinterpret_cast<const unsigned char*>(a.spart) + (size_t)bh * a.parts * PL::bytes,
                                    (uint32_t)(a.parts * PL::bytes));
        // one batch of PP partials: loads, then sums
        auto load_batch = [&](int pp, f32x4 (&tg)[C::PP][2 * C::KS], f32x4 (&tu)[C::PP][C::ET]) {
    #pragma unroll
            for (int q2 = 0; q2 < C::PP; ++q2) {
                const uint32_t pb = (uint32_t)((pp + q2) * PL::bytes);
    #pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    tg[q2][2 * ks] = __builtin_bit_cast(f32x4, bload16(rp, pb + PL::g_off + PL::frag_off(wave, ks, 0, lane)));
                    tg[q2][2 * ks + 1] = __builtin_bit_cast(f32x4, bload16(rp, pb + PL::g_off + PL::frag_off(wave, ks, 1, lane)));
                }
    #pragma unroll
                for (int i = 0; i < C::ET; ++i)          // U tile (e-tile wave, a-tile i)
                    tu[q2][i] = __builtin_bit_cast(f32x4, bload16(rp, pb + (uint32_t)(PL::u_off + (wave * PL::RT + i) * 1024 + lane * 16)));
            }
        };
        auto add_batch = [&](const f32x4 (&tg)[C::PP][2 * C::KS], const f32x4 (&tu)[C::PP][C::ET]) {
    #pragma unroll
            for (int q2 = 0; q2 < C::PP; ++q2) {
    #pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    glo[ks] += tg[q2][2 * ks];
                    ghi[ks] += tg[q2][2 * ks + 1];
                }
    #pragma unroll
                for (int i = 0; i < C::ET; ++i) su[i] += tu[q2][i];
            }
        };
        {
            f32x4 tg[C::PP][2 * C::KS], tu[C::PP][C::ET];
            load_batch(0, tg, tu);
    #pragma unroll
            for (int j = 0; j < C::PD; ++j) load_blk(j, ring[j]);
            add_batch(tg, tu);
        }
        for (int pp = C::PP; pp < a.parts; pp += C::PP) {
            f32x4 tg[C::PP][2 * C::KS], tu[C::PP][C::ET];
            load_batch(pp, tg, tu);
            add_batch(tg, tu);
        }
    } else {
        // ---- phase A: G (columns 16w..) and U^T (rows 16w..) of the whole frame
        constexpr int GPT = D / 8;                   // 16-byte feature groups per token
        constexpr int PDA = 4;                       // blocks of K, V and beta in flight (measured
                                                     // best: 3 and 6 are ~1 us slower, 5 spills)
        static_assert(32 * GPT == C::NTH, "two tokens per thread per block");
        constexpr int RT = D / 16;
        const int fgrp = tid % GPT, tp = tid / GPT;  // features 8 fgrp.., tokens 2 tp, 2 tp + 1
        const int nba = (N + BTA - 1) / BTA;
        const float inv_eps = 1.0f / a.eps, inv_n = N > 0 ? 1.0f / (float)N : 0.0f;
        const size_t tokf = (size_t)b * a.F * N;     // the frame's first token (F == 1)
        const uint32_t fbytes = N > 0 ? (uint32_t)(((size_t)(N - 1) * rowstride + D) * 2) : 0u;
        const rsrc_t rk = make_rsrc(static_cast<const T*>(a.k) + tokf * rowstride + (size_t)h * D, fbytes);
        const rsrc_t rv = make_rsrc(static_cast<const T*>(a.v) + tokf * rowstride + (size_t)h * D, fbytes);
        const rsrc_t rb = make_rsrc(a.beta + tokf * H + h, N > 0 ? (uint32_t)(((size_t)(N - 1) * H + 1) * 4) : 0u);
        struct KV {
            u32x4 k0, k1, v0, v1;
            float b0, b1;
        };
        auto load_kv = [&](int blk, KV& q2) {       // rows past N read as zeros
            const uint32_t t0 = (uint32_t)(blk * BTA + 2 * tp);
            const uint32_t o0 = t0 * row_bytes + (uint32_t)(fgrp * 16);
            q2.k0 = bload16(rk, o0);
            q2.k1 = bload16(rk, o0 + row_bytes);
            q2.v0 = bload16(rv, o0);
            q2.v1 = bload16(rv, o0 + row_bytes);
            q2.b0 = bload4f(rb, t0 * (uint32_t)H * 4u);
            q2.b1 = bload4f(rb, (t0 + 1u) * (uint32_t)H * 4u);
        };
        // key norms over the token's GPT lanes; rho k, beta rho k (bf16) and v
        // written transposed, the two tokens of a thread as one dword
        auto put_kv = [&](const KV& q2, unsigned char* buf) {
            float n0 = 0.f, n1 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x0 = bf2f((uint16_t)(q2.k0[e >> 1] >> (16 * (e & 1))));
                const float x1 = bf2f((uint16_t)(q2.k1[e >> 1] >> (16 * (e & 1))));
                n0 += x0 * x0;
                n1 += x1 * x1;
            }
            n0 = group_sum<GPT>(n0);
            n1 = group_sum<GPT>(n1);
            // 1 / max(|k|, eps) and beta (logits: sigmoid / N), as frame_gram forms them
            const float r0 = a.raw_keys ? 1.0f : fminf(__builtin_amdgcn_rsqf(n0), inv_eps);
            const float r1 = a.raw_keys ? 1.0f : fminf(__builtin_amdgcn_rsqf(n1), inv_eps);
            const float be0 = a.logits ? sigmoid_f(q2.b0) * inv_n : q2.b0;
            const float be1 = a.logits ? sigmoid_f(q2.b1) * inv_n : q2.b1;
            const float s0b = be0 * r0, s1b = be1 * r1;
            const int t = 2 * tp;
            if constexpr (TRK) {                     // token-major rows, one 16-byte chunk per array and token
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const u32x4 x = u ? q2.k1 : q2.k0;
                    const float rr = u ? r1 : r0, ss = u ? s1b : s0b;
                    u32x4 pk, bk;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const float lo = bf2f((uint16_t)(x[d] & 0xffffu)), hi = bf2f((uint16_t)(x[d] >> 16));
                        pk[d] = pack_bf16x2(rr * lo, rr * hi);
                        bk[d] = pack_bf16x2(ss * lo, ss * hi);
                    }
                    const int off = tok_off<ROWT>(t + u, 8 * fgrp);
                    *reinterpret_cast<u32x4*>(buf + off) = pk;
                    *reinterpret_cast<u32x4*>(buf + ARRA + off) = bk;
                    *reinterpret_cast<u32x4*>(buf + 2 * ARRA + off) = u ? q2.v1 : q2.v0;
                }
                return;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = 16 * (e & 1);
                const uint32_t kb0 = (q2.k0[e >> 1] >> sh) & 0xffffu, kb1 = (q2.k1[e >> 1] >> sh) & 0xffffu;
                const float x0 = bf2f((uint16_t)kb0), x1 = bf2f((uint16_t)kb1);
                const int off = lds_chunk<ROWA>(8 * fgrp + e, t >> 3) + (t & 7) * 2;
                *reinterpret_cast<uint32_t*>(buf + off) = pack_bf16x2(r0 * x0, r1 * x1);
                *reinterpret_cast<uint32_t*>(buf + ARRA + off) = pack_bf16x2(s0b * x0, s1b * x1);
                *reinterpret_cast<uint32_t*>(buf + 2 * ARRA + off) =
                    ((q2.v0[e >> 1] >> sh) & 0xffffu) | (((q2.v1[e >> 1] >> sh) & 0xffffu) << 16);
            }
        };
        f32x4 accg[RT], accu[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            accg[i] = f32x4{0, 0, 0, 0};
            accu[i] = f32x4{0, 0, 0, 0};
        }
        auto mfma_blk = [&](const unsigned char* buf) {
            if constexpr (TRK) {
#pragma unroll
                for (int ks = 0; ks < BTA / 32; ++ks) {
                    const int kb = 32 * ks + 8 * g;
                    const frag bx = tr_frag<ROWT>(buf + ARRA, 16 * wave, kb, r);       // beta rho K^T, rows e
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt)                                    // G[c][e]
                        io::mma(accg[mt], tr_frag<ROWT>(buf, 16 * mt, kb, r), bx);
#pragma unroll
                    for (int i = 0; i < RT; ++i)                                       // U^T[e][a]
                        io::mma(accu[i], bx, tr_frag<ROWT>(buf + 2 * ARRA, 16 * i, kb, r));
                }
                return;
            }
#pragma unroll
            for (int ks = 0; ks < BTA / 32; ++ks) {
                const frag bx = lds_frag<T, ROWA>(buf + ARRA, 16 * wave + r, ks, g);        // beta rho K^T, rows e
#pragma unroll
                for (int mt = 0; mt < RT; ++mt)                                             // G[c][e]
                    io::mma(accg[mt], lds_frag<T, ROWA>(buf, 16 * mt + r, ks, g), bx);
#pragma unroll
                for (int i = 0; i < RT; ++i)                                                // U^T[e][a]
                    io::mma(accu[i], bx, lds_frag<T, ROWA>(buf + 2 * ARRA, 16 * i + r, ks, g));
            }
        };
        KV ring_a[PDA];
#pragma unroll
        for (int j = 0; j < PDA; ++j) {
            load_kv(j, ring_a[j]);
            // keep each block's six loads together: issued in the loop's own
            // order (K, V, beta per block), the wait for a block's beta stays
            // exact; left free, the compiler moved every beta load behind all
            // K and V loads here, and the waits it then had to share with the
            // loop drained most of the ring before each block's beta was used
            asm volatile("" ::: "memory");
        }
        const int nfa = nba / PDA;
        for (int gi = 0; gi < nfa; ++gi) {
#pragma unroll
            for (int j = 0; j < PDA; ++j) {
                const int blk = gi * PDA + j;
                unsigned char* buf = smem + (blk & 1) * 3 * ARRA;
                put_kv(ring_a[j], buf);
                __syncthreads();
                load_kv(blk + PDA, ring_a[j]);       // past the frame: zeros, no traffic
                mfma_blk(buf);
            }
        }
#pragma unroll
        for (int j = 0; j < PDA; ++j) {
            const int blk = nfa * PDA + j;
            if (blk < nba) {
                unsigned char* buf = smem + (blk & 1) * 3 * ARRA;
                put_kv(ring_a[j], buf);
                __syncthreads();
                mfma_blk(buf);
            }
        }
        __syncthreads();                             // the LDS is staged with S_0 next
        load_s0();
#pragma unroll
        for (int j = 0; j < C::PD; ++j) load_blk(j, ring[j]);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            glo[ks] = accg[2 * ks];
            ghi[ks] = 2 * ks + 1 < RT ? accg[2 * ks + 1] : f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < C::ET; ++i) su[i] = accu[i];
    }
#pragma unroll
    for (int i = 0; i < C::PD0; ++i) {
        const int e4 = (tid + i * C::NTH) * 4, rr = e4 / D, cc = e4 % D;
        const f32x4 v = st0[i];
        if constexpr (sizeof(T) == 2)
            *reinterpret_cast<u32x2*>(sS0 + rr * C::ROWB + cc * 2) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        else
            *reinterpret_cast<f32x4*>(sS0 + rr * C::ROWB + cc * 4) = v;
    }
#pragma unroll
    for (int i = 0; i < C::ET; ++i) sn[i] = sn[i] * al + su[i];
    frag gm[C::KS];                                 // operand A: -alpha times the sums
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const f32x4 lo = glo[ks] * (-al), hi = ghi[ks] * (-al);
        if constexpr (sizeof(T) == 2)
            gm[ks] = u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                           pack_bf16x2(hi[2], hi[3])};
        else
            gm[ks] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (!FUSED && !kvalid) gm[ks] = io::zero();
    }
    __syncthreads();                                // S_0 staged
#pragma unroll
    for (int i = 0; i < C::ET; ++i) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int c0 = (ks * 32 + 8 * g) % D;
            const unsigned char* src = sS0 + (16 * i + r) * C::ROWB + c0 * C::SZ;
            frag sb;
            if constexpr (FUSED) {                  // columns 32ks + 4g + t, 32ks + 16 + 4g + t
                const unsigned char* row = sS0 + (16 * i + r) * C::ROWB;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(row + (ks * 32 + 4 * g) * 2);
                const u32x2 hi = ks * 32 + 16 < D ? *reinterpret_cast<const u32x2*>(row + (ks * 32 + 16 + 4 * g) * 2)
                                                  : u32x2{0u, 0u};
                sb = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else if constexpr (sizeof(T) == 2) {
                sb = *reinterpret_cast<const u32x4*>(src);
            } else {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
                sb = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
            if (!FUSED && !kvalid) sb = io::zero();
            io::mma(sn[i], gm[ks], sb);               // (S_0 Gm)^T += Gm^T S_0^T
        }
    }

    // ---- S_out (first range only) and the planes of S_1 in LDS
    if (part == 0 && a.S_out) {
#pragma unroll
        for (int i = 0; i < C::ET; ++i)
            *reinterpret_cast<f32x4*>(a.S_out + (size_t)bh * D * D + (size_t)(16 * i + r) * D + col0) = sn[i];
    }
#pragma unroll
    for (int i = 0; i < C::ET; ++i) {
        const int off = (16 * i + r) * C::ROWB + col0 * C::SZ;
        if constexpr (sizeof(T) == 2) {
            const f32x4 v = sn[i];
            const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
            const uint32_t l01 = pack_bf16x2(v[0] - bf2f(h01 & 0xffffu), v[1] - bf2f(h01 >> 16));
            const uint32_t l23 = pack_bf16x2(v[2] - bf2f(h23 & 0xffffu), v[3] - bf2f(h23 >> 16));
            *reinterpret_cast<u32x2*>(sS1 + off) = u32x2{h01, h23};
            *reinterpret_cast<u32x2*>(sS1 + C::PLANE + off) = u32x2{l01, l23};
        } else {
            *reinterpret_cast<f32x4*>(sS1 + off) = sn[i];
        }
    }
    __syncthreads();                                // S_1 planes complete
    // A fragments of O^T = S_1 Q^T: rows [16 wave, 16 wave + 16) of S_1
    frag ah[C::KS], alw[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const int c0 = (ks * 32 + 8 * g) % D;
        const unsigned char* src = sS1 + (16 * wave + r) * C::ROWB + c0 * C::SZ;
        if constexpr (sizeof(T) == 2) {
            ah[ks] = *reinterpret_cast<const u32x4*>(src);
            alw[ks] = *reinterpret_cast<const u32x4*>(src + C::PLANE);
        } else {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
            ah[ks] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        if (!kvalid) {
            ah[ks] = io::zero();
            alw[ks] = io::zero();
        }
        hold(ah[ks]);                               // read before the barrier, not after it
        if constexpr (sizeof(T) == 2) hold(alw[ks]);
    }
    __syncthreads();                                // LDS is reused for Q and O below
    if (nbeg >= nend) return;

    auto compute_blk = [&](const unsigned char* buf, unsigned char* obuf) {
#pragma unroll 1
        for (int sbk = 0; sbk < C::BT / 16; ++sbk) {     // 16-token sub-blocks
            frag bq[C::KS];
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int c0 = (ks * 32 + 8 * g) % D;
                const unsigned char* src = buf + (sbk * 16 + r) * C::ROWB + c0 * C::SZ;
                if constexpr (sizeof(T) == 2) {
                    bq[ks] = *reinterpret_cast<const u32x4*>(src);
                } else {
                    const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                    const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
                    bq[ks] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
                if (!kvalid) bq[ks] = io::zero();
            }
            f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                io::mma(acc, ah[ks], bq[ks]);
                if constexpr (sizeof(T) == 2) io::mma(acc, alw[ks], bq[ks]);
            }
            unsigned char* orow = obuf + (sbk * 16 + r) * C::ROWB;           // token sbk*16 + r
            if constexpr (sizeof(T) == 2)
                *reinterpret_cast<u32x2*>(orow + col0 * 2) =
                    u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            else
                *reinterpret_cast<f32x4*>(orow + col0 * 4) = acc;
        }
    };
    // whole rows of O block `blk` from its LDS tile; block -1 maps past the
    // resource and is dropped
    auto store_blk = [&](int blk, const unsigned char* obuf) {
        const uint32_t base = blk >= 0 ? (uint32_t)(blk * C::BT) * row_bytes : 0x80000000u;
#pragma unroll
        for (int i = 0; i < C::NST; ++i) {
            const int c = tid + C::NTH * i, n = c / C::LPR, pc = c % C::LPR;
            const u32x4 val = *reinterpret_cast<const u32x4*>(obuf + n * C::ROWB + pc * 16);
            bstore16(ro, base + (uint32_t)n * row_bytes + (uint32_t)(pc * 16), val);
        }
    };
    // the pipeline of the output pass: ring slot blk % PD, LDS buffer blk & 1,
    // one barrier per block; block blk-1's O tile is stored after the barrier
    unsigned char* const obase = smem + 2 * C::QBUF;
    const int nfull = nblk / C::PD;
    for (int gi = 0; gi < nfull; ++gi) {
#pragma unroll
        for (int j = 0; j < C::PD; ++j) {
            const int blk = gi * C::PD + j;
            unsigned char* buf = smem + (j & 1) * C::QBUF;
            put_blk(ring[j], buf);
            __syncthreads();
            store_blk(blk - 1, obase + ((j + 1) & 1) * C::QBUF);
            load_blk(blk + C::PD, ring[j]);         // past the range: zeros, no traffic
            compute_blk(buf, obase + (j & 1) * C::QBUF);
        }
    }
    const int rem = nblk - nfull * C::PD;
#pragma unroll
    for (int j = 0; j < C::PD; ++j) {
        if (j < rem) {
            const int blk = nfull * C::PD + j;
            unsigned char* buf = smem + (j & 1) * C::QBUF;
            put_blk(ring[j], buf);
            __syncthreads();
            store_blk(blk - 1, obase + ((j + 1) & 1) * C::QBUF);
            compute_blk(buf, obase + (j & 1) * C::QBUF);
        }
    }
    __syncthreads();
    store_blk(nblk - 1, obase + ((nblk - 1) & 1) * C::QBUF);
}

// ================================================================== state_copy
// S_final <- S0 (or zeros) for an empty scan (F == 0).  A plain kernel rather
// than a memset/memcpy node so the call stays capturable in a graph.
__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace gdn
