// gfx950 (MI355X) kernels for bidirectional (non-causal) linear attention.
//
// Operation (Flash Bi-directional Linear Attention README, intro; simple_la
// in its "Update" 2024-12-28; backward in "Update" 2024-12-30): per (batch,
// head), phi(x) = elu(x) + 1,
//   S = sum_t phi(k_t) v_t^T,  z = sum_t phi(k_t),
//   O_t = phi(q_t) S / (phi(q_t) . z + eps)     (simple_la: phi(q_t) S).
//
// Q and K have head size DK, V and O head size DV (each 32, 64, 96 or 128).
// Kernels, by step of the path:
//   fwd_state_w64_kernel (16-bit, DK = DV = 64), fwd_state_tile_kernel (the
//                      other 16-bit sizes) and fwd_state_kernel (fp32):
//                      phi(K)^T [V | 1] over a token slice on MFMA, one partial
//                      (S, z) per slice, or the state itself when a head is
//                      one slice;
//   combine_kernel     sums the partials of each head in ascending slice order;
//   fwd_output_kernel  O = phi(Q) S / (phi(Q) z + eps), S and z as MFMA operands;
//   bwd_dq_w64_kernel (16-bit, DK = DV = 64), bwd_dq_tile_kernel (the other
//                      16-bit sizes) and bwd_dq_kernel (fp32): dQ, plus
//                      partial dS = phi(Q)^T (dO / den) on MFMA and
//                      dz = sum_t c_t phi(q_t), combined like the forward state;
//   bwd_dkv_kernel     dK = (V dS^T + dz) * phi'(K), dV = phi(K) dS.
// The causal form (LA_CAUSAL; flash-linear-attention README, "Different forms
// of linear attention"), for every element type and head size up to 128,
// reuses the state reduction per segment and adds:
//   prefix_kernel, suffix_kernel  exclusive prefixes / suffixes of the
//                      per-segment sums, in place;
//   fwd_causal_kernel  the forward as a chunked scan of each segment (16-bit;
//                      head sizes 32 and 96 run padded to 64 and 128);
//   bwd_causal_q_kernel, bwd_causal_kv_kernel  the backward as a forward-order
//                      scan (dQ) and a reverse-order scan (dK, dV);
//   fwd_causal_f32_kernel, bwd_causal_q_f32_kernel, bwd_causal_kv_f32_kernel
//                      the same scans on fp32 operands.
// The optional query scale needs no kernel of its own (see Plan::eps).
//
// MFMA conventions (v_mfma_f32_16x16x32_{f16,bf16}; for fp32 operands eight
// v_mfma_f32_16x16x4f32 cover the same 32-long contraction): a wave holds A
// rows m = lane % 16, B columns n = lane % 16, each lane carrying 8 values of
// the contraction index for its lane group g = lane / 16; the result C[m][n]
// sits in lane (n + 16 g) at register r with m = 4 g + r. Which physical k the
// 8 values of a lane group stand for is free, as long as A and B agree, and
// the kernels use that freedom: a lane that loads D/4 contiguous features of
// one token row can feed them straight into B fragments, and the rows of A are
// permuted so that the same lane receives D/4 contiguous output features of
// that token, which it stores contiguously.
//
// Every tensor has its own layout (Layouts): batch, head and token strides in
// elements, dense [B, H, T, D] or [B, T, H, D] unless the caller passed
// strides; a row's D features are contiguous. The work split is a pure
// function of the shape and there are no floating-point atomics, so results
// are bit-identical across runs.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "la_internal.h"

namespace la {
namespace {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
enum FeatureMap { kPhiElu1 = 0, kPhiRelu = 1, kPhiIdentity = 2 };

template <typename T> struct Elt;
// kScaled: the fp32 states are multiplied by a power of two before they are
// rounded to this operand type (f16's range is too narrow for S, z, dS).
template <> struct Elt<float> { using frag = f32x8; static constexpr bool kScaled = false; };
template <> struct Elt<f16> { using frag = f16x8; static constexpr bool kScaled = true; };
template <> struct Elt<bf16> { using frag = bf16x8; static constexpr bool kScaled = false; };
template <typename T> using Frag = typename Elt<T>::frag;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes, the
// 8 bytes that lane i addresses become row i/4, columns 4(i%4)..4(i%4)+3 of a
// 4 x 16 block of 16-bit values, and lane j receives column j, rows 0..3 in
// order. Pointing lane i of group g at row (4 g' + i/4), column (c0 + 4(i%4))
// of a row-major tile therefore hands lane j the 4 consecutive rows of column
// c0 + j: an MFMA operand whose contraction index runs over tile rows.
__device__ __forceinline__ i16x4 lds_read_tr(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(const_cast<void*>(p)));
}

template <typename T>
__device__ __forceinline__ Frag<T> join_frag(i16x4 lo, i16x4 hi) {
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(Frag<T>, v);
}

// 16x16x16 MFMA on 16-bit operands held as raw bits (4 values per lane).
template <typename T> __device__ __forceinline__ f32x4 mma_k16(i16x4 a, i16x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mma_k16<f16>(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma_k16<bf16>(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Index of this thread's wave in the workgroup, as a value the compiler knows
// is the same on every lane of the wave (it lives in a scalar register).
// Branches on it, or on block indices derived from it, then compile to scalar
// branches. Computed as threadIdx.x / 64, the compiler cannot tell that it is
// wave-uniform and lowers such branches by masking lanes; the register
// allocator has then been seen to save a live vector register to an
// accumulation register inside one arm of such a branch and restore it after
// the join on every lane, which corrupts that register on the waves that took
// the other arm (wrong results, no error).
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Keeps the compiler from moving instructions across this point. Used between
// the load batches of a prefetch pipeline: the vector-memory counter retires
// loads in issue order, so batches must stay in the order they are consumed
// or the wait for the older batch would also drain the newer one.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Keeps this wave's LDS accesses in program order across the point. LDS
// instructions from one wave execute in order, so a read issued after a write
// to the same address sees the written value without waiting for it; only
// the compiler must not move accesses across (it would be free to for the
// transpose-read builtins it cannot prove alias the writes).
__device__ __forceinline__ void wave_lds_sync() { __asm__ volatile("" ::: "memory"); }

__device__ __forceinline__ f32x4 mma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// The feature map phi, chosen by la_problem.flags: elu(x) + 1 (the default),
// relu(x) or x. feature() returns phi(x) and phi'(x) in fp32.
//   elu + 1: evaluated piecewise, x + 1 for x > 0 and e^x otherwise (never
//     as expm1(x) + 1, which cancels for x << 0); both sides are computed and
//     one is selected, so no branch splits the wave (NaN falls to the exp
//     side and propagates). 16-bit inputs use the hardware exp2 on
//     x log2(e), fp32 inputs the accurate expf. phi' = 1 for x > 0, else e^x.
//   relu: x < 0 ? 0 : x (NaN propagates); phi' = 1 for x > 0, else 0.
//   identity: phi = x, phi' = 1.
template <int FM, typename T>
__device__ __forceinline__ void feature(float x, float& p, float& dp) {
    if constexpr (FM == kPhiRelu) {
        p = x < 0.f ? 0.f : x;
        dp = x > 0.f ? 1.f : 0.f;
    } else if constexpr (FM == kPhiIdentity) {
        p = x;
        dp = 1.f;
    } else {
        float e;
        if constexpr (std::is_same<T, float>::value) {
            e = expf(x);
        } else {
            e = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
        }
        p = x > 0.f ? x + 1.f : e;
        dp = x > 0.f ? 1.f : e;
    }
}

template <int FM, typename T>
__device__ __forceinline__ float phi(float x) {
    float p, dp;
    feature<FM, T>(x, p, dp);
    return p;
}

// phi'(x) from phi(x) alone: min(phi, 1) for elu + 1 (phi > 1 exactly where
// x > 0 and phi' = 1; elsewhere phi = e^x = phi'), [phi > 0] for relu, 1 for
// the identity.
template <int FM>
__device__ __forceinline__ float dphi_of(float p) {
    if constexpr (FM == kPhiRelu) return p > 0.f ? 1.f : 0.f;
    else if constexpr (FM == kPhiIdentity) return 1.f;
    else return fminf(p, 1.f);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }


// Hardware places workgroup b on XCD b % 8. Renumber so that consecutive
// logical ids (the slices or chunks of one head) share an XCD and its L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    if (n % 8 != 0) return b;
    return (b % 8) * (n / 8) + b / 8;
}

// N contiguous elements of a row; N * sizeof(T) is a multiple of 16 bytes.
template <typename T, int N>
struct alignas(16) Row {
    T e[N];
};

// Buffer-descriptor access to a slice of one head's rows. The descriptor
// covers exactly rows [r0, r1) of the head (rows rs elements apart; the span
// is below 2^31 bytes, as a whole head is), rows are counted from r0, and the
// hardware reads zeros for loads past r1 and drops stores there, even where
// the head continues: the kernels need no clamping or branches at the ragged
// end of a slice.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// phi of eight 16-bit values (one 16-byte row piece), each rounded to the
// element type: the bits of static_cast<T>(phi<FM, T>(x)) for every x. For
// f16 the work runs on packed halves, four instructions an element instead of
// about eight:
//   elu + 1 = max(x, 0) + e^min(x, 0). For x > 0 the exponential is exp2(0) =
//     1 and the f16 sum is x + 1 rounded once, as the fp32 sum rounded to f16
//     is (that sum is exact in fp32 wherever the f16 rounding could be near a
//     tie); for x <= 0 it is 0 plus e^x rounded to f16. The exponent x log2(e)
//     is formed in fp32 from the f16 input, as in feature(). The IEEE
//     minimum / maximum forms carry NaN through, and phi(inf) = inf,
//     phi(-inf) = 0 as before.
//   relu = maximum(x, 0) (+0 for an input of -0, where the scalar form keeps
//     -0: the same value).
// Other element types take the scalar form.
template <int FM, typename T>
__device__ __forceinline__ u32x4 phi8(u32x4 raw) {
    static_assert(sizeof(T) == 2, "eight 16-bit values in 16 bytes");
    if constexpr (FM == kPhiIdentity) {
        return raw;
    } else if constexpr (std::is_same<T, f16>::value) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        h2 x[4];
        __builtin_memcpy(x, &raw, sizeof(x));
        const h2 zero = {static_cast<f16>(0.f), static_cast<f16>(0.f)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (FM == kPhiRelu) {
                x[i] = __builtin_elementwise_maximum(x[i], zero);
            } else {
                const h2 mn = __builtin_elementwise_minimum(x[i], zero);
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(mn[0]), 1.4426950408889634f, 0.f));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(mn[1]), 1.4426950408889634f, 0.f));
                const h2 e = {static_cast<f16>(e0), static_cast<f16>(e1)};
                x[i] = __builtin_elementwise_maximum(x[i], zero) + e;
            }
        }
        u32x4 out;
        __builtin_memcpy(&out, x, sizeof(out));
        return out;
    } else {
        T v[8];
        __builtin_memcpy(v, &raw, sizeof(v));
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<T>(phi<FM, T>(to_f32(v[e])));
        u32x4 out;
        __builtin_memcpy(&out, v, sizeof(out));
        return out;
    }
}

// phi of eight 16-bit values in fp32: the values of phi<FM, T>(x), the same
// identities as phi8 with the final sum max(x, 0) + e formed in fp32 (one
// rounding, as x + 1 in the scalar form; 0 + e = e below zero).
template <int FM, typename T>
__device__ __forceinline__ void phi8_f32(u32x4 raw, float (&p)[8]) {
    static_assert(sizeof(T) == 2, "eight 16-bit values in 16 bytes");
    if constexpr (std::is_same<T, f16>::value && FM != kPhiIdentity) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        h2 x[4];
        __builtin_memcpy(x, &raw, sizeof(x));
        const h2 zero = {static_cast<f16>(0.f), static_cast<f16>(0.f)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h2 mx = __builtin_elementwise_maximum(x[i], zero);
            if constexpr (FM == kPhiRelu) {
                p[2 * i] = static_cast<float>(mx[0]);
                p[2 * i + 1] = static_cast<float>(mx[1]);
            } else {
                const h2 mn = __builtin_elementwise_minimum(x[i], zero);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(mn[h]), 1.4426950408889634f, 0.f));
                    p[2 * i + h] = __builtin_fmaf(static_cast<float>(mx[h]), 1.f, e);
                }
            }
        }
    } else {
        T v[8];
        __builtin_memcpy(v, &raw, sizeof(v));
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = phi<FM, T>(to_f32(v[e]));
    }
}

// phi and phi' of eight 16-bit values in fp32: the values feature() gives.
// For elu + 1 on f16 from the identities of phi8, with phi'(x) = e^min(x, 0)
// itself (exp2(0) = 1 for x > 0); the other cases take feature().
template <int FM, typename T>
__device__ __forceinline__ void feature8(u32x4 raw, float* p, float* dp) {
    static_assert(sizeof(T) == 2, "eight 16-bit values in 16 bytes");
    if constexpr (std::is_same<T, f16>::value && FM == kPhiElu1) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        h2 x[4];
        __builtin_memcpy(x, &raw, sizeof(x));
        const h2 zero = {static_cast<f16>(0.f), static_cast<f16>(0.f)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h2 mx = __builtin_elementwise_maximum(x[i], zero);
            const h2 mn = __builtin_elementwise_minimum(x[i], zero);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(mn[h]), 1.4426950408889634f, 0.f));
                p[2 * i + h] = __builtin_fmaf(static_cast<float>(mx[h]), 1.f, e);
                dp[2 * i + h] = e;
            }
        }
    } else {
        T v[8];
        __builtin_memcpy(v, &raw, sizeof(v));
#pragma unroll
        for (int e = 0; e < 8; ++e) feature<FM, T>(to_f32(v[e]), p[e], dp[e]);
    }
}

// keep ? x : 0 on a 16-byte row piece
__device__ __forceinline__ u32x4 keep_or_zero(u32x4 x, bool keep) {
    return keep ? x : u32x4{0u, 0u, 0u, 0u};
}

struct HeadBuf {
    __amdgpu_buffer_rsrc_t rsrc;
};
// Element offset of row 0 of head bh (B * H <= 2^24, so 32-bit division).
__device__ __forceinline__ int64_t head_offset(const Layout& L, int64_t bh) {
    const int64_t b = (int)bh / (int)L.H;
    return b * L.sb + (bh - b * L.H) * L.sh;
}

template <typename T>
__device__ __forceinline__ HeadBuf slice_buf(const T* base, const Layout& L, int64_t bh, int D, int64_t r0,
                                             int64_t r1) {
    const T* p = base + head_offset(L, bh) + r0 * L.rs;
    const int64_t bytes = r1 > r0 ? ((r1 - r0 - 1) * L.rs + D) * (int64_t)sizeof(T) : 0;
    return HeadBuf{__builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(p), 0, (int)bytes, 0x00020000)};
}
// The order in which a workgroup visits the n blocks of its slice, n padded
// up to a multiple of `group`: rotated by a per-workgroup multiple of `group`.
// Workgroups stream their slices side by side at the same pace; unrotated,
// they would all be at the same offset of slices whose bases are a fixed
// stride apart, and whether those simultaneous accesses pile onto the same
// DRAM channels would depend on where the buffers sit in physical memory.
// Indices at or past the padded count (the prefetches of the last turn, at
// most a few blocks) map to themselves, past the slice end, where the slice's
// buffer descriptors read zeros and drop stores; the clamp keeps them within
// 64 blocks of the end whatever the caller passes.
struct Rotation {
    int npad, R;
    __device__ Rotation(int n, int group, int wid) {
        npad = (n + group - 1) / group * group;
        const int nr = npad / group;
        R = nr > 0 ? group * ((wid * 7) % nr) : 0;
    }
    __device__ int operator()(int blk) const {
        if (blk >= npad) return min(blk, npad + 64);
        const int x = blk + R;
        return x >= npad ? x - npad : x;
    }
};

// Byte offset of element (row, col) of a slice whose rows are rs elements
// apart, for a buffer access, in unsigned 32-bit arithmetic (exact modulo
// 2^32). Offsets inside a slice are below 2^31 (the head size limit); rows
// past the end, which the kernels visit at most a few padded blocks (under
// a thousand rows) far, stay below 2^32, so their offsets still lie past the
// descriptor's range: such loads read zeros and such stores are dropped.
template <typename T>
__device__ __forceinline__ int buf_off(int64_t row, int64_t rs, int col) {
    return (int)((uint32_t)row * (uint32_t)(rs * (int)sizeof(T)) + (uint32_t)(col * (int)sizeof(T)));
}

// The offset of a 16-byte piece at element `col` of a row that a kernel built
// for rows of W elements holds with only REAL of them (a head size padded up
// inside the kernel): pieces at or past REAL get an offset past the range of
// every descriptor (heads span less than 2^31 bytes), so their loads read
// zeros and their stores are dropped. REAL = W leaves the offset as it is.
template <int W, int REAL>
__device__ __forceinline__ int pad_off(int off, int col) {
    if constexpr (REAL >= W) {
        return off;
    } else {
        return col < REAL ? off : (int)0x80000000u;
    }
}

// Cache policy of a buffer access (the instruction's cache-policy bits; hints
// only, results are the same). The 16-bit state reductions load K and V
// non-temporally: 104 -> 93 us at B8-H16-T16384-D64 f16 (207 -> 182 us at
// D128 bf16), with the rest of the step unchanged. Elsewhere it did not pay:
// on the output or K/V-side kernels' accesses it cost 5-25%, and on the dQ
// stores it only moved time from the K/V kernel to the dQ kernel (the
// write-back of lines left in the 256 MB infinity cache falls on whichever
// kernel runs next).
enum CachePolicy { kCacheDefault = 0, kNonTemporal = 2 };

template <int CP = kCacheDefault>
__device__ __forceinline__ uint4 buf_load16(const HeadBuf& b, int byte_off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b.rsrc, byte_off, 0, CP);
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CP = kCacheDefault>
__device__ __forceinline__ void buf_store16(const HeadBuf& b, int byte_off, uint4 x) {
    const u32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_amdgcn_raw_buffer_store_b128(v, b.rsrc, byte_off, 0, CP);
}

// Four fp32 values rounded to the 16-bit element type, as one 8-byte store.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ void buf_store4(const HeadBuf& b, int byte_off, f32x4 x) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = static_cast<T>(x[r]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), b.rsrc, byte_off, 0, 0);
}

// N contiguous elements of row `row` (rows rs elements apart) starting at
// element `col`, by buffer loads.
template <typename T, int N>
__device__ __forceinline__ void load_row_buf(Row<T, N>& r, const HeadBuf& b, int64_t row, int64_t rs, int col) {
    constexpr int NV = N * (int)sizeof(T) / 16;
    uint4* d = reinterpret_cast<uint4*>(r.e);
    const int off = buf_off<T>(row, rs, col);
#pragma unroll
    for (int i = 0; i < NV; ++i) d[i] = buf_load16(b, off + 16 * i);
}

// Stores a 16-row x D tile whose row n, columns [F g, F g + F), sit in lane
// n + 16 g, as full contiguous rows: the lanes first write their quarter rows
// to this wave's LDS staging area (row stride D + 16 bytes), then each lane
// reads 16 bytes back so that one store instruction covers whole 128-byte lines.
template <typename T, int D, int CP = kCacheDefault>
__device__ __forceinline__ void store_tile_rows(T* stage, const Row<T, D / 4>& vals, const HeadBuf& b,
                                                int64_t row0, int64_t rs) {
    constexpr int F = D / 4, EPC = 16 / (int)sizeof(T), LDR = D + EPC;
    constexpr int CPR = D / EPC;       // 16-byte chunks per row
    constexpr int NC = 16 * CPR / 64;  // chunks per lane (rows of CPR chunks, 16 rows)
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < F / EPC; ++i)
        *reinterpret_cast<uint4*>(&stage[m * LDR + F * g + EPC * i]) = reinterpret_cast<const uint4*>(vals.e)[i];
    wave_lds_sync();
    // chunk n = 64 k + lane of the tile: row n / CPR, chunk n % CPR of that row
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int n = 64 * k + lane, r = n / CPR, c = n % CPR;
        const uint4 x = *reinterpret_cast<const uint4*>(&stage[r * LDR + EPC * c]);
        buf_store16<CP>(b, buf_off<T>(row0 + r, rs, EPC * c), x);
    }
    wave_lds_sync();
}

// Same tile, each lane storing its own quarter row (for shapes whose LDS
// budget leaves no room for the staging area).
template <typename T, int D>
__device__ __forceinline__ void store_tile_quarters(const Row<T, D / 4>& vals, const HeadBuf& b, int64_t row0,
                                                    int64_t rs) {
    constexpr int F = D / 4, NV = F * (int)sizeof(T) / 16;
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int off = buf_off<T>(row0 + m, rs, F * g);
#pragma unroll
    for (int i = 0; i < NV; ++i) buf_store16(b, off + 16 * i, reinterpret_cast<const uint4*>(vals.e)[i]);
}

// Loads are unconditional: callers clamp the row index into the valid range
// and discard or zero what belongs to rows past the end. (Loads under a branch
// make the compiler drain every outstanding load at the join, which would
// serialise the prefetch pipelines.)
template <typename T, int N>
__device__ __forceinline__ void load_row(Row<T, N>& r, const T* __restrict__ p) {
    constexpr int NV = N * (int)sizeof(T) / 16;
    uint4* d = reinterpret_cast<uint4*>(r.e);
    const uint4* s = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < NV; ++i) d[i] = s[i];
}

template <typename T, int N>
__device__ __forceinline__ void zero_row_unless(Row<T, N>& r, bool keep) {
    constexpr int NV = N * (int)sizeof(T) / 16;
    uint4* d = reinterpret_cast<uint4*>(r.e);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        d[i].x = keep ? d[i].x : 0u;
        d[i].y = keep ? d[i].y : 0u;
        d[i].z = keep ? d[i].z : 0u;
        d[i].w = keep ? d[i].w : 0u;
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_row(T* __restrict__ p, const float (&x)[N]) {
    Row<T, N> r;
#pragma unroll
    for (int j = 0; j < N; ++j) r.e[j] = static_cast<T>(x[j]);
    constexpr int NV = N * (int)sizeof(T) / 16;
    const uint4* s = reinterpret_cast<const uint4*>(r.e);
    uint4* d = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < NV; ++i) d[i] = s[i];
}

// Workgroup-wide max and sum over NW waves: an xor tree inside each wave,
// then a pairwise tree over the waves in a fixed order. red holds NW floats.
template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red[wave_index()] = v;
    __syncthreads();
    float x[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) x[w] = red[w];
#pragma unroll
    for (int n = NW / 2; n > 0; n /= 2)
#pragma unroll
        for (int w = 0; w < n; ++w) x[w] = fmaxf(x[2 * w], x[2 * w + 1]);
    __syncthreads();
    return x[0];
}

template <int NW = kWaves>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red[wave_index()] = v;
    __syncthreads();
    float x[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) x[w] = red[w];
#pragma unroll
    for (int n = NW / 2; n > 0; n /= 2)
#pragma unroll
        for (int w = 0; w < n; ++w) x[w] = x[2 * w] + x[2 * w + 1];
    __syncthreads();
    return x[0];
}

// Exponent s with maxabs * 2^s in [2^14, 2^15): the largest state entry lands
// well inside f16's range and the rest keep f16's relative precision down to
// 2^-24 of it. Zero, inf or NaN: no scaling (inf/NaN then propagate).
__device__ __forceinline__ int scale_exp(float maxabs) {
    if (!(maxabs > 0.f) || !isfinite(maxabs)) return 0;
    int e;
    frexpf(maxabs, &e);  // maxabs = m 2^e, m in [0.5, 1)
    return min(max(15 - e, -120), 120);
}

// scale_exp for an exponent that is combined with others by taking the
// smallest: an all-zero block then gives the largest exponent, which leaves
// the others' choice alone.
__device__ __forceinline__ int scale_exp_for_min(float maxabs) { return maxabs == 0.f ? 120 : scale_exp(maxabs); }

// Fixed-order sum of the P partial (S, z) blocks of every head: one thread per
// 4 consecutive floats of a head's DK*DV + DK block, slices added in ascending
// order, eight 16-byte loads in flight per batch. A kernel of its own: the
// launch boundary makes every partial visible, which costs far less here than
// device-scope fences inside the producing kernel (each of those writes back
// and invalidates the XCD's L2).
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ part, int P,
                                                           float* __restrict__ outS,
                                                           float* __restrict__ outz, int64_t BH) {
    constexpr int E4 = (DK * DV + DK) / 4;
    constexpr int BPH = (E4 + kThreads - 1) / kThreads;  // blocks per head
    const int64_t bh = blockIdx.x / BPH;
    const int i = (blockIdx.x % BPH) * kThreads + threadIdx.x;
    if (bh >= BH || i >= E4) return;
    const float4* pb = reinterpret_cast<const float4*>(part) + bh * (int64_t)P * E4 + i;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < P; p0 += 8) {
        float4 x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = pb[(int64_t)min(p0 + j, P - 1) * E4];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (p0 + j < P) {
                acc.x += x[j].x;
                acc.y += x[j].y;
                acc.z += x[j].z;
                acc.w += x[j].w;
            }
    }
    const int idx = 4 * i;
    if (idx < DK * DV)
        *reinterpret_cast<float4*>(outS + bh * DK * DV + idx) = acc;
    else
        *reinterpret_cast<float4*>(outz + bh * DK + (idx - DK * DV)) = acc;
}

// Largest |x| over the NE floats at M, over an NT-thread workgroup: every
// thread issues its 16-byte loads at once (NE/4 is a multiple of NT).
template <int NE, int NT = kThreads>
__device__ __forceinline__ float block_absmax_matrix(const float* __restrict__ M, float* red) {
    constexpr int PER = NE / 4 / NT;
    static_assert(PER * 4 * NT == NE, "thread count must tile the matrix");
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = reinterpret_cast<const float4*>(M)[threadIdx.x + i * NT];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    return block_max<NT / 64>(mx, red);
}

// max |z_i| and sum z_i over the D-vector z, workgroup-wide, in a fixed order.
template <int D, int NT = kThreads>
__device__ __forceinline__ void block_vector_stats(const float* __restrict__ z, float* red, float& mx,
                                                   float& sum) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (threadIdx.x < D / 4) v = reinterpret_cast<const float4*>(z)[threadIdx.x];
    mx = block_max<NT / 64>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))), red);
    sum = block_sum<NT / 64>((v.x + v.y) + (v.z + v.w), red);
}

// A DK x DV fp32 matrix and a DK-vector staged in LDS, with their statistics.
// The matrix rows are DV + 1 floats apart, so that the fragment builders'
// column walks (lanes 16 rows or 16 columns apart) spread over the banks.
template <int DK, int DV>
struct StagedState {
    static constexpr int kLD = DV + 1;
    static constexpr int kFloats = DK * kLD + DK;  // matrix, then the vector
    float max_m, max_z, sum_z;
};

// Copies M and z from global memory into s (StagedState<DK, DV>::kFloats floats)
// with all of each thread's 16-byte loads in flight at once, and reduces
// max |M|, max |z| and sum z over the NT-thread workgroup in a fixed order
// (xor tree per wave, then a pairwise tree over the waves). Ends with a
// barrier; red holds 3 NT / 64 floats.
template <int DK, int DV, int NT = kThreads>
__device__ __forceinline__ StagedState<DK, DV> stage_state(const float* __restrict__ M,
                                                           const float* __restrict__ z, float* s, float* red) {
    constexpr int PER = DK * DV / 4 / NT, LD = StagedState<DK, DV>::kLD, NW = NT / 64;
    static_assert(PER * 4 * NT == DK * DV && DK / 4 <= NT, "thread count must tile the matrix");
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = reinterpret_cast<const float4*>(M)[tid + i * NT];
    float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < DK / 4) w = reinterpret_cast<const float4*>(z)[tid];
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = 4 * (tid + i * NT), r = e / DV, c = e % DV;
        float* d = s + r * LD + c;
        d[0] = v[i].x;
        d[1] = v[i].y;
        d[2] = v[i].z;
        d[3] = v[i].w;
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    if (tid < DK / 4) *reinterpret_cast<float4*>(s + DK * LD + 4 * tid) = w;
    float b = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
    float c = (w.x + w.y) + (w.z + w.w);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a = fmaxf(a, __shfl_xor(a, off));
        b = fmaxf(b, __shfl_xor(b, off));
        c += __shfl_xor(c, off);
    }
    if (lane == 0) {
        red[wave] = a;
        red[NW + wave] = b;
        red[2 * NW + wave] = c;
    }
    __syncthreads();
    float xa[NW], xb[NW], xc[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        xa[w] = red[w];
        xb[w] = red[NW + w];
        xc[w] = red[2 * NW + w];
    }
#pragma unroll
    for (int n = NW / 2; n > 0; n /= 2)
#pragma unroll
        for (int w = 0; w < n; ++w) {
            xa[w] = fmaxf(xa[2 * w], xa[2 * w + 1]);
            xb[w] = fmaxf(xb[2 * w], xb[2 * w + 1]);
            xc[w] = xc[2 * w] + xc[2 * w + 1];
        }
    StagedState<DK, DV> st;
    st.max_m = xa[0];
    st.max_z = xb[0];
    st.sum_z = xc[0];
    return st;
}

// ---------------------------------------------------------------------------
// Steps 1-3: split-T state reduction.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
struct StateShape {
    static constexpr int kEPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    static constexpr int kTT = 64;                    // tokens per tile
    static constexpr int kLDT = kTT + kEPC;           // LDS row stride (elements), +16 B pad
    static constexpr int kCK = DK / kEPC;             // chunks per K row
    static constexpr int kCV = DV / kEPC;             // chunks per V row
    static constexpr int kNK = kTT * kCK / kThreads;  // K chunks per thread per tile
    static constexpr int kNV = kTT * kCV / kThreads;  // V chunks per thread per tile
    static constexpr int kNI = DK / 32;               // 16-row blocks of S per wave
    static constexpr int kNJ = DV / 32;               // 16-column blocks of S per wave
    static constexpr int kKS = kTT / 32;              // 32-token MFMA steps per tile
    static_assert(kNK * kThreads == kTT * kCK && kNV * kThreads == kTT * kCV, "tile must split evenly");
};

// One workgroup reduces tokens [p L, min((p+1) L, T)) of head bh into partial
// (S, z), S = phi(K)^T V (DK x DV). Per 64-token tile the threads load the
// tile's 16-byte chunks in order (chunk n: row n / chunks-per-row), apply phi
// to K in fp32 and round it to the operand type, and write both tiles to LDS
// transposed ([feature][token]), so that MFMA fragments, which want 8
// consecutive tokens per lane, are single 16-byte LDS reads. The four waves
// split S two by two: wave w owns the row blocks of half (w % 2) and the
// column blocks of half (w / 2). z is summed in fp32 from the same rounded
// phi(k) values in LDS that the MFMA reads, one feature per thread, tokens in
// order. Rows past the slice end load a clamped row and are written as zeros.
template <typename T, int DK, int DV, int FM>
__global__ __launch_bounds__(kThreads) void fwd_state_kernel(
    const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ stS,
    float* __restrict__ stz, float* __restrict__ part, int64_t T_, const Layouts lay, int P, int64_t L) {
    using Sh = StateShape<T, DK, DV>;
    const Layout lk = lay.k, lv = lay.v;
    constexpr int EPC = Sh::kEPC, TT = Sh::kTT, LDT = Sh::kLDT, CK = Sh::kCK, CV = Sh::kCV, NK = Sh::kNK,
                  NV = Sh::kNV, NI = Sh::kNI, NJ = Sh::kNJ, KS = Sh::kKS;
    __shared__ __attribute__((aligned(16))) T sK[DK * LDT];
    __shared__ __attribute__((aligned(16))) T sV[DV * LDT];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int wi = wave & 1, wj = wave >> 1;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const T* kb = k + head_offset(lk, bh);
    const T* vb = v + head_offset(lv, bh);

    f32x4 acc[NI][NJ];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) acc[ii][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zacc = 0.f;

    uint4 rk[NK], rv[NV];
    auto load_tile = [&](int64_t ts) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, c = n % CK;
            const int64_t t = min(ts + r, t1 - 1);  // masked when written to LDS
            rk[i] = *reinterpret_cast<const uint4*>(kb + t * lk.rs + c * EPC);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, c = n % CV;
            const int64_t t = min(ts + r, t1 - 1);
            rv[i] = *reinterpret_cast<const uint4*>(vb + t * lv.rs + c * EPC);
        }
    };

    const int64_t ntile = (t1 > t0) ? (t1 - t0 + TT - 1) / TT : 0;
    if (ntile > 0) load_tile(t0);
    for (int64_t it = 0; it < ntile; ++it) {
        const int64_t ts = t0 + it * TT;
        __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, c = n % CK;
            const bool ok = ts + r < t1;
            const T* ke = reinterpret_cast<const T*>(&rk[i]);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                // padded rows must add nothing: phi(0) = 1, so mask after phi
                sK[(c * EPC + e) * LDT + r] = ok ? static_cast<T>(phi<FM, T>(to_f32(ke[e]))) : static_cast<T>(0.f);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, c = n % CV;
            const bool ok = ts + r < t1;
            const T* ve = reinterpret_cast<const T*>(&rv[i]);
#pragma unroll
            for (int e = 0; e < EPC; ++e) sV[(c * EPC + e) * LDT + r] = ok ? ve[e] : static_cast<T>(0.f);
        }
        __syncthreads();
        if (it + 1 < ntile) load_tile(ts + TT);  // in flight during the MFMA below
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int col = ks * 32 + grp * 8;
            Frag<T> a[NI];
#pragma unroll
            for (int ii = 0; ii < NI; ++ii)
                a[ii] = *reinterpret_cast<const Frag<T>*>(&sK[((wi * NI + ii) * 16 + m) * LDT + col]);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const Frag<T> b = *reinterpret_cast<const Frag<T>*>(&sV[((wj * NJ + jj) * 16 + m) * LDT + col]);
#pragma unroll
                for (int ii = 0; ii < NI; ++ii) acc[ii][jj] = mma(a[ii], b, acc[ii][jj]);
            }
        }
        if (tid < DK) {
            const T* row = &sK[tid * LDT];
#pragma unroll
            for (int c = 0; c < TT / EPC; ++c) {
                const uint4 x = *reinterpret_cast<const uint4*>(row + c * EPC);
                const T* xe = reinterpret_cast<const T*>(&x);
#pragma unroll
                for (int e = 0; e < EPC; ++e) zacc += to_f32(xe[e]);
            }
        }
    }

    float* oS;
    float* oz;
    if (P == 1) {
        oS = stS + bh * DK * DV;
        oz = stz + bh * DK;
    } else {
        oS = part + (bh * P + p) * (int64_t)(DK * DV + DK);
        oz = oS + DK * DV;
    }
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
        const int i0 = (wi * NI + ii) * 16 + 4 * grp;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) oS[(i0 + r) * DV + (wj * NJ + jj) * 16 + m] = acc[ii][jj][r];
    }
    if (tid < DK) oz[tid] = zacc;
}

// Steps 1-3 for 16-bit inputs at D = 64: every wave streams its own 32-token
// steps of the workgroup's slice (steps w, w + 4, ...) with two steps of loads
// in flight, and needs no workgroup barrier until the end. Per step a lane
// loads 16 bytes of 4 rows of K and of V (8 consecutive rows per wave
// instruction), applies phi to K in fp32, and stores both tiles row-major in
// the wave's own LDS area; transpose reads then give the MFMA operands
// directly: A = phi(K)^T (feature x token) and B = [V | 1] (token x feature).
// The wave accumulates the whole 64 x 64 S and z; the four waves' sums are
// added in a fixed order at the end.
struct StateW64 {
    static constexpr int kStep = 32;  // tokens per wave step
    static constexpr int kStages = 2; // steps of loads in flight per wave
    static constexpr int kLDR = 72;   // LDS row stride (elements): 144 B rows
    static constexpr int kTile = kStep * kLDR;
};

template <typename T, int FM>
__global__ __launch_bounds__(kThreads, 2) void fwd_state_w64_kernel(
    const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ stS,
    float* __restrict__ stz, float* __restrict__ part, int64_t T_, const Layouts lay, int P,
    int64_t L) {
    constexpr int D = 64, NB = 4, E = D * D + D;
    constexpr int STEP = StateW64::kStep, LDR = StateW64::kLDR, TILE = StateW64::kTile;
    constexpr int kTileBytes = kWaves * 2 * TILE * (int)sizeof(T);
    constexpr int kRedBytes = 2 * E * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) unsigned char smem[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int c = lane & 7, rg = lane >> 3;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const int nsteps = (int)(t1 > t0 ? (t1 - t0 + STEP - 1) / STEP : 0);
    T* sK = reinterpret_cast<T*>(smem) + wave * 2 * TILE;
    T* sV = sK + TILE;
    f32x4 acc[NB][NB + 1];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j <= NB; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<T>(1.f);

    struct Stage {
        uint4 k[4], v[4];
    };
    // Rows are counted from t0; rows past the slice end load as zeros and
    // phi(k) is masked for them. Steps go in rotated order, two per wave and
    // turn, with no early exit (an exit makes the compiler wait for every
    // load in flight where the paths join).
    const HeadBuf bk = slice_buf(k, lay.k, bh, D, t0, t1), bv = slice_buf(v, lay.v, bh, D, t0, t1);
    constexpr int NS = StateW64::kStages;
    const Rotation rot(nsteps, NS * kWaves, wid);
    auto issue = [&](Stage& st, int step) {
        const int ps = rot(step);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = (int64_t)ps * STEP + rg + 8 * r;
            st.k[r] = buf_load16<kNonTemporal>(bk, buf_off<T>(row, lay.k.rs, 8 * c));
            st.v[r] = buf_load16<kNonTemporal>(bv, buf_off<T>(row, lay.v.rs, 8 * c));
        }
    };
    // phi on K (fp32, rounded to T), padded rows zeroed after phi, row-major to LDS
    auto consume = [&](const Stage& st, int step) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rg + 8 * r;
            const bool ok = (int64_t)rot(step) * STEP + row < t1 - t0;
            const uint4 kr = st.k[r];
            *reinterpret_cast<u32x4*>(&sK[row * LDR + 8 * c]) = keep_or_zero(phi8<FM, T>(u32x4{kr.x, kr.y, kr.z, kr.w}), ok);
            *reinterpret_cast<uint4*>(&sV[row * LDR + 8 * c]) = st.v[r];
        }
    };
    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    auto mma_step = [&]() {
        wave_lds_sync();
        Frag<T> a[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            a[b] = join_frag<T>(lds_read_tr(&sK[rA * LDR + 16 * b + cA]),
                                lds_read_tr(&sK[(rA + 4) * LDR + 16 * b + cA]));
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const Frag<T> bv = join_frag<T>(lds_read_tr(&sV[rA * LDR + 16 * j + cA]),
                                            lds_read_tr(&sV[(rA + 4) * LDR + 16 * j + cA]));
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b][j] = mma(a[b], bv, acc[b][j]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][NB] = mma(a[b], ones, acc[b][NB]);
        wave_lds_sync();
    };

    // (written out for two stages: a loop over a stage array compiles to
    // register copies and shallower waits here)
    static_assert(NS == 2, "the loop below is written for two stages");
    if (nsteps > 0) {
        Stage s0, s1;
        issue(s0, wave);
        sched_fence();
        issue(s1, wave + kWaves);
        sched_fence();
        for (int st = wave; st < rot.npad; st += 2 * kWaves) {
            consume(s0, st);
            sched_fence();
            issue(s0, st + 2 * kWaves);
            sched_fence();
            mma_step();
            consume(s1, st + kWaves);
            sched_fence();
            issue(s1, st + 3 * kWaves);
            sched_fence();
            mma_step();
        }
    }

    // fixed-order sum of the four waves: (w0 + w2) + (w1 + w3)
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    if (wave >= 2) {
        float* dst = red + (wave - 2) * E;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * b + 4 * grp + r) * D + 16 * j + m] = acc[b][j][r];
            if (m == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[D * D + 16 * b + 4 * grp + r] = acc[b][NB][r];
        }
    }
    __syncthreads();
    if (wave < 2) {
        float* dst = red + wave * E;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int idx = (16 * b + 4 * grp + r) * D + 16 * j + m;
                    dst[idx] = acc[b][j][r] + dst[idx];
                }
            if (m == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int idx = D * D + 16 * b + 4 * grp + r;
                    dst[idx] = acc[b][NB][r] + dst[idx];
                }
        }
    }
    __syncthreads();
    float* oS;
    float* oz;
    if (P == 1) {
        oS = stS + bh * D * D;
        oz = stz + bh * D;
    } else {
        oS = part + (bh * P + p) * (int64_t)E;
        oz = oS + D * D;
    }
    for (int i = tid; i < E; i += kThreads) {
        const float x = red[i] + red[E + i];
        if (i < D * D)
            oS[i] = x;
        else
            oz[i - D * D] = x;
    }
}

// Steps 1-3 for 16-bit inputs, any (DK, DV): 64-token tiles of K and V
// staged row-major in LDS, double-buffered with one barrier per tile, the
// next two tiles' loads in flight. Each thread loads the tile's 16-byte
// chunks in order (chunk n: row n / chunks-per-row) and writes them to LDS as
// they are, K through phi; MFMA operands come from transposed LDS reads
// (A = phi(K)^T: feature x token, B = V: token x feature). The four waves
// split S two by two (wave w: row half w % 2, column half w / 2); the waves of
// column half 0 also multiply by a block of ones, which gives z from the same
// rounded phi(k). Rows past the slice end read as zeros (slice descriptors)
// and are zeroed after phi.
template <int DK, int DV>
struct StateTile {
    static constexpr int kTile = 64;     // tokens per tile
    // LDS row strides (elements): D + 16 puts four consecutive rows at least
    // 8 banks apart, so a transposed read of 4 rows x 32 bytes hits distinct banks
    static constexpr int kLDK = DK + 16;
    static constexpr int kLDV = DV + 16;
    static constexpr int kStages = 2;    // tiles of loads in flight
    static constexpr int kNI = DK / 32;  // 16-row blocks of S per wave
    static constexpr int kNJ = DV / 32;  // 16-column blocks of S per wave
};

template <typename T, int DK, int DV, int FM>
__global__ __launch_bounds__(kThreads, 2) void fwd_state_tile_kernel(
    const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ stS,
    float* __restrict__ stz, float* __restrict__ part, int64_t T_, const Layouts lay, int P,
    int64_t L) {
    using Sh = StateTile<DK, DV>;
    constexpr int TT = Sh::kTile, LDK = Sh::kLDK, LDV = Sh::kLDV, NI = Sh::kNI, NJ = Sh::kNJ;
    constexpr int CK = DK * (int)sizeof(T) / 16, CV = DV * (int)sizeof(T) / 16;  // chunks per row
    constexpr int NCK = TT * CK / kThreads, NCV = TT * CV / kThreads;           // per thread per tile
    constexpr int BUFK = TT * LDK, BUFV = TT * LDV;
    static_assert(sizeof(T) == 2, "transposed LDS reads take 16-bit elements");
    static_assert(NCK * kThreads == TT * CK && NCV * kThreads == TT * CV, "tile must split evenly");
    static_assert(Sh::kStages == 2, "the loop below is written for two stages");
    __shared__ __attribute__((aligned(16))) T sK[2 * BUFK];
    __shared__ __attribute__((aligned(16))) T sV[2 * BUFV];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int wi = wave & 1, wj = wave >> 1;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const int64_t len = t1 - t0;
    const int ntiles = (int)(len > 0 ? (len + TT - 1) / TT : 0);
    const Layout lk = lay.k, lv = lay.v;

    f32x4 acc[NI][NJ + 1];  // column NJ: z (waves of column half 0)
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int j = 0; j <= NJ; ++j) acc[ii][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<T>(1.f);

    struct Stage {
        u32x4 k[NCK], v[NCV];
    };
    const HeadBuf bk = slice_buf(k, lk, bh, DK, t0, t1), bv = slice_buf(v, lv, bh, DV, t0, t1);
    const Rotation rot(ntiles, Sh::kStages, wid);
    auto issue = [&](Stage& st, int tile) {
        const int row0 = rot(tile) * TT;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, c = n % CK;
            st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, buf_off<T>((int64_t)row0 + r, lk.rs, 8 * c), 0,
                                                            kNonTemporal);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, c = n % CV;
            st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(bv.rsrc, buf_off<T>((int64_t)row0 + r, lv.rs, 8 * c), 0,
                                                            kNonTemporal);
        }
    };
    auto consume = [&](const Stage& st, int tile, int buf) {
        const int64_t row0 = (int64_t)rot(tile) * TT;
        T* dK = sK + buf * BUFK;
        T* dV = sV + buf * BUFV;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, c = n % CK;
            const bool ok = row0 + r < len;
            *reinterpret_cast<u32x4*>(&dK[r * LDK + 8 * c]) = keep_or_zero(phi8<FM, T>(st.k[i]), ok);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, c = n % CV;
            *reinterpret_cast<u32x4*>(&dV[r * LDV + 8 * c]) = st.v[i];
        }
    };
    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    auto mma_tile = [&](int buf) {
        const T* K_ = sK + buf * BUFK;
        const T* V_ = sV + buf * BUFV;
#pragma unroll
        for (int ks = 0; ks < TT / 32; ++ks) {
            const int rb = 32 * ks + rA;
            Frag<T> a[NI];
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) {
                const int col = 16 * (wi * NI + ii) + cA;
                a[ii] = join_frag<T>(lds_read_tr(&K_[rb * LDK + col]), lds_read_tr(&K_[(rb + 4) * LDK + col]));
            }
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const int col = 16 * (wj * NJ + jj) + cA;
                const Frag<T> b = join_frag<T>(lds_read_tr(&V_[rb * LDV + col]), lds_read_tr(&V_[(rb + 4) * LDV + col]));
#pragma unroll
                for (int ii = 0; ii < NI; ++ii) acc[ii][jj] = mma(a[ii], b, acc[ii][jj]);
            }
            if (wj == 0) {
#pragma unroll
                for (int ii = 0; ii < NI; ++ii) acc[ii][NJ] = mma(a[ii], ones, acc[ii][NJ]);
            }
        }
    };

    if (ntiles > 0) {
        Stage s0, s1;
        issue(s0, 0);
        sched_fence();
        issue(s1, 1);
        sched_fence();
        for (int it = 0; it < rot.npad; it += 2) {
            consume(s0, it, 0);
            sched_fence();
            issue(s0, it + 2);
            sched_fence();
            __syncthreads();
            mma_tile(0);
            consume(s1, it + 1, 1);
            sched_fence();
            issue(s1, it + 3);
            sched_fence();
            __syncthreads();
            mma_tile(1);
        }
    }

    float* oS;
    float* oz;
    if (P == 1) {
        oS = stS + bh * DK * DV;
        oz = stz + bh * DK;
    } else {
        oS = part + (bh * P + p) * (int64_t)(DK * DV + DK);
        oz = oS + DK * DV;
    }
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
        const int i0 = (wi * NI + ii) * 16 + 4 * grp;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) oS[(i0 + r) * DV + (wj * NJ + jj) * 16 + m] = acc[ii][jj][r];
        if (wj == 0 && m == 0)
#pragma unroll
            for (int r = 0; r < 4; ++r) oz[i0 + r] = acc[ii][NJ][r];
    }
}

// ---------------------------------------------------------------------------
// Shared shape of the streaming kernels (output, bwd Q side, bwd K/V side).
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
struct StreamShape {
    static constexpr int kFK = DK / 4;    // Q/K-side features per lane (one quarter row)
    static constexpr int kFV = DV / 4;    // V/O-side features per lane
    static constexpr int kNBK = DK / 16;  // 16-row blocks over DK
    static constexpr int kNBV = DV / 16;  // 16-row blocks over DV
    static constexpr int kKSK = DK / 32;  // 32-long contraction steps over DK
    static constexpr int kKSV = DV / 32;  // 32-long contraction steps over DV
    static constexpr bool kSmall = sizeof(T) == 2 && DK <= 64 && DV <= 64;
    static constexpr int kU = kSmall ? 2 : 1;  // 16-token blocks per wave
    // 16-bit DK = DV = 128: eight waves share one copy of the (larger) fragments
    static constexpr int kWaves = (sizeof(T) == 2 && DK == 128 && DV == 128) ? 8 : ::la::kWaves;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kG = kWaves * kU * 16;  // tokens per workgroup iteration
    static constexpr int kStages = 2;            // blocks of loads in flight per wave
    // workgroups per CU the register budget is set for: 16-bit heads up to 64,
    // four (128 registers per lane); wider 16-bit heads, two for the output
    // kernel (128 registers) and one for the K/V kernel (256)
    static constexpr int kOutMinBlocks = (sizeof(T) == 2) ? (kSmall ? 4 : 2) : 1;
    static constexpr int kKvMinBlocks = kSmall ? 4 : 1;
    // The state is staged in LDS for the fragment builds except at
    // DK = DV = 128, where the staging area would halve the occupancy.
    static constexpr bool kStaged = !(DK == 128 && DV == 128);
};

// Fragment of an A operand built from an fp32 matrix M (rows LD floats apart)
// whose A rows run over DR indices and whose contraction runs over DC:
//   rows m of the 16-row block b stand for index (DR/4)*(m/4) + 4b + m%4,
//   the lane group's 8 contraction values stand for (DC/4)*g + 8s + e.
// If kTransposeSource, element = M[contraction][row] else M[row][contraction].
template <typename T, int DR, int DC, bool kTransposeSource, int LD>
__device__ __forceinline__ Frag<T> build_frag(const float* __restrict__ M, int b, int s, int m, int g,
                                              float scale) {
    constexpr int FR = DR / 4, FC = DC / 4;
    const int row = FR * (m >> 2) + 4 * b + (m & 3);
    const int k0 = FC * g + 8 * s;
    Frag<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = kTransposeSource ? M[(k0 + e) * LD + row] : M[row * LD + k0 + e];
        f[e] = static_cast<T>(x * scale);
    }
    return f;
}

// Fragment whose every row is the vector z: z[(DC/4)*g + 8s + e] (the
// contraction runs over DC).
template <typename T, int DC>
__device__ __forceinline__ Frag<T> build_zfrag(const float* __restrict__ z, int s, int g, float scale) {
    constexpr int F = DC / 4;
    Frag<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<T>(z[F * g + 8 * s + e] * scale);
    return f;
}

// Writes the workgroup's operand fragments to sA[f * 64 + lane], f < NF; wave w
// builds fragments w, w + 4, ... with all their loads issued together. make(f)
// returns fragment f (f is clamped, so its loads are unconditional).
template <typename T, int NF, int NW = kWaves, typename Make>
__device__ __forceinline__ void build_frags(Frag<T>* sA, Make make) {
    constexpr int PER = (NF + NW - 1) / NW;
    const int lane = threadIdx.x & 63, wave = wave_index();
    Frag<T> fr[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) fr[i] = make(min(wave + NW * i, NF - 1));
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (wave + NW * i < NF) sA[(wave + NW * i) * 64 + lane] = fr[i];
}

// ---------------------------------------------------------------------------
// Step 4: output.
// ---------------------------------------------------------------------------
// The NQ workgroups of head bh take its rounds of NW blocks (NW x 16 U tokens)
// in turn: workgroup ch takes rounds ch, ch + NQ, ..., so the workgroups of a
// head stream neighbouring tokens at any moment (B8-H16-T16384-D64 f16: 92.4 ->
// 85.9 us against contiguous, rotated chunks of LQ tokens). Per
// 16-token block a lane loads a quarter row of Q (DK/4 features), applies phi,
// and the wave computes O^T = S^T phi(Q)^T (rows permuted so each lane ends
// with DV/4 contiguous outputs of its token) and den = z . phi(q) from one more
// MFMA block whose rows are all z.
template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__((StreamShape<T, DK, DV>::kThreads), (StreamShape<T, DK, DV>::kOutMinBlocks)) void fwd_output_kernel(
    const T* __restrict__ q, const float* __restrict__ stS, const float* __restrict__ stz,
    T* __restrict__ o, int64_t T_, const Layouts lay, int NQ, int64_t LQ, float eps) {
    using Sh = StreamShape<T, DK, DV>;
    const Layout lk = lay.q, lv = lay.o;
    constexpr int FK = Sh::kFK, FV = Sh::kFV, NB = Sh::kNBV, KS = Sh::kKSK, U = Sh::kU, NW = Sh::kWaves,
                  NT = Sh::kThreads;
    constexpr int NFS = NB * KS;             // S fragments
    constexpr int NFR = NFS + (SIMPLE ? 0 : KS);  // + z fragments
    constexpr int LDR = DV + 16 / (int)sizeof(T);
    // The state is staged in LDS (sharing the store staging area, which the
    // loop alone uses) and the fragments are built from there.
    constexpr bool kStaged = Sh::kStaged;
    constexpr int kStoreBytes = NW * 16 * LDR * (int)sizeof(T);
    constexpr int kStBytes = kStaged ? StagedState<DK, DV>::kFloats * 4 : 0;
    __shared__ Frag<T> sA[NFR * 64];
    __shared__ __attribute__((aligned(16))) unsigned char sraw[kStoreBytes > kStBytes ? kStoreBytes : kStBytes];
    __shared__ float red[3 * NW];
    T* stage = reinterpret_cast<T*>(sraw);

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / NQ;
    const int ch = wid % NQ;
    (void)LQ;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const float* S = stS + bh * DK * DV;
    const float* z = stz + bh * DK;

    // The first two turns' loads are issued before the prologue, which they
    // overlap. Wave w takes block w of each of the workgroup's rounds, with the
    // loads of its next two blocks in flight while it computes one, two per
    // turn with no early exit; the descriptors cover the whole head, rows past
    // its end (the last round's tail, the padded turns) load as zeros and their
    // stores are dropped.
    constexpr int BT = 16 * U;
    const HeadBuf bq = slice_buf(q, lk, bh, DK, 0, T_), bo = slice_buf(o, lv, bh, DV, 0, T_);
    constexpr int NS = Sh::kStages;
    // rounds of NW blocks of the head, dealt to its NQ workgroups in turn
    constexpr int RT = NW * BT;
    const int64_t nrounds = (T_ + RT - 1) / RT;
    const int nmine = (int)(nrounds > ch ? (nrounds - ch + NQ - 1) / NQ : 0);
    const int nblk = nmine * NW;
    const int npad = (nblk + NS * NW - 1) / (NS * NW) * (NS * NW);
    auto row_of = [&](int blk) {
        return (blk < nblk ? ((int64_t)ch + (int64_t)NQ * (blk / NW)) * RT : T_) + (int64_t)BT * (blk % NW);
    };
    T* stg = stage + wave * 16 * LDR;
    auto issue = [&](Row<T, FK> (&b)[U], int blk) {
        const int64_t bs = row_of(blk);
#pragma unroll
        for (int u = 0; u < U; ++u) load_row_buf<T, FK>(b[u], bq, bs + 16 * u + m, lk.rs, FK * grp);
    };
    Row<T, FK> stg_q[NS][U];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        issue(stg_q[i], wave + i * NW);
        sched_fence();
    }
    int sS = 0, sz = 0;
    if constexpr (kStaged) {
        constexpr int LD = StagedState<DK, DV>::kLD;
        float* sSt = reinterpret_cast<float*>(sraw);
        const StagedState<DK, DV> st = stage_state<DK, DV, NT>(S, z, sSt, red);
        if constexpr (Elt<T>::kScaled) {
            sS = scale_exp(st.max_m);
            sz = scale_exp(st.max_z);
        }
        const float fS = ldexpf(1.f, sS), fz = ldexpf(1.f, sz);
        build_frags<T, NFR, NW>(sA, [&](int f) {
            return f < NFS ? build_frag<T, DV, DK, true, LD>(sSt, f / KS, f % KS, m, grp, fS)
                           : build_zfrag<T, DK>(sSt + DK * LD, max(f - NFS, 0), grp, fz);
        });
    } else {
        if constexpr (Elt<T>::kScaled) {
            float mz, zsum;
            sS = scale_exp(block_absmax_matrix<DK * DV, NT>(S, red));
            block_vector_stats<DK, NT>(z, red, mz, zsum);
            sz = scale_exp(mz);
        }
        const float fS = ldexpf(1.f, sS), fz = ldexpf(1.f, sz);
        build_frags<T, NFR, NW>(sA, [&](int f) {
            return f < NFS ? build_frag<T, DV, DK, true, DV>(S, f / KS, f % KS, m, grp, fS)
                           : build_zfrag<T, DK>(z, max(f - NFS, 0), grp, fz);
        });
    }
    __syncthreads();
    const float uS = ldexpf(1.f, -sS), uz = ldexpf(1.f, -sz);

    auto body = [&](Row<T, FK> (&qr)[U], int blk) {
        Frag<T> bq[U][KS];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if constexpr (sizeof(T) == 2) {
                    u32x4 raw;
                    __builtin_memcpy(&raw, &qr[u].e[8 * s], sizeof(raw));
                    bq[u][s] = __builtin_bit_cast(Frag<T>, phi8<FM, T>(raw));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) bq[u][s][e] = phi<FM, T>(qr[u].e[8 * s + e]);
                }
            }
        sched_fence();
        issue(qr, blk + NS * NW);
        sched_fence();
        f32x4 acc[U][NB], accd[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            accd[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[u][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const Frag<T> a = sA[(b * KS + s) * 64 + lane];
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u][b] = mma(a, bq[u][s], acc[u][b]);
            }
        if constexpr (!SIMPLE) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const Frag<T> a = sA[(NFS + s) * 64 + lane];
#pragma unroll
                for (int u = 0; u < U; ++u) accd[u] = mma(a, bq[u][s], accd[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Row<T, FV> out;
            if constexpr (SIMPLE) {
                const float f = uS * eps;  // simple_la: eps carries the query scale
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) out.e[4 * b + r] = static_cast<T>(acc[u][b][r] * f);
            } else {
                // one division per token: O = num 2^-sS / (den 2^-sz + eps)
                const float inv = uS / (accd[u][0] * uz + eps);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) out.e[4 * b + r] = static_cast<T>(acc[u][b][r] * inv);
            }
            store_tile_rows<T, DV>(stg, out, bo, row_of(blk) + 16 * u, lv.rs);
        }
    };
    for (int blk = wave; blk < npad; blk += NS * NW) {
#pragma unroll
        for (int i = 0; i < NS; ++i) body(stg_q[i], blk + i * NW);
    }
}

// ---------------------------------------------------------------------------
// Steps 5-6: backward, Q side.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
struct BwdQShape {
    static constexpr int kU = StreamShape<T, DK, DV>::kU;          // 16-token blocks per wave
    static constexpr int kG = kWaves * kU * 16;                     // tokens per iteration
    static constexpr int kLDT = kG + 16 / (int)sizeof(T);           // LDS row stride, +16 B
};

// One workgroup walks tokens [p LB, min((p+1) LB, T)) of head bh. Per token:
//   u = S dO_t (MFMA, S rows permuted as in the output kernel), den = z . phi(q)
//   (MFMA), r = phi(q) . u (lane partial + two cross-lane adds),
//   c = -r / den^2, dphi(q) = u / den + c z, dQ = dphi(q) * phi'(q),
//   dz += c phi(q) (fp32, per lane), and phi(q), w = dO 2^sw / den are written
//   to LDS transposed; then the workgroup accumulates dS += phi(Q)^T w on MFMA,
//   the four waves splitting dS two by two as in the state kernel.
// w carries the power of two 2^sw ~ sum(z) (f16 only) so that dO / den, about
// 1e-6 for long sequences, does not fall into f16 subnormals; dS is unscaled
// in fp32 when written.
template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ dout, const float* __restrict__ stS,
    const float* __restrict__ stz, T* __restrict__ dq, float* __restrict__ part,
    float* __restrict__ dS_out, float* __restrict__ dz_out, int64_t T_, const Layouts lay, int PB,
    int64_t LB, float eps) {
    using Sh = StreamShape<T, DK, DV>;
    const Layout lk = lay.q, lv = lay.dout, lg = lay.dq;
    using Bq = BwdQShape<T, DK, DV>;
    constexpr int FK = Sh::kFK, FV = Sh::kFV, NBK = Sh::kNBK, KSK = Sh::kKSK, KSV = Sh::kKSV;
    constexpr int U = Bq::kU, G = Bq::kG, LDT = Bq::kLDT;
    constexpr int NI = DK / 32, NJ = DV / 32;  // dS blocks per wave
    constexpr int NFS = NBK * KSV;
    constexpr int NFR = NFS + (SIMPLE ? 0 : KSK);
    __shared__ Frag<T> sA[NFR * 64];
    __shared__ __attribute__((aligned(16))) T sQ[DK * LDT];
    __shared__ __attribute__((aligned(16))) T sW[DV * LDT];
    __shared__ float sdz[kWaves][DK];
    __shared__ float red[4];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / PB;
    const int p = wid % PB;
    const int64_t t0 = (int64_t)p * LB;
    const int64_t t1 = min(t0 + LB, T_);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int wi = wave & 1, wj = wave >> 1;
    const float* S = stS + bh * DK * DV;
    const float* z = stz + bh * DK;

    int sS = 0, sz = 0, sw = 0;
    if constexpr (Elt<T>::kScaled) {
        float mz, zsum;
        sS = scale_exp(block_absmax_matrix<DK * DV>(S, red));
        block_vector_stats<DK>(z, red, mz, zsum);
        sz = scale_exp(mz);
        if constexpr (!SIMPLE) {
            if (zsum > 0.f && isfinite(zsum)) {
                int e;
                frexpf(zsum, &e);
                sw = min(max(e - 1, -120), 120);  // 2^sw <= sum(z) < 2^(sw+1)
            }
        }
    }
    {
        const float fS = ldexpf(1.f, sS), fz = ldexpf(1.f, sz);
        // captures by value: by reference, the choice between S and z
        // became a dynamically indexed load from a private copy of the captures
        build_frags<T, NFR>(sA, [=](int f) {
            return f < NFS ? build_frag<T, DK, DV, false, DV>(S, f / KSV, f % KSV, m, grp, fS)
                           : build_zfrag<T, DK>(z, max(f - NFS, 0), grp, fz);
        });
    }
    float zl[FK];
#pragma unroll
    for (int o = 0; o < FK; ++o) zl[o] = SIMPLE ? 0.f : z[FK * grp + o];
    __syncthreads();
    const float uS = ldexpf(1.f, -sS), uz = ldexpf(1.f, -sz), fw = ldexpf(1.f, sw);

    f32x4 dsacc[NI][NJ];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) dsacc[ii][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dzacc[FK];
#pragma unroll
    for (int o = 0; o < FK; ++o) dzacc[o] = 0.f;

    const T* qh = q + head_offset(lk, bh);
    const T* dh = dout + head_offset(lv, bh);
    T* gh = dq + head_offset(lg, bh);
    for (int64_t base = t0; base < t1; base += G) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = base + (wave * U + u) * 16 + m;
            const bool valid = t < t1;
            Row<T, FK> qr;
            Row<T, FV> dr;
            const int64_t tc = min(t, t1 - 1);  // rows past t1 are masked below
            load_row<T, FK>(qr, qh + tc * lk.rs + FK * grp);
            load_row<T, FV>(dr, dh + tc * lv.rs + FV * grp);
            float qt[FK];
#pragma unroll
            for (int o = 0; o < FK; ++o) qt[o] = phi<FM, T>(to_f32(qr.e[o]));
            Frag<T> bq[KSK], bd[KSV];
#pragma unroll
            for (int s = 0; s < KSK; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) bq[s][e] = static_cast<T>(qt[8 * s + e]);
#pragma unroll
            for (int s = 0; s < KSV; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) bd[s][e] = dr.e[8 * s + e];
            f32x4 au[NBK];
#pragma unroll
            for (int b = 0; b < NBK; ++b) au[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int s = 0; s < KSV; ++s) au[b] = mma(sA[(b * KSV + s) * 64 + lane], bd[s], au[b]);
            float dqt[FK], wv[FV];
            if constexpr (SIMPLE) {
#pragma unroll
                for (int b = 0; b < NBK; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dqt[4 * b + r] = au[b][r] * (uS * eps);  // eps: the query scale
#pragma unroll
                for (int o = 0; o < FV; ++o) wv[o] = to_f32(dr.e[o]);
            } else {
                f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSK; ++s) ad = mma(sA[(NFS + s) * 64 + lane], bq[s], ad);
                const float den = ad[0] * uz + eps;
                float uu[FK];
                float rr = 0.f;
#pragma unroll
                for (int b = 0; b < NBK; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uu[4 * b + r] = au[b][r] * uS;
                        rr += qt[4 * b + r] * uu[4 * b + r];
                    }
                rr += __shfl_xor(rr, 16);
                rr += __shfl_xor(rr, 32);
                const float inv = 1.f / den;
                const float c = -(rr * inv) * inv;
                const float ws = fw * inv;
#pragma unroll
                for (int o = 0; o < FK; ++o) {
                    dqt[o] = uu[o] * inv + c * zl[o];
                    if (valid) dzacc[o] += c * qt[o];
                }
#pragma unroll
                for (int o = 0; o < FV; ++o) wv[o] = to_f32(dr.e[o]) * ws;
            }
            if (valid) {
                float out[FK];
#pragma unroll
                for (int o = 0; o < FK; ++o) out[o] = dqt[o] * dphi_of<FM>(qt[o]);
                store_row<T, FK>(gh + t * lg.rs + FK * grp, out);
            }
            const int col = (wave * U + u) * 16 + m;
#pragma unroll
            for (int o = 0; o < FK; ++o)
                sQ[(FK * grp + o) * LDT + col] = valid ? static_cast<T>(qt[o]) : static_cast<T>(0.f);
#pragma unroll
            for (int o = 0; o < FV; ++o)
                sW[(FV * grp + o) * LDT + col] = valid ? static_cast<T>(wv[o]) : static_cast<T>(0.f);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < G / 32; ++ks) {
            const int col = ks * 32 + grp * 8;
            Frag<T> a[NI];
#pragma unroll
            for (int ii = 0; ii < NI; ++ii)
                a[ii] = *reinterpret_cast<const Frag<T>*>(&sQ[((wi * NI + ii) * 16 + m) * LDT + col]);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const Frag<T> bw = *reinterpret_cast<const Frag<T>*>(&sW[((wj * NJ + jj) * 16 + m) * LDT + col]);
#pragma unroll
                for (int ii = 0; ii < NI; ++ii) dsacc[ii][jj] = mma(a[ii], bw, dsacc[ii][jj]);
            }
        }
        __syncthreads();
    }

    float* oS;
    float* oz;
    if (PB == 1) {
        oS = dS_out + bh * DK * DV;
        oz = dz_out + bh * DK;
    } else {
        oS = part + (bh * PB + p) * (int64_t)(DK * DV + DK);
        oz = oS + DK * DV;
    }
    const float uw = ldexpf(1.f, -sw) * (SIMPLE ? eps : 1.f);  // simple_la: times the query scale
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
        const int i0 = (wi * NI + ii) * 16 + 4 * grp;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) oS[(i0 + r) * DV + (wj * NJ + jj) * 16 + m] = dsacc[ii][jj][r] * uw;
    }
    // dz: sum over the 16 token lanes of each lane group, then over waves, in a
    // fixed pattern.
#pragma unroll
    for (int o = 0; o < FK; ++o) {
        float x = dzacc[o];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if (m == 0) sdz[wave][FK * grp + o] = x;
    }
    __syncthreads();
    for (int i = tid; i < DK; i += kThreads) oz[i] = (sdz[0][i] + sdz[1][i]) + (sdz[2][i] + sdz[3][i]);
}

// Steps 5-6 for 16-bit inputs at D = 64, per wave: each wave walks its own
// 16-token steps (w, w + 4, ...) with two steps of Q and dO loads in flight.
// The loop takes two steps per turn with no early exit (an exit makes the
// compiler wait for every load in flight where the paths join): the slice's
// buffer descriptors read steps past the slice end as zeros, which add
// nothing, and drop their dQ stores.
// Per step it computes u = S dO_t, den and dQ as the workgroup kernel above.
// For the reduction over tokens it writes A_t = phi(q_t) 2^sw / den_t and the
// raw dO_t row-major into its own LDS area (one area per step of a turn),
// plus one more column beta_t = -r_t / den_t next to dO; after the turn's two
// steps it reads both back transposed (4 tokens of each step per lane) as
// the operands of 16x16x32 MFMAs over the turn's 32 tokens:
//   sum_t A_t dO_t^T = 2^sw dS   and   sum_t A_t beta_t = 2^sw dz
// (c_t phi(q_t) = (-r_t / den_t)(phi(q_t) / den_t)), so dS and dz share one
// operand and need no per-element work beyond the scaling of phi(q). Each
// wave holds its own 64 x 65 sums; waves are combined in a fixed order.
struct BwdQW64 {
    static constexpr int kStep = 16;   // tokens per wave step
    static constexpr int kStages = 2;  // steps of loads in flight per wave
    static constexpr int kRound = kStep * kWaves;
};

template <typename T, bool SIMPLE, int FM>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_w64_kernel(
    const T* __restrict__ q, const T* __restrict__ dout, const float* __restrict__ stS,
    const float* __restrict__ stz, T* __restrict__ dq, float* __restrict__ part,
    float* __restrict__ dS_out, float* __restrict__ dz_out, int64_t T_, const Layouts lay, int PB,
    int64_t LB, float eps) {
    constexpr int D = 64, F = 16, NB = 4, KS = 2, STEP = BwdQW64::kStep, E = D * D + D;
    constexpr int LDR = 88;                   // 176-byte rows: 64 features + the beta column block
    constexpr int NJ = NB + (SIMPLE ? 0 : 1);  // dS column blocks (+ dz)
    constexpr int NFS = NB * KS;
    constexpr int NFR = NFS + (SIMPLE ? 0 : KS);
    constexpr int kFragBytes = NFR * 64 * 16;
    constexpr int LDO = D + 16 / (int)sizeof(T);  // dQ staging row stride
    // per wave: the A and dO tiles of the two steps of a turn, then the dQ staging
    constexpr int kTileBytes = kWaves * (4 * STEP * LDR + 16 * LDO) * (int)sizeof(T);
    constexpr int kLoopBytes = kFragBytes + kTileBytes;
    constexpr int kRedBytes = 2 * E * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLoopBytes > kRedBytes ? kLoopBytes : kRedBytes];
    __shared__ float red12[12];
    __shared__ __attribute__((aligned(16))) float sZ[D];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / PB;
    const int p = wid % PB;
    const int64_t t0 = (int64_t)p * LB;
    const int64_t t1 = min(t0 + LB, T_);
    const int nsteps = (int)(t1 > t0 ? (t1 - t0 + STEP - 1) / STEP : 0);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const float* S = stS + bh * D * D;
    const float* z = stz + bh * D;
    Frag<T>* sA = reinterpret_cast<Frag<T>*>(smem);
    T* const sQ0 = reinterpret_cast<T*>(smem + kFragBytes) + wave * (4 * STEP * LDR + 16 * LDO);
    T* const sO = sQ0 + 4 * STEP * LDR;

    // A stage holds the loaded words as they are; unpacked at the load, the
    // halves would be carried around the loop and unpacking them would wait
    // for the loads right after they are issued.
    struct Stage {
        u32x4 q[2], d[2];
    };
    // Rows past the slice end load as zeros (dO = 0 gives u = 0, r = 0,
    // beta = 0, so such rows add nothing to dS or dz) and their dQ stores are
    // dropped. Rows are counted from t0.
    const HeadBuf bq = slice_buf(q, lay.q, bh, D, t0, t1), bd = slice_buf(dout, lay.dout, bh, D, t0, t1),
                  bdq = slice_buf(dq, lay.dq, bh, D, t0, t1);
    const Rotation rot(nsteps, BwdQW64::kStages * kWaves, wid);
    auto issue = [&](Stage& st, int step) {
        const int64_t row = (int64_t)rot(step) * STEP + m;
        const int oq = buf_off<T>(row, lay.q.rs, F * grp), od = buf_off<T>(row, lay.dout.rs, F * grp);
        st.q[0] = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, oq, 0, 0);
        st.q[1] = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, oq + 16, 0, 0);
        st.d[0] = __builtin_amdgcn_raw_buffer_load_b128(bd.rsrc, od, 0, 0);
        st.d[1] = __builtin_amdgcn_raw_buffer_load_b128(bd.rsrc, od + 16, 0, 0);
    };
    // The first two steps' loads are issued before the prologue, which they
    // overlap (with no steps they read zeros and the loop below does not run).
    constexpr int kStages = BwdQW64::kStages;
    Stage stg[kStages];
#pragma unroll
    for (int i = 0; i < kStages; ++i) {
        issue(stg[i], wave + i * kWaves);
        sched_fence();
    }
    // The state is staged in the tile area (which the loop alone uses) and
    // the fragments are built from there.
    static_assert(StagedState<D, D>::kFloats * 4 <= kTileBytes, "state staging exceeds the tile area");
    int sS = 0, sz = 0, sw = 0;
    {
        constexpr int LD = StagedState<D, D>::kLD;
        float* sSt = reinterpret_cast<float*>(smem + kFragBytes);
        const StagedState<D, D> st = stage_state<D, D>(S, z, sSt, red12);
        if constexpr (Elt<T>::kScaled) {
            sS = scale_exp(st.max_m);
            sz = scale_exp(st.max_z);
            if constexpr (!SIMPLE) {
                if (st.sum_z > 0.f && isfinite(st.sum_z)) {
                    int e;
                    frexpf(st.sum_z, &e);
                    sw = min(max(e - 1, -120), 120);  // 2^sw <= sum(z) < 2^(sw+1)
                }
            }
        }
        const float fS = ldexpf(1.f, sS), fz = ldexpf(1.f, sz);
        build_frags<T, NFR>(sA, [&](int f) {
            return f < NFS ? build_frag<T, D, D, false, LD>(sSt, f / KS, f % KS, m, grp, fS)
                           : build_zfrag<T, D>(sSt + D * LD, max(f - NFS, 0), grp, fz);
        });
        for (int i = tid; i < D; i += kThreads) sZ[i] = sSt[D * LD + i];
    }
    __syncthreads();
    const float uS = ldexpf(1.f, -sS), uz = ldexpf(1.f, -sz), fw = ldexpf(1.f, sw);

    f32x4 dsacc[NB][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) dsacc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int rA = 4 * grp + (m >> 2), cA = 4 * (m & 3);
    // step h of a turn writes its A and dO tiles to half h
    auto body = [&](Stage& st, int step, int h) {
        T* const sQ = sQ0 + h * 2 * STEP * LDR;
        T* const sW = sQ + STEP * LDR;
        sched_fence();  // keeps this stage's unpacking out of the previous step
        Row<T, F> lq;
        __builtin_memcpy(lq.e, st.q, sizeof(lq));
        float qt[F], dph[F];
        Frag<T> bq[KS], bd[KS];
#pragma unroll
        for (int s = 0; s < F / 8; ++s) {
            u32x4 raw;
            __builtin_memcpy(&raw, &lq.e[8 * s], sizeof(raw));
            feature8<FM, T>(raw, &qt[8 * s], &dph[8 * s]);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if constexpr (!SIMPLE)
#pragma unroll
                for (int e = 0; e < 8; ++e) bq[s][e] = static_cast<T>(qt[8 * s + e]);
            bd[s] = __builtin_bit_cast(Frag<T>, st.d[s]);
        }
        // dO rows go to LDS as loaded
        u32x4* dw4 = reinterpret_cast<u32x4*>(&sW[m * LDR + F * grp]);
        dw4[0] = st.d[0];
        dw4[1] = st.d[1];
        f32x4 au[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            au[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) au[b] = mma(sA[(b * KS + s) * 64 + lane], bd[s], au[b]);
        }
        // The stage's registers are free once the u products have read dO, so
        // the next load lands in the same registers and nothing is copied (and
        // waited for) where the loop closes.
        sched_fence();
        issue(st, step + BwdQW64::kStages * kWaves);
        sched_fence();
        float dqt[F];
        float aq = 1.f;  // factor on phi(q) in the reduction operand
        if constexpr (SIMPLE) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) dqt[4 * b + r] = au[b][r] * (uS * eps);  // eps: the query scale
        } else {
            f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) ad = mma(sA[(NFS + s) * 64 + lane], bq[s], ad);
            const float inv = 1.f / (ad[0] * uz + eps);
            float rr = 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) rr += qt[4 * b + r] * au[b][r];
            rr += __shfl_xor(rr, 16);
            rr += __shfl_xor(rr, 32);
            const float beta = -(rr * uS) * inv;  // -r / den
            const float cc = beta * inv;          // -r / den^2
            const float ku = uS * inv;
            const float* zl = &sZ[F * grp];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) dqt[4 * b + r] = au[b][r] * ku + cc * zl[4 * b + r];
            aq = fw * inv;
            if (grp == 0) sW[m * LDR + D] = static_cast<T>(beta);
        }
        Row<T, F> rq;
#pragma unroll
        for (int o = 0; o < F; ++o) rq.e[o] = static_cast<T>(qt[o] * aq);
        uint4* dq4 = reinterpret_cast<uint4*>(&sQ[m * LDR + F * grp]);
        dq4[0] = reinterpret_cast<const uint4*>(rq.e)[0];
        dq4[1] = reinterpret_cast<const uint4*>(rq.e)[1];
        {
            Row<T, F> out;
#pragma unroll
            for (int o = 0; o < F; ++o) out.e[o] = static_cast<T>(dqt[o] * dph[o]);
            store_tile_rows<T, D>(sO, out, bdq, (int64_t)rot(step) * STEP, lay.dq.rs);
        }
    };
    // sum over the 32 tokens of a turn on 16x16x32 MFMAs: values 0..3 of a
    // lane are tokens 4 grp + (0..3) of the first step, values 4..7 the same
    // rows of the second, in both operands
    auto reduce_turn = [&]() {
        const T* q0 = sQ0;
        const T* w0 = sQ0 + STEP * LDR;
        const T* q1 = sQ0 + 2 * STEP * LDR;
        const T* w1 = q1 + STEP * LDR;
        wave_lds_sync();
        Frag<T> a[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            a[b] = join_frag<T>(lds_read_tr(&q0[rA * LDR + 16 * b + cA]), lds_read_tr(&q1[rA * LDR + 16 * b + cA]));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const Frag<T> bw = join_frag<T>(lds_read_tr(&w0[rA * LDR + 16 * j + cA]), lds_read_tr(&w1[rA * LDR + 16 * j + cA]));
#pragma unroll
            for (int b = 0; b < NB; ++b) dsacc[b][j] = mma(a[b], bw, dsacc[b][j]);
        }
        wave_lds_sync();
    };

    static_assert(BwdQW64::kStages == 2, "a turn is the two steps whose tiles reduce_turn reads");
    for (int st = wave; st < rot.npad; st += kStages * kWaves) {
#pragma unroll
        for (int i = 0; i < kStages; ++i) body(stg[i], st + i * kWaves, i);
        reduce_turn();
    }

    // fixed-order sum of the four waves: (w0 + w2) + (w1 + w3); column 0 of
    // the last block holds dz
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    const float uw = ldexpf(1.f, -sw) * (SIMPLE ? eps : 1.f);  // simple_la: times the query scale
    if (wave >= 2) {
        float* dst = red + (wave - 2) * E;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * b + 4 * grp + r) * D + 16 * j + m] = dsacc[b][j][r] * uw;
            if (m == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[D * D + 16 * b + 4 * grp + r] = SIMPLE ? 0.f : dsacc[b][NJ - 1][r] * uw;
        }
    }
    __syncthreads();
    if (wave < 2) {
        float* dst = red + wave * E;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int idx = (16 * b + 4 * grp + r) * D + 16 * j + m;
                    dst[idx] = dsacc[b][j][r] * uw + dst[idx];
                }
            if (m == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int idx = D * D + 16 * b + 4 * grp + r;
                    dst[idx] = (SIMPLE ? 0.f : dsacc[b][NJ - 1][r] * uw) + dst[idx];
                }
        }
    }
    __syncthreads();
    float* oS;
    float* oz;
    if (PB == 1) {
        oS = dS_out + bh * D * D;
        oz = dz_out + bh * D;
    } else {
        oS = part + (bh * PB + p) * (int64_t)E;
        oz = oS + D * D;
    }
    for (int i = tid; i < E; i += kThreads) {
        const float x = red[i] + red[E + i];
        if (i < D * D)
            oS[i] = x;
        else
            oz[i - D * D] = x;
    }
}

// Steps 5-6 for 16-bit inputs, one wave per 16 rows of dS: DK / 16 waves take
// the 16-token steps of a round of DK tokens, each with two rounds of Q and dO
// loads in flight. Per step a wave computes u = S dO_t, den and dQ (staged
// for full-line stores through its own rows of the round tile), then writes
// A_t = phi(q_t) 2^sw / den_t, the raw dO_t and beta_t = -r_t / den_t to the
// round tile. After a barrier, wave w reduces the whole round into its 16
// rows of
//   sum_t A_t dO_t^T = 2^sw dS   and   sum_t A_t beta_t = 2^sw dz
// with 16x16x32 MFMAs on transposed LDS reads; a second barrier frees the
// tile for the next round. Rounds go in rotated order with no early exit;
// rows past the slice end load as zeros and add nothing.
template <int DK, int DV>
struct BwdQTile {
    static constexpr int kWaves = DK / 16;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kStep = 16;                // tokens per wave step
    static constexpr int kRound = kStep * kWaves;   // tokens per round
    // tile row strides (elements), the beta block after DV columns of the W
    // tile; D + 16 puts four consecutive rows 8 or more banks apart, so a
    // transposed read of 4 rows x 32 bytes hits distinct banks
    static constexpr int kLDA = DK + 16;
    static constexpr int kLDW = DV + 16;
    static constexpr int kStages = 2;               // rounds of loads in flight
    static constexpr int kMinBlocks = DK == 128 ? 1 : 2;
};

template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__((BwdQTile<DK, DV>::kThreads), (BwdQTile<DK, DV>::kMinBlocks)) void bwd_dq_tile_kernel(
    const T* __restrict__ q, const T* __restrict__ dout, const float* __restrict__ stS,
    const float* __restrict__ stz, T* __restrict__ dq, float* __restrict__ part,
    float* __restrict__ dS_out, float* __restrict__ dz_out, int64_t T_, const Layouts lay, int PB,
    int64_t LB, float eps) {
    using Sh = BwdQTile<DK, DV>;
    constexpr int FK = DK / 4, FV = DV / 4, NBK = DK / 16, NBV = DV / 16, KSK = DK / 32, KSV = DV / 32;
    constexpr int E = DK * DV + DK;
    constexpr int NW = Sh::kWaves, NT = Sh::kThreads, STEP = Sh::kStep;
    constexpr int RT = Sh::kRound, LDA = Sh::kLDA, LDW = Sh::kLDW;
    constexpr int NJ = NBV + (SIMPLE ? 0 : 1);  // dS column blocks (+ dz)
    constexpr int NFS = NBK * KSV;
    constexpr int NFR = NFS + (SIMPLE ? 0 : KSK);
    constexpr int NQK = FK * (int)sizeof(T) / 16;  // 16-byte words per quarter row of Q
    constexpr int NQV = FV * (int)sizeof(T) / 16;  // ... of dO
    constexpr int kFragBytes = NFR * 64 * 16;
    constexpr int kTileBytes = RT * (LDA + LDW) * (int)sizeof(T);  // A tile, then W tile
    constexpr int kStBytes = StagedState<DK, DV>::kFloats * 4;
    constexpr int kAreaBytes = kTileBytes > kStBytes ? kTileBytes : kStBytes;
    static_assert(sizeof(T) == 2, "transposed LDS reads take 16-bit elements");
    static_assert(Sh::kStages == 2, "the loop below is written for two stages");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kFragBytes + kAreaBytes];
    __shared__ float red[3 * NW];
    __shared__ float sZ[DK];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / PB;
    const int p = wid % PB;
    const int64_t t0 = (int64_t)p * LB;
    const int64_t t1 = min(t0 + LB, T_);
    const int nrounds = (int)(t1 > t0 ? (t1 - t0 + RT - 1) / RT : 0);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const Layout lk = lay.q, lv = lay.dout;
    const float* S = stS + bh * DK * DV;
    const float* z = stz + bh * DK;
    Frag<T>* sA = reinterpret_cast<Frag<T>*>(smem);
    T* tA = reinterpret_cast<T*>(smem + kFragBytes);
    T* tW = tA + RT * LDA;

    // The loaded words as they are (see the D = 64 kernel).
    struct Stage {
        u32x4 q[NQK], d[NQV];
    };
    const HeadBuf bq = slice_buf(q, lk, bh, DK, t0, t1), bd = slice_buf(dout, lv, bh, DV, t0, t1),
                  bdq = slice_buf(dq, lay.dq, bh, DK, t0, t1);
    const Rotation rot(nrounds, Sh::kStages, wid);
    auto issue = [&](Stage& st, int round) {
        const int64_t row = (int64_t)rot(round) * RT + wave * STEP + m;
        const int oq = buf_off<T>(row, lk.rs, FK * grp), od = buf_off<T>(row, lv.rs, FV * grp);
#pragma unroll
        for (int i = 0; i < (NQK > NQV ? NQK : NQV); ++i) {
            if (i < NQK) st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, oq + 16 * i, 0, 0);
            if (i < NQV) st.d[i] = __builtin_amdgcn_raw_buffer_load_b128(bd.rsrc, od + 16 * i, 0, 0);
        }
    };
    // The first two rounds' loads are issued before the prologue, which they
    // overlap (with no rounds they read zeros and the loop below does not run).
    Stage s0, s1;
    issue(s0, 0);
    sched_fence();
    issue(s1, 1);
    sched_fence();
    // The state is staged in the tile area (which the rounds alone use) and
    // the fragments are built from there.
    int sS = 0, sz = 0, sw = 0;
    {
        constexpr int LD = StagedState<DK, DV>::kLD;
        float* sSt = reinterpret_cast<float*>(tA);
        const StagedState<DK, DV> st = stage_state<DK, DV, NT>(S, z, sSt, red);
        if constexpr (Elt<T>::kScaled) {
            sS = scale_exp(st.max_m);
            sz = scale_exp(st.max_z);
            if constexpr (!SIMPLE) {
                if (st.sum_z > 0.f && isfinite(st.sum_z)) {
                    int e;
                    frexpf(st.sum_z, &e);
                    sw = min(max(e - 1, -120), 120);  // 2^sw <= sum(z) < 2^(sw+1)
                }
            }
        }
        const float fS = ldexpf(1.f, sS), fz = ldexpf(1.f, sz);
        // captures by value (see the generic dQ kernel)
        build_frags<T, NFR, NW>(sA, [=](int f) {
            return f < NFS ? build_frag<T, DK, DV, false, LD>(sSt, f / KSV, f % KSV, m, grp, fS)
                           : build_zfrag<T, DK>(sSt + DK * LD, max(f - NFS, 0), grp, fz);
        });
        for (int i = tid; i < DK; i += NT) sZ[i] = sSt[DK * LD + i];
    }
    __syncthreads();
    const float uS = ldexpf(1.f, -sS), uz = ldexpf(1.f, -sz), fw = ldexpf(1.f, sw);

    f32x4 dsacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) dsacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    const int row = wave * STEP + m;  // this lane's token within the round tile
    auto body = [&](Stage& st, int round) {
        sched_fence();
        Row<T, FK> lq;
        __builtin_memcpy(lq.e, st.q, sizeof(lq));
        float qt[FK];
        Frag<T> bqf[KSK], bdf[KSV];
#pragma unroll
        for (int o = 0; o < FK; ++o) qt[o] = phi<FM, T>(to_f32(lq.e[o]));
        if constexpr (!SIMPLE)
#pragma unroll
            for (int s = 0; s < KSK; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) bqf[s][e] = static_cast<T>(qt[8 * s + e]);
#pragma unroll
        for (int s = 0; s < KSV; ++s) bdf[s] = __builtin_bit_cast(Frag<T>, st.d[s]);
        // den first, so that the phi(q) fragments are dead before u
        float inv = 1.f;
        if constexpr (!SIMPLE) {
            f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSK; ++s) ad = mma(sA[(NFS + s) * 64 + lane], bqf[s], ad);
            inv = 1.f / (ad[0] * uz + eps);
        }
        f32x4 au[NBK];
#pragma unroll
        for (int b = 0; b < NBK; ++b) {
            au[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSV; ++s) au[b] = mma(sA[(b * KSV + s) * 64 + lane], bdf[s], au[b]);
        }
        // dO rows go to the round tile as loaded; then the stage is free
        {
            u32x4* dw = reinterpret_cast<u32x4*>(&tW[row * LDW + FV * grp]);
#pragma unroll
            for (int i = 0; i < NQV; ++i) dw[i] = st.d[i];
        }
        sched_fence();
        issue(st, round + Sh::kStages);
        sched_fence();
        float aq = 1.f;  // factor on phi(q) in the reduction operand
        float ku = SIMPLE ? uS * eps : uS, cc = 0.f;  // simple_la: eps carries the query scale
        if constexpr (!SIMPLE) {
            float rr = 0.f;
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) rr += qt[4 * b + r] * au[b][r];
            rr += __shfl_xor(rr, 16);
            rr += __shfl_xor(rr, 32);
            const float beta = -(rr * uS) * inv;  // -r / den
            cc = beta * inv;                      // -r / den^2
            ku = uS * inv;
            aq = fw * inv;
            if (grp == 0) tW[row * LDW + DV] = static_cast<T>(beta);
        }
        sched_fence();
        {
            Row<T, FK> out;
            const float* zl = &sZ[FK * grp];
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = 4 * b + r;
                    const float dqt = SIMPLE ? au[b][r] * ku : au[b][r] * ku + cc * zl[o];
                    out.e[o] = static_cast<T>(dqt * dphi_of<FM>(qt[o]));
                }
            // staged through this wave's own rows of the A tile (16 rows of
            // DK + 8 elements fit in its 16 rows of LDA), which are written
            // with A right after
            store_tile_rows<T, DK>(tA + wave * STEP * LDA, out, bdq, (int64_t)rot(round) * RT + wave * STEP, lay.dq.rs);
        }
        {
            Row<T, FK> rq;
#pragma unroll
            for (int o = 0; o < FK; ++o) rq.e[o] = static_cast<T>(qt[o] * aq);
            *reinterpret_cast<Row<T, FK>*>(&tA[row * LDA + FK * grp]) = rq;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < RT / 32; ++ks) {
            const int rb = 32 * ks + rA;
            const int col = 16 * wave + cA;
            const Frag<T> a = join_frag<T>(lds_read_tr(&tA[rb * LDA + col]), lds_read_tr(&tA[(rb + 4) * LDA + col]));
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const Frag<T> b = join_frag<T>(lds_read_tr(&tW[rb * LDW + 16 * j + cA]),
                                               lds_read_tr(&tW[(rb + 4) * LDW + 16 * j + cA]));
                dsacc[j] = mma(a, b, dsacc[j]);
            }
        }
        __syncthreads();
    };

    for (int r = 0; r < rot.npad; r += 2) {
        body(s0, r);
        body(s1, r + 1);
    }

    // wave w holds rows [16 w, 16 w + 16) of 2^sw dS; column 0 of the last
    // block holds 2^sw dz
    const float uw = ldexpf(1.f, -sw) * (SIMPLE ? eps : 1.f);  // simple_la: times the query scale
    float* oS;
    float* oz;
    if (PB == 1) {
        oS = dS_out + bh * DK * DV;
        oz = dz_out + bh * DK;
    } else {
        oS = part + (bh * PB + p) * (int64_t)E;
        oz = oS + DK * DV;
    }
#pragma unroll
    for (int j = 0; j < NBV; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) oS[(16 * wave + 4 * grp + r) * DV + 16 * j + m] = dsacc[j][r] * uw;
    if (m == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) oz[16 * wave + 4 * grp + r] = SIMPLE ? 0.f : dsacc[NJ - 1][r] * uw;
}

// ---------------------------------------------------------------------------
// Step 7: backward, K/V side.
// ---------------------------------------------------------------------------
// dphi(k_t) = dS v_t + dz and dv_t = dS^T phi(k_t): both are products of a
// fixed D x D matrix with a token's row, so each is one set of MFMA blocks with
// dS (or dS^T) as the A operand and the loaded K/V quarter rows as B.
// The NK workgroups of a head share its tokens by rounds of 16 NW tokens:
// workgroup ch takes rounds ch, ch + NK, ch + 2 NK, ..., so at any time the
// head's workgroups stream neighbouring rounds of its four tensors, and the
// heads' streams advance side by side. (Contiguous chunks per workgroup, the
// other choice, keep every workgroup on a separate stretch of all four
// tensors at once; how those concurrent streams fall on DRAM channels then
// depends on where the buffers sit, and the kernel ran 5-10% slower.)
template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__((StreamShape<T, DK, DV>::kThreads), (StreamShape<T, DK, DV>::kKvMinBlocks)) void bwd_dkv_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ dSg,
    const float* __restrict__ dzg, T* __restrict__ dk, T* __restrict__ dv, int64_t T_, const Layouts lay, int NK,
    int64_t LK) {
    using Sh = StreamShape<T, DK, DV>;
    const Layout lk = lay.k, lv = lay.v;
    constexpr int FK = Sh::kFK, FV = Sh::kFV, NBK = Sh::kNBK, NBV = Sh::kNBV, KSK = Sh::kKSK, KSV = Sh::kKSV,
                  NW = Sh::kWaves, NT = Sh::kThreads;
    constexpr int U = 1;  // one 16-token block per wave step; the prefetch gives the depth
    constexpr int NF1 = NBK * KSV;  // dK side: rows over DK, contraction over DV
    constexpr int NF2 = NBV * KSK;  // dV side: rows over DV, contraction over DK
    constexpr int DM = DK > DV ? DK : DV;
    constexpr int LDR = DM + 16 / (int)sizeof(T);
    constexpr int kFragBytes = (NF1 + NF2) * 64 * (int)sizeof(Frag<T>);
    // Store staging unless the fragments leave no room for it (fp32 at
    // DK = DV = 128): then the stores go out per lane.
    constexpr bool kStage = kFragBytes + NW * 16 * LDR * (int)sizeof(T) <= 150 * 1024;
    // The backward state is staged in LDS (sharing the store staging area,
    // which the loop alone uses) and the fragments are built from there,
    // where it fits beside them and except at DK = DV = 128.
    constexpr bool kStaged = Sh::kStaged && kFragBytes + StagedState<DK, DV>::kFloats * 4 <= 150 * 1024;
    constexpr int kStoreBytes = kStage ? NW * 16 * LDR * (int)sizeof(T) : 16;
    constexpr int kStBytes = kStaged ? StagedState<DK, DV>::kFloats * 4 : 0;
    __shared__ Frag<T> sA[(NF1 + NF2) * 64];
    __shared__ __attribute__((aligned(16))) unsigned char sraw[kStoreBytes > kStBytes ? kStoreBytes : kStBytes];
    __shared__ float red[3 * NW];
    T* stage = reinterpret_cast<T*>(sraw);

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / NK;
    const int ch = wid % NK;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const float* dS = dSg + bh * DK * DV;
    const float* dz = dzg + bh * DK;

    // The first two turns' loads are issued before the prologue, which they
    // overlap. The loop takes two rounds per turn with no early exit (an exit
    // makes the compiler wait for every load in flight where the paths join):
    // the head's buffer descriptors read rows past its end as zeros and drop
    // their stores.
    const HeadBuf bk = slice_buf(k, lk, bh, DK, 0, T_), bv_ = slice_buf(v, lv, bh, DV, 0, T_);
    const HeadBuf bdk = slice_buf(dk, lay.dk, bh, DK, 0, T_), bdv = slice_buf(dv, lay.dv, bh, DV, 0, T_);
    T* stg = stage + (kStage ? wave * 16 * LDR : 0);
    // The loaded words as they are (see the dQ kernel).
    constexpr int NQK = FK * (int)sizeof(T) / 16;  // 16-byte words per quarter row of K
    constexpr int NQV = FV * (int)sizeof(T) / 16;  // ... of V
    struct Stage {
        u32x4 k[U][NQK], v[U][NQV];
    };
    constexpr int NS = Sh::kStages;
    constexpr int RT = 16 * U * NW;  // tokens per round
    // this workgroup's rounds, padded to whole turns of NS
    const int64_t nrounds = (T_ + RT - 1) / RT;
    const int nmine = (int)(nrounds > ch ? (nrounds - ch + NK - 1) / NK : 0);
    const int npad = (nmine + NS - 1) / NS * NS;
    // first row of the wave's block of the workgroup's j-th round; the padded
    // rounds (and the prefetches past the last one) all read the rows just
    // past the head's end, zeros whose stores are dropped: their 32-bit
    // offsets stay below T + 64 rows, inside the head span the host checks
    auto row_of = [&](int j) {
        return (j < nmine ? ((int64_t)ch + (int64_t)NK * j) * RT : T_) + 16 * U * wave;
    };
    auto issue = [&](Stage& st, int blk) {
        const int64_t bs = row_of(blk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ok_ = buf_off<T>(bs + 16 * u + m, lk.rs, FK * grp);
            const int ov_ = buf_off<T>(bs + 16 * u + m, lv.rs, FV * grp);
#pragma unroll
            for (int i = 0; i < (NQK > NQV ? NQK : NQV); ++i) {
                if (i < NQK) st.k[u][i] = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, ok_ + 16 * i, 0, 0);
                if (i < NQV) st.v[u][i] = __builtin_amdgcn_raw_buffer_load_b128(bv_.rsrc, ov_ + 16 * i, 0, 0);
            }
        }
    };
    Stage stq[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        issue(stq[i], i);
        sched_fence();
    }
    // fragments [0, NF1): dK side, rows i, contraction j -> dS[i][j];
    // [NF1, NF1 + NF2): dV side, rows j, contraction i -> dS[i][j]
    int sD = 0;
    float dzl[FK];
    if constexpr (kStaged) {
        constexpr int LD = StagedState<DK, DV>::kLD;
        float* sSt = reinterpret_cast<float*>(sraw);
        const StagedState<DK, DV> st = stage_state<DK, DV, NT>(dS, dz, sSt, red);
        if constexpr (Elt<T>::kScaled) sD = scale_exp(st.max_m);
        const float fD = ldexpf(1.f, sD);
        build_frags<T, NF1 + NF2, NW>(sA, [&](int f) {
            return f < NF1 ? build_frag<T, DK, DV, false, LD>(sSt, f / KSV, f % KSV, m, grp, fD)
                           : build_frag<T, DV, DK, true, LD>(sSt, (f - NF1) / KSK, (f - NF1) % KSK, m, grp, fD);
        });
#pragma unroll
        for (int o = 0; o < FK; ++o) dzl[o] = SIMPLE ? 0.f : sSt[DK * LD + FK * grp + o];
    } else {
        if constexpr (Elt<T>::kScaled) sD = scale_exp(block_absmax_matrix<DK * DV, NT>(dS, red));
        const float fD = ldexpf(1.f, sD);
        build_frags<T, NF1 + NF2, NW>(sA, [&](int f) {
            return f < NF1 ? build_frag<T, DK, DV, false, DV>(dS, f / KSV, f % KSV, m, grp, fD)
                           : build_frag<T, DV, DK, true, DV>(dS, (f - NF1) / KSK, (f - NF1) % KSK, m, grp, fD);
        });
#pragma unroll
        for (int o = 0; o < FK; ++o) dzl[o] = SIMPLE ? 0.f : dz[FK * grp + o];
    }
    const float uD = ldexpf(1.f, -sD);
    __syncthreads();

    auto body = [&](Stage& st, int blk) {
        const int64_t base = row_of(blk);
        sched_fence();
        float dphik[U][FK];
        Frag<T> bk[U][KSK], bv[U][KSV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Row<T, FK> lk_;
            Row<T, FV> lv_;
            __builtin_memcpy(lk_.e, st.k[u], sizeof(lk_));
            __builtin_memcpy(lv_.e, st.v[u], sizeof(lv_));
            float kt[FK];
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int s = 0; s < FK / 8; ++s) {
                    u32x4 raw;
                    __builtin_memcpy(&raw, &lk_.e[8 * s], sizeof(raw));
                    feature8<FM, T>(raw, &kt[8 * s], &dphik[u][8 * s]);
                }
            } else {
#pragma unroll
                for (int o = 0; o < FK; ++o) feature<FM, T>(to_f32(lk_.e[o]), kt[o], dphik[u][o]);
            }
#pragma unroll
            for (int s = 0; s < KSK; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) bk[u][s][e] = static_cast<T>(kt[8 * s + e]);
#pragma unroll
            for (int s = 0; s < KSV; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[u][s][e] = lv_.e[8 * s + e];
        }
        f32x4 ak[U][NBK], av[U][NBV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int b = 0; b < NBK; ++b) ak[u][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < NBV; ++b) av[u][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (DK == DV) {
            // interleaved, as the two products share their loop shape
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int s = 0; s < KSV; ++s) {
                    const Frag<T> a1 = sA[(b * KSV + s) * 64 + lane];
                    const Frag<T> a2 = sA[(NF1 + b * KSK + s) * 64 + lane];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        ak[u][b] = mma(a1, bv[u][s], ak[u][b]);
                        av[u][b] = mma(a2, bk[u][s], av[u][b]);
                    }
                }
        } else {
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int s = 0; s < KSV; ++s) {
                    const Frag<T> a1 = sA[(b * KSV + s) * 64 + lane];
#pragma unroll
                    for (int u = 0; u < U; ++u) ak[u][b] = mma(a1, bv[u][s], ak[u][b]);
                }
#pragma unroll
            for (int b = 0; b < NBV; ++b)
#pragma unroll
                for (int s = 0; s < KSK; ++s) {
                    const Frag<T> a2 = sA[(NF1 + b * KSK + s) * 64 + lane];
#pragma unroll
                    for (int u = 0; u < U; ++u) av[u][b] = mma(a2, bk[u][s], av[u][b]);
                }
        }
        // the stage's registers are free once the products have read V
        sched_fence();
        issue(st, blk + NS);
        sched_fence();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Row<T, FK> gk;
            Row<T, FV> gv;
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = 4 * b + r;
                    gk.e[o] = static_cast<T>((ak[u][b][r] * uD + dzl[o]) * dphik[u][o]);
                }
#pragma unroll
            for (int b = 0; b < NBV; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) gv.e[4 * b + r] = static_cast<T>(av[u][b][r] * uD);
            if constexpr (kStage) {
                store_tile_rows<T, DK>(stg, gk, bdk, base + 16 * u, lay.dk.rs);
                store_tile_rows<T, DV>(stg, gv, bdv, base + 16 * u, lay.dv.rs);
            } else {
                store_tile_quarters<T, DK>(gk, bdk, base + 16 * u, lay.dk.rs);
                store_tile_quarters<T, DV>(gv, bdv, base + 16 * u, lay.dv.rs);
            }
        }
    };
    for (int j = 0; j < npad; j += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) body(stq[i], j + i);
    }
}

// ---------------------------------------------------------------------------
// Causal forward (LA_CAUSAL): token t attends to tokens s <= t.
// ---------------------------------------------------------------------------
// Each head's tokens are cut into the segments of the state reduction; a
// segment's exclusive prefix state (S, z of all earlier segments) comes from
// prefix_kernel. One workgroup walks its segment in 64-token chunks, in order,
// with the running state R, z of everything before the chunk on chip:
//   O_t = (phi(q_t) R + sum_{s in chunk, s <= t} a_ts v_s)
//         / (phi(q_t) z + sum_{s in chunk, s <= t} a_ts + eps),  a_ts = phi(q_t) . phi(k_s),
// then R += phi(K_c)^T V_c, z += sum phi(k). Per chunk, the four waves each
// take 16 query rows, one per lane (t = 16 wave + lane % 16), and
//   (a) compute a^T = phi(K) phi(Q)^T for them (key blocks above the diagonal
//       skipped, the diagonal block masked): in the MFMA result layout a
//       lane holds four consecutive keys of its query, which is the operand
//       layout of a contraction over keys, so a^T, rounded to 16 bits with a
//       power of two, feeds (b) straight from registers;
//   (b) compute O^T = [V | 1]^T a^T + [R | z]^T phi(Q)^T (V^T read
//       transposed from the chunk tile in the same key order; R^T and z as
//       16-bit copies in LDS), one reciprocal per lane, and store each lane's
//       four consecutive features of its O row as one 8-byte piece;
//   (c) add phi(K)^T V into their quarter of R's columns (fp32 registers;
//       wave 0 also keeps z) and publish it, scaled by the wave's own power
//       of two, into the other LDS copy of R^T for the next chunk.
// Two barriers per chunk; two chunks of loads in flight. Rows past the
// segment end load as zeros (K is zeroed after phi) and their stores are
// dropped.
// Four consecutive 16-bit values as one 8-byte LDS store.
template <typename T>
__device__ __forceinline__ void put4t(T* dst, f32x4 x, float f) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = static_cast<T>(x[r] * f);
    *reinterpret_cast<t4*>(dst) = y;
}

template <int DK, int DV>
struct CausalShape {
    static constexpr int kChunk = 64;                 // tokens per chunk
    static constexpr int kLDK = DK + 16;              // tQ, tK row stride (elements)
    static constexpr int kLDV = DV + 16;              // tV row stride
    static constexpr int kLDRT = DK + 8;              // R^T row stride (rows j, DK entries)
    static constexpr int kMinBlocks = (DK == 64 && DV == 64) ? 2 : 1;
};

// Largest x over the 64 lanes of the wave (x >= 0): DPP row shifts and
// broadcasts (lanes shifted in from outside a row read 0), then lane 63.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false)));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

template <typename T, int DK, int DV, bool SIMPLE, int FM, int DKR = DK, int DVR = DV>
__global__ __launch_bounds__(kThreads, (CausalShape<DK, DV>::kMinBlocks)) void fwd_causal_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ pre,
    T* __restrict__ o, int64_t T_, const Layouts lay, int P, int64_t L, float eps) {
    using Sh = CausalShape<DK, DV>;
    constexpr int C = Sh::kChunk, LDK = Sh::kLDK, LDV = Sh::kLDV, LDRT = Sh::kLDRT;
    constexpr int NBV = DV / 16;         // output column blocks
    constexpr int RJ = DV / 64;          // R column blocks per wave (a quarter of DV)
    constexpr int RI = DK / 16;          // R row blocks
    constexpr int KSK = DK / 32, KSC = C / 32;
    constexpr int CK = DK / 8, CV = DV / 8;  // 16-byte chunks per row
    constexpr int NCK = C * CK / kThreads, NCV = C * CV / kThreads;
    static_assert(sizeof(T) == 2, "transposed LDS reads take 16-bit elements");
    static_assert(NCK * kThreads == C * CK && NCV * kThreads == C * CV, "tiles must split evenly");
    static_assert(RJ >= 1 && RJ * 64 == DV, "each wave owns whole 16-column blocks of R");
    __shared__ __attribute__((aligned(16))) T tQ[C * LDK];
    __shared__ __attribute__((aligned(16))) T tK[C * LDK];
    __shared__ __attribute__((aligned(16))) T tV[C * LDV];
    __shared__ __attribute__((aligned(16))) T tRT[2][DV * LDRT];
    __shared__ __attribute__((aligned(16))) T tZ[2][DK];
    __shared__ int sExp[2][kWaves + 1];  // exponents of the R quarters, then of z

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const int64_t len = t1 - t0;
    const int nchunks = (int)(len > 0 ? (len + C - 1) / C : 0);
    const Layout lq = lay.q, lk = lay.k, lv = lay.v, lo = lay.o;

    // Running state: R[16 iR + 4 grp + r][16 (wave RJ + jR) + m] in accR[iR][jR][r];
    // z[16 iR + 4 grp + r] in accZ[iR][r] (wave 0). From the exclusive prefix.
    f32x4 accR[RI][RJ], accZ[RI];
    {
        const float* pS = (pre != nullptr && p > 0) ? pre + (bh * P + p) * (int64_t)(DKR * DVR + DKR) : nullptr;
#pragma unroll
        for (int iR = 0; iR < RI; ++iR) {
#pragma unroll
            for (int jR = 0; jR < RJ; ++jR)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    {
                        const int i = 16 * iR + 4 * grp + r, j = 16 * (wave * RJ + jR) + m;
                        accR[iR][jR][r] = (pS && i < DKR && j < DVR) ? pS[i * DVR + j] : 0.f;
                    }
#pragma unroll
            for (int r = 0; r < 4; ++r) accZ[iR][r] = (pS && 16 * iR + 4 * grp + r < DKR) ? pS[DKR * DVR + 16 * iR + 4 * grp + r] : 0.f;
        }
    }
    Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<T>(1.f);

    // this wave's quarter of R (as R^T) and z (wave 0) as 16-bit into copy `buf`
    auto publish = [&](int buf) {
        int sR = 0;
        if constexpr (Elt<T>::kScaled) {
            float mx = 0.f;
#pragma unroll
            for (int iR = 0; iR < RI; ++iR)
#pragma unroll
                for (int jR = 0; jR < RJ; ++jR)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(accR[iR][jR][r]));
            sR = scale_exp(wave_max_nonneg(mx));
        }
        const float fR = ldexpf(1.f, sR);
#pragma unroll
        for (int iR = 0; iR < RI; ++iR)
#pragma unroll
            for (int jR = 0; jR < RJ; ++jR)
                put4t(&tRT[buf][(16 * (wave * RJ + jR) + m) * LDRT + 16 * iR + 4 * grp], accR[iR][jR], fR);
        if (lane == 0) sExp[buf][wave] = sR;
        if constexpr (!SIMPLE) {
            if (wave == 0) {
                int sZ = 0;
                if constexpr (Elt<T>::kScaled) {
                    float mz = 0.f;
#pragma unroll
                    for (int iR = 0; iR < RI; ++iR)
#pragma unroll
                        for (int r = 0; r < 4; ++r) mz = fmaxf(mz, fabsf(accZ[iR][r]));
                    sZ = scale_exp(wave_max_nonneg(mz));
                }
                const float fZ = ldexpf(1.f, sZ);
                if (m == 0)
#pragma unroll
                    for (int iR = 0; iR < RI; ++iR) put4t(&tZ[buf][16 * iR + 4 * grp], accZ[iR], fZ);
                if (lane == 0) sExp[buf][kWaves] = sZ;
            }
        }
    };

    struct Stage {
        u32x4 q[NCK], k[NCK], v[NCV];
    };
    const HeadBuf bq = slice_buf(q, lq, bh, DKR, t0, t1), bk = slice_buf(k, lk, bh, DKR, t0, t1);
    const HeadBuf bv = slice_buf(v, lv, bh, DVR, t0, t1), bo = slice_buf(o, lo, bh, DVR, t0, t1);
    auto issue = [&](Stage& st, int c) {
        const int64_t row0 = (int64_t)c * C;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, cc = n % CK;
            st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, pad_off<DK, DKR>(buf_off<T>(row0 + r, lq.rs, 8 * cc), 8 * cc), 0, 0);
            st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, pad_off<DK, DKR>(buf_off<T>(row0 + r, lk.rs, 8 * cc), 8 * cc), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, cc = n % CV;
            st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(bv.rsrc, pad_off<DV, DVR>(buf_off<T>(row0 + r, lv.rs, 8 * cc), 8 * cc), 0, 0);
        }
    };
    auto consume = [&](const Stage& st, int c) {
        const int64_t row0 = (int64_t)c * C;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, cc = n % CK;
            // rows past the segment end and padded feature columns add nothing
            const bool okq = DKR == DK || 8 * cc < DKR, ok = okq && row0 + r < len;
            // rows past the segment end must add nothing: mask after phi
            *reinterpret_cast<u32x4*>(&tQ[r * LDK + 8 * cc]) = keep_or_zero(phi8<FM, T>(st.q[i]), okq);
            *reinterpret_cast<u32x4*>(&tK[r * LDK + 8 * cc]) = keep_or_zero(phi8<FM, T>(st.k[i]), ok);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, cc = n % CV;
            *reinterpret_cast<u32x4*>(&tV[r * LDV + 8 * cc]) = st.v[i];
        }
    };

    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    auto body = [&](Stage& st, int c) {
        const int cur = c & 1;
        const int64_t row0 = (int64_t)c * C;
        consume(st, c);
        __syncthreads();  // tiles of chunk c and the R^T, z copy `cur` are visible
        sched_fence();
        issue(st, c + 2);  // two chunks ahead; past the segment end these read zeros
        sched_fence();

        // (a) a^T[s][t] = phi(k_s) . phi(q_t) for the wave's query rows
        // t = 16 wave + m (one per lane) and the keys s = 16 sb + 4 grp + r of
        // block sb (the lane's four values). This result layout, with s along
        // a lane's values, is already the operand layout of the contraction
        // over s in (b), so a stays in registers. Slot i holds key block
        // sb = (wave - i) mod 4: slot 0 is the diagonal block (masked to
        // s <= t), slots 1 .. wave lie below it, and the slots past wave are
        // the blocks above the diagonal, which stay zero.
        f32x4 aa[C / 16];
#pragma unroll
        for (int i = 0; i < C / 16; ++i) aa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
            const Frag<T> bq = *reinterpret_cast<const Frag<T>*>(&tQ[(16 * wave + m) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
            for (int i = 0; i < C / 16; ++i) {
                if (i <= wave) {
                    const Frag<T> ak = *reinterpret_cast<const Frag<T>*>(&tK[(16 * (wave - i) + m) * LDK + 32 * ks + 8 * grp]);
                    aa[i] = mma(ak, bq, aa[i]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) aa[0][r] = 4 * grp + r > m ? 0.f : aa[0][r];
        int sA = 0;
        if constexpr (Elt<T>::kScaled) {
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < C / 16; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(aa[i][r]));
            sA = scale_exp(wave_max_nonneg(amax));
        }
        // operands over the keys of slots 2 ks and 2 ks + 1: values 0..3 of a
        // lane are the keys 16 sb + 4 grp + (0..3) of the first slot's block,
        // values 4..7 those of the second
        Frag<T> bA[KSC];
        {
            const float fA = ldexpf(1.f, sA);
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    bA[ks][r] = static_cast<T>(aa[2 * ks][r] * fA);
                    bA[ks][4 + r] = static_cast<T>(aa[2 * ks + 1][r] * fA);
                }
        }

        // (b) O^T = [V | 1]^T a^T + [R | z]^T phi(Q)^T, column t = 16 wave + m;
        // the denominator parts land in every row of dA and dR. The V^T
        // operand is read transposed with the key order of bA.
        f32x4 nA[NBV], nR[NBV], dA = f32x4{0.f, 0.f, 0.f, 0.f}, dR = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < NBV; ++jb) {
            nA[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
            nR[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int rT = 4 * grp + (m >> 2), cT = 4 * (m & 3);
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            if (2 * ks <= wave) {  // otherwise both slots lie above the diagonal
                const int r0 = 16 * ((wave - 2 * ks) & (C / 16 - 1)) + rT;
                const int r1 = 16 * ((wave - 2 * ks - 1) & (C / 16 - 1)) + rT;
#pragma unroll
                for (int jb = 0; jb < NBV; ++jb) {
                    const Frag<T> av = join_frag<T>(lds_read_tr(&tV[r0 * LDV + 16 * jb + cT]),
                                                    lds_read_tr(&tV[r1 * LDV + 16 * jb + cT]));
                    nA[jb] = mma(av, bA[ks], nA[jb]);
                }
                if constexpr (!SIMPLE) dA = mma(ones, bA[ks], dA);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
            const Frag<T> bq = *reinterpret_cast<const Frag<T>*>(&tQ[(16 * wave + m) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb) {
                const Frag<T> ar = *reinterpret_cast<const Frag<T>*>(&tRT[cur][(16 * jb + m) * LDRT + 32 * ks + 8 * grp]);
                nR[jb] = mma(ar, bq, nR[jb]);
            }
            if constexpr (!SIMPLE) {
                const Frag<T> az = *reinterpret_cast<const Frag<T>*>(&tZ[cur][32 * ks + 8 * grp]);
                dR = mma(az, bq, dR);
            }
        }
        {
            // one query row per lane: one reciprocal, and O row t's features
            // 16 jb + 4 grp .. + 3 as one 8-byte store per block
            const float uA = ldexpf(1.f, -sA);
            float inv = eps;  // simple_la: eps carries the query scale
            if constexpr (!SIMPLE) inv = __builtin_amdgcn_rcpf(dA[0] * uA + dR[0] * ldexpf(1.f, -sExp[cur][kWaves]) + eps);
            const float ia = uA * inv;
            const int64_t row = row0 + 16 * wave + m;
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb) {
                const float ir = ldexpf(1.f, -sExp[cur][jb / RJ]) * inv;
                f32x4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] = nA[jb][r] * ia + nR[jb][r] * ir;
                const int col = 16 * jb + 4 * grp;
                buf_store4<T>(bo, pad_off<DV, DVR>(buf_off<T>(row, lo.rs, col), col), y);
            }
        }

        // (c) R += phi(K)^T V on this wave's columns; z += sum_t phi(k_t) (wave 0)
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            const int rb = 32 * ks + rA;
            Frag<T> bvf[RJ];
#pragma unroll
            for (int jR = 0; jR < RJ; ++jR)
                bvf[jR] = join_frag<T>(lds_read_tr(&tV[rb * LDV + 16 * (wave * RJ + jR) + cA]),
                                       lds_read_tr(&tV[(rb + 4) * LDV + 16 * (wave * RJ + jR) + cA]));
#pragma unroll
            for (int iR = 0; iR < RI; ++iR) {
                const Frag<T> a = join_frag<T>(lds_read_tr(&tK[rb * LDK + 16 * iR + cA]),
                                               lds_read_tr(&tK[(rb + 4) * LDK + 16 * iR + cA]));
#pragma unroll
                for (int jR = 0; jR < RJ; ++jR) accR[iR][jR] = mma(a, bvf[jR], accR[iR][jR]);
                if constexpr (!SIMPLE) {
                    if (wave == 0) accZ[iR] = mma(a, ones, accZ[iR]);
                }
            }
        }
        publish(cur ^ 1);
        __syncthreads();  // every wave is done with the tiles and with copy `cur`
    };
    publish(0);
    // Two chunks of loads in flight. The chunk count is rounded up to even so
    // that the loop has no branch around loads (a branch makes the compiler
    // wait for every load in flight where the paths join): a chunk past the
    // segment end reads zeros, adds nothing to R and z, and stores nothing.
    if (nchunks > 0) {
        Stage s0, s1;
        issue(s0, 0);
        sched_fence();
        issue(s1, 1);
        sched_fence();
        for (int c = 0; c < nchunks; c += 2) {
            body(s0, c);
            body(s1, c + 1);
        }
    }
}

// Exclusive prefix of the P partial (S, z) blocks of every head, in place
// (block p becomes the sum of blocks 0 .. p-1), and their total into the
// state: the same fixed-order additions as combine_kernel, so where the
// segments are the bidirectional reduction's slices (every shape but 16-bit
// D = Dv = 64, which takes twice as many segments as slices) the state is
// bit-identical to the non-causal one.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void prefix_kernel(float* __restrict__ part, int P, float* __restrict__ outS,
                                                          float* __restrict__ outz, int64_t BH) {
    constexpr int E4 = (DK * DV + DK) / 4;
    constexpr int BPH = (E4 + kThreads - 1) / kThreads;  // blocks per head
    const int64_t bh = blockIdx.x / BPH;
    const int i = (blockIdx.x % BPH) * kThreads + threadIdx.x;
    if (bh >= BH || i >= E4) return;
    float4* pb = reinterpret_cast<float4*>(part) + bh * (int64_t)P * E4 + i;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < P; p0 += 8) {
        float4 x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = pb[(int64_t)min(p0 + j, P - 1) * E4];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (p0 + j < P) {
                pb[(int64_t)(p0 + j) * E4] = acc;
                acc.x += x[j].x;
                acc.y += x[j].y;
                acc.z += x[j].z;
                acc.w += x[j].w;
            }
    }
    const int idx = 4 * i;
    if (idx < DK * DV)
        *reinterpret_cast<float4*>(outS + bh * DK * DV + idx) = acc;
    else
        *reinterpret_cast<float4*>(outz + bh * DK + (idx - DK * DV)) = acc;
}

// ---------------------------------------------------------------------------
// Causal backward (LA_CAUSAL): the vector-Jacobian product of sum(O * dO)
// through the recurrent form, eps held constant.
// ---------------------------------------------------------------------------
// With the inclusive prefix states S_t = sum_{s<=t} phi(k_s) v_s^T and
// z_t = sum_{s<=t} phi(k_s):
//   den_t = phi(q_t) . z_t + eps,  w_t = 1 / den_t,  u_t = S_t dO_t,
//   c_t = -(phi(q_t) . u_t) w_t^2,  dphi(q_t) = w_t u_t + c_t z_t,
// and with the inclusive suffix sums G_s = sum_{t>=s} Qw_t dO_t^T and
// g_s = sum_{t>=s} c_t phi(q_t), where Qw_t = w_t phi(q_t):
//   dphi(k_s) = G_s v_s + g_s,  dV_s = G_s^T phi(k_s).
// simple_la: w = 1, c = 0. Two scans over the segments of the state
// reduction, in 64-token chunks:
//  bwd_causal_q_kernel walks its segment forward from the exclusive prefix
//   (R, z) of the earlier segments, as the causal forward does, and writes
//   dQ, w_t and c^_t = c_t / w_t per token, the exponent with which the
//   chunk's Qw was staged, and the segment's own sums of Qw_t dO_t^T and
//   c_t phi(q_t);
//  suffix_kernel turns those into exclusive suffixes (the later segments);
//  bwd_causal_kv_kernel walks its segment backward from that suffix (G, g),
//   staging Qw at the chunk's exponent, and writes dK and dV.
// Within a chunk, with a_ts = phi(q_t) . phi(k_s) and b_ts = dO_t . v_s:
//   dphi(q_t) = w_t (dO_t R^T) + c_t z + sum_{s<=t} (w_t b_ts + c_t) phi(k_s)
//   dphi(k_s) = G v_s + g + sum_{t>=s} (b_ts + c^_t) Qw_t
//   dV_s = G^T phi(k_s) + sum_{t>=s} (Qw_t . phi(k_s)) dO_t
// (R, z: everything before the chunk; G, g: everything after it).
// Both scans work in the transposed form of the causal forward: a lane owns
// one row of the chunk (a query in the dQ scan, a key in the K/V scan) and
// holds four consecutive entries of the other index in each 16 x 16 result,
// so a^T, b^T and the masked weights are the operands of the next
// contraction as they come out of the MFMAs, and every output row leaves as
// 8-byte pieces straight from the accumulators.
template <int DK, int DV>
struct CausalBwdShape {
    static constexpr int kChunk = 64;
    static constexpr int kLDK = DK + 16;      // tQ, tK row stride (elements)
    static constexpr int kLDV = DV + 16;      // tV, tD row stride
    static constexpr int kLDRT = DK + 8;      // R^T or G^T: rows j, DK entries
    static constexpr int kMinBlocks = (DK == 64 && DV == 64) ? 2 : 1;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over each row of 16 lanes (a lane group); every lane of the row gets
// the same total.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xb1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_f<0x4e>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    x += dpp_f<0x140>(x);  // row_mirror
    return x;
}

// A 16-bit fragment times a power of two, through fp32.
template <typename T>
__device__ __forceinline__ Frag<T> scale_frag(Frag<T> x, float f) {
    Frag<T> y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = static_cast<T>(static_cast<float>(x[e]) * f);
    return y;
}


// Forward-order scan of one segment: dQ, w and c^ per token, the chunk's Qw
// exponent, and (P > 1) the segment's sums of Qw dO^T and c phi(q). The four
// waves each own 16 query rows of the chunk and a quarter of the rows of R
// and of the G sum. Per chunk:
//   (a) a and b on the wave's rows (blocks above the diagonal skipped);
//   (b) Y = dO R^T (R^T as 16-bit in LDS, one power of two per owner wave);
//   (c) den and phi(q) . u per row from a, b, Y and phi(q) read at the
//       result positions, reduced over the 16 lanes of a row;
//   (d) P = mask(w b + c), staged transposed, times phi(K);
//   (e) dQ = (w Y + c z + P phi(K)) phi'(q), staged transposed and stored
//       as rows;
//   (f) R += phi(K)^T V, z += sum phi(k) on the wave's rows of R;
//   (g) Qw of the wave's rows into the shared Qw^T tile at the wave's own
//       power of two; after a barrier every wave takes the smallest of the
//       four exponents and rescales the other waves' columns to it as it
//       reads them for G += Qw^T dO.
// R^T and z are published at the top of the next chunk, after the barrier
// that ends this one. Three barriers per chunk; one chunk of loads in flight.
template <typename T, int DK, int DV, bool SIMPLE, int FM, int DKR = DK, int DVR = DV>
__global__ __launch_bounds__(kThreads, (CausalBwdShape<DK, DV>::kMinBlocks)) void bwd_causal_q_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ pre, T* __restrict__ dq, float* __restrict__ wc, int* __restrict__ es,
    float* __restrict__ gpart, int64_t T_, const Layouts lay, int P, int64_t L, int nche, float eps) {
    using Sh = CausalBwdShape<DK, DV>;
    constexpr int C = Sh::kChunk, LDK = Sh::kLDK, LDV = Sh::kLDV, LDRT = Sh::kLDRT;
    constexpr int NBI = DK / 16, NBV = DV / 16, NBC = C / 16;
    constexpr int RIW = DK / 64;  // 16-row blocks of R and of the G sum per wave
    constexpr int KSK = DK / 32, KSV = DV / 32, KSC = C / 32;
    constexpr int CK = DK / 8, CV = DV / 8;
    constexpr int NCK = C * CK / kThreads, NCV = C * CV / kThreads;
    static_assert(sizeof(T) == 2, "transposed LDS reads take 16-bit elements");
    static_assert(NCK * kThreads == C * CK && NCV * kThreads == C * CV, "tiles must split evenly");
    static_assert(RIW >= 1 && RIW * 64 == DK, "each wave owns whole 16-row blocks");
    __shared__ __attribute__((aligned(16))) T tQ[C * LDK];
    __shared__ __attribute__((aligned(16))) T tK[C * LDK];
    __shared__ __attribute__((aligned(16))) T tV[C * LDV];
    // With room in LDS the G update of a chunk runs in the next chunk (dO and
    // Qw tiles double-buffered, one barrier less per chunk); at DK = DV = 128
    // the second buffers do not fit and it runs after a barrier of its own.
    constexpr bool kDefer = !(DK == 128 && DV == 128);
    constexpr int NBUF = kDefer ? 2 : 1;
    __shared__ __attribute__((aligned(16))) T tD[NBUF][C * LDV];
    __shared__ __attribute__((aligned(16))) T tRT[DV * LDRT];
    // the Qw tiles' rows are 16 bytes longer than a row, not 32 as in tQ,
    // which keeps two workgroups' LDS within a CU's at DK = DV = 64
    constexpr int LDQ = DK + 8;
    __shared__ __attribute__((aligned(16))) T tQw[NBUF][C * LDQ];
    __shared__ __attribute__((aligned(16))) float sZ[DK];
    __shared__ int sExpR[kWaves], sExpQ[NBUF][kWaves];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const int64_t len = t1 - t0;
    // rounded up to even: the loop body comes in pairs (see below)
    const int nchunks = (int)(len > 0 ? (((len + C - 1) / C) + 1) / 2 * 2 : 0);
    const Layout lq = lay.q, lk = lay.k, lv = lay.v, ld = lay.dout;

    // R[16 (wave RIW + iR) + 4 grp + r][16 jb + m] in accR[iR][jb][r], z of
    // the same rows in accZ[iR][r], likewise the G sum in accG.
    f32x4 accR[RIW][NBV], accZ[RIW], accG[RIW][NBV];
    float gzp[NBI][4];  // sum of c_t phi(q_t)[16 ib + 4 grp + r] over this lane's query rows
    {
        const float* pS = (pre != nullptr && p > 0) ? pre + (bh * P + p) * (int64_t)(DKR * DVR + DKR) : nullptr;
#pragma unroll
        for (int iR = 0; iR < RIW; ++iR) {
            const int i0 = 16 * (wave * RIW + iR) + 4 * grp;
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb) {
                accG[iR][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    accR[iR][jb][r] = (pS && i0 + r < DKR && 16 * jb + m < DVR) ? pS[(i0 + r) * DVR + 16 * jb + m] : 0.f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) accZ[iR][r] = (pS && i0 + r < DKR) ? pS[DKR * DVR + i0 + r] : 0.f;
        }
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) gzp[ib][r] = 0.f;
    }
    Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<T>(1.f);

    auto publish = [&]() {
        int sR = 0;
        if constexpr (Elt<T>::kScaled) {
            float mx = 0.f;
#pragma unroll
            for (int iR = 0; iR < RIW; ++iR)
#pragma unroll
                for (int jb = 0; jb < NBV; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(accR[iR][jb][r]));
            sR = scale_exp(wave_max_nonneg(mx));
        }
        const float fR = ldexpf(1.f, sR);
#pragma unroll
        for (int iR = 0; iR < RIW; ++iR)
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb)
                put4t(&tRT[(16 * jb + m) * LDRT + 16 * (wave * RIW + iR) + 4 * grp], accR[iR][jb], fR);
        if (lane == 0) sExpR[wave] = sR;
        if constexpr (!SIMPLE) {
            if (m == 0)
#pragma unroll
                for (int iR = 0; iR < RIW; ++iR)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sZ[16 * (wave * RIW + iR) + 4 * grp + r] = accZ[iR][r];
        }
    };

    struct Stage {
        u32x4 q[NCK], k[NCK], v[NCV], d[NCV];
    };
    const HeadBuf bq = slice_buf(q, lq, bh, DKR, t0, t1), bk = slice_buf(k, lk, bh, DKR, t0, t1);
    const HeadBuf bv = slice_buf(v, lv, bh, DVR, t0, t1), bd = slice_buf(dout, ld, bh, DVR, t0, t1);
    const HeadBuf bdq = slice_buf(dq, lay.dq, bh, DKR, t0, t1);
    auto issue = [&](Stage& st, int c) {
        const int64_t row0 = (int64_t)c * C;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, cc = n % CK;
            st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, pad_off<DK, DKR>(buf_off<T>(row0 + r, lq.rs, 8 * cc), 8 * cc), 0, 0);
            st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, pad_off<DK, DKR>(buf_off<T>(row0 + r, lk.rs, 8 * cc), 8 * cc), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, cc = n % CV;
            st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(bv.rsrc, pad_off<DV, DVR>(buf_off<T>(row0 + r, lv.rs, 8 * cc), 8 * cc), 0, 0);
            st.d[i] = __builtin_amdgcn_raw_buffer_load_b128(bd.rsrc, pad_off<DV, DVR>(buf_off<T>(row0 + r, ld.rs, 8 * cc), 8 * cc), 0, 0);
        }
    };
    auto consume = [&](const Stage& st, int c) {
        const int64_t row0 = (int64_t)c * C;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int n = tid + kThreads * i, r = n / CK, cc = n % CK;
            // rows past the segment end and padded feature columns add nothing
            const bool okq = DKR == DK || 8 * cc < DKR, ok = okq && row0 + r < len;
            *reinterpret_cast<u32x4*>(&tQ[r * LDK + 8 * cc]) = keep_or_zero(phi8<FM, T>(st.q[i]), okq);
            *reinterpret_cast<u32x4*>(&tK[r * LDK + 8 * cc]) = keep_or_zero(phi8<FM, T>(st.k[i]), ok);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int n = tid + kThreads * i, r = n / CV, cc = n % CV;
            *reinterpret_cast<u32x4*>(&tV[r * LDV + 8 * cc]) = st.v[i];
            *reinterpret_cast<u32x4*>(&tD[c % NBUF][r * LDV + 8 * cc]) = st.d[i];
        }
    };

    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    float* wcb = wc + 2 * (bh * T_ + t0);
    int* esb = es + (bh * P + p) * (int64_t)nche;
    // G += Qw^T dO of chunk cg on this wave's rows of the G sum, at the
    // chunk's common exponent (the smallest of the four waves' exponents)
    auto gupdate = [&](int cg) {
        const int bf = cg % NBUF;
        int sM = 0;
        if constexpr (Elt<T>::kScaled) sM = min(min(sExpQ[bf][0], sExpQ[bf][1]), min(sExpQ[bf][2], sExpQ[bf][3]));
        if (tid == 0) esb[cg] = sM;
        const float uM = ldexpf(1.f, -sM);
#pragma unroll
        for (int iR = 0; iR < RIW; ++iR) {
            const int i0 = 16 * (wave * RIW + iR);
            Frag<T> qa[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const int rb = 32 * ks + rA;
                qa[ks] = join_frag<T>(lds_read_tr(&tQw[bf][rb * LDQ + i0 + cA]), lds_read_tr(&tQw[bf][(rb + 4) * LDQ + i0 + cA]));
                // tokens 32 ks + 8 grp .. + 7 were staged by wave 2 ks + grp / 2
                if constexpr (Elt<T>::kScaled) qa[ks] = scale_frag<T>(qa[ks], ldexpf(1.f, sM - sExpQ[bf][2 * ks + (grp >> 1)]));
            }
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb) {
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    const int rb = 32 * ks + rA;
                    const Frag<T> bd = join_frag<T>(lds_read_tr(&tD[bf][rb * LDV + 16 * jb + cA]),
                                                    lds_read_tr(&tD[bf][(rb + 4) * LDV + 16 * jb + cA]));
                    t = mma(qa[ks], bd, t);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) accG[iR][jb][r] += t[r] * uM;
            }
        }
    };
    auto body = [&](Stage& st, int c) {
        const int64_t row0 = (int64_t)c * C;
        publish();
        consume(st, c);
        __syncthreads();  // tiles of chunk c, R^T and z are visible
        sched_fence();
        issue(st, c + 1);  // past the segment end these read zeros
        sched_fence();

        // (a) a^T[s][t] = phi(k_s) . phi(q_t) and b^T[s][t] = v_s . dO_t for the
        // wave's query rows t = 16 wave + m (one per lane) and the keys
        // s = 16 sb + 4 grp + r of block sb (the lane's four values). With s
        // along a lane's values these results are already operands of the
        // contraction over s in (d). Slot i holds key block sb = (wave - i)
        // mod 4: slot 0 is the diagonal block (masked to s <= t), slots
        // 1 .. wave lie below it, and the slots past wave stay zero.
        f32x4 aa[NBC], bb[NBC];
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            aa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            bb[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        Frag<T> fd[KSV];  // dO row t
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
            fd[ks] = *reinterpret_cast<const Frag<T>*>(&tD[c % NBUF][(16 * wave + m) * LDV + 32 * ks + 8 * grp]);
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
            const Frag<T> bq = *reinterpret_cast<const Frag<T>*>(&tQ[(16 * wave + m) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
            for (int i = 0; i < NBC; ++i)
                if (i <= wave)
                    aa[i] = mma(*reinterpret_cast<const Frag<T>*>(&tK[(16 * (wave - i) + m) * LDK + 32 * ks + 8 * grp]),
                                bq, aa[i]);
        }
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
#pragma unroll
            for (int i = 0; i < NBC; ++i)
                if (i <= wave)
                    bb[i] = mma(*reinterpret_cast<const Frag<T>*>(&tV[(16 * (wave - i) + m) * LDV + 32 * ks + 8 * grp]),
                                fd[ks], bb[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool above = 4 * grp + r > m;
            aa[0][r] = above ? 0.f : aa[0][r];
            bb[0][r] = above ? 0.f : bb[0][r];
        }

        // (b) Y^T = R dO^T: rows i = 16 ib + 4 grp + r, column t; unscaled per
        // row block
        f32x4 Y[NBI];
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib) Y[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
            const int rb = 32 * ks + rA;
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib) {
                const Frag<T> ar = join_frag<T>(lds_read_tr(&tRT[rb * LDRT + 16 * ib + cA]),
                                                lds_read_tr(&tRT[(rb + 4) * LDRT + 16 * ib + cA]));
                Y[ib] = mma(ar, fd[ks], Y[ib]);
            }
        }
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib) {
            const float uR = ldexpf(1.f, -sExpR[ib / RIW]);
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[ib][r] *= uR;
        }

        // (c) phi(q_t) at the lane's features i = 16 ib + 4 grp + r (one
        // 8-byte read per block); den, w and c of the lane's query row: the
        // lane's partial sums, then over the four lane groups (every lane of
        // a row gets the same bits: the additions commute pairwise)
        float ph[NBI][4];
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            const t4 x = *reinterpret_cast<const t4*>(&tQ[(16 * wave + m) * LDK + 16 * ib + 4 * grp]);
#pragma unroll
            for (int r = 0; r < 4; ++r) ph[ib][r] = to_f32(x[r]);
        }
        const bool okt = row0 + 16 * wave + m < len;
        float w, cw;  // w_t and c_t of the lane's query row
        if constexpr (SIMPLE) {
            w = okt ? eps : 0.f;  // simple_la: eps carries the query scale
            cw = 0.f;
        } else {
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int i = NBC - 1; i >= 0; --i)
                if (i <= wave)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        sa += aa[i][r];
                        sb += aa[i][r] * bb[i][r];
                    }
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib) {
                const float4 z4 = *reinterpret_cast<const float4*>(&sZ[16 * ib + 4 * grp]);
                const float zr[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sa += ph[ib][r] * zr[r];
                    sb += ph[ib][r] * Y[ib][r];
                }
            }
            sa += __shfl_xor(sa, 16);
            sb += __shfl_xor(sb, 16);
            sa += __shfl_xor(sa, 32);
            sb += __shfl_xor(sb, 32);
            const float inv = __builtin_amdgcn_rcpf(sa + eps);  // v_rcp_f32, 1 ulp
            w = okt ? inv : 0.f;
            cw = okt ? -sb * inv * inv : 0.f;
            // w and c^ = c / w of row t, by the lanes of group 0
            if (grp == 0 && okt)
                *reinterpret_cast<float2*>(&wcb[2 * (row0 + 16 * wave + m)]) = make_float2(inv, -sb * inv);
        }

        // (d) P^T = mask(w b^T + c) in the slots of (a), rounded with a power of
        // two to operands over the keys of slots 2 ks and 2 ks + 1 (values
        // 0..3 of a lane from the first, 4..7 from the second), times phi(K)
        f32x4 pp[NBC];
        float pmx = 0.f;
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            pp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i <= wave) {  // blocks above the diagonal stay zero
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = SIMPLE ? bb[i][r] : w * bb[i][r] + cw;
                    pp[i][r] = i > 0 || 4 * grp + r <= m ? x : 0.f;
                    pmx = fmaxf(pmx, fabsf(pp[i][r]));
                }
            }
        }
        int sP = 0;
        if constexpr (Elt<T>::kScaled) sP = scale_exp(wave_max_nonneg(pmx));
        Frag<T> bP[KSC];
        {
            const float fP = ldexpf(1.f, sP);
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    bP[ks][r] = static_cast<T>(pp[2 * ks][r] * fP);
                    bP[ks][4 + r] = static_cast<T>(pp[2 * ks + 1][r] * fP);
                }
        }
        // pk^T = phi(K)^T P^T: rows i = 16 ib + 4 grp + r, column t
        f32x4 pk[NBI];
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib) pk[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int rT = 4 * grp + (m >> 2), cT = 4 * (m & 3);
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            if (2 * ks <= wave) {  // otherwise both slots lie above the diagonal
                const int r0 = 16 * ((wave - 2 * ks) & (NBC - 1)) + rT;
                const int r1 = 16 * ((wave - 2 * ks - 1) & (NBC - 1)) + rT;
#pragma unroll
                for (int ib = 0; ib < NBI; ++ib) {
                    const Frag<T> ak = join_frag<T>(lds_read_tr(&tK[r0 * LDK + 16 * ib + cT]),
                                                    lds_read_tr(&tK[r1 * LDK + 16 * ib + cT]));
                    pk[ib] = mma(ak, bP[ks], pk[ib]);
                }
            }
        }

        // (e) dQ^T = (w Y^T + c z + pk^T) phi'(q): the lane's four features of
        // row t, one 8-byte store per block
        {
            const float uP = ldexpf(1.f, -sP);
            const int64_t row = row0 + 16 * wave + m;
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib) {
                float zr[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (!SIMPLE) {
                    const float4 z4 = *reinterpret_cast<const float4*>(&sZ[16 * ib + 4 * grp]);
                    zr[0] = z4.x;
                    zr[1] = z4.y;
                    zr[2] = z4.z;
                    zr[3] = z4.w;
                }
                f32x4 g;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float d = SIMPLE ? w * (Y[ib][r] + pk[ib][r] * uP) : w * Y[ib][r] + cw * zr[r] + pk[ib][r] * uP;
                    g[r] = d * dphi_of<FM>(ph[ib][r]);
                }
                const int col = 16 * ib + 4 * grp;
                buf_store4<T>(bdq, pad_off<DK, DKR>(buf_off<T>(row, lay.dq.rs, col), col), g);
            }
        }

        // (f) R += phi(K)^T V and z += sum phi(k) on this wave's rows of R
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            const int rb = 32 * ks + rA;
            Frag<T> bvf[NBV];
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb)
                bvf[jb] = join_frag<T>(lds_read_tr(&tV[rb * LDV + 16 * jb + cA]),
                                       lds_read_tr(&tV[(rb + 4) * LDV + 16 * jb + cA]));
#pragma unroll
            for (int iR = 0; iR < RIW; ++iR) {
                const int i0 = 16 * (wave * RIW + iR);
                const Frag<T> a = join_frag<T>(lds_read_tr(&tK[rb * LDK + i0 + cA]),
                                               lds_read_tr(&tK[(rb + 4) * LDK + i0 + cA]));
#pragma unroll
                for (int jb = 0; jb < NBV; ++jb) accR[iR][jb] = mma(a, bvf[jb], accR[iR][jb]);
                if constexpr (!SIMPLE) accZ[iR] = mma(a, ones, accZ[iR]);
            }
        }

        // (g) Qw = w phi(q) of the wave's query rows into the Qw tile (rows t,
        // features i: one 8-byte store per block); c phi(q) into gzp
        {
            f32x4 qw[NBI];
            float qmx = 0.f;
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    qw[ib][r] = ph[ib][r] * w;
                    qmx = fmaxf(qmx, fabsf(qw[ib][r]));
                }
            int sQ = 0;
            if constexpr (Elt<T>::kScaled) sQ = scale_exp_for_min(wave_max_nonneg(qmx));
            const float fQ = ldexpf(1.f, sQ);
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib) put4t(&tQw[c % NBUF][(16 * wave + m) * LDQ + 16 * ib + 4 * grp], qw[ib], fQ);
            if (lane == 0) sExpQ[c % NBUF][wave] = sQ;
            if constexpr (!SIMPLE) {
#pragma unroll
                for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
                    for (int r = 0; r < 4; ++r) gzp[ib][r] += cw * ph[ib][r];
            }
        }
        if constexpr (kDefer) {
            if (c > 0) gupdate(c - 1);  // its tiles are the other buffers
        } else {
            __syncthreads();  // the Qw tile and its four exponents are visible
            gupdate(c);
        }
        __syncthreads();  // every wave is done with this chunk's tiles, R^T, z and the older Qw, dO tiles
    };
    // One chunk of loads in flight (a chunk's work outlasts the load latency
    // many times over; a second stage only adds registers). The chunk count is
    // even (the K/V scan indexes the exponents the same way); a chunk past the
    // segment end reads zeros, adds nothing and stores nothing.
    if (nchunks > 0) {
        Stage st;
        issue(st, 0);
        sched_fence();
        for (int c = 0; c < nchunks; ++c) body(st, c);
        if constexpr (kDefer) gupdate(nchunks - 1);  // after the last chunk's closing barrier
    }
    if (gpart != nullptr) {
        float* gp = gpart + (bh * P + p) * (int64_t)(DKR * DVR + DKR);
#pragma unroll
        for (int iR = 0; iR < RIW; ++iR) {
            const int i0 = 16 * (wave * RIW + iR) + 4 * grp;
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (i0 + r < DKR && 16 * jb + m < DVR) gp[(i0 + r) * DVR + 16 * jb + m] = accG[iR][jb][r];
        }
        // g: the lanes' sums over their query rows (the 16 lanes of a group),
        // then over the four waves in order
        float* red = reinterpret_cast<float*>(tQ);  // free after the last barrier
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = row16_sum(gzp[ib][r]);
                if (m == 0) red[wave * DK + 16 * ib + 4 * grp + r] = x;
            }
        __syncthreads();
        if (tid < DKR) gp[DKR * DVR + tid] = ((red[tid] + red[DK + tid]) + red[2 * DK + tid]) + red[3 * DK + tid];
    }
}

// Exclusive suffix of the P partial (G, g) blocks of every head, in place:
// block p becomes the sum of blocks p + 1 .. P - 1, added from the last down.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void suffix_kernel(float* __restrict__ part, int P, int64_t BH) {
    constexpr int E4 = (DK * DV + DK) / 4;
    constexpr int BPH = (E4 + kThreads - 1) / kThreads;
    const int64_t bh = blockIdx.x / BPH;
    const int i = (blockIdx.x % BPH) * kThreads + threadIdx.x;
    if (bh >= BH || i >= E4) return;
    float4* pb = reinterpret_cast<float4*>(part) + bh * (int64_t)P * E4 + i;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p1 = P; p1 > 0; p1 -= 8) {
        float4 x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = pb[(int64_t)max(p1 - 1 - j, 0) * E4];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (p1 - 1 - j >= 0) {
                pb[(int64_t)(p1 - 1 - j) * E4] = acc;
                acc.x += x[j].x;
                acc.y += x[j].y;
                acc.z += x[j].z;
                acc.w += x[j].w;
            }
    }
}

// Reverse-order scan of one segment: dK and dV. The four waves each own 16
// key rows of the chunk and a quarter of the rows of G. Qw = w phi(q) is
// staged at the exponent bwd_causal_q_kernel chose for the chunk. Per chunk:
//   (a) a~[s][t] = phi(k_s) . Qw_t and b[s][t] = v_s . dO_t for t >= s;
//   (b) dK = ((mask(b + c^) Qw) + V G^T + g) phi'(k): the first product
//       from the transposed staging of mask(b + c^), V G^T from G^T in LDS
//       (one power of two per owner wave, constant along each result column);
//   (c) dV = a~ dO + phi(K) G: phi(K) G sums over the owners' quarters, so
//       the A operand is rescaled per quarter to the smallest exponent;
//   (d) G += Qw^T dO, g += Qw^T c^ on the wave's rows of G.
// G^T and g are published at the top of the next chunk. Two barriers per chunk.
template <typename T, int DK, int DV, bool SIMPLE, int FM, int DKR = DK, int DVR = DV>
__global__ __launch_bounds__(kThreads, (CausalBwdShape<DK, DV>::kMinBlocks)) void bwd_causal_kv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ wc, const int* __restrict__ es, const float* __restrict__ suf, T* __restrict__ dk,
    T* __restrict__ dv, int64_t T_, const Layouts lay, int P, int64_t L, int nche, float qscale) {
    using Sh = CausalBwdShape<DK, DV>;
    constexpr int C = Sh::kChunk, LDK = Sh::kLDK, LDV = Sh::kLDV, LDRT = Sh::kLDRT;
    constexpr int NBI = DK / 16, NBV = DV / 16, NBC = C / 16;
    constexpr int RIW = DK / 64;
    constexpr int KSK = DK / 32, KSV = DV / 32, KSC = C / 32;
    constexpr int CK = DK / 8, CV = DV / 8;
    constexpr int NCK = C * CK / kThreads, NCV = C * CV / kThreads;
    constexpr int QW = DK / 4;  // columns of G^T per owner wave
    static_assert(sizeof(T) == 2, "transposed LDS reads take 16-bit elements");
    static_assert(NCK * kThreads == C * CK && NCV * kThreads == C * CV, "tiles must split evenly");
    static_assert(RIW >= 1 && RIW * 64 == DK, "each wave owns whole 16-row blocks");
    __shared__ __attribute__((aligned(16))) T tQ[C * LDK];  // Qw, scaled
    __shared__ __attribute__((aligned(16))) T tK[C * LDK];
    __shared__ __attribute__((aligned(16))) T tV[C * LDV];
    __shared__ __attribute__((aligned(16))) T tD[C * LDV];
    __shared__ __attribute__((aligned(16))) T tGT[DV * LDRT];
    __shared__ __attribute__((aligned(16))) float sGz[DK];
    __shared__ __attribute__((aligned(16))) float sC[C];
    __shared__ __attribute__((aligned(16))) T sCh[C];  // c^ as 16-bit operands, scaled by 2^scale_exp(max |c^|)
    __shared__ int sExpG[kWaves];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const int64_t len = t1 - t0;
    const int nreal = (int)(len > 0 ? (len + C - 1) / C : 0);
    const int nchunks = (nreal + 1) / 2 * 2;
    const Layout lq = lay.q, lk = lay.k, lv = lay.v, ld = lay.dout;

    f32x4 accG[RIW][NBV], accGz[RIW];
    {
        const float* pG = suf != nullptr ? suf + (bh * P + p) * (int64_t)(DKR * DVR + DKR) : nullptr;
#pragma unroll
        for (int iR = 0; iR < RIW; ++iR) {
            const int i0 = 16 * (wave * RIW + iR) + 4 * grp;
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    accG[iR][jb][r] = (pG && i0 + r < DKR && 16 * jb + m < DVR) ? pG[(i0 + r) * DVR + 16 * jb + m] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) accGz[iR][r] = (pG && i0 + r < DKR) ? pG[DKR * DVR + i0 + r] : 0.f;
        }
    }

    auto publish = [&]() {
        int sG = 0;
        if constexpr (Elt<T>::kScaled) {
            float mx = 0.f;
#pragma unroll
            for (int iR = 0; iR < RIW; ++iR)
#pragma unroll
                for (int jb = 0; jb < NBV; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(accG[iR][jb][r]));
            sG = scale_exp_for_min(wave_max_nonneg(mx));
        }
        const float fG = ldexpf(1.f, sG);
#pragma unroll
        for (int iR = 0; iR < RIW; ++iR)
#pragma unroll
            for (int jb = 0; jb < NBV; ++jb)
                put4t(&tGT[(16 * jb + m) * LDRT + 16 * (wave * RIW + iR) + 4 * grp], accG[iR][jb], fG);
        if (lane == 0) sExpG[wave] = sG;
        if constexpr (!SIMPLE) {
            if (m == 0)
#pragma unroll
                for (int iR = 0; iR < RIW; ++iR)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sGz[16 * (wave * RIW + iR) + 4 * grp + r] = accGz[iR][r];
        }
    };

    struct Stage {
        u32x4 q[NCK], k[NCK], v[NCV], d[NCV];
        unsigned w, ch;  // w and c^ of token `lane` of the chunk
        int es;
    };
    const HeadBuf bq = slice_buf(q, lq, bh, DKR, t0, t1), bk = slice_buf(k, lk, bh, DKR, t0, t1);
    const HeadBuf bv = slice_buf(v, lv, bh, DVR, t0, t1), bd = slice_buf(dout, ld, bh, DVR, t0, t1);
    const HeadBuf bdk = slice_buf(dk, lay.dk, bh, DKR, t0, t1), bdv = slice_buf(dv, lay.dv, bh, DVR, t0, t1);
    // w and c^ of the segment's tokens (8 bytes each); zeros past the end
    const HeadBuf bwc{__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(wc + 2 * (bh * T_ + t0)), 0,
                                                        (int)(len > 0 ? 8 * len : 0), 0x00020000)};
    const int* esb = es + (bh * P + p) * (int64_t)nche;
    // step n of the walk visits chunk nchunks - 1 - n; the prefetch after the
    // first chunk goes to a chunk past the segment end, which reads zeros
    auto chunk_of = [&](int n) { return n < nchunks ? nchunks - 1 - n : n; };
    auto issue = [&](Stage& st, int n) {
        const int c = chunk_of(n);
        const int64_t row0 = (int64_t)c * C;
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int nn = tid + kThreads * i, r = nn / CK, cc = nn % CK;
            st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, pad_off<DK, DKR>(buf_off<T>(row0 + r, lq.rs, 8 * cc), 8 * cc), 0, 0);
            st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, pad_off<DK, DKR>(buf_off<T>(row0 + r, lk.rs, 8 * cc), 8 * cc), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int nn = tid + kThreads * i, r = nn / CV, cc = nn % CV;
            st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(bv.rsrc, pad_off<DV, DVR>(buf_off<T>(row0 + r, lv.rs, 8 * cc), 8 * cc), 0, 0);
            st.d[i] = __builtin_amdgcn_raw_buffer_load_b128(bd.rsrc, pad_off<DV, DVR>(buf_off<T>(row0 + r, ld.rs, 8 * cc), 8 * cc), 0, 0);
        }
        if constexpr (!SIMPLE) {
            // two dword loads: the 8-byte buffer-load builtin drops the upper dword with this compiler
            const int off = (int)((uint32_t)(row0 + lane) * 8u);
            st.w = __builtin_amdgcn_raw_buffer_load_b32(bwc.rsrc, off, 0, 0);
            st.ch = __builtin_amdgcn_raw_buffer_load_b32(bwc.rsrc, off + 4, 0, 0);
        }
        // the exponent of a written chunk (chunks past the end hold zeros, any finite scale will do)
        st.es = nreal > 0 ? esb[min(c, nreal - 1)] : 0;
    };
    // returns the chunk's Qw exponent
    auto consume = [&](const Stage& st, int n, float& cmx) -> int {
        const int c = chunk_of(n);
        const int64_t row0 = (int64_t)c * C;
        const int sQ = st.es;
        const float fQ = ldexpf(1.f, sQ);
        float wl = 1.f, cl = 0.f;
        if constexpr (!SIMPLE) {
            wl = __builtin_bit_cast(float, st.w);
            cl = __builtin_bit_cast(float, st.ch);
        }
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int nn = tid + kThreads * i, r = nn / CK, cc = nn % CK;
            // rows past the segment end and padded feature columns add nothing
            const bool ok = (DKR == DK || 8 * cc < DKR) && row0 + r < len;
            float wt = qscale;  // simple_la: w is the query scale
            if constexpr (!SIMPLE) wt = __shfl(wl, r);
            const float f = ok ? wt * fQ : 0.f;
            float pq[8];
            phi8_f32<FM, T>(st.q[i], pq);
            Row<T, 8> qt;
#pragma unroll
            for (int e = 0; e < 8; ++e) qt.e[e] = static_cast<T>(pq[e] * f);
            *reinterpret_cast<Row<T, 8>*>(&tQ[r * LDK + 8 * cc]) = qt;
            *reinterpret_cast<u32x4*>(&tK[r * LDK + 8 * cc]) = keep_or_zero(phi8<FM, T>(st.k[i]), ok);
        }
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int nn = tid + kThreads * i, r = nn / CV, cc = nn % CV;
            *reinterpret_cast<u32x4*>(&tV[r * LDV + 8 * cc]) = st.v[i];
            *reinterpret_cast<u32x4*>(&tD[r * LDV + 8 * cc]) = st.d[i];
        }
        if constexpr (!SIMPLE) {
            cmx = wave_max_nonneg(fabsf(cl));  // the same in every wave
            if (wave == 0) {
                int sC2 = 0;
                if constexpr (Elt<T>::kScaled) sC2 = scale_exp(cmx);
                sC[lane] = cl;
                sCh[lane] = static_cast<T>(cl * ldexpf(1.f, sC2));
            }
        }
        return sQ;
    };

    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    auto body = [&](Stage& st, int n) {
        const int c = chunk_of(n);
        const int64_t row0 = (int64_t)c * C;
        publish();
        float cmx = 0.f;
        const int sQ = consume(st, n, cmx);
        __syncthreads();  // tiles, G^T and g are visible
        sched_fence();
        issue(st, n + 1);
        sched_fence();
        const float uQ = ldexpf(1.f, -sQ);

        // (a) a~^T[t][s] = Qw_t . phi(k_s) and b^T[t][s] = dO_t . v_s for the
        // wave's keys s = 16 wave + m (one per lane) and the queries
        // t = 16 tb + 4 grp + r of block tb (the lane's four values): with t
        // along a lane's values these results are already operands of the
        // contractions over t in (b) and (c). Slot i holds query block
        // tb = wave + i: slot 0 is the diagonal block (masked to t >= s), and
        // the slots with wave + i past the last block stay zero.
        f32x4 aa[NBC], bb[NBC];
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            aa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            bb[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        Frag<T> fk[KSK], fv[KSV];  // phi(k_s), v_s
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
            fk[ks] = *reinterpret_cast<const Frag<T>*>(&tK[(16 * wave + m) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
            fv[ks] = *reinterpret_cast<const Frag<T>*>(&tV[(16 * wave + m) * LDV + 32 * ks + 8 * grp]);
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
#pragma unroll
            for (int i = 0; i < NBC; ++i)
                if (wave + i < NBC)
                    aa[i] = mma(*reinterpret_cast<const Frag<T>*>(&tQ[(16 * (wave + i) + m) * LDK + 32 * ks + 8 * grp]),
                                fk[ks], aa[i]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
#pragma unroll
            for (int i = 0; i < NBC; ++i)
                if (wave + i < NBC)
                    bb[i] = mma(*reinterpret_cast<const Frag<T>*>(&tD[(16 * (wave + i) + m) * LDV + 32 * ks + 8 * grp]),
                                fv[ks], bb[i]);
        float pmx = 0.f, amx = 0.f;
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            if (wave + i >= NBC) continue;  // below the diagonal: never computed, stay zero
            float ch[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (!SIMPLE) {
                const float4 c4 = *reinterpret_cast<const float4*>(&sC[16 * (wave + i) + 4 * grp]);
                ch[0] = c4.x;
                ch[1] = c4.y;
                ch[2] = c4.z;
                ch[3] = c4.w;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = i > 0 || 4 * grp + r >= m;
                aa[i][r] = keep ? aa[i][r] : 0.f;
                bb[i][r] = keep ? bb[i][r] + ch[r] : 0.f;  // now mask(b + c^)
                pmx = fmaxf(pmx, fabsf(bb[i][r]));
                amx = fmaxf(amx, fabsf(aa[i][r]));
            }
        }
        // phi(k_s) at the lane's features i = 16 ib + 4 grp + r
        float pk[NBI][4];
#pragma unroll
        for (int ib = 0; ib < NBI; ++ib) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            const t4 x = *reinterpret_cast<const t4*>(&tK[(16 * wave + m) * LDK + 16 * ib + 4 * grp]);
#pragma unroll
            for (int r = 0; r < 4; ++r) pk[ib][r] = to_f32(x[r]);
        }
        // operands over the queries of slots 2 ks and 2 ks + 1 (values 0..3 of
        // a lane from the first, 4..7 from the second), read transposed from a
        // query-major tile with the same order
        const int rT = 4 * grp + (m >> 2), cT = 4 * (m & 3);
        auto pack = [&](const f32x4 (&x)[NBC], int sx, Frag<T> (&f)[KSC]) {
            const float fx = ldexpf(1.f, sx);
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f[ks][r] = static_cast<T>(x[2 * ks][r] * fx);
                    f[ks][4 + r] = static_cast<T>(x[2 * ks + 1][r] * fx);
                }
        };
        const int64_t srow = row0 + 16 * wave + m;

        // (b) dK^T = Qw^T mask(b + c^)^T + G V^T + g, times phi'(k): rows i, column s
        {
            int sP = 0;
            if constexpr (Elt<T>::kScaled) sP = scale_exp(wave_max_nonneg(pmx));
            Frag<T> bP[KSC];
            pack(bb, sP, bP);
            f32x4 x1[NBI], x2[NBI];
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib) {
                x1[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
                x2[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                if (wave + 2 * ks < NBC) {  // otherwise both slots lie below the diagonal
                    const int r0 = 16 * ((wave + 2 * ks) & (NBC - 1)) + rT;
                    const int r1 = 16 * ((wave + 2 * ks + 1) & (NBC - 1)) + rT;
#pragma unroll
                    for (int ib = 0; ib < NBI; ++ib) {
                        const Frag<T> aq = join_frag<T>(lds_read_tr(&tQ[r0 * LDK + 16 * ib + cT]),
                                                        lds_read_tr(&tQ[r1 * LDK + 16 * ib + cT]));
                        x1[ib] = mma(aq, bP[ks], x1[ib]);
                    }
                }
            }
#pragma unroll
            for (int ks = 0; ks < KSV; ++ks) {
                const int rb = 32 * ks + rA;
#pragma unroll
                for (int ib = 0; ib < NBI; ++ib) {
                    const Frag<T> ag = join_frag<T>(lds_read_tr(&tGT[rb * LDRT + 16 * ib + cA]),
                                                    lds_read_tr(&tGT[(rb + 4) * LDRT + 16 * ib + cA]));
                    x2[ib] = mma(ag, fv[ks], x2[ib]);
                }
            }
            const float u1 = ldexpf(1.f, -sP) * uQ;
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib) {
                const float u2 = ldexpf(1.f, -sExpG[ib / RIW]);
                float gz[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (!SIMPLE) {
                    const float4 g4 = *reinterpret_cast<const float4*>(&sGz[16 * ib + 4 * grp]);
                    gz[0] = g4.x;
                    gz[1] = g4.y;
                    gz[2] = g4.z;
                    gz[3] = g4.w;
                }
                f32x4 g;
#pragma unroll
                for (int r = 0; r < 4; ++r) g[r] = (x1[ib][r] * u1 + x2[ib][r] * u2 + gz[r]) * dphi_of<FM>(pk[ib][r]);
                const int col = 16 * ib + 4 * grp;
                buf_store4<T>(bdk, pad_off<DK, DKR>(buf_off<T>(srow, lay.dk.rs, col), col), g);
            }
        }

        // (c) dV^T = dO^T a~^T + G^T phi(K)^T: rows j, column s
        {
            int sA = 0;
            if constexpr (Elt<T>::kScaled) sA = scale_exp(wave_max_nonneg(amx));
            Frag<T> bA[KSC];
            pack(aa, sA, bA);
            f32x4 y1[NBV], y2[NBV];
#pragma unroll
            for (int jv = 0; jv < NBV; ++jv) {
                y1[jv] = f32x4{0.f, 0.f, 0.f, 0.f};
                y2[jv] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                if (wave + 2 * ks < NBC) {
                    const int r0 = 16 * ((wave + 2 * ks) & (NBC - 1)) + rT;
                    const int r1 = 16 * ((wave + 2 * ks + 1) & (NBC - 1)) + rT;
#pragma unroll
                    for (int jv = 0; jv < NBV; ++jv) {
                        const Frag<T> ad = join_frag<T>(lds_read_tr(&tD[r0 * LDV + 16 * jv + cT]),
                                                        lds_read_tr(&tD[r1 * LDV + 16 * jv + cT]));
                        y1[jv] = mma(ad, bA[ks], y1[jv]);
                    }
                }
            }
            int sM = 0;
            if constexpr (Elt<T>::kScaled) sM = min(min(sExpG[0], sExpG[1]), min(sExpG[2], sExpG[3]));
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) {
                // features 32 ks + 8 grp .. + 7 of G^T were published by wave (32 ks + 8 grp) / QW
                Frag<T> b = fk[ks];
                if constexpr (Elt<T>::kScaled) b = scale_frag<T>(b, ldexpf(1.f, sM - sExpG[(32 * ks + 8 * grp) / QW]));
#pragma unroll
                for (int jv = 0; jv < NBV; ++jv)
                    y2[jv] = mma(*reinterpret_cast<const Frag<T>*>(&tGT[(16 * jv + m) * LDRT + 32 * ks + 8 * grp]), b,
                                 y2[jv]);
            }
            const float u1 = ldexpf(1.f, -sA) * uQ, u2 = ldexpf(1.f, -sM);
#pragma unroll
            for (int jv = 0; jv < NBV; ++jv) {
                f32x4 g;
#pragma unroll
                for (int r = 0; r < 4; ++r) g[r] = y1[jv][r] * u1 + y2[jv][r] * u2;
                const int col = 16 * jv + 4 * grp;
                buf_store4<T>(bdv, pad_off<DV, DVR>(buf_off<T>(srow, lay.dv.rs, col), col), g);
            }
        }

        // (d) G += Qw^T dO, g += Qw^T c^ on this wave's rows of G
        {
            int sC2 = 0;
            if constexpr (!SIMPLE && Elt<T>::kScaled) sC2 = scale_exp(cmx);  // the scale of sCh
#pragma unroll
            for (int iR = 0; iR < RIW; ++iR) {
                const int i0 = 16 * (wave * RIW + iR);
                Frag<T> qa[KSC];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    const int rb = 32 * ks + rA;
                    qa[ks] = join_frag<T>(lds_read_tr(&tQ[rb * LDK + i0 + cA]), lds_read_tr(&tQ[(rb + 4) * LDK + i0 + cA]));
                }
#pragma unroll
                for (int jv = 0; jv < NBV; ++jv) {
                    f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) {
                        const int rb = 32 * ks + rA;
                        const Frag<T> b = join_frag<T>(lds_read_tr(&tD[rb * LDV + 16 * jv + cA]),
                                                       lds_read_tr(&tD[(rb + 4) * LDV + 16 * jv + cA]));
                        t = mma(qa[ks], b, t);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) accG[iR][jv][r] += t[r] * uQ;
                }
                if constexpr (!SIMPLE) {
                    f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) {
                        const Frag<T> cf = *reinterpret_cast<const Frag<T>*>(&sCh[32 * ks + 8 * grp]);
                        t = mma(qa[ks], cf, t);
                    }
                    const float u = uQ * ldexpf(1.f, -sC2);
#pragma unroll
                    for (int r = 0; r < 4; ++r) accGz[iR][r] += t[r] * u;
                }
            }
        }
        __syncthreads();  // every wave is done with the tiles, G^T and g
    };
    if (nchunks > 0) {
        Stage st;
        issue(st, 0);
        sched_fence();
        for (int n = 0; n < nchunks; ++n) body(st, n);
    }
}

// ---------------------------------------------------------------------------
// Causal scans on fp32 operands (fp32 inputs, every head size up to 128).
// ---------------------------------------------------------------------------
// The same recurrences, segments, prefix and suffix kernels and workspace as
// the 16-bit scans, in a plainer form. A chunk's tiles are staged in LDS as
// fp32 (phi applied on the way, rows past the segment end zeroed), the running
// state (R, z forward; G, g in the reverse scan) stays in LDS, and every
// product is cut into 16 x 16 result tiles dealt round-robin to the four
// waves, each tile a chain of 16x16x4 fp32 MFMAs reading both operands from
// LDS. fp32 MFMA runs at the fp32 vector rate, so these scans are bound by
// their products (about 4 D Dv + 2 C (D + Dv) multiply-adds per token), not by
// HBM. Chunks are 32 tokens: a 128 x 128 fp32 state plus the chunk's tiles
// fit one workgroup's LDS. The next chunk's loads are in flight in registers
// while a chunk is processed.
struct CF {
    static constexpr int C = 32;             // tokens per chunk (kThreads / 8: eight lanes per row)
    static constexpr int NT = C / 16;        // 16-token blocks per chunk
    static constexpr int NL = NT * (NT + 1) / 2;  // blocks on or below the diagonal
    static constexpr int LC = C + 4;         // row stride of C x C tiles (floats)
};
static_assert(CF::C * 8 == kThreads, "the per-row steps take eight lanes per row");

// Block (tb, sb), sb <= tb, of the n-th block on or below the diagonal.
__device__ __forceinline__ void lower_block(int n, int& tb, int& sb) {
    tb = 0;
    while (n > tb) {
        n -= tb + 1;
        ++tb;
    }
    sb = n;
}

// acc[m][n] += sum_{k0 <= k < k1} X(m, k) Y(n, k) over one 16 x 16 tile on
// 16x16x4 fp32 MFMA. X(m, k) = x[m ldx + k] when XK (k contiguous), else
// x[k ldx + m]; the same for Y. With XS, X(m, k) is also multiplied by xs[k].
// Lane (m, g) = (lane % 16, lane / 16) feeds k = k' + 4 g + e to the e-th
// MFMA of each 16-wide step k' (the same permutation of the contraction index
// for both operands). k0 and k1 are multiples of 16. The result sits in the
// MFMA layout: lane (m, g), register r holds row 4 g + r, column m.
template <bool XK, bool YK, bool XS = false>
__device__ __forceinline__ f32x4 tile_f32(f32x4 acc, const float* x, int ldx, const float* y, int ldy, int k0,
                                          int k1, const float* xs = nullptr) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll 2
    for (int kk = k0; kk < k1; kk += 16) {
        const int k = kk + 4 * g;
        float a[4], b[4];
        if constexpr (XK) {
            const float4 t = *reinterpret_cast<const float4*>(x + m * ldx + k);
            a[0] = t.x, a[1] = t.y, a[2] = t.z, a[3] = t.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = x[(k + e) * ldx + m];
        }
        if constexpr (YK) {
            const float4 t = *reinterpret_cast<const float4*>(y + m * ldy + k);
            b[0] = t.x, b[1] = t.y, b[2] = t.z, b[3] = t.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = y[(k + e) * ldy + m];
        }
        if constexpr (XS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] *= xs[k + e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    }
    return acc;
}

// One chunk (CF::C rows of W elements) of a tensor in flight: 16-byte pieces
// dealt over the workgroup's threads, loaded unconditionally through the
// segment's buffer descriptor (rows past its end read zeros).
template <typename T, int W>
struct ChunkLoad {
    static constexpr int VEC = 16 / (int)sizeof(T), PPR = W / VEC, NP = CF::C * PPR;
    static constexpr int NPT = (NP + kThreads - 1) / kThreads;
    u32x4 x[NPT];
    __device__ __forceinline__ void issue(const HeadBuf& b, int64_t rs, int64_t row0) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int n = min((int)threadIdx.x + kThreads * i, NP - 1);
            x[i] = __builtin_amdgcn_raw_buffer_load_b128(b.rsrc, buf_off<T>(row0 + n / PPR, rs, VEC * (n % PPR)), 0, 0);
        }
    }
    // Row r, element j of the chunk goes to dst[r ld + j] as f(r, value).
    template <typename F>
    __device__ __forceinline__ void put(float* dst, int ld, F f) const {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int n = (int)threadIdx.x + kThreads * i;
            if (NP % kThreads == 0 || n < NP) {
                const int r = n / PPR, c0 = VEC * (n % PPR);
                const T* e = reinterpret_cast<const T*>(&x[i]);
                float y[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) y[j] = f(r, to_f32(e[j]));
#pragma unroll
                for (int j = 0; j < VEC; j += 4)
                    *reinterpret_cast<float4*>(dst + r * ld + c0 + j) = make_float4(y[j], y[j + 1], y[j + 2], y[j + 3]);
            }
        }
    }
};

// Rows [0, CF::C) of an fp32 LDS tile (row stride ld) rounded to T and stored
// as 16-byte pieces at rows row0.. of a segment (rows past its end dropped).
template <typename T, int W>
__device__ __forceinline__ void store_chunk(const float* src, int ld, const HeadBuf& b, int64_t rs, int64_t row0) {
    constexpr int VEC = 16 / (int)sizeof(T), PPR = W / VEC, NP = CF::C * PPR;
    for (int n = threadIdx.x; n < NP; n += kThreads) {
        const int r = n / PPR, c0 = VEC * (n % PPR);
        Row<T, VEC> out;
#pragma unroll
        for (int j = 0; j < VEC; ++j) out.e[j] = static_cast<T>(src[r * ld + c0 + j]);
        buf_store16(b, buf_off<T>(row0 + r, rs, c0), *reinterpret_cast<const uint4*>(out.e));
    }
}

// Causal forward, fp32 operands: one workgroup per segment, 32-token chunks
// in order. Per chunk, with R, z the state before it:
//   A = mask(phi(Q) phi(K)^T) (s <= t), 1/den_t = 1 / (phi(q_t) . z + sum_s A_ts + eps),
//   O = (phi(Q) R + A V) / den (simple_la: times the query scale instead),
//   R += phi(K)^T V, z += sum_s phi(k_s).
template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__(kThreads) void fwd_causal_f32_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ pre,
    T* __restrict__ o, int64_t T_, const Layouts lay, int P, int64_t L, float eps) {
    constexpr int C = CF::C, NT = CF::NT, NL = CF::NL, LC = CF::LC;
    constexpr int NI = DK / 16, NJ = DV / 16, LK = DK + 4, LV = DV + 4;
    __shared__ __attribute__((aligned(16))) float sR[DK * LV];
    __shared__ __attribute__((aligned(16))) float sQ[C * LK];
    __shared__ __attribute__((aligned(16))) float sK[C * LK];
    __shared__ __attribute__((aligned(16))) float sV[C * LV];
    __shared__ __attribute__((aligned(16))) float sO[C * LV];
    __shared__ __attribute__((aligned(16))) float sA[C * LC];
    __shared__ float sZ[DK], sRcp[C];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, g = lane >> 4;
    const int64_t t0 = (int64_t)p * L, t1 = min(t0 + L, T_), len = t1 - t0;
    const int nch = (int)(len > 0 ? (len + C - 1) / C : 0);

    const float* st = pre ? pre + (bh * P + p) * (int64_t)(DK * DV + DK) : nullptr;
    for (int e = tid; e < DK * DV; e += kThreads) sR[(e / DV) * LV + e % DV] = st ? st[e] : 0.f;
    for (int e = tid; e < DK; e += kThreads) sZ[e] = st ? st[DK * DV + e] : 0.f;

    const HeadBuf bq = slice_buf(q, lay.q, bh, DK, t0, t1), bk = slice_buf(k, lay.k, bh, DK, t0, t1);
    const HeadBuf bv = slice_buf(v, lay.v, bh, DV, t0, t1), bo = slice_buf(o, lay.o, bh, DV, t0, t1);
    ChunkLoad<T, DK> lq, lk;
    ChunkLoad<T, DV> lv;
    lq.issue(bq, lay.q.rs, 0);
    lk.issue(bk, lay.k.rs, 0);
    lv.issue(bv, lay.v.rs, 0);

    for (int c = 0; c < nch; ++c) {
        const int nvalid = (int)min((int64_t)C, len - (int64_t)c * C);
        const auto feat = [&](int r, float x) { return r < nvalid ? phi<FM, T>(x) : 0.f; };
        lq.put(sQ, LK, feat);
        lk.put(sK, LK, feat);
        lv.put(sV, LV, [](int, float x) { return x; });
        const int64_t next = (int64_t)min(c + 1, nch - 1) * C;
        lq.issue(bq, lay.q.rs, next);
        lk.issue(bk, lay.k.rs, next);
        lv.issue(bv, lay.v.rs, next);
        __syncthreads();

        for (int n = wave; n < NL; n += kWaves) {
            int tb, sb;
            lower_block(n, tb, sb);
            const f32x4 a = tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sQ + 16 * tb * LK, LK, sK + 16 * sb * LK,
                                                 LK, 0, DK);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sA[(16 * tb + 4 * g + r) * LC + 16 * sb + m] = (sb < tb || m <= 4 * g + r) ? a[r] : 0.f;
        }
        __syncthreads();

        {
            // eight lanes per row
            const int t = tid >> 3, sub = tid & 7;
            if constexpr (SIMPLE) {
                if (sub == 0) sRcp[t] = eps;  // the query scale
            } else {
                float den = 0.f;
                for (int s = sub; s <= t; s += 8) den += sA[t * LC + s];
                for (int i = sub; i < DK; i += 8) den += sQ[t * LK + i] * sZ[i];
                den += __shfl_xor(den, 1);
                den += __shfl_xor(den, 2);
                den += __shfl_xor(den, 4);
                if (sub == 0) sRcp[t] = 1.f / (den + eps);
            }
        }
        __syncthreads();

#pragma unroll 1
        for (int jj = 0; jj < NT * NJ / kWaves; ++jj) {
            const int n = wave + kWaves * jj, tb = n / NJ, jb = n % NJ;
            f32x4 acc = tile_f32<true, false>(f32x4{0.f, 0.f, 0.f, 0.f}, sQ + 16 * tb * LK, LK, sR + 16 * jb, LV, 0, DK);
            acc = tile_f32<true, false>(acc, sA + 16 * tb * LC, LC, sV + 16 * jb, LV, 0, 16 * (tb + 1));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tb + 4 * g + r;
                sO[row * LV + 16 * jb + m] = acc[r] * sRcp[row];
            }
        }
        __syncthreads();

#pragma unroll 1
        for (int jj = 0; jj < NI * NJ / kWaves; ++jj) {
            const int n = wave + kWaves * jj, ib = n / NJ, jb = n % NJ;
            float* rt = sR + 16 * ib * LV + 16 * jb;
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = rt[(4 * g + r) * LV + m];
            acc = tile_f32<false, false>(acc, sK + 16 * ib, LK, sV + 16 * jb, LV, 0, C);
#pragma unroll
            for (int r = 0; r < 4; ++r) rt[(4 * g + r) * LV + m] = acc[r];
        }
        for (int i = tid; i < DK; i += kThreads) {
            float s = 0.f;
            for (int r = 0; r < C; ++r) s += sK[r * LK + i];
            sZ[i] += s;
        }
        store_chunk<T, DV>(sO, LV, bo, lay.o.rs, (int64_t)c * C);
        __syncthreads();
    }
}

// Forward-order dQ scan, fp32 operands. Per chunk, with R, z the state
// before it (the quantities of the 16-bit scan's comment):
//   A = mask(phi(Q) phi(K)^T), B = mask(dO V^T) (s <= t), Y = dO R^T;
//   den_t = phi(q_t) . z + sum_s A_ts + eps, w_t = 1 / den_t,
//   c_t = -(phi(q_t) . Y_t + sum_s A_ts B_ts) w_t^2   (simple_la: w = scale, c = 0);
//   P = mask(w B + c), dphi(Q) = w Y + c z^T + P phi(K), dQ = dphi(Q) phi'(Q);
//   R += phi(K)^T V, z += sum_s phi(k_s);
// and w_t, c^_t = c_t / w_t per token into wc (normalised mode). With
// gpart (P > 1) the segment's own sums G = sum_t w_t phi(q_t) dO_t^T and
// g = sum_t c_t phi(q_t) are kept (G in registers, spread over the waves) and
// written there at the end.
template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__(kThreads) void bwd_causal_q_f32_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ pre, T* __restrict__ dq, float* __restrict__ wc, float* __restrict__ gpart, int64_t T_,
    const Layouts lay, int P, int64_t L, float eps) {
    constexpr int C = CF::C, NT = CF::NT, NL = CF::NL, LC = CF::LC;
    constexpr int NI = DK / 16, NJ = DV / 16, LK = DK + 4, LV = DV + 4;
    constexpr int NY = NT * NI / kWaves;  // dQ tiles per wave
    constexpr int NG = NI * NJ / kWaves;  // G tiles per wave
    __shared__ __attribute__((aligned(16))) float sR[DK * LV];
    __shared__ __attribute__((aligned(16))) float sQ[C * LK];
    __shared__ __attribute__((aligned(16))) float sK[C * LK];
    __shared__ __attribute__((aligned(16))) float sV[C * LV];
    __shared__ __attribute__((aligned(16))) float sD[C * LV];
    __shared__ __attribute__((aligned(16))) float sA[C * LC];
    __shared__ __attribute__((aligned(16))) float sB[C * LC];
    __shared__ float sZ[DK], sPart[NI * C], sW[C], sC[C];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, g = lane >> 4;
    const int64_t t0 = (int64_t)p * L, t1 = min(t0 + L, T_), len = t1 - t0;
    const int nch = (int)(len > 0 ? (len + C - 1) / C : 0);

    const float* st = pre ? pre + (bh * P + p) * (int64_t)(DK * DV + DK) : nullptr;
    for (int e = tid; e < DK * DV; e += kThreads) sR[(e / DV) * LV + e % DV] = st ? st[e] : 0.f;
    for (int e = tid; e < DK; e += kThreads) sZ[e] = st ? st[DK * DV + e] : 0.f;

    const HeadBuf bq = slice_buf(q, lay.q, bh, DK, t0, t1), bk = slice_buf(k, lay.k, bh, DK, t0, t1);
    const HeadBuf bv = slice_buf(v, lay.v, bh, DV, t0, t1), bd = slice_buf(dout, lay.dout, bh, DV, t0, t1);
    const HeadBuf bdq = slice_buf(dq, lay.dq, bh, DK, t0, t1);
    ChunkLoad<T, DK> lq, lk;
    ChunkLoad<T, DV> lv, ld;
    lq.issue(bq, lay.q.rs, 0);
    lk.issue(bk, lay.k.rs, 0);
    lv.issue(bv, lay.v.rs, 0);
    ld.issue(bd, lay.dout.rs, 0);

    const bool sums = gpart != nullptr;
    f32x4 G[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) G[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float gsum = 0.f;  // thread i < DK: g_i

    for (int c = 0; c < nch; ++c) {
        const int nvalid = (int)min((int64_t)C, len - (int64_t)c * C);
        const auto feat = [&](int r, float x) { return r < nvalid ? phi<FM, T>(x) : 0.f; };
        const auto raw = [](int, float x) { return x; };
        lq.put(sQ, LK, feat);
        lk.put(sK, LK, feat);
        lv.put(sV, LV, raw);
        ld.put(sD, LV, raw);
        const int64_t next = (int64_t)min(c + 1, nch - 1) * C;
        lq.issue(bq, lay.q.rs, next);
        lk.issue(bk, lay.k.rs, next);
        lv.issue(bv, lay.v.rs, next);
        ld.issue(bd, lay.dout.rs, next);
        __syncthreads();

        // (a) A and B on the blocks on or below the diagonal; Y on this
        // wave's tiles, with its share of phi(q) . Y per row
        for (int n = wave; n < 2 * NL; n += kWaves) {
            const bool isA = n < NL;
            if (SIMPLE && isA) continue;
            int tb, sb;
            lower_block(isA ? n : n - NL, tb, sb);
            const f32x4 a = isA ? tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sQ + 16 * tb * LK, LK,
                                                       sK + 16 * sb * LK, LK, 0, DK)
                                : tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sD + 16 * tb * LV, LV,
                                                       sV + 16 * sb * LV, LV, 0, DV);
            float* dst = isA ? sA : sB;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * tb + 4 * g + r) * LC + 16 * sb + m] = (sb < tb || m <= 4 * g + r) ? a[r] : 0.f;
        }
        f32x4 Y[NY];
#pragma unroll
        for (int jj = 0; jj < NY; ++jj) {
            const int n = wave + kWaves * jj, tb = n / NI, ib = n % NI;
            Y[jj] = tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sD + 16 * tb * LV, LV, sR + 16 * ib * LV, LV, 0, DV);
            if constexpr (!SIMPLE) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * tb + 4 * g + r;
                    const float d = row16_sum(Y[jj][r] * sQ[row * LK + 16 * ib + m]);
                    if (m == 0) sPart[ib * C + row] = d;
                }
            }
        }
        __syncthreads();

        // (b) per row (eight lanes each): w, c, P = mask(w B + c) in place of B
        {
            const int t = tid >> 3, sub = tid & 7;
            const bool ok = t < nvalid;
            float w, cc = 0.f;
            if constexpr (SIMPLE) {
                w = ok ? eps : 0.f;  // the query scale
            } else {
                float den = 0.f, dot = 0.f;  // phi(q) . z_t and phi(q) . u_t
                for (int s = sub; s <= t; s += 8) {
                    den += sA[t * LC + s];
                    dot += sA[t * LC + s] * sB[t * LC + s];
                }
                for (int i = sub; i < DK; i += 8) den += sQ[t * LK + i] * sZ[i];
                for (int ib = sub; ib < NI; ib += 8) dot += sPart[ib * C + t];
#pragma unroll
                for (int x = 1; x < 8; x <<= 1) {
                    den += __shfl_xor(den, x);
                    dot += __shfl_xor(dot, x);
                }
                w = ok ? 1.f / (den + eps) : 0.f;
                const float chat = -dot * w;  // c / w
                cc = chat * w;
                if (ok && sub == 0) {
                    float* wt = wc + (bh * T_ + t0 + (int64_t)c * C + t) * 2;
                    wt[0] = w;
                    wt[1] = chat;
                }
            }
            if (sub == 0) {
                sW[t] = w;
                sC[t] = cc;
            }
            for (int s = sub; s < C; s += 8) sB[t * LC + s] = s <= t ? w * sB[t * LC + s] + cc : 0.f;
        }
        __syncthreads();

        // (c) dQ on this wave's tiles (kept in Y); the segment sums
#pragma unroll
        for (int jj = 0; jj < NY; ++jj) {
            const int n = wave + kWaves * jj, tb = n / NI, ib = n % NI;
            const f32x4 pk = tile_f32<true, false>(f32x4{0.f, 0.f, 0.f, 0.f}, sB + 16 * tb * LC, LC, sK + 16 * ib, LK,
                                                   0, 16 * (tb + 1));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tb + 4 * g + r, col = 16 * ib + m;
                const float d = sW[row] * Y[jj][r] + sC[row] * sZ[col] + pk[r];
                Y[jj][r] = d * dphi_of<FM>(sQ[row * LK + col]);
            }
        }
        if (sums) {
#pragma unroll
            for (int jj = 0; jj < NG; ++jj) {
                const int n = wave + kWaves * jj, ib = n / NJ, jb = n % NJ;
                G[jj] = tile_f32<false, false, true>(G[jj], sQ + 16 * ib, LK, sD + 16 * jb, LV, 0, C, sW);
            }
            if (tid < DK) {
                float s = 0.f;
                for (int r = 0; r < C; ++r) s += sC[r] * sQ[r * LK + tid];
                gsum += s;
            }
        }
        __syncthreads();

        // (d) dQ into sQ's place; R += phi(K)^T V, z += sum phi(k)
#pragma unroll
        for (int jj = 0; jj < NY; ++jj) {
            const int n = wave + kWaves * jj, tb = n / NI, ib = n % NI;
#pragma unroll
            for (int r = 0; r < 4; ++r) sQ[(16 * tb + 4 * g + r) * LK + 16 * ib + m] = Y[jj][r];
        }
#pragma unroll 1
        for (int jj = 0; jj < NI * NJ / kWaves; ++jj) {
            const int n = wave + kWaves * jj, ib = n / NJ, jb = n % NJ;
            float* rt = sR + 16 * ib * LV + 16 * jb;
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = rt[(4 * g + r) * LV + m];
            acc = tile_f32<false, false>(acc, sK + 16 * ib, LK, sV + 16 * jb, LV, 0, C);
#pragma unroll
            for (int r = 0; r < 4; ++r) rt[(4 * g + r) * LV + m] = acc[r];
        }
        for (int i = tid; i < DK; i += kThreads) {
            float s = 0.f;
            for (int r = 0; r < C; ++r) s += sK[r * LK + i];
            sZ[i] += s;
        }
        __syncthreads();
        store_chunk<T, DK>(sQ, LK, bdq, lay.dq.rs, (int64_t)c * C);
        __syncthreads();
    }

    if (sums) {
        float* gp = gpart + (bh * P + p) * (int64_t)(DK * DV + DK);
#pragma unroll
        for (int jj = 0; jj < NG; ++jj) {
            const int n = wave + kWaves * jj, ib = n / NJ, jb = n % NJ;
#pragma unroll
            for (int r = 0; r < 4; ++r) gp[(16 * ib + 4 * g + r) * DV + 16 * jb + m] = G[jj][r];
        }
        if (tid < DK) gp[DK * DV + tid] = gsum;
    }
}

// Reverse-order dK, dV scan, fp32 operands: chunks from the segment's last
// to its first, starting from the suffix (G, g) of the later segments. Per
// chunk, with Qw_t = w_t phi(q_t) and G, g the sums over everything after it:
//   P~[s][t] = mask(v_s . dO_t + c^_t) w_t,  A~[s][t] = mask(phi(k_s) . phi(q_t)) w_t  (t >= s);
//   dK = (V G^T + g + P~ phi(Q)) phi'(K),  dV = phi(K) G + A~ dO;
//   G += Qw^T dO,  g += sum_t c^_t Qw_t.
template <typename T, int DK, int DV, bool SIMPLE, int FM>
__global__ __launch_bounds__(kThreads) void bwd_causal_kv_f32_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ wc, const float* __restrict__ suf, T* __restrict__ dk, T* __restrict__ dv, int64_t T_,
    const Layouts lay, int P, int64_t L, float qscale) {
    constexpr int C = CF::C, NT = CF::NT, NL = CF::NL, LC = CF::LC;
    constexpr int NI = DK / 16, NJ = DV / 16, LK = DK + 4, LV = DV + 4;
    constexpr int NDK = NT * NI / kWaves, NDV = NT * NJ / kWaves;
    __shared__ __attribute__((aligned(16))) float sG[DK * LV];
    __shared__ __attribute__((aligned(16))) float sQ[C * LK];
    __shared__ __attribute__((aligned(16))) float sK[C * LK];
    __shared__ __attribute__((aligned(16))) float sV[C * LV];
    __shared__ __attribute__((aligned(16))) float sD[C * LV];
    __shared__ __attribute__((aligned(16))) float sP[C * LC];
    __shared__ __attribute__((aligned(16))) float sT[C * LC];
    __shared__ float sg[DK], sW[C], sCh[C];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, g = lane >> 4;
    const int64_t t0 = (int64_t)p * L, t1 = min(t0 + L, T_), len = t1 - t0;
    const int nch = (int)(len > 0 ? (len + C - 1) / C : 0);

    const float* st = suf ? suf + (bh * P + p) * (int64_t)(DK * DV + DK) : nullptr;
    for (int e = tid; e < DK * DV; e += kThreads) sG[(e / DV) * LV + e % DV] = st ? st[e] : 0.f;
    for (int e = tid; e < DK; e += kThreads) sg[e] = st ? st[DK * DV + e] : 0.f;

    const HeadBuf bq = slice_buf(q, lay.q, bh, DK, t0, t1), bk = slice_buf(k, lay.k, bh, DK, t0, t1);
    const HeadBuf bv = slice_buf(v, lay.v, bh, DV, t0, t1), bd = slice_buf(dout, lay.dout, bh, DV, t0, t1);
    const HeadBuf bdk = slice_buf(dk, lay.dk, bh, DK, t0, t1), bdv = slice_buf(dv, lay.dv, bh, DV, t0, t1);
    ChunkLoad<T, DK> lq, lk;
    ChunkLoad<T, DV> lv, ld;
    const int64_t first = (int64_t)max(nch - 1, 0) * C;
    lq.issue(bq, lay.q.rs, first);
    lk.issue(bk, lay.k.rs, first);
    lv.issue(bv, lay.v.rs, first);
    ld.issue(bd, lay.dout.rs, first);
    // w_t, c^_t of this thread's row (tid < C) of the chunk in flight
    const float* wch = wc + (bh * T_ + t0) * 2;
    float nw = 0.f, nch_ = 0.f;
    const auto load_wc = [&](int cidx) {
        if constexpr (!SIMPLE) {
            if (tid < C && len > 0) {
                const int64_t t = min((int64_t)cidx * C + tid, len - 1);
                nw = wch[2 * t];
                nch_ = wch[2 * t + 1];
            }
        }
    };
    load_wc(max(nch - 1, 0));

    for (int c = nch - 1; c >= 0; --c) {
        const int nvalid = (int)min((int64_t)C, len - (int64_t)c * C);
        const auto feat = [&](int r, float x) { return r < nvalid ? phi<FM, T>(x) : 0.f; };
        const auto raw = [](int, float x) { return x; };
        lq.put(sQ, LK, feat);
        lk.put(sK, LK, feat);
        lv.put(sV, LV, raw);
        ld.put(sD, LV, raw);
        if (tid < C) {
            const bool ok = tid < nvalid;
            sW[tid] = ok ? (SIMPLE ? qscale : nw) : 0.f;
            sCh[tid] = ok && !SIMPLE ? nch_ : 0.f;
        }
        const int64_t next = (int64_t)max(c - 1, 0) * C;
        lq.issue(bq, lay.q.rs, next);
        lk.issue(bk, lay.k.rs, next);
        lv.issue(bv, lay.v.rs, next);
        ld.issue(bd, lay.dout.rs, next);
        load_wc(max(c - 1, 0));
        __syncthreads();

        // (a) P~ and A~ on the blocks on or above the diagonal (t >= s)
        for (int n = wave; n < 2 * NL; n += kWaves) {
            const bool isP = n < NL;
            int tb, sb;
            lower_block(isP ? n : n - NL, tb, sb);  // tb >= sb: key block sb, query block tb
            const f32x4 a = isP ? tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sV + 16 * sb * LV, LV,
                                                       sD + 16 * tb * LV, LV, 0, DV)
                                : tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sK + 16 * sb * LK, LK,
                                                       sQ + 16 * tb * LK, LK, 0, DK);
            float* dst = isP ? sP : sT;
            const int t = 16 * tb + m;
            const float wt = sW[t], ct = isP ? sCh[t] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * sb + 4 * g + r) * LC + t] = (sb < tb || m >= 4 * g + r) ? (a[r] + ct) * wt : 0.f;
        }
        __syncthreads();

        // (b) dK and dV on this wave's tiles
        f32x4 rk[NDK], rv[NDV];
#pragma unroll
        for (int jj = 0; jj < NDK; ++jj) {
            const int n = wave + kWaves * jj, sb = n / NI, ib = n % NI;
            f32x4 acc = tile_f32<true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, sV + 16 * sb * LV, LV, sG + 16 * ib * LV, LV,
                                             0, DV);
            acc = tile_f32<true, false>(acc, sP + 16 * sb * LC, LC, sQ + 16 * ib, LK, 16 * sb, C);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * sb + 4 * g + r, col = 16 * ib + m;
                rk[jj][r] = (acc[r] + sg[col]) * dphi_of<FM>(sK[row * LK + col]);
            }
        }
#pragma unroll
        for (int jj = 0; jj < NDV; ++jj) {
            const int n = wave + kWaves * jj, sb = n / NJ, jb = n % NJ;
            f32x4 acc = tile_f32<true, false>(f32x4{0.f, 0.f, 0.f, 0.f}, sK + 16 * sb * LK, LK, sG + 16 * jb, LV, 0, DK);
            rv[jj] = tile_f32<true, false>(acc, sT + 16 * sb * LC, LC, sD + 16 * jb, LV, 16 * sb, C);
        }
        __syncthreads();

        // (c) G += Qw^T dO, g += sum c^ Qw; dK, dV into the K and V tiles
#pragma unroll 1
        for (int jj = 0; jj < NI * NJ / kWaves; ++jj) {
            const int n = wave + kWaves * jj, ib = n / NJ, jb = n % NJ;
            float* gt = sG + 16 * ib * LV + 16 * jb;
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gt[(4 * g + r) * LV + m];
            acc = tile_f32<false, false, true>(acc, sQ + 16 * ib, LK, sD + 16 * jb, LV, 0, C, sW);
#pragma unroll
            for (int r = 0; r < 4; ++r) gt[(4 * g + r) * LV + m] = acc[r];
        }
        for (int i = tid; i < DK; i += kThreads) {
            float s = 0.f;
            for (int r = 0; r < C; ++r) s += sCh[r] * sW[r] * sQ[r * LK + i];
            sg[i] += s;
        }
#pragma unroll
        for (int jj = 0; jj < NDK; ++jj) {
            const int n = wave + kWaves * jj, sb = n / NI, ib = n % NI;
#pragma unroll
            for (int r = 0; r < 4; ++r) sK[(16 * sb + 4 * g + r) * LK + 16 * ib + m] = rk[jj][r];
        }
#pragma unroll
        for (int jj = 0; jj < NDV; ++jj) {
            const int n = wave + kWaves * jj, sb = n / NJ, jb = n % NJ;
#pragma unroll
            for (int r = 0; r < 4; ++r) sV[(16 * sb + 4 * g + r) * LV + 16 * jb + m] = rv[jj][r];
        }
        __syncthreads();
        store_chunk<T, DK>(sK, LK, bdk, lay.dk.rs, (int64_t)c * C);
        store_chunk<T, DV>(sV, LV, bdv, lay.dv.rs, (int64_t)c * C);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Head size 256 (DK = DV = 256, 16-bit inputs): wide kernels.
// ---------------------------------------------------------------------------
// A 256 x 256 fp32 state (256 KB) fits neither one wave's registers nor a
// workgroup's LDS, so these kernels run eight waves per workgroup and split
// the state among them: wave w owns 32 of its rows (or columns), and tiles of
// tokens are shared through LDS. Per 16 or 32 tokens the waves also split the
// products: wave w computes 32 of the 256 output features of every token.
// MFMA conventions as above; where a wave's results are token rows, the rows
// of its two 16-row A blocks are permuted so that lane (t + 16 g) ends with the
// eight contiguous features 32 w + 8 g .. + 7 of token t (block b gives
// 32 w + 8 g + 4 b + r in register r), which it stores as one 16-byte piece.
struct Wide {
    static constexpr int D = 256;
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    // token-major LDS tile row stride (elements): four consecutive rows fall
    // 8 banks apart, so transposed reads of 4 rows x 32 bytes do not conflict
    static constexpr int kLD = D + 16;
    static constexpr int kCPR = D * 2 / 16;  // 16-byte chunks per 16-bit row: 32
    // the state or output feature that row m of A block b (0, 1) of wave w
    // stands for, in the permuted order
    static __device__ __forceinline__ int feat(int w, int b, int m) { return 32 * w + 8 * (m >> 2) + 4 * b + (m & 3); }
};

// Largest |x| over n floats at M (n a multiple of 4 NT), over an NT-thread
// workgroup, in a fixed order: each thread walks its float4s in turn.
template <int NT>
__device__ __forceinline__ float block_absmax_loop(const float* __restrict__ M, int n, float* red) {
    float mx = 0.f;
    for (int i = threadIdx.x; i < n / 4; i += NT) {
        const float4 v = reinterpret_cast<const float4*>(M)[i];
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    return block_max<NT / 64>(mx, red);
}

// A operand of wave w, 16-row block b, contraction step s of a 256 x 256 fp32
// matrix M (rows 256 floats apart), rows in the permuted order of Wide::feat,
// contraction index 32 s + 8 g + e, scaled and rounded to T:
//   kRowsAreColumns = false: element M[feat][k]; true: element M[k][feat].
template <typename T, bool kRowsAreColumns>
__device__ __forceinline__ Frag<T> wide_frag(const float* __restrict__ M, int w, int b, int s, int m, int g,
                                             float scale) {
    const int f = Wide::feat(w, b, m), k0 = 32 * s + 8 * g;
    Frag<T> r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = kRowsAreColumns ? M[(k0 + e) * Wide::D + f] : M[f * Wide::D + k0 + e];
        r[e] = static_cast<T>(x * scale);
    }
    return r;
}

// Steps 1-3 at D = 256: one workgroup reduces tokens [p L, min((p+1) L, T))
// of head bh into a partial (S, z) (or the state itself when a head is one
// slice). Per 32-token tile the threads load K and V (two 16-byte chunks of
// each per thread), apply phi to K in fp32 and round it to T (zero past the
// slice end), and store both tiles token-major in LDS (two buffers, one
// barrier per tile, the next two tiles' loads in flight). Wave w accumulates
// rows 32 w .. 32 w + 31 of S over all 256 columns (32 blocks) and of z (a
// block of ones as B), from transposed LDS reads: A = phi(K)^T, B = V.
template <typename T, int FM>
__global__ __launch_bounds__(Wide::kThreads, 1) void fwd_state_wide_kernel(
    const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ stS, float* __restrict__ stz,
    float* __restrict__ part, int64_t T_, const Layouts lay, int P, int64_t L) {
    constexpr int D = Wide::D, NT = Wide::kThreads, LD = Wide::kLD, CPR = Wide::kCPR, E = D * D + D;
    constexpr int TT = 32;                // tokens per tile
    constexpr int NCH = TT * CPR / NT;    // chunks of each tensor per thread per tile: 2
    constexpr int NJ = D / 16;            // column blocks: 16
    __shared__ __attribute__((aligned(16))) T sK[2][TT * LD];
    __shared__ __attribute__((aligned(16))) T sV[2][TT * LD];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / P;
    const int p = wid % P;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)p * L;
    const int64_t t1 = min(t0 + L, T_);
    const int64_t len = t1 - t0;
    const int ntiles = (int)(len > 0 ? (len + TT - 1) / TT : 0);
    const int npad = (ntiles + 1) / 2 * 2;

    f32x4 acc[2][NJ + 1];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j <= NJ; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<T>(1.f);

    // Rows are counted from t0; tiles past the slice end read zeros (and K is
    // zeroed after phi there), so the loop always runs whole pairs of tiles.
    const HeadBuf bk = slice_buf(k, lay.k, bh, D, t0, t1), bv = slice_buf(v, lay.v, bh, D, t0, t1);
    struct Stage {
        u32x4 k[NCH], v[NCH];
    };
    auto issue = [&](Stage& st, int tile) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int n = tid + NT * i, r = n / CPR, c = n % CPR;
            const int64_t row = (int64_t)tile * TT + r;
            st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, buf_off<T>(row, lay.k.rs, 8 * c), 0, kNonTemporal);
            st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(bv.rsrc, buf_off<T>(row, lay.v.rs, 8 * c), 0, kNonTemporal);
        }
    };
    auto put = [&](const Stage& st, int tile, int buf) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int n = tid + NT * i, r = n / CPR, c = n % CPR;
            const bool ok = (int64_t)tile * TT + r < len;
            Row<T, 8> kr;
            __builtin_memcpy(kr.e, &st.k[i], 16);
            Row<T, 8> kt;
#pragma unroll
            for (int e = 0; e < 8; ++e) kt.e[e] = ok ? static_cast<T>(phi<FM, T>(to_f32(kr.e[e]))) : static_cast<T>(0.f);
            *reinterpret_cast<uint4*>(&sK[buf][r * LD + 8 * c]) = *reinterpret_cast<const uint4*>(kt.e);
            *reinterpret_cast<u32x4*>(&sV[buf][r * LD + 8 * c]) = st.v[i];
        }
    };
    const int rA = 8 * grp + (m >> 2), cA = 4 * (m & 3);
    auto mma_tile = [&](int buf) {
        const T* kk = sK[buf];
        const T* vv = sV[buf];
        Frag<T> a[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int cb = 16 * (2 * wave + rb) + cA;
            a[rb] = join_frag<T>(lds_read_tr(&kk[rA * LD + cb]), lds_read_tr(&kk[(rA + 4) * LD + cb]));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const Frag<T> b = join_frag<T>(lds_read_tr(&vv[rA * LD + 16 * j + cA]),
                                           lds_read_tr(&vv[(rA + 4) * LD + 16 * j + cA]));
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) acc[rb][j] = mma(a[rb], b, acc[rb][j]);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[rb][NJ] = mma(a[rb], ones, acc[rb][NJ]);
    };

    if (ntiles > 0) {
        Stage s0, s1;
        issue(s0, 0);
        sched_fence();
        issue(s1, 1);
        sched_fence();
        for (int tile = 0; tile < npad; tile += 2) {
            put(s0, tile, 0);
            sched_fence();
            issue(s0, tile + 2);
            sched_fence();
            __syncthreads();
            mma_tile(0);
            put(s1, tile + 1, 1);
            sched_fence();
            issue(s1, tile + 3);
            sched_fence();
            __syncthreads();
            mma_tile(1);
        }
    }

    float* oS;
    float* oz;
    if (P == 1) {
        oS = stS + bh * D * D;
        oz = stz + bh * D;
    } else {
        oS = part + (bh * P + p) * (int64_t)E;
        oz = oS + D * D;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row0 = 32 * wave + 16 * rb + 4 * grp;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) oS[(row0 + r) * D + 16 * j + m] = acc[rb][j][r];
        if (m == 0)
#pragma unroll
            for (int r = 0; r < 4; ++r) oz[row0 + r] = acc[rb][NJ][r];
    }
}

// Step 4 at D = 256: one workgroup streams tokens [ch LQ, min((ch+1) LQ, T))
// of head bh in 16-token blocks. The threads load a block of Q (one 16-byte
// chunk each: the 32 threads of a token row are 32 lanes of one wave), apply
// phi in fp32, store phi(q) rounded to T token-major in LDS and reduce
// den = phi(q) . z + eps over the row's lanes with xor shuffles (z in fp32);
// after a barrier wave w multiplies the block by its 32 columns of S, held
// as 16 fragments in registers since the prologue (A = S^T, rows permuted,
// B = phi(Q)^T read straight from the token-major tile), scales by 1 / den and
// stores eight contiguous outputs per lane. Two LDS buffers, one barrier per
// block, the loads of the next four blocks in flight, two workgroups per CU.
template <typename T, bool SIMPLE, int FM>
__global__ __launch_bounds__(Wide::kThreads, 2) void fwd_output_wide_kernel(
    const T* __restrict__ q, const float* __restrict__ stS, const float* __restrict__ stz, T* __restrict__ o,
    int64_t T_, const Layouts lay, int NQ, int64_t LQ, float eps) {
    constexpr int D = Wide::D, NT = Wide::kThreads, LD = Wide::kLD, CPR = Wide::kCPR, KS = D / 32;
    constexpr int BT = 16;  // tokens per block
    constexpr int NS = 4;   // blocks of loads in flight per thread
    static_assert(BT * CPR == NT, "one chunk per thread per block");
    __shared__ __attribute__((aligned(16))) T sQ[2][BT * LD];
    __shared__ float sDen[2][BT];
    __shared__ float sZ[D];
    __shared__ float red[NT / 64];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / NQ;
    const int ch = wid % NQ;
    const int64_t c0 = (int64_t)ch * LQ;
    const int64_t c1 = min(c0 + LQ, T_);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int lr = tid / CPR, lc = tid % CPR;  // the chunk this thread loads: token row, 16-byte column
    const float* S = stS + bh * D * D;
    const float* z = stz + bh * D;
    const int nblk = (int)(c1 > c0 ? (c1 - c0 + BT - 1) / BT : 0);
    const int npad = (nblk + NS - 1) / NS * NS;

    const HeadBuf bq = slice_buf(q, lay.q, bh, D, c0, c1), bo = slice_buf(o, lay.o, bh, D, c0, c1);
    auto issue = [&](u32x4& x, int blk) {
        x = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, buf_off<T>((int64_t)blk * BT + lr, lay.q.rs, 8 * lc), 0, 0);
    };
    u32x4 x[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        issue(x[i], i);
        sched_fence();
    }

    // prologue: z to LDS; S^T fragments of this wave's 32 columns, scaled by 2^sS (f16)
    for (int i = tid; i < D; i += NT) sZ[i] = z[i];
    int sS = 0;
    if constexpr (Elt<T>::kScaled) sS = scale_exp(block_absmax_loop<NT>(S, D * D, red));
    const float fS = ldexpf(1.f, sS), uS = ldexpf(1.f, -sS);
    Frag<T> a[2][KS];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int s = 0; s < KS; ++s) a[b][s] = wide_frag<T, true>(S, wave, b, s, m, grp, fS);
    __syncthreads();

    auto put = [&](const u32x4& x, int buf) {
        Row<T, 8> raw, ph;
        __builtin_memcpy(raw.e, &x, 16);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ph.e[e] = static_cast<T>(phi<FM, T>(to_f32(raw.e[e])));
            d += to_f32(ph.e[e]) * sZ[8 * lc + e];
        }
        *reinterpret_cast<uint4*>(&sQ[buf][lr * LD + 8 * lc]) = *reinterpret_cast<const uint4*>(ph.e);
        if constexpr (!SIMPLE) {
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) d += __shfl_xor(d, off);  // the 32 lanes of this row
            if (lc == 0) sDen[buf][lr] = d;
        }
    };
    auto compute = [&](int blk, int buf) {
        const T* qq = sQ[buf];
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const Frag<T> bq_ = __builtin_bit_cast(Frag<T>, *reinterpret_cast<const u32x4*>(&qq[m * LD + 32 * s + 8 * grp]));
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[b] = mma(a[b][s], bq_, acc[b]);
        }
        float f;
        if constexpr (SIMPLE) f = uS * eps;  // simple_la: eps carries the query scale
        else f = uS / (sDen[buf][m] + eps);
        Row<T, 8> out;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) out.e[4 * b + r] = static_cast<T>(acc[b][r] * f);
        buf_store16(bo, buf_off<T>((int64_t)blk * BT + m, lay.o.rs, 32 * wave + 8 * grp), *reinterpret_cast<const uint4*>(out.e));
    };

    // (written out per stage: each stage keeps its own registers)
    for (int blk = 0; blk < npad; blk += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            put(x[i], i & 1);
            sched_fence();
            issue(x[i], blk + i + NS);
            sched_fence();
            __syncthreads();
            compute(blk + i, i & 1);
        }
    }
}

// Step 7 at D = 256: one workgroup of 16 waves streams tokens [ch LK,
// min((ch+1) LK, T)) of head bh in 16-token blocks. The threads load a block
// of K (the first 512) and of V (the others), one 16-byte chunk each, and
// store phi(k) rounded to T, phi'(k) in fp32 and V token-major in LDS. Waves
// 0-7 compute dK, wave w its features 32 w .. 32 w + 31 with A = dS (rows i,
// contraction over V's features) and B = V^T; waves 8-15 compute dV with
// A = dS^T (rows j, contraction over K's features) and B = phi(K)^T. Each
// wave's 16 fragments stay in registers from the prologue on; B is read
// straight from the token-major tiles.
//   dK_t = (dS v_t + dz) * phi'(k_t),  dV_t = dS^T phi(k_t)
// Two LDS buffers, one barrier per block, the next two blocks' loads in flight.
struct WideKV {
    static constexpr int kWaves = 16;
    static constexpr int kThreads = 64 * kWaves;
};

template <typename T, bool SIMPLE, int FM>
__global__ __launch_bounds__(WideKV::kThreads, 1) void bwd_dkv_wide_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ dSg, const float* __restrict__ dzg,
    T* __restrict__ dk, T* __restrict__ dv, int64_t T_, const Layouts lay, int NK, int64_t LK) {
    constexpr int D = Wide::D, NT = WideKV::kThreads, LD = Wide::kLD, CPR = Wide::kCPR, KS = D / 32;
    constexpr int BT = 16;
    constexpr int NS = 2;       // blocks of loads in flight per thread (4 measured slower)
    constexpr int LDP = D + 4;  // row stride (floats) of the phi'(k) tile
    static_assert(2 * BT * CPR == NT, "one chunk of K or V per thread per block");
    __shared__ __attribute__((aligned(16))) T sK[2][BT * LD];
    __shared__ __attribute__((aligned(16))) T sV[2][BT * LD];
    __shared__ __attribute__((aligned(16))) float sP[2][BT * LDP];
    __shared__ float sZd[D];
    __shared__ float red[NT / 64];

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / NK;
    const int ch = wid % NK;
    const int64_t c0 = (int64_t)ch * LK;
    const int64_t c1 = min(c0 + LK, T_);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const bool vside = wave >= 8;  // uniform over the wave: dV (true) or dK
    const int fw = wave & 7;       // the wave's group of 32 features
    const int lt = tid & (NT / 2 - 1), lr = lt / CPR, lc = lt % CPR;  // the chunk this thread loads
    const float* dS = dSg + bh * D * D;
    const float* dz = dzg + bh * D;
    const int nblk = (int)(c1 > c0 ? (c1 - c0 + BT - 1) / BT : 0);
    const int npad = (nblk + NS - 1) / NS * NS;

    const HeadBuf bk = slice_buf(k, lay.k, bh, D, c0, c1), bv = slice_buf(v, lay.v, bh, D, c0, c1);
    const HeadBuf bdk = slice_buf(dk, lay.dk, bh, D, c0, c1), bdv = slice_buf(dv, lay.dv, bh, D, c0, c1);
    auto issue = [&](u32x4& x, int blk) {
        const int64_t row = (int64_t)blk * BT + lr;
        // the dV waves (the upper half of the threads) load V, the dK waves K
        if (vside) x = __builtin_amdgcn_raw_buffer_load_b128(bv.rsrc, buf_off<T>(row, lay.v.rs, 8 * lc), 0, 0);
        else x = __builtin_amdgcn_raw_buffer_load_b128(bk.rsrc, buf_off<T>(row, lay.k.rs, 8 * lc), 0, 0);
    };
    u32x4 x[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        issue(x[i], i);
        sched_fence();
    }

    // prologue: this wave's 16 fragments of dS (dK side) or dS^T (dV side),
    // scaled by 2^sD (f16); dz to LDS
    int sD = 0;
    if constexpr (Elt<T>::kScaled) sD = scale_exp(block_absmax_loop<NT>(dS, D * D, red));
    const float fD = ldexpf(1.f, sD), uD = ldexpf(1.f, -sD);
    Frag<T> a[2][KS];
    if (vside) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s = 0; s < KS; ++s) a[b][s] = wide_frag<T, true>(dS, fw, b, s, m, grp, fD);
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s = 0; s < KS; ++s) a[b][s] = wide_frag<T, false>(dS, fw, b, s, m, grp, fD);
    }
    for (int i = tid; i < D; i += NT) sZd[i] = SIMPLE ? 0.f : dz[i];

    auto put = [&](const u32x4& x, int buf) {
        if (vside) {
            *reinterpret_cast<u32x4*>(&sV[buf][lr * LD + 8 * lc]) = x;
        } else {
            Row<T, 8> raw, ph;
            __builtin_memcpy(raw.e, &x, 16);
            float dp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float pv;
                feature<FM, T>(to_f32(raw.e[e]), pv, dp[e]);
                ph.e[e] = static_cast<T>(pv);
            }
            *reinterpret_cast<uint4*>(&sK[buf][lr * LD + 8 * lc]) = *reinterpret_cast<const uint4*>(ph.e);
            float4* pp = reinterpret_cast<float4*>(&sP[buf][lr * LDP + 8 * lc]);
            pp[0] = make_float4(dp[0], dp[1], dp[2], dp[3]);
            pp[1] = make_float4(dp[4], dp[5], dp[6], dp[7]);
        }
    };
    auto compute = [&](int blk, int buf) {
        const T* src = vside ? sK[buf] : sV[buf];
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const Frag<T> b_ = __builtin_bit_cast(Frag<T>, *reinterpret_cast<const u32x4*>(&src[m * LD + 32 * s + 8 * grp]));
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[b] = mma(a[b][s], b_, acc[b]);
            if (s % 2 == 1) sched_fence();  // two steps' operands in flight: 16 fragments stay resident
        }
        const int f0 = 32 * fw + 8 * grp;
        const int64_t row = (int64_t)blk * BT + m;
        Row<T, 8> out;
        if (vside) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) out.e[4 * b + r] = static_cast<T>(acc[b][r] * uD);
            buf_store16(bdv, buf_off<T>(row, lay.dv.rs, f0), *reinterpret_cast<const uint4*>(out.e));
        } else {
            const float* pp = &sP[buf][m * LDP + f0];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = 4 * b + r;
                    out.e[e] = static_cast<T>((acc[b][r] * uD + sZd[f0 + e]) * pp[e]);
                }
            buf_store16(bdk, buf_off<T>(row, lay.dk.rs, f0), *reinterpret_cast<const uint4*>(out.e));
        }
    };
    __syncthreads();

    for (int blk = 0; blk < npad; blk += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            put(x[i], i & 1);
            sched_fence();
            issue(x[i], blk + i + NS);
            sched_fence();
            __syncthreads();
            compute(blk + i, i & 1);
        }
    }
}

// Steps 5-6 at D = 256: one workgroup reduces tokens [p LB, min((p+1) LB, T))
// of head bh into partial (dS, dz) and writes their dQ, in 16-token blocks.
// Lane (t + 16 g) of wave w owns features 32 w + 8 g .. + 7 of token t of the
// block: it loads that 16-byte piece of Q (kept in registers) and of dO
// (stored token-major in LDS, double-buffered, for all waves), and
//   (a) u = S dO for the wave's features (A = S, 16 fragments of this wave's
//       rows kept in LDS since the prologue: with 32 rows of the fp32 dS sums
//       per wave in registers, S does not fit there as well; B = dO^T read
//       straight from the tile), phi(q) and phi'(q) in fp32, and over its
//       eight features the partial sums of r = phi(q) . u and of
//       phi(q) . z, which the waves publish per token;
//   (b) after a barrier: r and den = phi(q) . z + eps summed over the waves in
//       a fixed order, c = -r / den^2, dQ = (u / den + c z) * phi'(q) stored
//       as one 16-byte piece; A_t = phi(q_t) 2^sw / den_t to the wave's own
//       token-major LDS tile, read back transposed as the A operand of
//       dS += A^T dO (16x16x16 over the block's tokens, B = dO read transposed
//       from the shared tile); dz += c phi(q) in fp32 per lane.
// simple_la: den = 1, c = 0, A = phi(q). Two barriers per block; the loads of
// the next four blocks in flight in registers. Rows past the slice end load
// zeros: dO = 0 adds nothing to dS or dz, and their dQ stores are dropped.
template <typename T, bool SIMPLE, int FM>
__global__ __launch_bounds__(Wide::kThreads, 1) void bwd_dq_wide_kernel(
    const T* __restrict__ q, const T* __restrict__ dout, const float* __restrict__ stS,
    const float* __restrict__ stz, T* __restrict__ dq, float* __restrict__ part, float* __restrict__ dS_out,
    float* __restrict__ dz_out, int64_t T_, const Layouts lay, int PB, int64_t LB, float eps) {
    constexpr int D = Wide::D, NT = Wide::kThreads, NW = Wide::kWaves, LD = Wide::kLD;
    constexpr int KS = D / 32, NJ = D / 16, E = D * D + D;
    constexpr int BT = 16;
    // blocks of loads in flight per thread: normalised mode needs the
    // registers for r and den, which leave room for two
    constexpr int NS = SIMPLE ? 4 : 2;
    constexpr int LDA = 48;  // row stride (elements) of a wave's A tile: 32 features + 16
    __shared__ __attribute__((aligned(16))) Frag<T> sSf[NW * 2 * KS * 64];
    __shared__ __attribute__((aligned(16))) T sO[2][BT * LD];
    __shared__ __attribute__((aligned(16))) T sA[NW][BT * LDA];
    __shared__ float sR[2][NW][BT];
    __shared__ float sDn[2][NW][BT];
    __shared__ float sZ[D];
    float* red = &sR[0][0][0];  // the prologue's reductions (sR is free until the loop)

    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = wid / PB;
    const int p = wid % PB;
    const int64_t t0 = (int64_t)p * LB;
    const int64_t t1 = min(t0 + LB, T_);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int m = lane & 15, grp = lane >> 4;
    const int f0 = 32 * wave + 8 * grp;  // the lane's eight features
    const float* S = stS + bh * D * D;
    const float* z = stz + bh * D;
    const int nblk = (int)(t1 > t0 ? (t1 - t0 + BT - 1) / BT : 0);
    const int npad = (nblk + NS - 1) / NS * NS;

    const HeadBuf bq = slice_buf(q, lay.q, bh, D, t0, t1), bd = slice_buf(dout, lay.dout, bh, D, t0, t1),
                  bdq = slice_buf(dq, lay.dq, bh, D, t0, t1);
    struct Stage {
        u32x4 q, d;
    };
    auto issue = [&](Stage& st, int blk) {
        const int64_t row = (int64_t)blk * BT + m;
        st.q = __builtin_amdgcn_raw_buffer_load_b128(bq.rsrc, buf_off<T>(row, lay.q.rs, f0), 0, 0);
        st.d = __builtin_amdgcn_raw_buffer_load_b128(bd.rsrc, buf_off<T>(row, lay.dout.rs, f0), 0, 0);
    };
    Stage stg[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        issue(stg[i], i);
        sched_fence();
    }

    // prologue: this wave's S fragments (rows in the permuted order) to LDS,
    // scaled by 2^sS (f16); z to LDS; the exponent sw with 2^sw <= sum(z) <
    // 2^(sw+1) that keeps A_t near 1 (f16)
    int sS = 0, sw = 0;
    if constexpr (Elt<T>::kScaled) {
        sS = scale_exp(block_absmax_loop<NT>(S, D * D, red));
        if constexpr (!SIMPLE) {
            float zs = 0.f;
            if (tid < D / 4) {
                const float4 zz = reinterpret_cast<const float4*>(z)[tid];
                zs = (zz.x + zz.y) + (zz.z + zz.w);
            }
            const float sum = block_sum<NT / 64>(zs, red);
            if (sum > 0.f && isfinite(sum)) {
                int e;
                frexpf(sum, &e);
                sw = min(max(e - 1, -120), 120);
            }
        }
    }
    const float fS = ldexpf(1.f, sS), uS = ldexpf(1.f, -sS), fw = ldexpf(1.f, sw);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sSf[((2 * wave + b) * KS + s) * 64 + lane] = wide_frag<T, false>(S, wave, b, s, m, grp, fS);
    for (int i = tid; i < D; i += NT) sZ[i] = z[i];

    f32x4 dsacc[2][NJ];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < NJ; ++j) dsacc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dzp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dzp[e] = 0.f;
    T* aw = sA[wave];
    const int rA = 4 * grp + (m >> 2), cA = 4 * (m & 3);

    auto compute = [&](const Stage& st, int blk, int buf) {
        *reinterpret_cast<u32x4*>(&sO[buf][m * LD + f0]) = st.d;
        Row<T, 8> raw;
        __builtin_memcpy(raw.e, &st.q, 16);
        float ph[8], dph[8];
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            feature<FM, T>(to_f32(raw.e[e]), ph[e], dph[e]);
            dp += ph[e] * sZ[f0 + e];
        }
        __syncthreads();  // the block's dO tile is complete
        // (a) u = S dO for the wave's features, r and den over them
        f32x4 u[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const T* oo = sO[buf];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const Frag<T> b_ = __builtin_bit_cast(Frag<T>, *reinterpret_cast<const u32x4*>(&oo[m * LD + 32 * s + 8 * grp]));
#pragma unroll
            for (int b = 0; b < 2; ++b) u[b] = mma(sSf[((2 * wave + b) * KS + s) * 64 + lane], b_, u[b]);
        }
        float uu[8];
        float rp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uu[e] = u[e >> 2][e & 3] * uS;
            rp += ph[e] * uu[e];
        }
        float inv = 1.f, cc = 0.f;
        if constexpr (!SIMPLE) {
            rp += __shfl_xor(rp, 16);
            rp += __shfl_xor(rp, 32);
            dp += __shfl_xor(dp, 16);
            dp += __shfl_xor(dp, 32);
            if (grp == 0) {
                sR[buf][wave][m] = rp;
                sDn[buf][wave][m] = dp;
            }
            __syncthreads();
            float r = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                r += sR[buf][w][m];
                den += sDn[buf][w][m];
            }
            inv = 1.f / (den + eps);
            cc = -r * inv * inv;
        }
        // (b) dQ, then the reduction operand and dz
        Row<T, 8> out;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float g = SIMPLE ? uu[e] * eps : uu[e] * inv + cc * sZ[f0 + e];  // simple_la: eps carries the query scale
            out.e[e] = static_cast<T>(g * dph[e]);
        }
        buf_store16(bdq, buf_off<T>((int64_t)blk * BT + m, lay.dq.rs, f0), *reinterpret_cast<const uint4*>(out.e));
        Row<T, 8> at;
        const float fa = SIMPLE ? 1.f : fw * inv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            at.e[e] = static_cast<T>(ph[e] * fa);
            dzp[e] += cc * ph[e];
        }
        *reinterpret_cast<uint4*>(&aw[m * LDA + 8 * grp]) = *reinterpret_cast<const uint4*>(at.e);
        wave_lds_sync();
        i16x4 a[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) a[rb] = lds_read_tr(&aw[rA * LDA + 16 * rb + cA]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const i16x4 bw = lds_read_tr(&oo[rA * LD + 16 * j + cA]);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) dsacc[rb][j] = mma_k16<T>(a[rb], bw, dsacc[rb][j]);
        }
        wave_lds_sync();
        sched_fence();  // one block at a time: the dS sums take half the registers
    };
    __syncthreads();  // the S fragments and z are in LDS

    // (written out per stage: each stage keeps its own registers). Block n
    // writes dO tile n % 2, last read by block n - 2: the two barriers of
    // block n - 1 lie between.
    for (int blk = 0; blk < npad; blk += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const Stage cur = stg[i];
            sched_fence();
            issue(stg[i], blk + i + NS);
            sched_fence();
            compute(cur, blk + i, i & 1);
        }
    }

    // dz over the lanes of each feature group (tokens), in a fixed order
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) dzp[e] += __shfl_xor(dzp[e], off);
    float* oS;
    float* oz;
    if (PB == 1) {
        oS = dS_out + bh * D * D;
        oz = dz_out + bh * D;
    } else {
        oS = part + (bh * PB + p) * (int64_t)E;
        oz = oS + D * D;
    }
    const float uw = ldexpf(1.f, -sw) * (SIMPLE ? eps : 1.f);  // simple_la: times the query scale
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row0 = 32 * wave + 16 * rb + 4 * grp;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) oS[(row0 + r) * D + 16 * j + m] = dsacc[rb][j][r] * uw;
    }
    if (m == 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) oz[f0 + e] = SIMPLE ? 0.f : dzp[e];
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
constexpr bool kWaveKernels = (sizeof(T) == 2 && DK == 64 && DV == 64);
template <typename T, int DK, int DV>
constexpr bool kTileKernels = (sizeof(T) == 2 && !kWaveKernels<T, DK, DV>);

template <typename X>
struct Same {
    using type = X;
};

// Launches kernel on stream s with the arguments converted to its parameter
// types, and returns the status of this launch (not an error that an earlier
// HIP call of the caller left behind).
template <typename... KArgs>
hipError_t launch(void (*kernel)(KArgs...), int64_t blocks, int threads, hipStream_t s,
                  typename Same<KArgs>::type... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks), dim3(threads), argv, 0,
                           s);
}

// After a split reduction (P > 1 slices per head), sum the partials.
template <int DK, int DV>
hipError_t launch_combine(int P, const float* part, float* outS, float* outz, int64_t BH, hipStream_t s) {
    if (P <= 1) return hipSuccess;
    constexpr int E4 = (DK * DV + DK) / 4;
    return launch(combine_kernel<DK, DV>, BH * ((E4 + kThreads - 1) / kThreads), kThreads, s, part, P, outS, outz,
                  BH);
}

// The state reduction kernel alone: partials into the workspace (P > 1) or
// the state itself (P = 1).
template <typename T, int DK, int DV, int FM>
hipError_t launch_state_reduction(const Plan& p, const void* k, const void* v, float* state, float* part,
                                  hipStream_t s) {
    const int64_t nblk = p.BH * p.P;
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    float* sz = state + p.BH * DK * DV;
    if constexpr (kWaveKernels<T, DK, DV>)
        return launch(fwd_state_w64_kernel<T, FM>, nblk, kThreads, s, kk, vv, state, sz, part, p.T, p.lay, p.P, p.L);
    else if constexpr (kTileKernels<T, DK, DV>)
        return launch(fwd_state_tile_kernel<T, DK, DV, FM>, nblk, kThreads, s, kk, vv, state, sz, part, p.T,
                      p.lay, p.P, p.L);
    else
        return launch(fwd_state_kernel<T, DK, DV, FM>, nblk, kThreads, s, kk, vv, state, sz, part, p.T, p.lay,
                      p.P, p.L);
}

template <typename T, int DK, int DV, int FM>
hipError_t fwd_state_fm(const Plan& p, const void* k, const void* v, float* state, void* ws,
                       hipStream_t s) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_part);
    const hipError_t e = launch_state_reduction<T, DK, DV, FM>(p, k, v, state, part, s);
    if (e != hipSuccess) return e;
    return launch_combine<DK, DV>(p.P, part, state, state + p.BH * DK * DV, p.BH, s);
}

// The D = 256 unit's launchers (16-bit only; the problem checks keep fp32 and
// mixed sizes away from them).
template <typename T, int FM>
hipError_t wide_fwd_state_fm(const Plan& p, const void* k, const void* v, float* state, void* ws, hipStream_t s) {
    constexpr int D = Wide::D;
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_part);
    const hipError_t e = launch(fwd_state_wide_kernel<T, FM>, p.BH * p.P, Wide::kThreads, s, static_cast<const T*>(k),
                                static_cast<const T*>(v), state, state + p.BH * D * D, part, p.T, p.lay, p.P, p.L);
    if (e != hipSuccess) return e;
    return launch_combine<D, D>(p.P, part, state, state + p.BH * D * D, p.BH, s);
}
template <typename T, int FM>
hipError_t wide_fwd_output_fm(const Plan& p, const void* q, const float* state, void* o, hipStream_t s) {
    constexpr int D = Wide::D;
    const T* qq = static_cast<const T*>(q);
    T* oo = static_cast<T*>(o);
    const float* sz = state + p.BH * D * D;
    if (p.simple)
        return launch(fwd_output_wide_kernel<T, true, FM>, p.BH * p.NQ, Wide::kThreads, s, qq, state, sz, oo, p.T,
                      p.lay, p.NQ, p.LQ, p.eps);
    return launch(fwd_output_wide_kernel<T, false, FM>, p.BH * p.NQ, Wide::kThreads, s, qq, state, sz, oo, p.T, p.lay,
                  p.NQ, p.LQ, p.eps);
}
template <typename T, int FM>
hipError_t wide_bwd_dq_fm(const Plan& p, const void* q, const void* dout, const float* state, void* dq, void* ws,
                          hipStream_t s) {
    constexpr int D = Wide::D;
    char* w = static_cast<char*>(ws);
    float* part = reinterpret_cast<float*>(w + p.off_part);
    float* dS = reinterpret_cast<float*>(w + p.off_dstate);
    float* dz = dS + p.BH * D * D;
    const T* qq = static_cast<const T*>(q);
    const T* dd = static_cast<const T*>(dout);
    const float* sz = state + p.BH * D * D;
    T* g = static_cast<T*>(dq);
    const hipError_t e =
        p.simple ? launch(bwd_dq_wide_kernel<T, true, FM>, p.BH * p.PB, Wide::kThreads, s, qq, dd, state, sz, g, part,
                          dS, dz, p.T, p.lay, p.PB, p.LB, p.eps)
                 : launch(bwd_dq_wide_kernel<T, false, FM>, p.BH * p.PB, Wide::kThreads, s, qq, dd, state, sz, g, part,
                          dS, dz, p.T, p.lay, p.PB, p.LB, p.eps);
    if (e != hipSuccess) return e;
    return launch_combine<D, D>(p.PB, part, dS, dz, p.BH, s);
}
template <typename T, int FM>
hipError_t wide_bwd_dkv_fm(const Plan& p, const void* k, const void* v, void* dk, void* dv, void* ws, hipStream_t s) {
    constexpr int D = Wide::D;
    const float* dS = reinterpret_cast<const float*>(static_cast<char*>(ws) + p.off_dstate);
    const float* dz = dS + p.BH * D * D;
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* gk = static_cast<T*>(dk);
    T* gv = static_cast<T*>(dv);
    if (p.simple)
        return launch(bwd_dkv_wide_kernel<T, true, FM>, p.BH * p.NK, WideKV::kThreads, s, kk, vv, dS, dz, gk, gv, p.T,
                      p.lay, p.NK, p.LK);
    return launch(bwd_dkv_wide_kernel<T, false, FM>, p.BH * p.NK, WideKV::kThreads, s, kk, vv, dS, dz, gk, gv, p.T,
                  p.lay, p.NK, p.LK);
}
// Token split of the D = 256 kernels: one workgroup per CU for the
// reductions (each writes a 263 KB partial), two turns of the chip for the
// streaming steps.
SplitCfg wide_split_config(int step) {
    switch (step) {
        case kStepState:
        case kStepCausalState: return {64, 256};
        case kStepBwdQ: return {32, 256};
        case kStepBwdKV: return {32, 512};
        default: return {32, 512};
    }
}

// 16-bit elements take the 16-bit causal scans, built for head sizes 64 and
// 128: a head size of 32 or 96 runs the kernel for the next of them with the
// missing feature columns read as zeros (phi of them zeroed too) and never
// stored; fp32 elements take the fp32-operand scans.
template <typename T, int DK, int DV>
constexpr bool kCausalKernels = sizeof(T) == 2;
template <int D>
constexpr int kCausalPad = D <= 64 ? 64 : 128;

// Causal forward: segment states, their exclusive prefixes in place (and the
// full state), then the chunked scan of every segment.
template <typename T, int DK, int DV, int FM>
hipError_t fwd_causal_fm(const Plan& p, const void* q, const void* k, const void* v, void* o, float* state,
                         void* ws, hipStream_t s) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_part);
    hipError_t e = launch_state_reduction<T, DK, DV, FM>(p, k, v, state, part, s);
    if (e != hipSuccess) return e;
    if (p.P > 1) {
        constexpr int E4 = (DK * DV + DK) / 4;
        e = launch(prefix_kernel<DK, DV>, p.BH * ((E4 + kThreads - 1) / kThreads), kThreads, s, part, p.P, state,
                   state + p.BH * DK * DV, p.BH);
        if (e != hipSuccess) return e;
    }
    const float* pre = p.P > 1 ? part : nullptr;
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* oo = static_cast<T*>(o);
    const int64_t nblk = p.BH * p.P;
    if constexpr (kCausalKernels<T, DK, DV>) {
        constexpr int DKP = kCausalPad<DK>, DVP = kCausalPad<DV>;
        if (p.simple)
            return launch(fwd_causal_kernel<T, DKP, DVP, true, FM, DK, DV>, nblk, kThreads, s, qq, kk, vv, pre, oo,
                          p.T, p.lay, p.P, p.L, p.eps);
        return launch(fwd_causal_kernel<T, DKP, DVP, false, FM, DK, DV>, nblk, kThreads, s, qq, kk, vv, pre, oo, p.T,
                      p.lay, p.P, p.L, p.eps);
    } else {
        if (p.simple)
            return launch(fwd_causal_f32_kernel<T, DK, DV, true, FM>, nblk, kThreads, s, qq, kk, vv, pre, oo, p.T,
                          p.lay, p.P, p.L, p.eps);
        return launch(fwd_causal_f32_kernel<T, DK, DV, false, FM>, nblk, kThreads, s, qq, kk, vv, pre, oo, p.T,
                      p.lay, p.P, p.L, p.eps);
    }
}

// Causal backward: segment states and their exclusive prefixes (as in the
// causal forward; with reuse_prefix they are already in the workspace, where
// the forward left them), the forward-order dQ scan, the exclusive suffixes
// of its per-segment (G, g) sums, then the reverse-order dK, dV scan.
template <typename T, int DK, int DV, int FM>
hipError_t bwd_causal_fm(const Plan& p, const void* q, const void* k, const void* v, const void* dout, void* dq,
                         void* dk, void* dv, void* ws, hipStream_t s) {
    char* w = static_cast<char*>(ws);
    float* part = reinterpret_cast<float*>(w + p.off_part);
    float* gpart = reinterpret_cast<float*>(w + p.off_cgpart);
    float* wcp = reinterpret_cast<float*>(w + p.off_cwc);
    int* esp = reinterpret_cast<int*>(w + p.off_ces);
    float* total = reinterpret_cast<float*>(w + p.off_fstate);  // the full state; not needed here
    constexpr int E4 = (DK * DV + DK) / 4;
    const int64_t nred = p.BH * ((E4 + kThreads - 1) / kThreads);
    hipError_t e;
    if (p.P > 1 && !p.reuse_prefix) {
        e = launch_state_reduction<T, DK, DV, FM>(p, k, v, total, part, s);
        if (e != hipSuccess) return e;
        e = launch(prefix_kernel<DK, DV>, nred, kThreads, s, part, p.P, total, total + p.BH * DK * DV, p.BH);
        if (e != hipSuccess) return e;
    }
    const float* pre = p.P > 1 ? part : nullptr;
    float* gp = p.P > 1 ? gpart : nullptr;
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    const T* dd = static_cast<const T*>(dout);
    T* dqq = static_cast<T*>(dq);
    T* dkk = static_cast<T*>(dk);
    T* dvv = static_cast<T*>(dv);
    const int64_t nblk = p.BH * p.P;
    constexpr int DKP = kCausalPad<DK>, DVP = kCausalPad<DV>;
    if constexpr (kCausalKernels<T, DK, DV>) {
        e = p.simple ? launch(bwd_causal_q_kernel<T, DKP, DVP, true, FM, DK, DV>, nblk, kThreads, s, qq, kk, vv, dd,
                              pre, dqq, wcp, esp, gp, p.T, p.lay, p.P, p.L, p.nche, p.eps)
                     : launch(bwd_causal_q_kernel<T, DKP, DVP, false, FM, DK, DV>, nblk, kThreads, s, qq, kk, vv, dd,
                              pre, dqq, wcp, esp, gp, p.T, p.lay, p.P, p.L, p.nche, p.eps);
    } else {
        e = p.simple ? launch(bwd_causal_q_f32_kernel<T, DK, DV, true, FM>, nblk, kThreads, s, qq, kk, vv, dd, pre,
                              dqq, wcp, gp, p.T, p.lay, p.P, p.L, p.eps)
                     : launch(bwd_causal_q_f32_kernel<T, DK, DV, false, FM>, nblk, kThreads, s, qq, kk, vv, dd, pre,
                              dqq, wcp, gp, p.T, p.lay, p.P, p.L, p.eps);
    }
    if (e != hipSuccess) return e;
    if (p.P > 1) {
        e = launch(suffix_kernel<DK, DV>, nred, kThreads, s, gpart, p.P, p.BH);
        if (e != hipSuccess) return e;
    }
    if constexpr (kCausalKernels<T, DK, DV>) {
        return p.simple ? launch(bwd_causal_kv_kernel<T, DKP, DVP, true, FM, DK, DV>, nblk, kThreads, s, qq, kk, vv,
                                 dd, wcp, esp, gp, dkk, dvv, p.T, p.lay, p.P, p.L, p.nche, p.eps)
                        : launch(bwd_causal_kv_kernel<T, DKP, DVP, false, FM, DK, DV>, nblk, kThreads, s, qq, kk, vv,
                                 dd, wcp, esp, gp, dkk, dvv, p.T, p.lay, p.P, p.L, p.nche, 1.f);
    } else {
        return p.simple ? launch(bwd_causal_kv_f32_kernel<T, DK, DV, true, FM>, nblk, kThreads, s, qq, kk, vv, dd,
                                 wcp, gp, dkk, dvv, p.T, p.lay, p.P, p.L, p.eps)
                        : launch(bwd_causal_kv_f32_kernel<T, DK, DV, false, FM>, nblk, kThreads, s, qq, kk, vv, dd,
                                 wcp, gp, dkk, dvv, p.T, p.lay, p.P, p.L, p.eps);
    }
}

template <typename T, int DK, int DV, int FM>
hipError_t fwd_output_fm(const Plan& p, const void* q, const float* state, void* o, hipStream_t s) {
    const int64_t nblk = p.BH * p.NQ;
    constexpr int nt = StreamShape<T, DK, DV>::kThreads;
    const T* qq = static_cast<const T*>(q);
    const float* sz = state + p.BH * DK * DV;
    T* oo = static_cast<T*>(o);
    if (p.simple)
        return launch(fwd_output_kernel<T, DK, DV, true, FM>, nblk, nt, s, qq, state, sz, oo, p.T, p.lay, p.NQ, p.LQ,
                      p.eps);
    return launch(fwd_output_kernel<T, DK, DV, false, FM>, nblk, nt, s, qq, state, sz, oo, p.T, p.lay, p.NQ, p.LQ,
                  p.eps);
}

template <typename T, int DK, int DV, int FM>
hipError_t bwd_dq_fm(const Plan& p, const void* q, const void* dout, const float* state, void* dq,
                    void* ws, hipStream_t s) {
    const int64_t nblk = p.BH * p.PB;
    char* w = static_cast<char*>(ws);
    float* part = reinterpret_cast<float*>(w + p.off_part);
    float* dst = reinterpret_cast<float*>(w + p.off_dstate);
    const T* qq = static_cast<const T*>(q);
    const T* dd = static_cast<const T*>(dout);
    const float* sS = state;
    const float* sz = state + p.BH * DK * DV;
    T* g = static_cast<T*>(dq);
    float* dS = dst;
    float* dz = dst + p.BH * DK * DV;
    hipError_t e;
    if constexpr (kWaveKernels<T, DK, DV>) {
        e = p.simple ? launch(bwd_dq_w64_kernel<T, true, FM>, nblk, kThreads, s, qq, dd, sS, sz, g, part, dS, dz, p.T,
                              p.lay, p.PB, p.LB, p.eps)
                     : launch(bwd_dq_w64_kernel<T, false, FM>, nblk, kThreads, s, qq, dd, sS, sz, g, part, dS, dz, p.T,
                              p.lay, p.PB, p.LB, p.eps);
    } else if constexpr (kTileKernels<T, DK, DV>) {
        constexpr int nt = BwdQTile<DK, DV>::kThreads;
        e = p.simple ? launch(bwd_dq_tile_kernel<T, DK, DV, true, FM>, nblk, nt, s, qq, dd, sS, sz, g, part, dS, dz,
                              p.T, p.lay, p.PB, p.LB, p.eps)
                     : launch(bwd_dq_tile_kernel<T, DK, DV, false, FM>, nblk, nt, s, qq, dd, sS, sz, g, part, dS, dz,
                              p.T, p.lay, p.PB, p.LB, p.eps);
    } else {
        e = p.simple ? launch(bwd_dq_kernel<T, DK, DV, true, FM>, nblk, kThreads, s, qq, dd, sS, sz, g, part, dS, dz,
                              p.T, p.lay, p.PB, p.LB, p.eps)
                     : launch(bwd_dq_kernel<T, DK, DV, false, FM>, nblk, kThreads, s, qq, dd, sS, sz, g, part, dS, dz,
                              p.T, p.lay, p.PB, p.LB, p.eps);
    }
    if (e != hipSuccess) return e;
    return launch_combine<DK, DV>(p.PB, part, dS, dz, p.BH, s);
}

template <typename T, int DK, int DV, int FM>
hipError_t bwd_dkv_fm(const Plan& p, const void* k, const void* v, void* dk, void* dv, void* ws,
                     hipStream_t s) {
    const int64_t nblk = p.BH * p.NK;
    constexpr int nt = StreamShape<T, DK, DV>::kThreads;
    const float* dst = reinterpret_cast<const float*>(static_cast<char*>(ws) + p.off_dstate);
    const float* dz = dst + p.BH * DK * DV;
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* gk = static_cast<T*>(dk);
    T* gv = static_cast<T*>(dv);
    if (p.simple)
        return launch(bwd_dkv_kernel<T, DK, DV, true, FM>, nblk, nt, s, kk, vv, dst, dz, gk, gv, p.T, p.lay, p.NK,
                      p.LK);
    return launch(bwd_dkv_kernel<T, DK, DV, false, FM>, nblk, nt, s, kk, vv, dst, dz, gk, gv, p.T, p.lay, p.NK,
                  p.LK);
}

// The feature map is a template parameter of every kernel: one switch here.
#define LA_FEATURE_MAP(FN, ...)                                                    \
    switch (p.fm) {                                                                \
        case kPhiRelu: return FN<T, DK, DV, kPhiRelu>(p, __VA_ARGS__);             \
        case kPhiIdentity: return FN<T, DK, DV, kPhiIdentity>(p, __VA_ARGS__);     \
        default: return FN<T, DK, DV, kPhiElu1>(p, __VA_ARGS__);                   \
    }

template <typename T, int DK, int DV>
hipError_t fwd_state_t(const Plan& p, const void* k, const void* v, float* state, void* ws, hipStream_t s) {
    LA_FEATURE_MAP(fwd_state_fm, k, v, state, ws, s);
}
template <typename T, int DK, int DV>
hipError_t fwd_output_t(const Plan& p, const void* q, const float* state, void* o, hipStream_t s) {
    LA_FEATURE_MAP(fwd_output_fm, q, state, o, s);
}
template <typename T, int DK, int DV>
hipError_t fwd_causal_t(const Plan& p, const void* q, const void* k, const void* v, void* o, float* state, void* ws,
                        hipStream_t s) {
    LA_FEATURE_MAP(fwd_causal_fm, q, k, v, o, state, ws, s);
}
template <typename T, int DK, int DV>
hipError_t bwd_causal_t(const Plan& p, const void* q, const void* k, const void* v, const void* dout, void* dq,
                        void* dk, void* dv, void* ws, hipStream_t s) {
    LA_FEATURE_MAP(bwd_causal_fm, q, k, v, dout, dq, dk, dv, ws, s);
}
template <typename T, int DK, int DV>
hipError_t bwd_dq_t(const Plan& p, const void* q, const void* dout, const float* state, void* dq, void* ws,
                    hipStream_t s) {
    LA_FEATURE_MAP(bwd_dq_fm, q, dout, state, dq, ws, s);
}
template <typename T, int DK, int DV>
hipError_t bwd_dkv_t(const Plan& p, const void* k, const void* v, void* dk, void* dv, void* ws, hipStream_t s) {
    LA_FEATURE_MAP(bwd_dkv_fm, k, v, dk, dv, ws, s);
}

// Grid targets of the tile kernels, in workgroups: enough that each CU has
// about 64 KB of loads in flight (a tile kernel's workgroup keeps two tiles or
// rounds of DK + DV wide rows in flight), within 2 to 8 workgroups per CU of
// the 256 for the state; for dQ (DK / 16 waves per workgroup) at least 8
// waves and at most 8 workgroups per CU.
constexpr int64_t clamp_wgs(int64_t per_cu, int64_t lo, int64_t hi) {
    return 256 * (per_cu < lo ? lo : per_cu > hi ? hi : per_cu);
}
template <int DK, int DV>
constexpr int64_t kStateTileWgs = clamp_wgs(512 / (DK + DV), 2, 8);
template <int DK, int DV>
constexpr int64_t kBwdQTileWgs = clamp_wgs(16384 / (DK * (DK + DV)), (128 + DK - 1) / DK, 8);

template <typename T, int DK, int DV>
SplitCfg split_config_t(int step) {
    switch (step) {
        case kStepState:
            // one workgroup per CU at D = 64: 89.8 us against 93.3 us at two
            // (B8-H16-T16384-D64 f16; T = 4096: 31.8 against 35.6 us)
            if constexpr (kWaveKernels<T, DK, DV>) return {int64_t(StateW64::kStep) * kWaves * StateW64::kStages, 256};
            else if constexpr (kTileKernels<T, DK, DV>)
                return {int64_t(StateTile<DK, DV>::kTile) * StateTile<DK, DV>::kStages, kStateTileWgs<DK, DV>};
            else return {StateShape<T, DK, DV>::kTT, 1024};
        case kStepCausalState:
            // the causal scans' segments: two workgroups per CU at D = 64
            if constexpr (kWaveKernels<T, DK, DV>) return {int64_t(StateW64::kStep) * kWaves * StateW64::kStages, 512};
            else if constexpr (kTileKernels<T, DK, DV>)
                return {int64_t(StateTile<DK, DV>::kTile) * StateTile<DK, DV>::kStages, kStateTileWgs<DK, DV>};
            else return {StateShape<T, DK, DV>::kTT, 1024};
        case kStepBwdQ:
            if constexpr (kWaveKernels<T, DK, DV>) return {int64_t(BwdQW64::kRound) * BwdQW64::kStages, 512};
            else if constexpr (kTileKernels<T, DK, DV>)
                return {int64_t(BwdQTile<DK, DV>::kRound) * BwdQTile<DK, DV>::kStages, kBwdQTileWgs<DK, DV>};
            else return {BwdQShape<T, DK, DV>::kG, 1024};
        case kStepBwdKV:
            // the rounds of a head are dealt to its workgroups in turn (see the
            // kernel); for 16-bit heads up to 64 wide (four workgroups per CU)
            // a grid of two full turns of the chip measured best: 187 us
            // against 200 us at one turn and 201 us with contiguous chunks
            // (B8-H16-T16384-D64 f16)
            return {int64_t(StreamShape<T, DK, DV>::kStages) * 16 * StreamShape<T, DK, DV>::kWaves,
                    StreamShape<T, DK, DV>::kSmall ? 2048 : 1024,
                    // and at most 1024 tokens per workgroup where that asks for
                    // more: B2-H8-T262144-D64 bf16 417 us against 440 us at 2048
                    // workgroups (2048 tokens each); the headline shape is at
                    // 1024 tokens already
                    StreamShape<T, DK, DV>::kSmall ? 1024 : 0};
        default:
            // the output: at least four turns of the pipeline per workgroup, so
            // that short sequences do not spend their workgroups on prologues
            // (B8-H16-T4096-D64 f16: 34.9 -> 29.2 us; T = 16384 unchanged)
            return {4 * StreamShape<T, DK, DV>::kStages * StreamShape<T, DK, DV>::kG, 2048};
    }
}

// ---------------------------------------------------------------------------
// This compilation unit: one element type and one Q/K head size, every V head
// size. The build compiles the file once per (LA_UNIT_DTYPE, LA_UNIT_DK).
// ---------------------------------------------------------------------------
#if !defined(LA_UNIT_DTYPE) || !defined(LA_UNIT_DK)
#error "compile once per unit with -DLA_UNIT_DTYPE=<0|1|2> (la_dtype) -DLA_UNIT_DK=<32|64|96|128|256>"
#endif

template <int DT> struct UnitType;
template <> struct UnitType<0> { using type = float; };
template <> struct UnitType<1> { using type = f16; };
template <> struct UnitType<2> { using type = bf16; };
using UT = UnitType<LA_UNIT_DTYPE>::type;
constexpr int UDK = LA_UNIT_DK;

#if LA_UNIT_DK == 256
// D = DV = 256, 16-bit: the wide kernels (no causal form at this size).
#define LA_WIDE_MAP(FN, ...)                                                       \
    switch (p.fm) {                                                                \
        case kPhiRelu: return FN<UT, kPhiRelu>(p, __VA_ARGS__);                    \
        case kPhiIdentity: return FN<UT, kPhiIdentity>(p, __VA_ARGS__);            \
        default: return FN<UT, kPhiElu1>(p, __VA_ARGS__);                          \
    }
static_assert(sizeof(UT) == 2, "head size 256 is built for 16-bit inputs only");
hipError_t unit_fwd_state(const Plan& p, const void* k, const void* v, float* state, void* ws, hipStream_t s) {
    LA_WIDE_MAP(wide_fwd_state_fm, k, v, state, ws, s);
}
hipError_t unit_fwd_output(const Plan& p, const void* q, const float* state, void* o, hipStream_t s) {
    LA_WIDE_MAP(wide_fwd_output_fm, q, state, o, s);
}
hipError_t unit_bwd_dq(const Plan& p, const void* q, const void* dout, const float* state, void* dq, void* ws,
                       hipStream_t s) {
    LA_WIDE_MAP(wide_bwd_dq_fm, q, dout, state, dq, ws, s);
}
hipError_t unit_bwd_dkv(const Plan& p, const void* k, const void* v, void* dk, void* dv, void* ws, hipStream_t s) {
    LA_WIDE_MAP(wide_bwd_dkv_fm, k, v, dk, dv, ws, s);
}
hipError_t unit_fwd_causal(const Plan&, const void*, const void*, const void*, void*, float*, void*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t unit_bwd_causal(const Plan&, const void*, const void*, const void*, const void*, void*, void*, void*, void*,
                           hipStream_t) {
    return hipErrorInvalidValue;
}
SplitCfg unit_split_config(int step, int) { return wide_split_config(step); }
#undef LA_WIDE_MAP
#else
#define LA_DV_DISPATCH(FN, ...)                                       \
    switch (p.DV) {                                                   \
        case 32: return FN<UT, UDK, 32>(p, __VA_ARGS__);              \
        case 64: return FN<UT, UDK, 64>(p, __VA_ARGS__);              \
        case 96: return FN<UT, UDK, 96>(p, __VA_ARGS__);              \
        case 128: return FN<UT, UDK, 128>(p, __VA_ARGS__);            \
        default: return hipErrorInvalidValue;                         \
    }

hipError_t unit_fwd_state(const Plan& p, const void* k, const void* v, float* state, void* ws, hipStream_t s) {
    LA_DV_DISPATCH(fwd_state_t, k, v, state, ws, s);
}
hipError_t unit_fwd_output(const Plan& p, const void* q, const float* state, void* o, hipStream_t s) {
    LA_DV_DISPATCH(fwd_output_t, q, state, o, s);
}
hipError_t unit_fwd_causal(const Plan& p, const void* q, const void* k, const void* v, void* o, float* state,
                           void* ws, hipStream_t s) {
    LA_DV_DISPATCH(fwd_causal_t, q, k, v, o, state, ws, s);
}
hipError_t unit_bwd_dq(const Plan& p, const void* q, const void* dout, const float* state, void* dq, void* ws,
                       hipStream_t s) {
    LA_DV_DISPATCH(bwd_dq_t, q, dout, state, dq, ws, s);
}
hipError_t unit_bwd_dkv(const Plan& p, const void* k, const void* v, void* dk, void* dv, void* ws, hipStream_t s) {
    LA_DV_DISPATCH(bwd_dkv_t, k, v, dk, dv, ws, s);
}
hipError_t unit_bwd_causal(const Plan& p, const void* q, const void* k, const void* v, const void* dout, void* dq,
                           void* dk, void* dv, void* ws, hipStream_t s) {
    LA_DV_DISPATCH(bwd_causal_t, q, k, v, dout, dq, dk, dv, ws, s);
}
SplitCfg unit_split_config(int step, int DV) {
    switch (DV) {
        case 32: return split_config_t<UT, UDK, 32>(step);
        case 64: return split_config_t<UT, UDK, 64>(step);
        case 96: return split_config_t<UT, UDK, 96>(step);
        default: return split_config_t<UT, UDK, 128>(step);
    }
}

#endif

const KernelSet kUnitSet = {unit_fwd_state, unit_fwd_output, unit_bwd_dq,    unit_bwd_dkv,
                             unit_split_config, unit_fwd_causal, unit_bwd_causal};

}  // namespace

#define LA_UNIT_NAME2(dt, dk) kernel_set_##dt##_##dk
#define LA_UNIT_NAME(dt, dk) LA_UNIT_NAME2(dt, dk)
const KernelSet* LA_UNIT_NAME(LA_UNIT_DTYPE, LA_UNIT_DK)() { return &kUnitSet; }

}  // namespace la
