// common.hpp -- device helpers shared by the gfx950 kernels of libatomattn.
//
// Storage types: float (fp32) or bf16_t (bfloat16 bits). All arithmetic is
// fp32. Matrix products run on the CDNA4 matrix cores (MFMA) with 16-byte
// per-lane operand chunks:
//   * 32x32 output tiles (projections): v_mfma_f32_32x32x16_bf16 for bf16,
//     four v_mfma_f32_32x32x2_f32 for fp32;
//   * 16x16 output tiles (slot attention): v_mfma_f32_16x16x32_bf16, or four
//     v_mfma_f32_16x16x4_f32.
// The k order inside a chunk is a free choice (a matrix product sums over k
// in any order), so each lane always supplies 16 contiguous bytes of its
// row (A operand) or column (B operand): lane half h (32x32) or lane
// quarter g (16x16) supplies k = chunk_base + h*HALF + e (resp. g*QUARTER+e).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace waa {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) {
    return __uint_as_float(((uint32_t)x) << 16);
}

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
// fp32 -> bf16, round to nearest even (NaN stays NaN): the gfx950
// conversion instruction (v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) {
    return __builtin_bit_cast(bf16_t, (__bf16)x);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values -> two bf16 packed in one word (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 16 bytes of storage-type values -> 16/sizeof(T) floats.
template <typename T>
__device__ __forceinline__ void unpack16(uint4 v, float *out) {
    if constexpr (sizeof(T) == 4) {
        out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// 16/sizeof(T) floats -> 16 bytes of storage-type values (round to nearest
// even for bf16).
template <typename T>
__device__ __forceinline__ uint4 pack16(const float *in) {
    if constexpr (sizeof(T) == 4) {
        return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                          __float_as_uint(in[3]));
    } else {
        return make_uint4(pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                          pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7]));
    }
}

// Logistic function from e = exp(-|z|) in (0, 1]: 1/(1+e) for z >= 0 and
// e/(1+e) below, so a very negative argument keeps its tiny (down to
// subnormal) value instead of 1 - 1. exp2f keeps subnormal results (the
// compiler range-scales them); the reciprocal is the hardware one (1 ulp).
__device__ __forceinline__ float sigmoid_f(float z) {
    const float e = exp2f(-fabsf(z) * 1.4426950408889634f);
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return z >= 0.0f ? r : e * r;
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// ---------------------------------------------------------- reductions
// Butterfly reductions over aligned lane groups of width W (power of 2).

template <int W> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1)
        v += __shfl_xor(v, m, W);
    return v;
}
template <int W> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1)
        v = fmaxf(v, __shfl_xor(v, m, W));
    return v;
}
// Reductions over aligned groups of 16 lanes with DPP lane permutations
// (pure VALU, no LDS traffic): swap neighbours, swap pairs, mirror within
// 8, mirror within 16 -- after the four steps every lane holds the result.
__device__ __forceinline__ float dpp_f(float v, int ctrl) {
    switch (ctrl) {
    case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    }
}
// Sum over aligned groups of 8 lanes (the first three steps of sum16).
__device__ __forceinline__ float sum8(float v) {
    v += dpp_f(v, 0xB1);
    v += dpp_f(v, 0x4E);
    v += dpp_f(v, 0x141);
    return v;
}
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f(v, 0xB1);
    v += dpp_f(v, 0x4E);
    v += dpp_f(v, 0x141);
    v += dpp_f(v, 0x140);
    return v;
}
// Row sum over the TPR threads of a tile row (aligned lane groups of 8 or 16).
template <int TPR> __device__ __forceinline__ float row_sum(float x) {
    return TPR == 16 ? sum16(x) : sum8(x);
}
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, dpp_f(v, 0xB1));
    v = fmaxf(v, dpp_f(v, 0x4E));
    v = fmaxf(v, dpp_f(v, 0x141));
    v = fmaxf(v, dpp_f(v, 0x140));
    return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        v = min(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        v = max(v, __shfl_xor(v, m, 64));
    return v;
}

// -------------------------------------------------------- MFMA wrappers

template <typename T> struct Mma32;
template <> struct Mma32<bf16_t> {
    static constexpr int KC = 16;  // k values per 16-byte chunk
    static constexpr int HALF = 8; // k values per lane half
    __device__ static __forceinline__ void mma(f32x16_t &acc, uint4 a, uint4 b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
            acc, 0, 0, 0);
    }
};
template <> struct Mma32<float> {
    static constexpr int KC = 8;
    static constexpr int HALF = 4;
    __device__ static __forceinline__ void mma(f32x16_t &acc, uint4 a, uint4 b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
};

template <typename T> struct Mma16;
template <> struct Mma16<bf16_t> {
    static constexpr int KC = 32;
    static constexpr int QUARTER = 8;
    __device__ static __forceinline__ void mma(f32x4_t &acc, uint4 a, uint4 b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
            acc, 0, 0, 0);
    }
};
template <> struct Mma16<float> {
    static constexpr int KC = 16;
    static constexpr int QUARTER = 4;
    __device__ static __forceinline__ void mma(f32x4_t &acc, uint4 a, uint4 b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
};

// Output element v of a 32x32 accumulator in this lane: (row, col).
__device__ __forceinline__ int acc32_row(int v, int lane) {
    return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}
__device__ __forceinline__ int acc32_col(int lane) { return lane & 31; }
// Output element v of a 16x16 accumulator in this lane.
__device__ __forceinline__ int acc16_row(int v, int lane) { return (lane >> 4) * 4 + v; }
__device__ __forceinline__ int acc16_col(int lane) { return lane & 15; }

// Padding (in elements) that makes a row pitch 16 bytes longer than the
// data, so that the 32 rows of an operand tile start in different LDS banks.
template <typename T> constexpr int pad16() { return 16 / (int)sizeof(T); }

// Matrix products acc1 += A1 @ B1 (and, with DUAL, acc2 += A2 @ B2) over
// nk1 (nk2) 16-byte k-chunks, nk >= 1.
// A: LDS tiles, row-major, pitch lda elements (16-byte aligned rows); with
//    SPLIT each is an unevaluated sum hi + lo of two tiles in the storage
//    type (for bf16 it keeps ~16 mantissa bits of an fp32 activation at
//    twice the MFMA work).
// B: packed weight blocks (see pack.hip): chunk kc of the column block at
//    B[kc*64 + lane], 16 bytes per lane, read from L2.
// Software pipeline: P B chunks per product are in flight; each chunk is
// consumed and its register refilled with the chunk P ahead. Every load
// is unconditional (indices clamp to the last chunk, so the tail re-reads
// it), which lets the compiler wait for exactly the chunk it needs instead
// of draining all loads; the A chunks of a group are read from LDS together.
// P: pipeline depth in 16-byte chunks per product (4 by default; 2 saves
// registers where that lets more workgroups fit a CU).
template <typename T, bool DUAL, bool SPLIT, int P = 4>
__device__ __forceinline__ void gemm_pipe(f32x16_t &acc1, const T *A1, const T *A1lo,
                                          int lda1, int nk1, const uint4 *__restrict__ B1,
                                          f32x16_t &acc2, const T *A2, const T *A2lo,
                                          int lda2, int nk2, const uint4 *__restrict__ B2) {
    constexpr int KC = Mma32<T>::KC;
    const int lane = threadIdx.x & 63;
    const int o1 = (lane & 31) * lda1 + (lane >> 5) * Mma32<T>::HALF;
    const int o2 = DUAL ? (lane & 31) * lda2 + (lane >> 5) * Mma32<T>::HALF : 0;
    const int nk = DUAL ? (nk1 > nk2 ? nk1 : nk2) : nk1;
    const int l1 = nk1 - 1, l2 = DUAL ? nk2 - 1 : 0;
    uint4 b1[P], b2[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        b1[j] = B1[(j < l1 ? j : l1) * 64 + lane];
        if (DUAL)
            b2[j] = B2[(j < l2 ? j : l2) * 64 + lane];
    }
    for (int kb = 0; kb < nk; kb += P) {
        uint4 x1[P], x1l[P], x2[P], x2l[P];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int k1 = kb + j < l1 ? kb + j : l1;
            x1[j] = *reinterpret_cast<const uint4 *>(A1 + o1 + k1 * KC);
            if (SPLIT)
                x1l[j] = *reinterpret_cast<const uint4 *>(A1lo + o1 + k1 * KC);
            if (DUAL) {
                const int k2 = kb + j < l2 ? kb + j : l2;
                x2[j] = *reinterpret_cast<const uint4 *>(A2 + o2 + k2 * KC);
                if (SPLIT)
                    x2l[j] = *reinterpret_cast<const uint4 *>(A2lo + o2 + k2 * KC);
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int k = kb + j;
            if (k < nk1) {
                Mma32<T>::mma(acc1, x1[j], b1[j]);
                if (SPLIT)
                    Mma32<T>::mma(acc1, x1l[j], b1[j]);
            }
            if (DUAL && k < nk2) {
                Mma32<T>::mma(acc2, x2[j], b2[j]);
                if (SPLIT)
                    Mma32<T>::mma(acc2, x2l[j], b2[j]);
            }
            const int n1 = k + P < l1 ? k + P : l1;
            b1[j] = B1[n1 * 64 + lane];
            if (DUAL) {
                const int n2 = k + P < l2 ? k + P : l2;
                b2[j] = B2[n2 * 64 + lane];
            }
        }
    }
}

template <typename T, bool SPLIT = false, int P = 4>
__device__ __forceinline__ void gemm2(f32x16_t &acc1, const T *A1, const T *A1lo, int lda1,
                                      int nk1, const uint4 *__restrict__ B1, f32x16_t &acc2,
                                      const T *A2, const T *A2lo, int lda2, int nk2,
                                      const uint4 *__restrict__ B2) {
    gemm_pipe<T, true, SPLIT, P>(acc1, A1, A1lo, lda1, nk1, B1, acc2, A2, A2lo, lda2, nk2, B2);
}

template <typename T, bool SPLIT = false, int P = 4>
__device__ __forceinline__ void gemm1(f32x16_t &acc, const T *A, const T *Alo, int lda, int nk,
                                      const uint4 *__restrict__ B) {
    gemm_pipe<T, false, SPLIT, P>(acc, A, Alo, lda, nk, B, acc, A, Alo, lda, 0, B);
}

// Store x into a split operand pair: hi = x rounded to T, lo = the rest
// rounded to T (for fp32 storage lo is not used).
template <typename T>
__device__ __forceinline__ void put_split(T *hi, T *lo, int idx, float x) {
    const T h = from_f<T>(x);
    hi[idx] = h;
    if (lo != nullptr)
        lo[idx] = from_f<T>(x - to_f(h));
}

__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        z[i] = 0.0f;
    return z;
}
__device__ __forceinline__ f32x4_t zero4() {
    f32x4_t z;
    z[0] = z[1] = z[2] = z[3] = 0.0f;
    return z;
}

// ------------------------------------------------------- AF3 pair bias
// ("windowed_atom_attention", Required behavior, AF3 encoder page): the
// bias of head h for a slot with pair row x (V channels) is
// LN(x) . (pair_scale * w_pair[:, h]). With d = x - x[0] (shifted data
// keeps the one-pass variance well conditioned):
//   LN(x) . w_h = rstd * (sum_v d_v w_vh - mean(d) * sum_v w_vh),
//   rstd = 1 / sqrt(mean(d^2) - mean(d)^2 + eps).

// LDS weights: w4[v] = pair_scale[v] * w_pair[v][0..3] (heads past H are
// zero), and partial column sums wpart[2][4] (lanes of one head reduced
// per wave; V <= 32). Every thread of the (>= 128-thread) block calls it.
template <typename T>
__device__ __forceinline__ void pair_weights_put(T sv, T wv, int V, int H, float *w4,
                                                 float *wpart) {
    const int i = threadIdx.x;
    float w = 0.0f;
    if (i < V * 4) {
        w = i % 4 < H ? to_f(sv) * to_f(wv) : 0.0f;
        w4[i] = w;
    }
    if (i < 128) { // waves 0 and 1 (whole waves): sum over the lanes of head i % 4
        w += __shfl_xor(w, 4);
        w += __shfl_xor(w, 8);
        w += __shfl_xor(w, 16);
        w += __shfl_xor(w, 32);
        if ((i & 63) < 4)
            wpart[(i >> 6) * 4 + (i & 3)] = w;
    }
}
// The two factors of this thread's weight, loaded unconditionally (indices
// clamped; the values of threads past V * 4 are not used), so that a
// kernel can issue them early and store them later with pair_weights_put.
template <typename T>
__device__ __forceinline__ void pair_weights_load(const T *ps, const T *wp, int V, int H, T &sv,
                                                  T &wv) {
    const int i = threadIdx.x;
    const int v = min(i / 4, V - 1), h = min(i % 4, H - 1);
    sv = ps[v];
    wv = wp[v * H + h];
}
template <typename T>
__device__ __forceinline__ void pair_weights(const T *ps, const T *wp, int V, int H, float *w4,
                                             float *wpart) {
    T sv, wv;
    pair_weights_load<T>(ps, wp, V, H, sv, wv);
    pair_weights_put<T>(sv, wv, V, H, w4, wpart);
}

// Column sums of the weights (after a barrier that follows pair_weights).
__device__ __forceinline__ float4 pair_wsum(const float *wpart) {
    const float4 a = reinterpret_cast<const float4 *>(wpart)[0];
    const float4 b = reinterpret_cast<const float4 *>(wpart)[1];
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Bias of heads 0..3 for G slots whose pair rows (NV 16-byte vectors each)
// are in registers; w4p from pair_weights, ws from pair_wsum.
template <typename T, int NV, int G>
__device__ __forceinline__ void pair_bias_rows(const uint4 (&rows)[G][NV], const float4 *w4p,
                                               float4 ws, float eps, float (&out)[G][4]) {
    constexpr int E = 16 / sizeof(T);
    constexpr float kInvV = 1.0f / (float)(NV * E);
    float x0[G], sd[G], sq[G], bb[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float t[E];
        unpack16<T>(rows[g][0], t);
        x0[g] = t[0];
        sd[g] = sq[g] = 0.0f;
#pragma unroll
        for (int h = 0; h < 4; ++h)
            bb[g][h] = 0.0f;
    }
#pragma unroll
    for (int pt = 0; pt < NV; ++pt) {
        float xv[G][E];
#pragma unroll
        for (int g = 0; g < G; ++g)
            unpack16<T>(rows[g][pt], xv[g]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float4 w4 = w4p[pt * E + e]; // one broadcast read, all heads
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float dv = xv[g][e] - x0[g];
                sd[g] += dv;
                sq[g] = fmaf(dv, dv, sq[g]);
                bb[g][0] = fmaf(dv, w4.x, bb[g][0]);
                bb[g][1] = fmaf(dv, w4.y, bb[g][1]);
                bb[g][2] = fmaf(dv, w4.z, bb[g][2]);
                bb[g][3] = fmaf(dv, w4.w, bb[g][3]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float md = sd[g] * kInvV;
        const float var = fmaxf(fmaf(sq[g], kInvV, -md * md), 0.0f);
        const float rstd = rsqrtf(var + eps);
        out[g][0] = (bb[g][0] - md * ws.x) * rstd;
        out[g][1] = (bb[g][1] - md * ws.y) * rstd;
        out[g][2] = (bb[g][2] - md * ws.z) * rstd;
        out[g][3] = (bb[g][3] - md * ws.w) * rstd;
    }
}

// Zero the padding columns A .. vt_pitch(A)-1 of the transposed V rows
// ([B][HD][pitch]); row i goes to workgroup i % nwg.
template <typename T>
__device__ __forceinline__ void zero_vt_pad(T *vt, int B, int HD, int A, int wg, int nwg) {
    const int pitch = vt_pitch(A), w = pitch - A;
    for (int64_t i = wg; i < (int64_t)B * HD; i += nwg)
        for (int e = threadIdx.x; e < w; e += blockDim.x)
            vt[i * pitch + A + e] = (T)0;
}

// Load / store of a V at a 32-bit byte offset from a base pointer. With a
// base that is uniform over the wave this is the scalar-base addressing form
// (64-bit base in scalar registers, 32-bit offset per lane): no 64-bit
// address arithmetic and one vector register per address.
template <typename V>
__device__ __forceinline__ V ld_off(const void *base, uint32_t bytes) {
    return *reinterpret_cast<const V *>(reinterpret_cast<const char *>(base) + bytes);
}
template <typename V>
__device__ __forceinline__ void st_off(void *base, uint32_t bytes, V v) {
    *reinterpret_cast<V *>(reinterpret_cast<char *>(base) + bytes) = v;
}

// Map the hardware dispatch order (round-robin over the 8 XCDs of MI355X)
// to a logical block index such that consecutive logical blocks run on the
// same XCD and share its L2. Bijective on [0, nblk).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    const int X = 8;
    const int full = (nblk / X) * X;
    if (bid >= full)
        return bid;
    return (bid % X) * (full / X) + bid / X;
}

// 32 x 16 output strips of a 32-row tile (8-wave workgroups): the same
// product as gemm_pipe on 16x16 MFMA tiles, c[0] for rows 0-15 and c[1] for
// rows 16-31, both fed by one B chunk. B: packed strips (pack.hip, strip
// layout): chunk kc at B[kc*64 + lane], lane quarter g = lane/16 holding
// k = kc*KC + g*QUARTER + e of column lane%16. nk in 16-byte k-chunks of
// Mma16<T>::KC.
template <typename T, bool DUAL, bool SPLIT, int P = 4>
__device__ __forceinline__ void gemm_pipe16(f32x4_t (&c1)[2], const T *A1, const T *A1lo,
                                            int lda1, int nk1, const uint4 *__restrict__ B1,
                                            f32x4_t (&c2)[2], const T *A2, const T *A2lo,
                                            int lda2, int nk2, const uint4 *__restrict__ B2) {
    constexpr int KC = Mma16<T>::KC, QU = Mma16<T>::QUARTER;
    const int lane = threadIdx.x & 63;
    const int o1 = (lane & 15) * lda1 + (lane >> 4) * QU, h1 = 16 * lda1;
    const int o2 = DUAL ? (lane & 15) * lda2 + (lane >> 4) * QU : 0, h2 = DUAL ? 16 * lda2 : 0;
    const int nk = DUAL ? (nk1 > nk2 ? nk1 : nk2) : nk1;
    const int l1 = nk1 - 1, l2 = DUAL ? nk2 - 1 : 0;
    uint4 b1[P], b2[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        b1[j] = B1[(j < l1 ? j : l1) * 64 + lane];
        if (DUAL)
            b2[j] = B2[(j < l2 ? j : l2) * 64 + lane];
    }
    for (int kb = 0; kb < nk; kb += P) {
        uint4 x1[P][2], x1l[P][2], x2[P][2], x2l[P][2];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int k1 = kb + j < l1 ? kb + j : l1;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                x1[j][t] = *reinterpret_cast<const uint4 *>(A1 + o1 + t * h1 + k1 * KC);
                if (SPLIT)
                    x1l[j][t] = *reinterpret_cast<const uint4 *>(A1lo + o1 + t * h1 + k1 * KC);
            }
            if (DUAL) {
                const int k2 = kb + j < l2 ? kb + j : l2;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    x2[j][t] = *reinterpret_cast<const uint4 *>(A2 + o2 + t * h2 + k2 * KC);
                    if (SPLIT)
                        x2l[j][t] = *reinterpret_cast<const uint4 *>(A2lo + o2 + t * h2 + k2 * KC);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int k = kb + j;
            if (k < nk1) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    Mma16<T>::mma(c1[t], x1[j][t], b1[j]);
                    if (SPLIT)
                        Mma16<T>::mma(c1[t], x1l[j][t], b1[j]);
                }
            }
            if (DUAL && k < nk2) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    Mma16<T>::mma(c2[t], x2[j][t], b2[j]);
                    if (SPLIT)
                        Mma16<T>::mma(c2[t], x2l[j][t], b2[j]);
                }
            }
            const int n1 = k + P < l1 ? k + P : l1;
            b1[j] = B1[n1 * 64 + lane];
            if (DUAL) {
                const int n2 = k + P < l2 ? k + P : l2;
                b2[j] = B2[n2 * 64 + lane];
            }
        }
    }
}

// Output layouts of the GEMM stages of a 32-row tile, as policies:
//  Blk32<T>: 32x32 blocks (4-wave workgroups), 16 accumulator elements a
//            lane, packed weights in the block layout;
//  Blk16<T>: 32x16 strips (8-wave workgroups), 8 elements a lane, packed
//            weights in the strip layout.
// BW: output columns per block; NW: waves per workgroup; KC: k values per
// 16-byte chunk; row(i, lane) / col(lane): the tile row and block column of
// accumulator element i; colsum: the sum over the lanes that hold one
// column (whose owner lanes are col_owner).
template <typename T> struct Blk32 {
    static constexpr int BW = 32, NW = 4, NE = 16, KC = Mma32<T>::KC;
    struct Acc {
        f32x16_t a;
    };
    __device__ static __forceinline__ Acc zero() { return Acc{zero16()}; }
    __device__ static __forceinline__ float at(const Acc &x, int i) { return x.a[i]; }
    __device__ static __forceinline__ void put(Acc &x, int i, float v) { x.a[i] = v; }
    __device__ static __forceinline__ int row(int i, int lane) { return acc32_row(i, lane); }
    __device__ static __forceinline__ int col(int lane) { return lane & 31; }
    __device__ static __forceinline__ float colsum(float x) { return x + __shfl_xor(x, 32); }
    __device__ static __forceinline__ bool col_owner(int lane) { return lane < 32; }
    template <bool DUAL, bool SPLIT, int P>
    __device__ static __forceinline__ void pipe(Acc &c1, const T *A1, const T *A1lo, int lda1,
                                                int nk1, const uint4 *B1, Acc &c2, const T *A2,
                                                const T *A2lo, int lda2, int nk2, const uint4 *B2) {
        gemm_pipe<T, DUAL, SPLIT, P>(c1.a, A1, A1lo, lda1, nk1, B1, c2.a, A2, A2lo, lda2, nk2, B2);
    }
};
template <typename T> struct Blk16 {
    static constexpr int BW = 16, NW = 8, NE = 8, KC = Mma16<T>::KC;
    struct Acc {
        f32x4_t t[2];
    };
    __device__ static __forceinline__ Acc zero() { return Acc{{zero4(), zero4()}}; }
    __device__ static __forceinline__ float at(const Acc &x, int i) { return x.t[i >> 2][i & 3]; }
    __device__ static __forceinline__ void put(Acc &x, int i, float v) { x.t[i >> 2][i & 3] = v; }
    __device__ static __forceinline__ int row(int i, int lane) {
        return (i >> 2) * 16 + (lane >> 4) * 4 + (i & 3);
    }
    __device__ static __forceinline__ int col(int lane) { return lane & 15; }
    __device__ static __forceinline__ float colsum(float x) {
        x += __shfl_xor(x, 16);
        return x + __shfl_xor(x, 32);
    }
    __device__ static __forceinline__ bool col_owner(int lane) { return lane < 16; }
    template <bool DUAL, bool SPLIT, int P>
    __device__ static __forceinline__ void pipe(Acc &c1, const T *A1, const T *A1lo, int lda1,
                                                int nk1, const uint4 *B1, Acc &c2, const T *A2,
                                                const T *A2lo, int lda2, int nk2, const uint4 *B2) {
        gemm_pipe16<T, DUAL, SPLIT, P>(c1.t, A1, A1lo, lda1, nk1, B1, c2.t, A2, A2lo, lda2, nk2, B2);
    }
};

// One GEMM stage of a 32-row tile in layout L (one wave per output block,
// blocks nb = wave, wave + NW, ...): for every block nb < nblocks,
// x1 = A1 @ B1[nb] (and x2 = A2 @ B2[nb]), then epi(r, c, x1, x2) for each
// accumulator element of the lane (tile row r, stage column c). B1[nb]
// starts at B1 + nb * bs1 (16-byte units); nk in chunks of L::KC.
template <typename L, typename T, bool DUAL, bool SPLIT, int P = 4, typename Epi>
__device__ __forceinline__ void gemm_stage(int nblocks, const T *A1, const T *A1lo, int lda1,
                                           int nk1, const uint4 *B1, int64_t bs1,
                                           const T *A2, const T *A2lo, int lda2, int nk2,
                                           const uint4 *B2, int64_t bs2, Epi &&epi) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int nb = wave; nb < nblocks; nb += L::NW) {
        typename L::Acc a1 = L::zero(), a2 = L::zero();
        L::template pipe<DUAL, SPLIT, P>(a1, A1, A1lo, lda1, nk1, B1 + nb * bs1,
                                         a2, A2, A2lo, lda2, nk2, DUAL ? B2 + nb * bs2 : B1);
        const int c0 = nb * L::BW + L::col(lane);
#pragma unroll
        for (int i = 0; i < L::NE; ++i)
            epi(L::row(i, lane), c0, L::at(a1, i), DUAL ? L::at(a2, i) : 0.0f);
    }
}

// gemm_stage whose epilogue also receives a per-column value v = colv(c)
// (a bias or scale entry), read before the block's products so that its
// load overlaps them instead of waiting in the epilogue:
// epi(r, c, x1, x2, v).
template <typename L, typename T, bool DUAL, bool SPLIT, int P = 4, typename Col, typename Epi>
__device__ __forceinline__ void gemm_stage_cv(int nblocks, const T *A1, const T *A1lo, int lda1,
                                              int nk1, const uint4 *B1, int64_t bs1,
                                              const T *A2, const T *A2lo, int lda2, int nk2,
                                              const uint4 *B2, int64_t bs2, Col &&colv, Epi &&epi) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int nb = wave; nb < nblocks; nb += L::NW) {
        const int c0 = nb * L::BW + L::col(lane);
        const float cv = colv(c0);
        typename L::Acc a1 = L::zero(), a2 = L::zero();
        L::template pipe<DUAL, SPLIT, P>(a1, A1, A1lo, lda1, nk1, B1 + nb * bs1,
                                         a2, A2, A2lo, lda2, nk2, DUAL ? B2 + nb * bs2 : B1);
#pragma unroll
        for (int i = 0; i < L::NE; ++i)
            epi(L::row(i, lane), c0, L::at(a1, i), DUAL ? L::at(a2, i) : 0.0f, cv);
    }
}

// gemm_stage with a block epilogue: epi_blk(nb, a1, a2) receives the whole
// accumulators of block nb (for epilogues that group elements, e.g. runs of
// consecutive rows: elements 4m .. 4m+3 of a lane are rows L::row(4m) + 0..3
// of one column in both layouts).
template <typename L, typename T, bool DUAL, bool SPLIT, int P = 4, typename Epi>
__device__ __forceinline__ void gemm_stage_blk(int nblocks, const T *A1, const T *A1lo, int lda1,
                                               int nk1, const uint4 *B1, int64_t bs1,
                                               const T *A2, const T *A2lo, int lda2, int nk2,
                                               const uint4 *B2, int64_t bs2, Epi &&epi_blk) {
    const int wave = threadIdx.x >> 6;
    for (int nb = wave; nb < nblocks; nb += L::NW) {
        typename L::Acc a1 = L::zero(), a2 = L::zero();
        L::template pipe<DUAL, SPLIT, P>(a1, A1, A1lo, lda1, nk1, B1 + nb * bs1,
                                         a2, A2, A2lo, lda2, nk2, DUAL ? B2 + nb * bs2 : B1);
        epi_blk(nb, a1, a2);
    }
}

} // namespace waa
