// slot.hip -- masked slot attention, one block of 16 query atoms per
// workgroup (4 waves).
//
// What it computes ("windowed_atom_attention", Required behavior; the AF3
// and ESMFold2 encoder pages): a slot (a, k) with key id j is allowed iff
// 0 <= j < A, atoms a and j are usable, window_mask[a, k], and |j - a| <=
// radius when radius >= 0. Logits are Q[a].K[j]/sqrt(D) plus, for AF3, the
// per-head pair bias (LN(pair[a, k]) * pair_scale) @ w_pair. A softmax over
// the allowed slots of the row (every slot its own term, repeats included)
// gives attention[b, h, a, k]; a row without allowed slots is exactly zero.
// o[a, h] = sum_k w_k V[j_k, h].
//
// How: the 16 queries of a block see a narrow band of key ids (the supplied
// windows are local), so the workgroup stages the K and V rows of that band
// [jlo, jhi] for one head in LDS (coalesced row loads, up to 128 rows per
// chunk), computes the dense 16 x rows score tile Q K^T on MFMA (fp32
// operands: Q and K are kept in fp32 because they set the logits), reads each
// slot's logit out of that tile by its key id, does the softmax in
// registers (16 lanes per query), scatters the weights into a dense
// 16 x rows probability tile (repeated ids add up) and gets o = P V on MFMA.
// Key ids outside one chunk are handled by looping over chunks of the band,
// so any key_index is correct; the windowed layouts need one chunk.
// Masks and the pair bias are computed first with fully coalesced loads of
// key_index, window_mask and pair; disallowed slots never load their pair
// row, so NaN payloads there never enter arithmetic.
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace waa {

constexpr int kQB = 16;     // queries per workgroup
constexpr int kRMAX = 128;  // key rows per staged chunk

struct SlotLayout {
    int dkS, dkSp, dk, dkp, vtp, sp;
    size_t o_rel, o_beta, o_wpr, o_kst, o_vst, o_s, o_p, total;
};

__host__ __device__ inline size_t sal16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline SlotLayout slot_layout(int K, int H, int D, int V,
                                                  int esz, int style) {
    SlotLayout L;
    const int kc = esz == 2 ? 32 : 16; // MFMA k per chunk of the P V product
    L.dkS = (D + 15) / 16 * 16;          // fp32 score product: 16 per chunk
    L.dkSp = L.dkS + 4;
    L.dk = (D + kc - 1) / kc * kc;
    L.dkp = L.dk + 16 / esz;
    L.vtp = kRMAX + 8; // bf16 transposed V pitch
    L.sp = kRMAX + 4;
    size_t o = 0;
    L.o_rel = o; o = sal16(o + (size_t)kQB * K * 4);
    L.o_beta = o;
    if (style == STYLE_AF3)
        o = sal16(o + (size_t)H * kQB * K * 4);
    L.o_wpr = o;
    if (style == STYLE_AF3)
        o = sal16(o + (size_t)V * H * 4);
    L.o_kst = o; o = sal16(o + (size_t)kRMAX * L.dkSp * 4);
    L.o_vst = o;
    if (esz == 2)
        o = sal16(o + (size_t)L.dk * L.vtp * esz);
    else
        o = sal16(o + (size_t)kRMAX * L.dkp * esz);
    L.o_s = o; o = sal16(o + (size_t)kQB * L.sp * 4);
    L.o_p = o; o = sal16(o + (size_t)kQB * L.sp * 4);
    L.total = o;
    return L;
}

size_t slot_lds_bytes(const Dims &d, int dtype, int style) {
    return slot_layout(d.K, d.H, d.D, d.V, dtype ? 2 : 4, style).total;
}

int slot_supported(const Dims &d, int dtype, int style) {
    if (d.D % 16 != 0 || d.D > 128 || d.K > 512)
        return 0;
    if (style == STYLE_AF3 && (d.V % 8 != 0 || d.V > 64))
        return 0;
    return slot_lds_bytes(d, dtype, style) <= kMaxLds;
}

// Stage rows [c0, c0+rows) of head h of src ([.., HD], storage dtype) into
// dst[r][d] (pitch dkp), zero-filling rows up to rpad and columns up to dk.
template <typename T>
__device__ __forceinline__ void stage_rows(T *dst, int dkp, const T *src,
                                           int64_t row0, int HD, int hD, int D,
                                           int dk, int rows, int rpad) {
    constexpr int E = 16 / sizeof(T);
    const int vpr = dk / E;
    for (int idx = threadIdx.x; idx < rpad * vpr; idx += 256) {
        const int r = idx / vpr, dv = (idx % vpr) * E;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < rows && dv < D)
            val = *reinterpret_cast<const uint4 *>(src + (row0 + r) * HD + hD + dv);
        *reinterpret_cast<uint4 *>(dst + r * dkp + dv) = val;
    }
}

// bf16 V rows staged transposed: dst[d][r] (pitch vtp), so that the B
// operand of P V (k = key row) is 16 contiguous bytes per lane.
__device__ __forceinline__ void stage_rows_t(bf16_t *dst, int vtp,
                                             const bf16_t *src, int64_t row0,
                                             int HD, int hD, int D, int dk,
                                             int rows, int rpad) {
    const int vpr = dk / 8;
    for (int idx = threadIdx.x; idx < rpad * vpr; idx += 256) {
        const int r = idx / vpr, dv = (idx % vpr) * 8;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < rows && dv < D)
            val = *reinterpret_cast<const uint4 *>(src + (row0 + r) * HD + hD + dv);
        const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dst[(dv + 2 * e) * vtp + r] = (bf16_t)(w[e] & 0xffffu);
            dst[(dv + 2 * e + 1) * vtp + r] = (bf16_t)(w[e] >> 16);
        }
    }
}

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

// P operand (probabilities, fp32 in LDS) as a 16-byte chunk of T.
template <typename T>
__device__ __forceinline__ uint4 p_chunk(const float *src);
template <> __device__ __forceinline__ uint4 p_chunk<float>(const float *src) {
    return *reinterpret_cast<const uint4 *>(src);
}
template <> __device__ __forceinline__ uint4 p_chunk<bf16_t>(const float *src) {
    const float4 lo = *reinterpret_cast<const float4 *>(src);
    const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
    uint4 r;
    r.x = (uint32_t)from_f<bf16_t>(lo.x) | ((uint32_t)from_f<bf16_t>(lo.y) << 16);
    r.y = (uint32_t)from_f<bf16_t>(lo.z) | ((uint32_t)from_f<bf16_t>(lo.w) << 16);
    r.z = (uint32_t)from_f<bf16_t>(hi.x) | ((uint32_t)from_f<bf16_t>(hi.y) << 16);
    r.w = (uint32_t)from_f<bf16_t>(hi.z) | ((uint32_t)from_f<bf16_t>(hi.w) << 16);
    return r;
}

template <typename T, int STYLE, int SPL>
__global__ __launch_bounds__(256) void k_slot(SlotArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_lo, s_hi;
    constexpr int KC = Mma16<T>::KC, QU = Mma16<T>::QUARTER;
    const int A = p.A, K = p.K, H = p.H, D = p.D, V = p.V, HD = H * D;
    const int nqb = (A + kQB - 1) / kQB;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int b = wg / nqb, a0 = (wg % nqb) * kQB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = tid >> 4, j16 = tid & 15;
    const int a = a0 + q;
    const bool qin = a < A;
    const int64_t bA = (int64_t)b * A;
    const SlotLayout L = slot_layout(K, H, D, V, sizeof(T), STYLE);
    int *rel_s = reinterpret_cast<int *>(smem + L.o_rel);
    float *beta = reinterpret_cast<float *>(smem + L.o_beta);
    float *wpr = reinterpret_cast<float *>(smem + L.o_wpr);
    float *kst = reinterpret_cast<float *>(smem + L.o_kst);
    T *vst = reinterpret_cast<T *>(smem + L.o_vst);
    float *sbuf = reinterpret_cast<float *>(smem + L.o_s);
    float *pbuf = reinterpret_cast<float *>(smem + L.o_p);
    const float *qg = reinterpret_cast<const float *>(p.q); // fp32 logit operands
    const float *kg = reinterpret_cast<const float *>(p.k);
    const T *vg = reinterpret_cast<const T *>(p.v);
    T *att = reinterpret_cast<T *>(p.attention);
    T *og = reinterpret_cast<T *>(p.o);

    if (tid == 0) {
        s_lo = INT_MAX;
        s_hi = -1;
    }
    if (STYLE == STYLE_AF3) {
        const T *ps = reinterpret_cast<const T *>(p.pair_scale);
        const T *wp = reinterpret_cast<const T *>(p.w_pair);
        for (int i = tid; i < V * H; i += 256)
            wpr[i] = to_f(ps[i / H]) * to_f(wp[i]);
    }
    // ---- masks: coalesced over the block's QB*K slots
    int lo = INT_MAX, hi = -1;
    for (int s = tid; s < kQB * K; s += 256) {
        const int qq = s / K, k = s - qq * K;
        const int aa = a0 + qq;
        int rel = -1;
        if (aa < A) {
            const int64_t nn = bA + aa;
            const int64_t j = p.key_index[nn * K + k];
            if (j >= 0 && j < A && p.usable[nn] && p.window_mask[nn * K + k] &&
                p.usable[bA + j]) {
                const int64_t dist = j > aa ? j - aa : aa - j;
                if (p.radius < 0 || dist <= p.radius) {
                    rel = (int)j;
                    lo = min(lo, rel);
                    hi = max(hi, rel);
                }
            }
        }
        rel_s[s] = rel;
    }
    __syncthreads();
    lo = wave_min_i(lo);
    hi = wave_max_i(hi);
    if (lane == 0) {
        atomicMin(&s_lo, lo);
        atomicMax(&s_hi, hi);
    }
    // ---- AF3 pair bias, coalesced 16-byte loads of the allowed pair rows
    if (STYLE == STYLE_AF3) {
        constexpr int E = 16 / sizeof(T);
        const int vps = V / E; // 16-byte vectors per slot row (1, 2, 4 or 8)
        const T *pair = reinterpret_cast<const T *>(p.pair);
        const int total = kQB * K * vps;
        const int rounds = (total + 255) / 256;
        for (int it = 0; it < rounds; ++it) {
            const int idx = it * 256 + tid;
            const bool live = idx < total;
            const int s = live ? idx / vps : 0;
            const int part = live ? idx - s * vps : 0;
            const bool ok = live && rel_s[s] >= 0;
            float x[E];
            if (ok) {
                const int qq = s / K, k = s - qq * K;
                const int64_t nn = bA + a0 + qq;
                unpack16<T>(*reinterpret_cast<const uint4 *>(pair + (nn * K + k) * V + part * E), x);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    x[e] = 0.0f;
            }
            float sm = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                sm += x[e];
            for (int m = 1; m < vps; m <<= 1)
                sm += __shfl_xor(sm, m, 64);
            const float mean = sm / (float)V;
            float sq = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                x[e] -= mean;
                sq += x[e] * x[e];
            }
            for (int m = 1; m < vps; m <<= 1)
                sq += __shfl_xor(sq, m, 64);
            const float rstd = 1.0f / sqrtf(sq / (float)V + p.eps);
            for (int h = 0; h < H; ++h) {
                float bh = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    bh += x[e] * wpr[(part * E + e) * H + h];
                for (int m = 1; m < vps; m <<= 1)
                    bh += __shfl_xor(bh, m, 64);
                if (ok && part == 0) {
                    const int qq = s / K, k = s - qq * K;
                    beta[(h * kQB + qq) * K + k] = bh * rstd;
                }
            }
        }
    }
    __syncthreads();
    const int jlo = s_lo, jhi = s_hi;

    // this thread's slots for the softmax: query q, k = j16*SPL + i
    int rel[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int k = j16 * SPL + i;
        rel[i] = k < K ? rel_s[q * K + k] : -1;
    }

    if (jhi < 0) {
        // no allowed slot anywhere in the block: all-zero rows
        if (qin) {
            for (int h = 0; h < H; ++h) {
#pragma unroll
                for (int i = 0; i < SPL; ++i) {
                    const int k = j16 * SPL + i;
                    if (k < K)
                        att[(((int64_t)b * H + h) * A + a) * K + k] = from_f<T>(0.0f);
                }
            }
            for (int c = j16; c < HD; c += 16)
                og[(bA + a) * HD + c] = from_f<T>(0.0f);
        }
        return;
    }

    const int span = jhi - jlo + 1;
    const int nch = (span + kRMAX - 1) / kRMAX;
    const int nkq = L.dkS / 16;
    const int g = lane >> 4, l16 = lane & 15;
    const float scale = p.inv_sqrt_d;

    for (int h = 0; h < H; ++h) {
        // A operand of S: this lane's query row, 16-byte k chunks
        uint4 qf[8];
        {
            const int aq = a0 + l16;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                qf[kc] = make_uint4(0, 0, 0, 0);
                const int d0 = kc * 16 + g * 4;
                if (kc < nkq && aq < A && d0 < D)
                    qf[kc] = *reinterpret_cast<const uint4 *>(qg + (bA + aq) * HD + h * D + d0);
            }
        }
        float lg[SPL];
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            lg[i] = -INFINITY;

        for (int c = 0; c < nch; ++c) {
            const int c0 = jlo + c * kRMAX;
            const int rows = min(kRMAX, jhi + 1 - c0);
            const int rpad = (rows + 31) / 32 * 32;
            stage_rows<float>(kst, L.dkSp, kg, bA + c0, HD, h * D, D, L.dkS, rows, rpad);
            if (nch == 1) {
                if constexpr (sizeof(T) == 2)
                    stage_rows_t(reinterpret_cast<bf16_t *>(vst), L.vtp,
                                 reinterpret_cast<const bf16_t *>(vg), bA + c0, HD,
                                 h * D, D, L.dk, rows, rpad);
                else
                    stage_rows<T>(vst, L.dkp, vg, bA + c0, HD, h * D, D, L.dk, rows, rpad);
            }
            __syncthreads();
            for (int cb = wave; cb < rpad / 16; cb += 4) {
                f32x4_t acc = zero4();
                const float *krow = kst + (cb * 16 + l16) * L.dkSp + g * 4;
#pragma unroll
                for (int kc = 0; kc < 8; ++kc)
                    if (kc < nkq)
                        Mma16<float>::mma(acc, qf[kc], *reinterpret_cast<const uint4 *>(krow + kc * 16));
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    sbuf[acc16_row(v, lane) * L.sp + cb * 16 + acc16_col(lane)] = acc[v];
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const int r = rel[i] - c0;
                if (rel[i] >= 0 && r >= 0 && r < rows) {
                    float l = sbuf[q * L.sp + r] * scale;
                    if (STYLE == STYLE_AF3)
                        l += beta[(h * kQB + q) * K + j16 * SPL + i];
                    lg[i] = l;
                }
            }
            if (nch > 1)
                __syncthreads();
        }

        // masked softmax over the row: 16 lanes per query
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (rel[i] >= 0)
                m = fmaxf(m, lg[i]);
        m = group_max<16>(m);
        float w[SPL];
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            w[i] = rel[i] >= 0 ? __expf(lg[i] - m) : 0.0f;
            sum += w[i];
        }
        sum = group_sum<16>(sum);
        const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            w[i] *= inv;
        if (qin) {
            T *arow = att + (((int64_t)b * H + h) * A + a) * K;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const int k = j16 * SPL + i;
                if (k < K)
                    arow[k] = from_f<T>(w[i]);
            }
        }

        // o = P V, P scattered by key id (repeats add up)
        f32x4_t oacc[2] = {zero4(), zero4()};
        for (int c = 0; c < nch; ++c) {
            const int c0 = jlo + c * kRMAX;
            const int rows = min(kRMAX, jhi + 1 - c0);
            const int rpad = (rows + 31) / 32 * 32;
            if (nch > 1) {
                if constexpr (sizeof(T) == 2)
                    stage_rows_t(reinterpret_cast<bf16_t *>(vst), L.vtp,
                                 reinterpret_cast<const bf16_t *>(vg), bA + c0, HD,
                                 h * D, D, L.dk, rows, rpad);
                else
                    stage_rows<T>(vst, L.dkp, vg, bA + c0, HD, h * D, D, L.dk, rows, rpad);
            }
            for (int i = tid; i < kQB * rpad; i += 256) {
                const int rr = i / rpad, cc = i - rr * rpad;
                pbuf[rr * L.sp + cc] = 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const int r = rel[i] - c0;
                if (rel[i] >= 0 && r >= 0 && r < rows)
                    atomicAdd(&pbuf[q * L.sp + r], w[i]);
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int db = wave + 4 * t;
                if (db * 16 < D) {
                    const float *prow = pbuf + l16 * L.sp + g * QU;
                    for (int kc = 0; kc < rpad / KC; ++kc) {
                        const uint4 av = p_chunk<T>(prow + kc * KC);
                        uint4 bv;
                        if constexpr (sizeof(T) == 2) {
                            bv = *reinterpret_cast<const uint4 *>(
                                vst + (db * 16 + l16) * L.vtp + kc * KC + g * QU);
                        } else {
                            const T *vc = vst + (kc * KC + g * QU) * L.dkp + db * 16 + l16;
                            bv.x = __float_as_uint(vc[0]);
                            bv.y = __float_as_uint(vc[L.dkp]);
                            bv.z = __float_as_uint(vc[2 * L.dkp]);
                            bv.w = __float_as_uint(vc[3 * L.dkp]);
                        }
                        Mma16<T>::mma(oacc[t], av, bv);
                    }
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int db = wave + 4 * t;
            if (db * 16 < D) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int aq = a0 + acc16_row(v, lane);
                    if (aq < A)
                        og[(bA + aq) * HD + h * D + db * 16 + acc16_col(lane)] =
                            from_f<T>(oacc[t][v]);
                }
            }
        }
    }
}

template <typename T, int STYLE>
static const void *pick_slot(int spl) {
    switch (spl) {
    case 1: return (const void *)k_slot<T, STYLE, 1>;
    case 2: return (const void *)k_slot<T, STYLE, 2>;
    case 4: return (const void *)k_slot<T, STYLE, 4>;
    case 8: return (const void *)k_slot<T, STYLE, 8>;
    case 16: return (const void *)k_slot<T, STYLE, 16>;
    default: return (const void *)k_slot<T, STYLE, 32>;
    }
}

hipError_t launch_slot(const SlotArgs &a, int dtype, int style, hipStream_t s) {
    int spl = 1;
    while (spl * 16 < a.K)
        spl *= 2;
    const Dims d{a.B, a.A, 1, a.K, 32, 32, a.H, a.D, a.V, 32, 32};
    const size_t lds = slot_lds_bytes(d, dtype, style);
    const void *fn;
    if (dtype == 0)
        fn = style == STYLE_AF3 ? pick_slot<float, STYLE_AF3>(spl) : pick_slot<float, STYLE_ESM>(spl);
    else
        fn = style == STYLE_AF3 ? pick_slot<bf16_t, STYLE_AF3>(spl) : pick_slot<bf16_t, STYLE_ESM>(spl);
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int grid = a.B * ((a.A + kQB - 1) / kQB);
    void *args[] = {(void *)&a};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(256), args, lds, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

} // namespace waa
