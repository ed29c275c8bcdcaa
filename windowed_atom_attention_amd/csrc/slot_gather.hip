// slot_gather.hip -- the slot-attention step for query blocks whose key ids
// span a wide band ("windowed_atom_attention", Required behavior: key slots
// hold global within-batch atom ids, any table is allowed).
//
// The slot kernel (slot_kernel.hpp) multiplies a block's 16 queries against
// the contiguous band of key rows its slots reach: for local windows that
// band is about K rows and every row is read once for the whole block. For
// a block whose band is wider than kWideChunks chunks (scattered ids) that
// work grows with the band, not with K, so the slot kernel hands the block
// to a queue instead (wide[0] = count, wide[1..] = block ids) and this
// kernel computes it by gathers: one wave per query, the logits of its
// slots against their K rows (fp32), the masked softmax, and o from the
// selected rows of the row-major V copy the projection kernel writes. Cost
// per slot and head: one K row (D fp32) and one V row (D values) -- the
// bytes of a table with no locality, independent of how far apart the ids
// are. Results follow the same rules as the slot kernel (allowed slots,
// exact-zero empty rows, repeated ids as separate terms).
#include "kernels.hpp"
#include "common.hpp"

namespace waa {

namespace {

constexpr int kQBg = 16; // queries per block (as the slot kernel)
constexpr int kHGg = 4;  // AF3: at most four heads (the slot kernel's bound)
constexpr int kMaxKg = 256;
constexpr int kPairVg = 32;

// sum over slots s of w[s] times the D values at rows[kid[s] * HD + off ..]
// (storage type T, 16 bytes per lane): lane group g takes slots g, g + SP,
// ... in order, four slots' loads in flight; groups are added by lane
// exchanges. Every lane returns its E = 16/sizeof(T) channels of the total,
// channels E * (lane % (D/E)) ..
template <typename T, int D>
__device__ __forceinline__ void gather_rowsum(const float *w, const int *kid, int K,
                                              const T *rows, int HD, int off, int lane,
                                              float (&acc)[16 / sizeof(T)]) {
    constexpr int E = 16 / sizeof(T), L = D / E, SP = 64 / L;
    const int g = lane / L, q = lane - g * L;
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0f;
    for (int s0 = 0; s0 < K; s0 += 4 * SP) {
        uint4 r[4];
        float ww[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + u * SP + g;
            ww[u] = s < K ? w[s] : 0.0f;
            r[u] = make_uint4(0, 0, 0, 0);
            if (ww[u] != 0.0f)
                r[u] = *reinterpret_cast<const uint4 *>(rows + (int64_t)kid[s] * HD + off + q * E);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float x[E];
            unpack16<T>(r[u], x);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] += ww[u] * x[e];
        }
    }
#pragma unroll
    for (int o = L; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] += __shfl_xor(acc[e], o);
}

template <typename T, int STYLE, int D>
__global__ __launch_bounds__(256) void k_slot_gather(SlotArgs p) {
    extern __shared__ float smem[];
    const int count = p.wide[0];
    if ((int)blockIdx.x >= count)
        return;
    const int wg = p.wide[1 + blockIdx.x];
    const int A = p.A, K = p.K, H = p.H, HD = H * D;
    const int nqb = (A + kQBg - 1) / kQBg;
    const int b = wg / nqb, a0 = (wg % nqb) * kQBg;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float *base = smem + w * (2 * K + K * H + HD);
    int *skid = reinterpret_cast<int *>(base);
    float *sP = base + K;
    float *sbeta = sP + K;
    float *sq = sbeta + K * H;
    const int64_t bA = (int64_t)b * A;
    const float *qg = reinterpret_cast<const float *>(p.q);
    const float *kg = reinterpret_cast<const float *>(p.k);
    const T *vr = reinterpret_cast<const T *>(p.vrows);
    T *att = reinterpret_cast<T *>(p.attention);
    T *og = reinterpret_cast<T *>(p.o);
    constexpr int E = 16 / sizeof(T);

    for (int it = 0; it < kQBg / 4; ++it) {
        const int a = a0 + w * (kQBg / 4) + it;
        const bool live = a < A;
        const int64_t n = bA + (live ? a : 0);
        const bool qu = live && p.usable[n];
        for (int s = lane; s < K; s += 64) {
            const int64_t e = n * K + s;
            const int64_t j = p.key_index[e];
            bool ok = qu && j >= 0 && j < A && p.window_mask[e];
            if (ok)
                ok = p.usable[bA + j] && (p.radius < 0 || (j > a ? j - a : a - j) <= p.radius);
            skid[s] = ok ? (int)(bA + j) : -1;
            if (STYLE == STYLE_AF3) {
                float bt[kHGg];
#pragma unroll
                for (int h = 0; h < kHGg; ++h)
                    bt[h] = 0.0f;
                if (ok && p.pbias) {
                    const float4 v = reinterpret_cast<const float4 *>(p.pbias)[e];
                    bt[0] = v.x; bt[1] = v.y; bt[2] = v.z; bt[3] = v.w;
                } else if (ok) {
                    // (LN(pair row) * pair_scale) @ w_pair
                    const T *pr = reinterpret_cast<const T *>(p.pair) + e * p.V;
                    const T *ps = reinterpret_cast<const T *>(p.pair_scale);
                    const T *wp = reinterpret_cast<const T *>(p.w_pair);
                    float x[kPairVg];
                    float m = 0.0f;
#pragma unroll
                    for (int v = 0; v < kPairVg; ++v) {
                        x[v] = v < p.V ? to_f(pr[v]) : 0.0f;
                        m += x[v];
                    }
                    m /= (float)p.V;
                    float q2 = 0.0f;
#pragma unroll
                    for (int v = 0; v < kPairVg; ++v) {
                        const float d = v < p.V ? x[v] - m : 0.0f;
                        q2 += d * d;
                    }
                    const float r = 1.0f / sqrtf(q2 / (float)p.V + p.eps);
#pragma unroll
                    for (int v = 0; v < kPairVg; ++v)
                        if (v < p.V) {
                            const float xn = (x[v] - m) * r * to_f(ps[v]);
#pragma unroll
                            for (int h = 0; h < kHGg; ++h)
                                if (h < H)
                                    bt[h] += xn * to_f(wp[v * H + h]);
                        }
                }
                for (int h = 0; h < H; ++h)
                    sbeta[s * H + h] = bt[h];
            }
        }
        for (int i = lane; i < HD; i += 64)
            sq[i] = qg[n * HD + i];
        __syncthreads();
        for (int h = 0; h < H; ++h) {
            float l[kMaxKg / 64];
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < kMaxKg / 64; ++c) {
                const int s = lane + 64 * c;
                l[c] = -INFINITY;
                if (s < K && skid[s] >= 0) {
                    const float4 *kr = reinterpret_cast<const float4 *>(kg + (int64_t)skid[s] * HD + h * D);
                    float4 r4[D / 4];
#pragma unroll
                    for (int i = 0; i < D / 4; ++i)
                        r4[i] = kr[i];
                    const float *qv = sq + h * D;
                    float dot = 0.0f;
#pragma unroll
                    for (int i = 0; i < D / 4; ++i)
                        dot += qv[4 * i] * r4[i].x + qv[4 * i + 1] * r4[i].y +
                               qv[4 * i + 2] * r4[i].z + qv[4 * i + 3] * r4[i].w;
                    l[c] = dot * p.inv_sqrt_d + (STYLE == STYLE_AF3 ? sbeta[s * H + h] : 0.0f);
                    mx = fmaxf(mx, l[c]);
                }
            }
            mx = group_max<64>(mx);
            float sum = 0.0f;
#pragma unroll
            for (int c = 0; c < kMaxKg / 64; ++c) {
                const int s = lane + 64 * c;
                if (s < K && skid[s] >= 0) {
                    l[c] = expf(l[c] - mx);
                    sum += l[c];
                }
            }
            sum = group_sum<64>(sum);
            const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
            T *ar = att + (((int64_t)b * H + h) * A + (live ? a : 0)) * K;
#pragma unroll
            for (int c = 0; c < kMaxKg / 64; ++c) {
                const int s = lane + 64 * c;
                if (s < K) {
                    const float pw = skid[s] >= 0 ? l[c] * inv : 0.0f;
                    sP[s] = pw;
                    if (live)
                        ar[s] = from_f<T>(pw);
                }
            }
            __syncthreads();
            float acc[E];
            gather_rowsum<T, D>(sP, skid, K, vr, HD, h * D, lane, acc);
            if (live && lane < D / E)
                *reinterpret_cast<uint4 *>(og + n * HD + h * D + lane * E) = pack16<T>(acc);
            __syncthreads();
        }
    }
}

template <typename T, int STYLE>
hipError_t launch_gather_t(const SlotArgs &a, hipStream_t s) {
    const int grid = a.B * ((a.A + kQBg - 1) / kQBg);
    const size_t lds = 4 * sizeof(float) * (size_t)(2 * a.K + a.K * a.H + a.H * a.D);
    const void *fn;
    switch (a.D) {
    case 16: fn = reinterpret_cast<const void *>(k_slot_gather<T, STYLE, 16>); break;
    case 32: fn = reinterpret_cast<const void *>(k_slot_gather<T, STYLE, 32>); break;
    case 64: fn = reinterpret_cast<const void *>(k_slot_gather<T, STYLE, 64>); break;
    case 128: fn = reinterpret_cast<const void *>(k_slot_gather<T, STYLE, 128>); break;
    default: return hipErrorInvalidValue;
    }
    allow_lds(fn, lds);
    SlotArgs args = a;
    void *kargs[] = {(void *)&args};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(256), kargs, lds, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

} // namespace

size_t slot_gather_lds_bytes(int K, int H, int D) {
    return 4 * sizeof(float) * (size_t)(2 * K + K * H + H * D);
}

hipError_t launch_slot_gather(const SlotArgs &a, int dtype, int style, hipStream_t s) {
    if (!a.wide || !a.vrows)
        return hipSuccess;
    if (style == STYLE_AF3)
        return dtype ? launch_gather_t<bf16_t, STYLE_AF3>(a, s) : launch_gather_t<float, STYLE_AF3>(a, s);
    return dtype ? launch_gather_t<bf16_t, STYLE_ESM>(a, s) : launch_gather_t<float, STYLE_ESM>(a, s);
}

} // namespace waa
