// slot.hip -- masked slot attention, one block of 16 query atoms per
// workgroup (4 waves, 16 threads per query).
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
// How:
//  * Each thread owns SPL consecutive slots of one query. It loads their key
//    ids and window bits, then (only for slots that can be allowed) the key
//    usability and the pair rows, all loads issued before any is used, and
//    keeps the mask and the per-head pair bias in registers. Disallowed
//    slots never load their pair row, so NaN payloads never enter arithmetic.
//  * The 16 queries of a block see a narrow band [jlo, jhi] of key ids (the
//    supplied windows are local). Each wave takes one head: it computes the
//    dense 16 x band score tile Q K^T on MFMA with both operands read from
//    L2 straight into registers (Q and K are fp32: they set the logits) and
//    leaves it in LDS. Every thread then reads its slots' logits out of the
//    tiles by key id, does the softmax in registers and scatters the weights
//    into dense 16 x band probability tiles (repeated ids add up). Each wave
//    then forms o = P V for its head on MFMA, reading V from the transposed
//    copy the prep kernel writes, so a lane's operand is 16 contiguous bytes.
//    Three barriers per block; heads run in parallel on the four waves.
//  * A band wider than 128 rows is processed in chunks (any key_index is
//    correct; the windowed layouts need a single chunk).
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace waa {

constexpr int kQB = 16;     // queries per workgroup
constexpr int kRMAX = 128;  // key rows per chunk of the band
constexpr int kHG = 4;      // heads per pass (one per wave)

struct SlotLayout {
    int sp;
    size_t o_wpr, o_s, o_p, o_tag, total;
};

__host__ __device__ inline size_t sal16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline SlotLayout slot_layout(int H, int V, int style) {
    SlotLayout L;
    L.sp = kRMAX + 4;
    size_t o = 0;
    L.o_wpr = o; // pair_scale * w_pair as [V][4] (heads padded to 4)
    if (style == STYLE_AF3)
        o = sal16(o + (size_t)V * kHG * 4);
    L.o_s = o; o = sal16(o + (size_t)kHG * kQB * L.sp * 4);
    L.o_p = o; o = sal16(o + (size_t)kHG * kQB * L.sp * 4);
    L.o_tag = o; o = sal16(o + (size_t)kQB * kRMAX * 4); // writer of each P cell
    L.total = o;
    return L;
}

size_t slot_lds_bytes(const Dims &d, int dtype, int style) {
    (void)dtype;
    return slot_layout(d.H, d.V, style).total;
}

__host__ __device__ inline int slot_spl(int K) { return K <= 16 ? 1 : (K <= 128 ? 8 : 16); }

int slot_supported(const Dims &d, int dtype, int style) {
    const int esz = dtype ? 2 : 4;
    if ((d.D != 16 && d.D != 32 && d.D != 64 && d.D != 128) || d.K > 256)
        return 0;
    if (style == STYLE_AF3 && (d.V % 8 != 0 || d.V * esz > 64 || d.H > kHG))
        return 0;
    return slot_lds_bytes(d, dtype, style) <= kMaxLds;
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

// 16 bytes of the transposed V row `src` starting at key row r (of A rows):
// one vector load when all its rows exist, else row by row with zeros past
// the batch's last atom (the pitch padding is never read).
template <typename T>
__device__ __forceinline__ uint4 vt_chunk(const T *src, int r, int A) {
    constexpr int E = 16 / sizeof(T);
    if (r + E <= A)
        return *reinterpret_cast<const uint4 *>(src + r);
    T tmp[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        tmp[e] = r + e < A ? src[r + e] : (T)0;
    uint4 v;
    __builtin_memcpy(&v, tmp, 16);
    return v;
}

template <typename T, int STYLE, int SPL, int DK>
__global__ __launch_bounds__(256, 2) void k_slot(SlotArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_lo, s_hi;
    constexpr int KC = Mma16<T>::KC, QU = Mma16<T>::QUARTER;
    constexpr int E = 16 / sizeof(T);
    constexpr int NKQ = DK / 16;                     // fp32 k chunks of Q.K
    constexpr int NDB = DK / 16;                     // 16-wide output blocks of o
    constexpr int CBG = DK <= 32 ? 4 : (DK == 64 ? 2 : 1); // score blocks per load batch
    const int A = p.A, K = p.K, H = p.H, V = p.V, HD = H * DK;
    const int nqb = (A + kQB - 1) / kQB;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int b = wg / nqb, a0 = (wg % nqb) * kQB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = tid >> 4, j16 = tid & 15;
    const int g = lane >> 4, l16 = lane & 15;
    const int a = a0 + q;
    const bool qin = a < A;
    const int64_t bA = (int64_t)b * A;
    const int64_t nrow = bA + (qin ? a : 0);
    const int k0 = j16 * SPL;
    const SlotLayout L = slot_layout(H, V, STYLE);
    float *wpr = reinterpret_cast<float *>(smem + L.o_wpr);
    float *sbuf = reinterpret_cast<float *>(smem + L.o_s);
    float *pbuf = reinterpret_cast<float *>(smem + L.o_p);
    const float *qg = reinterpret_cast<const float *>(p.q); // fp32 logit operands
    const float *kg = reinterpret_cast<const float *>(p.k);
    const T *vtg = reinterpret_cast<const T *>(p.v);        // [B][HD][vt_pitch(A)]
    const int vtp = vt_pitch(A);
    T *att = reinterpret_cast<T *>(p.attention);
    T *og = reinterpret_cast<T *>(p.o);

    // ---- masks of this thread's slots; all loads issued before use
    int64_t kid[SPL];
    bool wmv[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int k = k0 + i;
        kid[i] = -1;
        wmv[i] = false;
        if (qin && k < K) {
            kid[i] = p.key_index[nrow * K + k];
            wmv[i] = p.window_mask[nrow * K + k] != 0;
        }
    }
    const bool qok = qin && p.usable[nrow];
    if (tid == 0) {
        s_lo = INT_MAX;
        s_hi = -1;
    }
    if (STYLE == STYLE_AF3) {
        const T *ps = reinterpret_cast<const T *>(p.pair_scale);
        const T *wp = reinterpret_cast<const T *>(p.w_pair);
        for (int i = tid; i < V * kHG; i += 256) {
            const int v = i / kHG, h = i % kHG;
            wpr[i] = h < H ? to_f(ps[v]) * to_f(wp[v * H + h]) : 0.0f;
        }
    }
    for (int i = tid; i < kHG * kQB * L.sp / 4; i += 256)
        reinterpret_cast<float4 *>(pbuf)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    bool cand[SPL];
    uint8_t uj[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int64_t j = kid[i];
        const int64_t dist = j > a ? j - a : a - j;
        cand[i] = qok && wmv[i] && j >= 0 && j < A && (p.radius < 0 || dist <= p.radius);
        uj[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i)
        if (cand[i])
            uj[i] = p.usable[bA + kid[i]];

    // ---- AF3 pair bias per slot and head (H <= 4), in registers
    float beta[SPL][kHG];
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
        for (int h = 0; h < kHG; ++h)
            beta[i][h] = 0.0f;
    __syncthreads(); // wpr, pbuf zero, s_lo/s_hi initialised
    if (STYLE == STYLE_AF3) {
        const T *pair = reinterpret_cast<const T *>(p.pair);
        const int vps = V / E; // 16-byte vectors per pair row (<= 4)
#pragma unroll
        for (int g0 = 0; g0 < SPL; g0 += 4) {
            uint4 pb[4][4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    pb[ii][pt] = make_uint4(0, 0, 0, 0);
                    const int i = g0 + ii;
                    if (i < SPL && pt < vps && cand[i])
                        pb[ii][pt] = *reinterpret_cast<const uint4 *>(
                            pair + (nrow * K + k0 + i) * V + pt * E);
                }
            }
            // normalised rows y = (x - mean) * rstd of the (up to) 4 slots
            float y[4][4 * E];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    unpack16<T>(pb[ii][pt], y[ii] + pt * E);
                float sm = 0.0f;
#pragma unroll
                for (int v = 0; v < 4 * E; ++v)
                    if (v < V)
                        sm += y[ii][v];
                const float mean = sm / (float)V;
                float sq = 0.0f;
#pragma unroll
                for (int v = 0; v < 4 * E; ++v) {
                    y[ii][v] = v < V ? y[ii][v] - mean : 0.0f;
                    sq += y[ii][v] * y[ii][v];
                }
                const float rstd = 1.0f / sqrtf(sq / (float)V + p.eps);
#pragma unroll
                for (int v = 0; v < 4 * E; ++v)
                    y[ii][v] *= rstd;
            }
            // beta[i][h] = y . (pair_scale * w_pair)[:, h]; one broadcast
            // 16-byte LDS read serves all four heads of a channel
#pragma unroll
            for (int v = 0; v < 4 * E; ++v) {
                if (v < V) {
                    const float4 w4 = *reinterpret_cast<const float4 *>(wpr + v * kHG);
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int i = g0 + ii;
                        if (i < SPL) {
                            beta[i][0] += y[ii][v] * w4.x;
                            beta[i][1] += y[ii][v] * w4.y;
                            beta[i][2] += y[ii][v] * w4.z;
                            beta[i][3] += y[ii][v] * w4.w;
                        }
                    }
                }
            }
        }
    }
    int rel[SPL];
    int lo = INT_MAX, hi = -1;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        rel[i] = (cand[i] && uj[i]) ? (int)kid[i] : -1;
        if (rel[i] >= 0) {
            lo = min(lo, rel[i]);
            hi = max(hi, rel[i]);
        }
    }
    lo = wave_min_i(lo);
    hi = wave_max_i(hi);
    if (lane == 0) {
        atomicMin(&s_lo, lo);
        atomicMax(&s_hi, hi);
    }
    __syncthreads();
    const int jhi = s_hi;

    // whole-vector attention stores when rows and slot groups are 16-byte
    // multiples (attention rows then start 16-byte aligned)
    const bool vec_att = (SPL * (int)sizeof(T)) % 16 == 0 && (K % SPL) == 0 &&
                         ((uintptr_t)att & 15) == 0;
    auto store_att = [&](int h, const float *w) {
        if (!qin || k0 >= K) // K % SPL == 0 on the vector path: k0 < K means k0 + SPL <= K
            return;
        T *arow = att + (((int64_t)b * H + h) * A + a) * K;
        if (vec_att) {
            T tmp[SPL];
#pragma unroll
            for (int i = 0; i < SPL; ++i)
                tmp[i] = from_f<T>(w[i]);
#pragma unroll
            for (int i = 0; i < SPL * (int)sizeof(T) / 16; ++i) {
                uint4 v4;
                __builtin_memcpy(&v4, tmp + i * E, 16);
                *reinterpret_cast<uint4 *>(arow + k0 + i * E) = v4;
            }
        } else {
#pragma unroll
            for (int i = 0; i < SPL; ++i)
                if (k0 + i < K)
                    arow[k0 + i] = from_f<T>(w[i]);
        }
    };

    if (jhi < 0) {
        // no allowed slot anywhere in the block: all-zero rows
        float zw[SPL];
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            zw[i] = 0.0f;
        for (int h = 0; h < H; ++h)
            store_att(h, zw);
        if (qin)
            for (int c = j16; c < HD; c += 16)
                og[nrow * HD + c] = from_f<T>(0.0f);
        return;
    }

    const int jal = s_lo & ~7; // band start, aligned for the transposed V rows
    const int span = jhi + 1 - jal;
    const int nch = (span + kRMAX - 1) / kRMAX;
    const float scale = p.inv_sqrt_d;
    float *swave = sbuf + wave * kQB * L.sp; // this wave's head tiles
    // Unique writer of each probability cell (query, key row): every
    // allowed slot writes its slot index into the tag tile and the one
    // whose index survives writes the cell with a plain store; the others
    // (repeated key ids in a row) add their weights with LDS atomics after
    // a barrier. A wide band (several chunks) adds every weight atomically.
    int *tag = reinterpret_cast<int *>(smem + L.o_tag);
    bool win[SPL];
    int lose_any = 0;
    if (nch == 1) {
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (rel[i] >= 0)
                tag[q * kRMAX + rel[i] - jal] = k0 + i;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            win[i] = rel[i] >= 0 && tag[q * kRMAX + rel[i] - jal] == k0 + i;
            lose_any |= (rel[i] >= 0 && !win[i]) ? 1 : 0;
        }
    } else {
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            win[i] = false;
        lose_any = 1;
    }
    lose_any = __syncthreads_or(lose_any);
    float *pwave = pbuf + wave * kQB * L.sp;

    for (int hg = 0; hg < H; hg += kHG) {
        const int hw = hg + wave; // this wave's head in the S and P V products
        const bool hv = hw < H;
        // Q fragments (A operand of S): query row l16, fp32
        uint4 qf[NKQ];
        {
            const int aq = a0 + l16;
#pragma unroll
            for (int kc = 0; kc < NKQ; ++kc) {
                qf[kc] = make_uint4(0, 0, 0, 0);
                if (hv && aq < A)
                    qf[kc] = *reinterpret_cast<const uint4 *>(qg + (bA + aq) * HD + hw * DK + kc * 16 + g * 4);
            }
        }
        float lg[SPL][kHG];
#pragma unroll
        for (int i = 0; i < SPL; ++i)
#pragma unroll
            for (int hh = 0; hh < kHG; ++hh)
                lg[i][hh] = -INFINITY;

        for (int c = 0; c < nch; ++c) {
            const int c0 = jal + c * kRMAX;
            const int rows = min(kRMAX, jhi + 1 - c0);
            const int ncb = (rows + 15) / 16;
            if (hv) {
                for (int cb0 = 0; cb0 < ncb; cb0 += CBG) {
                    f32x4_t acc[CBG];
                    uint4 kb[CBG][NKQ];
#pragma unroll
                    for (int t = 0; t < CBG; ++t) {
                        acc[t] = zero4();
                        const int r = (cb0 + t) * 16 + l16;
#pragma unroll
                        for (int kc = 0; kc < NKQ; ++kc) {
                            kb[t][kc] = make_uint4(0, 0, 0, 0);
                            if (r < rows)
                                kb[t][kc] = *reinterpret_cast<const uint4 *>(
                                    kg + (bA + c0 + r) * HD + hw * DK + kc * 16 + g * 4);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < CBG; ++t)
#pragma unroll
                        for (int kc = 0; kc < NKQ; ++kc)
                            Mma16<float>::mma(acc[t], qf[kc], kb[t][kc]);
#pragma unroll
                    for (int t = 0; t < CBG; ++t)
                        if (cb0 + t < ncb)
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                swave[acc16_row(v, lane) * L.sp + (cb0 + t) * 16 + acc16_col(lane)] = acc[t][v];
                }
            }
            __syncthreads();
#pragma unroll
            for (int hh = 0; hh < kHG; ++hh) {
                if (hg + hh >= H)
                    break;
                const float *sh = sbuf + (hh * kQB + q) * L.sp;
#pragma unroll
                for (int i = 0; i < SPL; ++i) {
                    const int r = rel[i] - c0;
                    if (rel[i] >= 0 && r >= 0 && r < rows) {
                        float l = sh[r] * scale;
                        if (STYLE == STYLE_AF3)
                            l += beta[i][hh];
                        lg[i][hh] = l;
                    }
                }
            }
            if (nch > 1)
                __syncthreads();
        }

        // masked softmax per head over the row: 16 lanes per query
#pragma unroll
        for (int hh = 0; hh < kHG; ++hh) {
            if (hg + hh >= H)
                break;
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < SPL; ++i)
                if (rel[i] >= 0)
                    m = fmaxf(m, lg[i][hh]);
            m = max16(m);
            float w[SPL];
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                w[i] = rel[i] >= 0 ? __expf(lg[i][hh] - m) : 0.0f;
                sum += w[i];
            }
            sum = sum16(sum);
            const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                w[i] *= inv;
                lg[i][hh] = w[i];
            }
            store_att(hg + hh, w);
        }

        // o = P V per head; P scattered by key id (repeats add up)
        f32x4_t oacc[NDB];
#pragma unroll
        for (int t = 0; t < NDB; ++t)
            oacc[t] = zero4();
        for (int c = 0; c < nch; ++c) {
            const int c0 = jal + c * kRMAX;
            const int rows = min(kRMAX, jhi + 1 - c0);
            const int rpad = (rows + 31) / 32 * 32;
#pragma unroll
            for (int hh = 0; hh < kHG; ++hh) {
                if (hg + hh >= H)
                    break;
                float *ph = pbuf + (hh * kQB + q) * L.sp;
#pragma unroll
                for (int i = 0; i < SPL; ++i) {
                    const int r = rel[i] - c0;
                    if (win[i])
                        ph[r] = lg[i][hh];
                }
            }
            if (lose_any) {
                __syncthreads();
#pragma unroll
                for (int hh = 0; hh < kHG; ++hh) {
                    if (hg + hh >= H)
                        break;
                    float *ph = pbuf + (hh * kQB + q) * L.sp;
#pragma unroll
                    for (int i = 0; i < SPL; ++i) {
                        const int r = rel[i] - c0;
                        if (rel[i] >= 0 && !win[i] && r >= 0 && r < rows)
                            atomicAdd(&ph[r], lg[i][hh]);
                    }
                }
            }
            __syncthreads();
            if (hv) {
                const float *prow = pwave + l16 * L.sp + g * QU;
                const T *vrow = vtg + ((int64_t)b * HD + hw * DK) * vtp;
                for (int kc = 0; kc < rpad / KC; ++kc) {
                    const uint4 av = p_chunk<T>(prow + kc * KC);
                    const int r = c0 + kc * KC + g * QU;
#pragma unroll
                    for (int t = 0; t < NDB; ++t) {
                        const uint4 bv = vt_chunk<T>(vrow + (int64_t)(t * 16 + l16) * vtp, r, A);
                        Mma16<T>::mma(oacc[t], av, bv);
                    }
                }
                // leave this wave's P tile zero for the next chunk / head group
                for (int i = lane; i < kQB * L.sp / 4; i += 64)
                    reinterpret_cast<float4 *>(pwave)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            __syncthreads();
        }
        if (hv) {
#pragma unroll
            for (int t = 0; t < NDB; ++t) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int aq = a0 + acc16_row(v, lane);
                    if (aq < A)
                        og[(bA + aq) * HD + hw * DK + t * 16 + acc16_col(lane)] = from_f<T>(oacc[t][v]);
                }
            }
        }
    }
}

template <typename T, int STYLE, int SPL>
static const void *pick_slot_d(int D) {
    switch (D) {
    case 16: return (const void *)k_slot<T, STYLE, SPL, 16>;
    case 32: return (const void *)k_slot<T, STYLE, SPL, 32>;
    case 64: return (const void *)k_slot<T, STYLE, SPL, 64>;
    default: return (const void *)k_slot<T, STYLE, SPL, 128>;
    }
}

template <typename T, int STYLE>
static const void *pick_slot(int spl, int D) {
    switch (spl) {
    case 1: return pick_slot_d<T, STYLE, 1>(D);
    case 8: return pick_slot_d<T, STYLE, 8>(D);
    default: return pick_slot_d<T, STYLE, 16>(D);
    }
}

hipError_t launch_slot(const SlotArgs &a, int dtype, int style, hipStream_t s) {
    const int spl = slot_spl(a.K);
    const Dims d{a.B, a.A, 1, a.K, 32, 32, a.H, a.D, a.V, 32, 32};
    const size_t lds = slot_lds_bytes(d, dtype, style);
    const void *fn;
    if (style == STYLE_AF3)
        fn = dtype == 0 ? pick_slot<float, STYLE_AF3>(spl, a.D) : pick_slot<bf16_t, STYLE_AF3>(spl, a.D);
    else
        fn = dtype == 0 ? pick_slot<float, STYLE_ESM>(spl, a.D) : pick_slot<bf16_t, STYLE_ESM>(spl, a.D);
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int grid = a.B * ((a.A + kQB - 1) / kQB);
    void *args[] = {(void *)&a};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(256), args, lds, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

// Transposed copy of v ([B][A][HD] -> [B][HD][vt_pitch(A)]), for the
// standalone slot-attention entry point.
template <typename T>
__global__ __launch_bounds__(256) void k_vt(const T *v, T *vt, int B, int A, int HD,
                                            int pitch) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per = (int64_t)A * HD;
    if (i >= per * B)
        return;
    const int64_t b = i / per;
    const int64_t r = i - b * per;
    const int aa = (int)(r / HD), c = (int)(r - (int64_t)aa * HD);
    vt[(b * HD + c) * pitch + aa] = v[i];
}

hipError_t launch_vt(const void *v, void *vt, int B, int A, int HD, int dtype,
                     hipStream_t s) {
    const int64_t total = (int64_t)A * HD * B;
    const int64_t grid = (total + 255) / 256;
    if (dtype == 0)
        hipLaunchKernelGGL(k_vt<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float *)v, (float *)vt, B, A, HD, vt_pitch(A));
    else
        hipLaunchKernelGGL(k_vt<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const bf16_t *)v, (bf16_t *)vt, B, A, HD, vt_pitch(A));
    return hipGetLastError();
}

} // namespace waa
