// post.hip -- everything after the slot attention, one 32-atom tile per
// workgroup ("windowed_atom_attention", Required behavior):
//   u  = (o * G) flattened head-major @ w_attention_out   (no bias)
//   x1 = x0 + g_att * u        (AF3 g_att = sigmoid(c@w_rg[0] + b_rg[0]) on
//                               the raw condition; ESMFold2 g_att = m2, raw)
//   z  = A_2(x1) (AF3) or RMS(x1)*(1 + m4) + m3 (ESMFold2)  -- on the NEW x
//   t  = (SiLU(z @ w_ff_gate) * (z @ w_ff_up)) @ w_ff_out
//   x2 = x1 + g_tr * t, hidden = select(usable, x2, 0)
//   decoder: position_update = select(usable,
//              (LN(hidden)*readout_scale [+ readout_bias]) @ w_readout, 0)
// The entry state x0 and the conditioning are recomputed from the inputs
// (two small GEMMs cost far less than storing and re-reading four C-wide
// vectors per atom). All matrix products run on MFMA: 32x32 blocks with
// four waves, or, for grids of at most one tile per CU, 32x16 strips with
// eight waves (two per SIMD, so one wave's epilogue runs under the other's
// MFMAs); each dual GEMM's epilogue applies the elementwise step in
// registers.
//
// pool: encoder mean-pool, atomics-free. A tile owns every token whose
// first usable atom lies in it; it walks its atoms in index order and, for
// the last open token, continues into the following atoms until that
// token's atoms end. Requires usable atoms sorted by atom_to_token within a
// batch; a violation sets the status word.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace waa {

struct PostLayout {
    int xp, ldS, ldC, ldHD, ldH;
    size_t o_st, o_us, o_key, o_seg, o_opC, o_opC2, o_opU, o_opZ, o_opH, total;
};

// Transition width handled per pass (h is staged that many columns at a
// time): 128, or all of M when the grid has at most one tile per CU and LDS
// allows (then LDS does not limit occupancy).
constexpr int kMC = 128;
__host__ __device__ inline int post_pass_width(const Dims &d, int wide) {
    return wide ? d.M : (d.M < kMC ? d.M : kMC);
}

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline PostLayout post_layout(const Dims &d, int esz, int style, int wide) {
    PostLayout L;
    L.xp = d.C + 4;
    L.ldS = d.S + 16 / esz;
    L.ldC = d.C + 16 / esz;
    L.ldHD = d.H * d.D + 16 / esz;
    L.ldH = post_pass_width(d, wide) + 16 / esz;
    size_t o = 32 * (size_t)L.xp * 4;
    L.o_st = o; o += 32 * 4 * 4;
    L.o_us = o; o += 32;
    L.o_key = o; o += 32 * 4;      // (batch, token) key of each row, -1 if unusable
    L.o_seg = o; o += 4 * 33 * 4;  // segment of each row; segment keys, counts; count
    L.o_opC = o; o = al16(o + 32 * (size_t)L.ldS * esz);
    L.o_opC2 = o; // LN(c) * cond_scale[2] (AF3)
    if (style == STYLE_AF3)
        o = al16(o + 32 * (size_t)L.ldS * esz);
    // one tile holds, in turn, o*G (until x1) and a chunk of h (transition)
    const int w = L.ldHD > L.ldH ? L.ldHD : L.ldH;
    L.o_opU = L.o_opH = o;
    o = al16(o + 32 * (size_t)w * esz);
    L.o_opZ = o; o = al16(o + 32 * (size_t)L.ldC * esz);
    L.total = o;
    return L;
}

size_t post_lds_bytes(const Dims &d, int dtype, int style) {
    return post_layout(d, dtype ? 2 : 4, style, 0).total;
}

// NW waves (4: 32x32 output blocks, several workgroups per CU; 8: 32x16
// strips, two waves per SIMD for grids of at most one tile per CU), TPR =
// 64*NW/32 threads per tile row.
template <typename T, int STYLE, int STAGE, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : (sizeof(T) == 2 ? 3 : 2)) void k_post(BlockArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NT = 64 * NW, TPR = NT / 32;
    using G = typename std::conditional<NW == 8, Blk16<T>, Blk32<T>>::type;
    using Acc = typename G::Acc;
    constexpr int BW = G::BW;
    // GEMM pipeline depth: 2 for bf16 keeps the kernel at three
    // workgroups per CU
    constexpr int PP = sizeof(T) == 2 ? 2 : 4;
    const Dims d = p.d;
    const int N = d.B * d.A, C = d.C, S = d.S, HD = d.H * d.D, M = d.M;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = tid / TPR, sub = tid % TPR;
    const int n0 = blockIdx.x * 32;
    const int n = n0 + row;
    const bool inb = n < N;
    constexpr int E = 16 / sizeof(T);
    const PostLayout L = post_layout(d, sizeof(T), STYLE, p.post_wide);
    const int MCW = post_pass_width(d, p.post_wide);
    float *xs = reinterpret_cast<float *>(smem);
    float *st = reinterpret_cast<float *>(smem + L.o_st);
    uint8_t *us = smem + L.o_us;
    T *opC = reinterpret_cast<T *>(smem + L.o_opC);
    T *opC2 = reinterpret_cast<T *>(smem + L.o_opC2);
    T *opU = reinterpret_cast<T *>(smem + L.o_opU);
    T *opZ = reinterpret_cast<T *>(smem + L.o_opZ);
    T *opH = reinterpret_cast<T *>(smem + L.o_opH);

    // the row's usability and token, loaded unconditionally (row 0 past
    // the end) so that the row loads below go out without waiting for them
    const int64_t nc = inb ? n : 0;
    const uint8_t usv = p.usable[nc];
    const int64_t tkr = p.atom_to_token[nc];
    const bool u = inb && usv;
    const int b = inb ? n / d.A : 0;
    int *rkey = reinterpret_cast<int *>(smem + L.o_key);
    if (sub == 0) {
        us[row] = u;
        if (STAGE == STAGE_ENCODER)
            rkey[row] = u ? b * d.T + (int)tkr : -1;
    }
    {
        // entry state (as the prep kernel builds it), condition (raw for the
        // AF3 gates, SiLU for the ESMFold2 modulation) and o*G rounded to
        // the storage type; every load of a round is issued before the
        // rows are converted into LDS
        // rows past the end read row 0 (loads are unconditional; the values
        // of unusable or missing rows are replaced by zeros after the load)
        const T *ar = reinterpret_cast<const T *>(p.atom) + nc * C;
        const T *cr = reinterpret_cast<const T *>(p.condition) + nc * S;
        const T *orow = reinterpret_cast<const T *>(p.o) + nc * HD;
        const T *grow = reinterpret_cast<const T *>(p.g) + nc * HD;
        // (a usable atom's token is in range; others read token 0, unused)
        const int64_t tk = tkr >= 0 && tkr < d.T ? tkr : 0;
        const float *tp = p.tokproj + ((int64_t)b * d.T + tk) * C;
        const int nvC = C / E, nvS = S / E, nvH = HD / E;
        const int nvmax = nvC > nvS ? (nvC > nvH ? nvC : nvH) : (nvS > nvH ? nvS : nvH);
        constexpr int RV = sizeof(T) == 2 ? 2 : 4; // vectors per array and thread in one round
        // AF3 with the condition row in one round: its values stay in
        // registers for the statistics and LN(c) * cond_scale[2] (no LDS
        // re-read), and the cond_scale[2] vectors load with the rows
        const T *cscale2 = reinterpret_cast<const T *>(p.cond_scale) + 2 * S;
        const bool keepc = STYLE == STYLE_AF3 && nvS <= RV * TPR;
        float ck[RV][E];
        uint4 vs[RV];
        float csum = 0.0f;
        for (int base = sub; base < nvmax; base += RV * TPR) {
            uint4 va[RV], vc[RV], vo[RV], vg[RV];
            float vt[RV][E]; // decoder: the gathered token projection
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                const int vi = base + j * TPR;
                va[j] = *reinterpret_cast<const uint4 *>(ar + min(vi, nvC - 1) * E);
                vc[j] = *reinterpret_cast<const uint4 *>(cr + min(vi, nvS - 1) * E);
                vo[j] = *reinterpret_cast<const uint4 *>(orow + min(vi, nvH - 1) * E);
                vg[j] = *reinterpret_cast<const uint4 *>(grow + min(vi, nvH - 1) * E);
                if (STYLE == STYLE_AF3)
                    vs[j] = *reinterpret_cast<const uint4 *>(cscale2 + min(vi, nvS - 1) * E);
                const uint4 z = make_uint4(0, 0, 0, 0);
                if (!u) {
                    va[j] = z;
                    vc[j] = z;
                }
                if (!inb)
                    vo[j] = vg[j] = z;
                if constexpr (STAGE == STAGE_DECODER) {
#pragma unroll
                    for (int t = 0; t < E / 4; ++t) {
                        float4 f = *reinterpret_cast<const float4 *>(tp + min(vi, nvC - 1) * E + 4 * t);
                        if (!u)
                            f = make_float4(0.f, 0.f, 0.f, 0.f);
                        vt[j][4 * t + 0] = f.x; vt[j][4 * t + 1] = f.y;
                        vt[j][4 * t + 2] = f.z; vt[j][4 * t + 3] = f.w;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                const int vi = base + j * TPR;
                if (vi < nvC) {
                    float xv[E];
                    unpack16<T>(va[j], xv);
                    if constexpr (STAGE == STAGE_DECODER) {
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            xv[e] += vt[j][e];
                    }
#pragma unroll
                    for (int e = 0; e < E; e += 4)
                        *reinterpret_cast<float4 *>(xs + row * L.xp + vi * E + e) =
                            make_float4(xv[e], xv[e + 1], xv[e + 2], xv[e + 3]);
                }
                if (vi < nvS) {
                    float cv[E];
                    unpack16<T>(vc[j], cv);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        csum += cv[e];
                        ck[j][e] = cv[e];
                        if (STYLE != STYLE_AF3)
                            cv[e] = silu_f(cv[e]);
                    }
                    // (AF3: the raw condition, already in the storage type)
                    *reinterpret_cast<uint4 *>(opC + row * L.ldS + vi * E) =
                        STYLE == STYLE_AF3 ? vc[j] : pack16<T>(cv);
                }
                if (vi < nvH) {
                    float ov[E], gv[E];
                    unpack16<T>(vo[j], ov);
                    unpack16<T>(vg[j], gv);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        ov[e] *= gv[e];
                    *reinterpret_cast<uint4 *>(opU + row * L.ldHD + vi * E) = pack16<T>(ov);
                }
            }
        }
        if (STYLE == STYLE_AF3) {
            // c_2 = LN(c) * cond_scale[2], each thread on its own entries of
            // opC (written above by the same thread: no barrier needed)
            const float mc = row_sum<TPR>(csum) / (float)S;
            if (keepc) {
                float q = 0.0f;
#pragma unroll
                for (int j = 0; j < RV; ++j)
                    if (sub + j * TPR < nvS)
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const float t = ck[j][e] - mc;
                            q += t * t;
                        }
                const float rc = 1.0f / sqrtf(row_sum<TPR>(q) / (float)S + p.eps);
#pragma unroll
                for (int j = 0; j < RV; ++j) {
                    const int vi = sub + j * TPR;
                    if (vi < nvS) {
                        float sc[E];
                        unpack16<T>(vs[j], sc);
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            sc[e] *= (ck[j][e] - mc) * rc;
                        *reinterpret_cast<uint4 *>(opC2 + row * L.ldS + vi * E) = pack16<T>(sc);
                    }
                }
            } else {
            float q = 0.0f;
            for (int vi = sub; vi < nvS; vi += TPR)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float t = to_f(opC[row * L.ldS + vi * E + e]) - mc;
                    q += t * t;
                }
            const float rc = 1.0f / sqrtf(row_sum<TPR>(q) / (float)S + p.eps);
            const T *cscale = reinterpret_cast<const T *>(p.cond_scale) + 2 * S;
            for (int vi = sub; vi < nvS; vi += TPR) {
                float sc[E];
                unpack16<T>(*reinterpret_cast<const uint4 *>(cscale + vi * E), sc);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int c = vi * E + e;
                    opC2[row * L.ldS + c] = from_f<T>((to_f(opC[row * L.ldS + c]) - mc) * rc * sc[e]);
                }
            }
            }
        }
    }
    __syncthreads();

    const int nkS = S / G::KC, nkC = C / G::KC;
    const int nkHD = HD / G::KC, nkM = M / G::KC;

    // x1 = x0 + g_att * (o*G) @ w_attention_out
    {
        const T *brg = reinterpret_cast<const T *>(p.b_rg);
        const int64_t offg = STYLE == STYLE_AF3 ? p.off.w_rg[0] : p.off.w_mod[2];
        gemm_stage_cv<G, T, true, false, PP>(
            C / BW, opU, nullptr, L.ldHD, nkHD, p.pk + p.off.w_ao, (int64_t)nkHD * 64,
            opC, nullptr, L.ldS, nkS, p.pk + offg, (int64_t)nkS * 64,
            [&](int c) { return STYLE == STYLE_AF3 ? to_f(brg[c]) : 0.0f; },
            [&](int r, int c, float x1, float x2, float bg) {
                const float gate = STYLE == STYLE_AF3 ? sigmoid_f(x2 + bg) : x2;
                xs[r * L.xp + c] += gate * x1;
            });
    }
    __syncthreads();
    // statistics of the NEW state for the transition norm: each thread reads
    // 16-byte pieces of its row (channels 4*sub + 4*TPR*k ..), several
    // reads in flight per loop step (single-float reads in a loop of
    // runtime length had each waited for the previous one: 3.8 k cycles per
    // workgroup on a 24576-atom bf16 workload)
    {
        const float *xr = xs + row * L.xp;
        if (STYLE == STYLE_AF3) {
            float s = 0.0f;
#pragma unroll 4
            for (int c = 4 * sub; c < C; c += 4 * TPR) {
                const float4 v = *reinterpret_cast<const float4 *>(xr + c);
                s += (v.x + v.y) + (v.z + v.w);
            }
            const float mean = row_sum<TPR>(s) / (float)C;
            float q = 0.0f;
#pragma unroll 4
            for (int c = 4 * sub; c < C; c += 4 * TPR) {
                const float4 v = *reinterpret_cast<const float4 *>(xr + c);
                const float t0 = v.x - mean, t1 = v.y - mean, t2 = v.z - mean, t3 = v.w - mean;
                q += (t0 * t0 + t1 * t1) + (t2 * t2 + t3 * t3);
            }
            const float rstd = 1.0f / sqrtf(row_sum<TPR>(q) / (float)C + p.eps);
            if (sub == 0) {
                st[row * 4 + 0] = mean;
                st[row * 4 + 1] = rstd;
            }
        } else {
            float q = 0.0f;
#pragma unroll 4
            for (int c = 4 * sub; c < C; c += 4 * TPR) {
                const float4 v = *reinterpret_cast<const float4 *>(xr + c);
                q += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
            }
            const float rstd = 1.0f / sqrtf(row_sum<TPR>(q) / (float)C + p.eps);
            if (sub == 0) {
                st[row * 4 + 0] = 0.0f;
                st[row * 4 + 1] = rstd;
            }
        }
    }
    __syncthreads();
    // z = transition-normalised x1
    {
        const T *bsc = reinterpret_cast<const T *>(p.b_scale);
        const T *opz = STYLE == STYLE_AF3 ? opC2 : opC;
        const int64_t o1 = STYLE == STYLE_AF3 ? p.off.w_scale[2] : p.off.w_mod[3];
        const int64_t o2 = STYLE == STYLE_AF3 ? p.off.w_shift[2] : p.off.w_mod[4];
        gemm_stage_cv<G, T, true, false, PP>(
            C / BW, opz, nullptr, L.ldS, nkS, p.pk + o1, (int64_t)nkS * 64,
            opz, nullptr, L.ldS, nkS, p.pk + o2, (int64_t)nkS * 64,
            [&](int c) { return STYLE == STYLE_AF3 ? to_f(bsc[2 * C + c]) : 0.0f; },
            [&](int r, int c, float x1, float x2, float bs) {
                const float xn = (xs[r * L.xp + c] - st[r * 4 + 0]) * st[r * 4 + 1];
                float z;
                if (STYLE == STYLE_AF3)
                    z = xn * sigmoid_f(x1 + bs) + x2;
                else
                    z = xn * (1.0f + x2) + x1;
                opZ[r * L.ldC + c] = from_f<T>(z);
            });
    }
    __syncthreads();
    // x2 = x1 + g_tr * (h @ w_ff_out), h = SiLU(z @ w_ff_gate) * (z @ w_ff_up),
    // with h staged MCW columns at a time. Output columns go in groups of
    // NW blocks (one per wave), so each wave carries its block of
    // h @ w_ff_out in registers across the passes; with more than one group
    // and M > MCW the h chunks are recomputed per group.
    // hidden = select(usable, x2, 0).
    {
        constexpr int KC = G::KC;
        const T *brg = reinterpret_cast<const T *>(p.b_rg);
        const int64_t offg = STYLE == STYLE_AF3 ? p.off.w_rg[1] : p.off.w_mod[5];
        const bool single = M <= MCW;
        for (int cg = 0; cg < C / BW; cg += NW) {
            const int nb = cg + wave;
            const bool own = nb < C / BW;
            // the gate bias of this lane's column, loaded before the products
            const float bias =
                STYLE == STYLE_AF3 ? to_f(brg[C + min(nb, C / BW - 1) * BW + G::col(lane)]) : 0.0f;
            Acc acc = G::zero(), ga = G::zero();
            for (int m0 = 0; m0 < M; m0 += MCW) {
                const int mc = M - m0 < MCW ? M - m0 : MCW;
                if (cg == 0 || !single) {
                    if (m0 > 0 || cg > 0)
                        __syncthreads(); // the previous chunk of h has been consumed
                    gemm_stage<G, T, true, false, PP>(
                        mc / BW, opZ, nullptr, L.ldC, nkC, p.pk + p.off.ff_gate + (int64_t)(m0 / BW) * nkC * 64,
                        (int64_t)nkC * 64, opZ, nullptr, L.ldC, nkC,
                        p.pk + p.off.ff_up + (int64_t)(m0 / BW) * nkC * 64, (int64_t)nkC * 64,
                        [&](int r, int c, float x1, float x2) {
                            opH[r * L.ldH + c] = from_f<T>(silu_f(x1) * x2);
                        });
                    __syncthreads();
                }
                if (!own)
                    continue;
                const uint4 *wo = p.pk + p.off.ff_out + ((int64_t)nb * nkM + m0 / KC) * 64;
                if (m0 + MCW >= M)
                    G::template pipe<true, false, PP>(acc, opH, nullptr, L.ldH, mc / KC, wo,
                                                      ga, opC, nullptr, L.ldS, nkS,
                                                      p.pk + offg + (int64_t)nb * nkS * 64);
                else
                    G::template pipe<false, false, PP>(acc, opH, nullptr, L.ldH, mc / KC, wo,
                                                       acc, opH, nullptr, L.ldH, 0, wo);
            }
            if (own) {
                const int c = nb * BW + G::col(lane);
#pragma unroll
                for (int i = 0; i < G::NE; ++i) {
                    const int r = G::row(i, lane);
                    const float gv = G::at(ga, i);
                    const float gate = STYLE == STYLE_AF3 ? sigmoid_f(gv + bias) : gv;
                    const float x2 = xs[r * L.xp + c] + gate * G::at(acc, i);
                    xs[r * L.xp + c] = us[r] ? x2 : 0.0f;
                }
            }
        }
    }
    // hidden rows are complete in xs: each thread stores 16-byte pieces of
    // its row (and, for the encoder, the same values as the pooling operand)
    __syncthreads();
    {
        T *hrow = reinterpret_cast<T *>(p.hidden) + (int64_t)(inb ? n : 0) * C;
        for (int vi = sub; vi < C / E; vi += TPR) {
            T tmp[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                tmp[e] = from_f<T>(xs[row * L.xp + vi * E + e]);
            uint4 v4;
            __builtin_memcpy(&v4, tmp, 16);
            if (inb)
                *reinterpret_cast<uint4 *>(hrow + vi * E) = v4;
            if (STAGE == STAGE_ENCODER)
                *reinterpret_cast<uint4 *>(opZ + row * L.ldC + vi * E) = v4;
        }
    }
    if (STAGE == STAGE_ENCODER) {
        // ---- pooling: ReLU(hidden @ w_pool) of this tile's rows, summed per
        // segment of consecutive usable rows with one (batch, token) key.
        // Segments inside the tile are complete tokens (keys are sorted) and
        // their means are written here; the first and the last segment may
        // continue in neighbouring tiles and go to this tile's record for
        // the pooling fix-up kernel.
        int *segid = reinterpret_cast<int *>(smem + L.o_seg);
        int *skey = segid + 32, *scnt = segid + 64, *snum = segid + 96;
        if (wave == 0) {
            const int k = lane < 32 ? rkey[lane] : -1;
            const uint64_t um = __ballot(k >= 0);
            const uint64_t below = um & ((1ull << lane) - 1ull);
            const int prev = below ? 63 - __clzll((long long)below) : -1;
            const int pk = prev >= 0 ? rkey[prev] : -1;
            const bool start = k >= 0 && (prev < 0 || pk != k);
            const uint64_t sm = __ballot(start);
            const int sidx = __popcll(sm & ((2ull << lane) - 1ull)) - 1;
            if (lane < 32)
                segid[lane] = k >= 0 ? sidx : -1;
            if (start) {
                const uint64_t above = sm & ~((2ull << lane) - 1ull);
                const int nxt = above ? __ffsll((long long)above) - 1 : 32;
                const uint64_t span = ((nxt >= 64 ? 0ull : (1ull << nxt)) - 1ull) & ~((1ull << lane) - 1ull);
                skey[sidx] = k;
                scnt[sidx] = __popcll(um & span);
            }
            // keys must not decrease along the usable rows (sorted tokens)
            const bool bad = k >= 0 && prev >= 0 && pk > k;
            if (__ballot(bad) != 0ull && lane == 0 && p.status != nullptr)
                p.status[0] = 1;
            if (lane == 0)
                snum[0] = __popcll(sm);
        }
        __syncthreads();
        const int nseg = snum[0];
        const int tile = blockIdx.x;
        float *rsum = p.pool_sum + (int64_t)tile * 2 * d.U;
        if (tid == 0) {
            int *ri = p.pool_int + (int64_t)tile * 8;
            ri[0] = nseg;
            ri[1] = nseg > 0 ? skey[0] : -1;
            ri[2] = nseg > 0 ? scnt[0] : 0;
            ri[3] = nseg > 1 ? skey[nseg - 1] : -1;
            ri[4] = nseg > 1 ? scnt[nseg - 1] : 0;
        }
        if (nseg > 0) {
            T *tout = reinterpret_cast<T *>(p.token_output);
            int sv[G::NE]; // segment of each accumulator row of the lane
#pragma unroll
            for (int i = 0; i < G::NE; ++i)
                sv[i] = segid[G::row(i, lane)];
            // segment sums of one ReLU'd column block: the lane's rows, then
            // the other lanes of its column (colsum)
            auto pool_block = [&](Acc &acc, int nb) {
                const int col = nb * BW + G::col(lane);
#pragma unroll
                for (int i = 0; i < G::NE; ++i)
                    G::put(acc, i, fmaxf(G::at(acc, i), 0.0f));
                for (int s = 0; s < nseg; ++s) {
                    float part = 0.0f;
#pragma unroll
                    for (int i = 0; i < G::NE; ++i)
                        part += sv[i] == s ? G::at(acc, i) : 0.0f;
                    part = G::colsum(part);
                    if (G::col_owner(lane)) {
                        if (s == 0)
                            rsum[col] = part;
                        else if (s == nseg - 1)
                            rsum[d.U + col] = part;
                        else
                            tout[(int64_t)skey[s] * d.U + col] = from_f<T>(part / (float)scnt[s]);
                    }
                }
            };
            // two column blocks per GEMM call where the wave has two left
            const int nbU = d.U / BW;
            for (int nb0 = wave; nb0 < nbU; nb0 += 2 * NW) {
                const int nb1 = nb0 + NW;
                Acc a1 = G::zero(), a2 = G::zero();
                const uint4 *w0 = p.pk + p.off.w_pool + (int64_t)nb0 * nkC * 64;
                if (nb1 < nbU) {
                    G::template pipe<true, false, PP>(a1, opZ, nullptr, L.ldC, nkC, w0,
                                                      a2, opZ, nullptr, L.ldC, nkC,
                                                      p.pk + p.off.w_pool + (int64_t)nb1 * nkC * 64);
                    pool_block(a1, nb0);
                    pool_block(a2, nb1);
                } else {
                    G::template pipe<false, false, PP>(a1, opZ, nullptr, L.ldC, nkC, w0,
                                                       a1, opZ, nullptr, L.ldC, 0, w0);
                    pool_block(a1, nb0);
                }
            }
        }
    }
    if (STAGE == STAGE_DECODER) {
        const float *xr = xs + row * L.xp;
        float s = 0.0f;
#pragma unroll 4
        for (int c = 4 * sub; c < C; c += 4 * TPR) {
            const float4 v = *reinterpret_cast<const float4 *>(xr + c);
            s += (v.x + v.y) + (v.z + v.w);
        }
        const float mean = row_sum<TPR>(s) / (float)C;
        float q = 0.0f;
#pragma unroll 4
        for (int c = 4 * sub; c < C; c += 4 * TPR) {
            const float4 v = *reinterpret_cast<const float4 *>(xr + c);
            const float t0 = v.x - mean, t1 = v.y - mean, t2 = v.z - mean, t3 = v.w - mean;
            q += (t0 * t0 + t1 * t1) + (t2 * t2 + t3 * t3);
        }
        const float rstd = 1.0f / sqrtf(row_sum<TPR>(q) / (float)C + p.eps);
        const T *rs = reinterpret_cast<const T *>(p.readout_scale);
        const T *rb = reinterpret_cast<const T *>(p.readout_bias);
        const T *wr = reinterpret_cast<const T *>(p.w_readout);
        float acc0 = 0.0f, acc1 = 0.0f, acc2 = 0.0f;
        // RU columns per step, their parameter loads issued together
        // (clamped) before any is used: one L2 wait per step
        constexpr int RU = 8;
        for (int c0 = sub; c0 < C; c0 += RU * TPR) {
            T rsv[RU], rbv[RU], w0[RU], w1[RU], w2[RU];
#pragma unroll
            for (int k = 0; k < RU; ++k) {
                const int c = min(c0 + k * TPR, C - 1);
                rsv[k] = rs[c];
                rbv[k] = STYLE == STYLE_ESM ? rb[c] : T{};
                w0[k] = wr[c * 3 + 0];
                w1[k] = wr[c * 3 + 1];
                w2[k] = wr[c * 3 + 2];
            }
#pragma unroll
            for (int k = 0; k < RU; ++k) {
                const int c = c0 + k * TPR;
                if (c < C) {
                    float z = (xr[c] - mean) * rstd * to_f(rsv[k]);
                    if (STYLE == STYLE_ESM)
                        z += to_f(rbv[k]);
                    acc0 += z * to_f(w0[k]);
                    acc1 += z * to_f(w1[k]);
                    acc2 += z * to_f(w2[k]);
                }
            }
        }
        acc0 = row_sum<TPR>(acc0);
        acc1 = row_sum<TPR>(acc1);
        acc2 = row_sum<TPR>(acc2);
        if (sub == 0 && inb) {
            T *pu = reinterpret_cast<T *>(p.position_update) + (int64_t)n * 3;
            const bool ok = us[row];
            pu[0] = from_f<T>(ok ? acc0 : 0.0f);
            pu[1] = from_f<T>(ok ? acc1 : 0.0f);
            pu[2] = from_f<T>(ok ? acc2 : 0.0f);
        }
    }
}

hipError_t launch_post(const BlockArgs &a, int dtype, int style, int stage,
                       hipStream_t s) {
    const int N = a.d.B * a.d.A;
    const int grid = (N + 31) / 32;
    BlockArgs b = a;
    const int esz = dtype ? 2 : 4;
    b.post_wide = grid <= device_cus() && post_layout(a.d, esz, style, 1).total <= kMaxLds;
    const size_t lds = post_layout(a.d, esz, style, b.post_wide).total;
    const void *fn = nullptr;
#define WAA_PICK(T, ST, SG) fn = a.nw8 ? (const void *)k_post<T, ST, SG, 8> : (const void *)k_post<T, ST, SG, 4>
    if (dtype == 0) {
        if (style == STYLE_AF3) { if (stage == STAGE_ENCODER) WAA_PICK(float, 0, 0); else WAA_PICK(float, 0, 1); }
        else { if (stage == STAGE_ENCODER) WAA_PICK(float, 1, 0); else WAA_PICK(float, 1, 1); }
    } else {
        if (style == STYLE_AF3) { if (stage == STAGE_ENCODER) WAA_PICK(bf16_t, 0, 0); else WAA_PICK(bf16_t, 0, 1); }
        else { if (stage == STAGE_ENCODER) WAA_PICK(bf16_t, 1, 0); else WAA_PICK(bf16_t, 1, 1); }
    }
#undef WAA_PICK
    allow_lds(fn, lds);
    void *args[] = {(void *)&b};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(a.nw8 ? 512 : 256), args, lds, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

// --------------------------------------------------------------- pool fix-up

// Tokens whose atoms cross tile boundaries: every tile's record holds the
// sums and counts of its first and last segment (post kernel). A tile owns
// its last segment (when it has two or more) and its first segment unless
// that continues the last segment of the previous non-empty tile; the owner
// adds the first-segment sums of the following tiles while they continue the
// token (a single-segment tile passes it on), in tile order, and writes the
// mean. Keys that decrease across tiles set the status word.
template <typename T>
__global__ __launch_bounds__(256) void k_pool_fix(BlockArgs p) {
    const int t = blockIdx.x, ntile = gridDim.x, U = p.d.U, tid = threadIdx.x;
    const int *ri = p.pool_int;
    const float *rs = p.pool_sum;
    // Everything the common case needs is loaded at once, before any of it
    // is used: this tile's record and both segment sums, the previous
    // tile's record, the next tile's record and first-segment sums (indices
    // clamped; a token rarely spans more than two tiles, the loops below
    // cover the rest).
    const int tp = t > 0 ? t - 1 : 0, tn = t + 1 < ntile ? t + 1 : t;
    int rec[8], prv[8], nxt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        rec[k] = ri[t * 8 + k];
        prv[k] = ri[tp * 8 + k];
        nxt[k] = ri[tn * 8 + k];
    }
    float s0[2], s1[2], n0[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int col = min(tid + 256 * i, U - 1);
        s0[i] = rs[((int64_t)t * 2 + 0) * U + col];
        s1[i] = rs[((int64_t)t * 2 + 1) * U + col];
        n0[i] = rs[(int64_t)tn * 2 * U + col];
    }
    const int nseg = rec[0];
    if (nseg == 0)
        return;
    int prev_last = -1;
    if (t > 0) {
        if (prv[0] != 0) {
            prev_last = prv[0] == 1 ? prv[1] : prv[3];
        } else {
            int u = t - 2;
            while (u >= 0 && ri[u * 8] == 0)
                --u;
            prev_last = u < 0 ? -1 : (ri[u * 8] == 1 ? ri[u * 8 + 1] : ri[u * 8 + 3]);
        }
    }
    const int fkey = rec[1];
    if (prev_last > fkey && tid == 0 && p.status != nullptr)
        p.status[0] = 1;
    T *tout = reinterpret_cast<T *>(p.token_output);
    for (int which = 0; which < 2; ++which) {
        int key, cnt;
        bool may_continue;
        float acc[2];
        if (which == 0) {
            if (prev_last == fkey)
                continue;
            key = fkey;
            cnt = rec[2];
            may_continue = nseg == 1;
            acc[0] = s0[0];
            acc[1] = s0[1];
        } else {
            if (nseg < 2)
                continue;
            key = rec[3];
            cnt = rec[4];
            may_continue = true;
            acc[0] = s1[0];
            acc[1] = s1[1];
        }
        int v = t + 1;
        if (may_continue && v < ntile && nxt[0] != 0) { // the next tile, from the loads above
            if (nxt[1] != key) {
                may_continue = false;
            } else {
                cnt += nxt[2];
                acc[0] += n0[0];
                acc[1] += n0[1];
                may_continue = nxt[0] == 1;
                ++v;
            }
        }
        for (; may_continue && v < ntile; ++v) {
            const int ns = ri[v * 8];
            if (ns == 0)
                continue;
            if (ri[v * 8 + 1] != key)
                break;
            cnt += ri[v * 8 + 2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int col = tid + 256 * i;
                if (col < U)
                    acc[i] += rs[(int64_t)v * 2 * U + col];
            }
            may_continue = ns == 1;
        }
        const float inv = 1.0f / (float)cnt;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = tid + 256 * i;
            if (col < U)
                tout[(int64_t)key * U + col] = from_f<T>(acc[i] * inv);
        }
    }
}

hipError_t launch_pool(const BlockArgs &a, int dtype, hipStream_t s) {
    const int grid = (a.d.B * a.d.A + 31) / 32;
    if (dtype == 0)
        hipLaunchKernelGGL(k_pool_fix<float>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_pool_fix<bf16_t>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace waa
