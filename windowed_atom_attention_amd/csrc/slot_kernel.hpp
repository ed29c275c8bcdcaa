// slot_kernel.hpp -- masked slot attention, one block of 16 query atoms per
// workgroup (4 waves and 16 threads per query, or 8 waves and 32 threads per
// query). Included by the translation units that instantiate it
// (slot_af3_f32.hip, slot_af3_bf16.hip, slot_af3_pre.hip, slot_esm.hip);
// the launcher lives in slot.hip.
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
//  * Each thread owns SPL slots of one query, strided by the threads per
//    query (thread j of a query has slots j, j+16, ... in the 16-thread
//    form), so that the threads of a query touch consecutive slots:
//    coalesced key-id, window, pair and attention rows, and distinct LDS
//    banks for the tile and tag cells of windowed key lists. It loads their
//    key ids and window bits, the pair rows of all its slots (or their
//    precomputed bias) and then gathers the key usability of every slot,
//    all unconditionally. The pair bias of every slot and head is
//    formed in registers from one pass over the row: with d = x - x[0]
//    (shifted data keeps the variance well conditioned),
//      LN(x) . w_h = rstd * (sum_v d_v w_vh - mean(d) * sum_v w_vh),
//      rstd = 1 / sqrt(mean(d^2) - mean(d)^2 + eps).
//    Bias values of slots that are not allowed are never used, so a NaN
//    payload in such a row never reaches an output.
//  * The 16 queries of a block see a narrow band [jlo, jhi] of key ids (the
//    supplied windows are local). Each wave takes one head: it computes the
//    dense 16 x band score tile Q K^T on MFMA with both operands read from
//    L2 straight into registers (Q and K are fp32: they set the logits) and
//    leaves it in LDS. Every thread reads its slots' logits out of the tiles
//    by key id and does the softmax in registers. The same LDS then holds
//    the dense 16 x band probability tiles: zeroed, filled with each slot's
//    weight by key id (a repeated id in a row adds up), and multiplied by V
//    on MFMA per head, V read from the transposed copy the prep kernel
//    writes so that a lane's operand is 16 contiguous bytes.
//  * A band wider than 128 rows is processed in chunks (any key_index is
//    correct; the windowed layouts need a single chunk).
#pragma once

#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace waa {

constexpr int kQB = 16;     // queries per workgroup
constexpr int kRMAX = 128;  // key rows per chunk of the band
constexpr int kHG = 4;      // heads per pass (one per wave)

struct SlotLayout {
    int sp;
    size_t o_wpr, o_t, o_tag, total;
};

__host__ __device__ inline size_t sal16(size_t x) { return (x + 15) & ~(size_t)15; }

// LDS: AF3 pair weights pair_scale * w_pair as [V][4] (heads padded to 4)
// and two partial column sums [2][4]; the score / probability tiles
// [4][16][sp] fp32; the writer tag of each probability cell [16][128].
__host__ __device__ inline SlotLayout slot_layout(int H, int V, int style) {
    (void)H;
    SlotLayout L;
    L.sp = kRMAX + 4;
    size_t o = 0;
    L.o_wpr = o;
    if (style == STYLE_AF3)
        o = sal16(o + (size_t)(V + 2) * kHG * 4);
    L.o_t = o; o = sal16(o + (size_t)kHG * kQB * L.sp * 4);
    L.o_tag = o; o = sal16(o + (size_t)kQB * kRMAX * 4);
    L.total = o;
    return L;
}

// Slots per thread for K and TQ threads per query (16 or 32).
__host__ __device__ inline int slot_spl(int K, int tq) {
    return tq == 32 ? (K <= 32 ? 1 : (K <= 128 ? 4 : 8)) : (K <= 16 ? 1 : (K <= 128 ? 8 : 16));
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
    return make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                      pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w));
}

// NV: 16-byte vectors per AF3 pair row (V = NV * 16 / sizeof(T)), or 0
// when the AF3 pair bias comes precomputed (p.pbias); 1 for ESMFold2, which
// has no pair input.
// TQ: threads per query (16: 256-thread workgroups, one wave per head,
// three workgroups per CU; 32: 512-thread workgroups, two waves per head
// splitting the score blocks and the output channels, half the slots and
// registers per thread, two workgroups per CU -- for grids of at most about
// two blocks per CU, where more waves per block shorten its latency chain).
template <typename T, int STYLE, int SPL, int DK, int NV, int TQ>
__global__ __launch_bounds__(kQB * TQ, TQ == 32 ? 4 : (SPL >= 16 ? 2 : 3)) void k_slot(SlotArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_lo, s_hi;
    constexpr int KC = Mma16<T>::KC, QU = Mma16<T>::QUARTER;
    constexpr int E = 16 / sizeof(T);
    constexpr bool PRE = STYLE == STYLE_AF3 && NV == 0;  // pair bias read from p.pbias
    constexpr bool FUSED = STYLE == STYLE_AF3 && NV > 0; // pair bias from the pair rows
    constexpr int NVB = NV > 0 ? NV : 1;
    constexpr int VV = NV * E;                       // AF3 pair channels
    constexpr int NKQ = DK / 16;                     // fp32 k chunks of Q.K
    constexpr int NDB = DK / 16;                     // 16-wide output blocks of o
    constexpr int NVC = kRMAX / KC;                  // P V k chunks of a full band chunk
    constexpr int NDBW0 = (DK / 16) / ((kQB * TQ) / 64 / kHG) > 0 ? (DK / 16) / ((kQB * TQ) / 64 / kHG) : 1;
    constexpr int VG = NVC < 8 / NDBW0 ? NVC : (8 / NDBW0 > 0 ? 8 / NDBW0 : 1); // V chunks per load batch (<= 8 vectors)
    constexpr int CBG = DK <= 32 ? 4 : (DK == 64 ? 2 : 1); // score blocks per load batch
    const int A = p.A, K = p.K, H = p.H, HD = H * DK;
    const int nqb = (A + kQB - 1) / kQB;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int b = wg / nqb, a0 = (wg % nqb) * kQB;
    constexpr int NT = kQB * TQ, NSUB = NT / 64 / kHG; // threads; waves per head
    constexpr int NDBW = NDB / NSUB > 0 ? NDB / NSUB : 1;  // output blocks of o per wave
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = tid / TQ, jq = tid % TQ;
    const int hsl = wave % kHG, hsub = wave / kHG; // head slot and sub-wave of this wave
    const int g = lane >> 4, l16 = lane & 15;
    const int a = a0 + q;
    const bool qin = a < A;
    const int64_t bA = (int64_t)b * A;
    const int64_t nrow = bA + (qin ? a : 0);
    // addresses: 64-bit bases uniform over the workgroup (scalar registers)
    // plus 32-bit per-thread offsets
    const int64_t row0 = bA + a0;          // first query row of the block
    const uint32_t qr = qin ? (uint32_t)q : 0u; // this thread's row in the block (clamped)
    // slot i of the thread is key slot jq + TQ*i of the query: for every i
    // the TQ threads of a query touch consecutive slots (coalesced rows,
    // conflict-free tile and tag cells for windowed key lists)
    const SlotLayout L = slot_layout(H, VV, STYLE);
    float *wpr = reinterpret_cast<float *>(smem + L.o_wpr);
    float *tile = reinterpret_cast<float *>(smem + L.o_t);
    const float *qg = reinterpret_cast<const float *>(p.q); // fp32 logit operands
    const float *kg = reinterpret_cast<const float *>(p.k);
    const T *vtg = reinterpret_cast<const T *>(p.v);        // [B][HD][vt_pitch(A)]
    const int vtp = vt_pitch(A);
    T *att = reinterpret_cast<T *>(p.attention);
    T *og = reinterpret_cast<T *>(p.o);

    // AF3 pair weight factors (first: the wait for them covers nothing else)
    T psv{}, wpv{};
    if (FUSED)
        pair_weights_load<T>(reinterpret_cast<const T *>(p.pair_scale),
                             reinterpret_cast<const T *>(p.w_pair), VV, H, psv, wpv);
    // ---- key ids and window bits of this thread's slots (loads clamped
    // into the row; slots past its end are marked missing), and the
    // query's usability, unconditionally. Issued before the pair rows:
    // loads return in order, so the key-id chain (ids, then the key
    // usability gather) does not wait for the pair rows.
    const uint8_t uq = ld_off<uint8_t>(p.usable + row0, qr);
    int64_t kid[SPL];
    bool wmv[SPL];
    const int64_t *kib = p.key_index + row0 * K;
    const uint8_t *wmb = p.window_mask + row0 * K;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int k = jq + TQ * i;
        const uint32_t off = qr * (uint32_t)K + (uint32_t)min(k, K - 1);
        kid[i] = ld_off<int64_t>(kib, off * 8u);
        wmv[i] = ld_off<uint8_t>(wmb, off) != 0;
        if (!qin || k >= K) {
            kid[i] = -1;
            wmv[i] = false;
        }
    }
    // ---- row-major copy of this block's V rows (for the gather path of
    // other blocks): one 16-byte vector of one channel's consecutive atoms
    // from the transposed copy per thread, stored element by element; the
    // stores need no wait and overlap the loads below
    if (p.vrows_out) {
        constexpr int CH = kQB / E; // 16-byte vectors per channel
        T *vrw = reinterpret_cast<T *>(p.vrows_out);
        for (int t = tid; t < HD * CH; t += NT) {
            const int c = t / CH, q0 = (t - c * CH) * E;
            const uint4 vv = ld_off<uint4>(vtg + ((int64_t)b * HD + c) * vtp,
                                           (uint32_t)(a0 + q0) * (uint32_t)sizeof(T));
            const T *ve = reinterpret_cast<const T *>(&vv);
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (a0 + q0 + e < A)
                    vrw[(row0 + q0 + e) * HD + c] = ve[e];
        }
    }
    // ---- AF3 pair rows of this thread's slots, in groups of GS slots: the
    // first group (both, when there are two) is in flight from the start,
    // each later group while the previous one is reduced. Loads are issued
    // unconditionally (a load in a branch makes every later wait cover it):
    // rows past the end of a ragged key list re-read the last row, threads
    // without slots read the query's last row, rows of unusable queries are
    // loaded but unused.
    const int nsl = !qin || K <= jq ? 0 : min(SPL, (K - jq + TQ - 1) / TQ); // slots that exist
    constexpr int GS = SPL < 4 ? SPL : (NV <= 2 ? 4 : (NV * (int)sizeof(T) <= 8 ? 2 : 1));
    constexpr int NG = SPL / GS;
    uint4 pbuf[2][GS][NVB];
    const int slast = max(nsl, 1) - 1;
    const T *pairb = reinterpret_cast<const T *>(p.pair) + row0 * K * VV;
    const uint32_t prow = (qr * (uint32_t)K + (uint32_t)min(jq, K - 1)) * VV;
    auto load_group = [&](uint4 (&dst)[GS][NVB], int g0) {
#pragma unroll
        for (int ii = 0; ii < GS; ++ii) {
            const uint32_t src = prow + (uint32_t)(min(g0 + ii, slast) * TQ * VV);
#pragma unroll
            for (int pt = 0; pt < NV; ++pt)
                dst[ii][pt] = ld_off<uint4>(pairb, (src + pt * E) * (uint32_t)sizeof(T));
        }
    };
    // (two groups take the registers of the double buffer)
    if (FUSED) {
        load_group(pbuf[0], 0);
        if (NG == 2)
            load_group(pbuf[1], GS);
    }
    // precomputed pair bias of the thread's slots (clamped as the rows)
    float4 pbv[PRE ? SPL : 1];
    if (PRE) {
        const float4 *pbb = reinterpret_cast<const float4 *>(p.pbias) + row0 * K;
        const uint32_t pbr = qr * (uint32_t)K + (uint32_t)min(jq, K - 1);
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            pbv[i] = ld_off<float4>(pbb, (pbr + (uint32_t)(min(i, slast) * TQ)) * 16u);
    }

    const bool qok = qin && uq != 0;
    if (tid == 0) {
        s_lo = INT_MAX;
        s_hi = -1;
    }
    bool cand[SPL];
    uint8_t uj[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int64_t j = kid[i];
        const int64_t dist = j > a ? j - a : a - j;
        cand[i] = qok && wmv[i] && j >= 0 && j < A && (p.radius < 0 || dist <= p.radius);
        uj[i] = 0;
    }
    // key usability of every slot, loaded unconditionally (ids clamped into
    // the batch) so that all SPL loads are in flight together; used (with
    // cand) only once the pair bias is formed
#pragma unroll
    for (int i = 0; i < SPL; ++i)
        uj[i] = ld_off<uint8_t>(p.usable + bA, (uint32_t)min(max(kid[i], (int64_t)0), (int64_t)A - 1));
    if (FUSED)
        pair_weights_put<T>(psv, wpv, VV, H, wpr, wpr + VV * 4);

    // ---- AF3 pair bias per slot and head (H <= 4), in registers
    float beta[SPL][kHG];
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
        for (int h = 0; h < kHG; ++h)
            beta[i][h] = 0.0f;
    __syncthreads(); // wpr, s_lo/s_hi initialised
    if (FUSED && nsl > 0) {
        const float4 *w4p = reinterpret_cast<const float4 *>(wpr);
        const float4 ws = pair_wsum(wpr + VV * 4);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (NG > 2 && gi + 1 < NG)
                load_group(pbuf[(gi + 1) & 1], (gi + 1) * GS);
            if (!qok)
                continue;
            float bb[GS][4];
            pair_bias_rows<T, NVB, GS>(pbuf[gi & 1], w4p, ws, p.eps, bb);
#pragma unroll
            for (int ii = 0; ii < GS; ++ii)
#pragma unroll
                for (int h = 0; h < kHG; ++h)
                    beta[gi * GS + ii][h] = bb[ii][h];
        }
    }
    if (PRE && nsl > 0) {
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            beta[i][0] = pbv[i].x;
            beta[i][1] = pbv[i].y;
            beta[i][2] = pbv[i].z;
            beta[i][3] = pbv[i].w;
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

    // Attention rows of one head. For bf16 rows of whole 16-byte vectors
    // (one fitting the query's 512-byte row of the tag tile, which is free
    // by the time the weights exist) the values pass through that row so
    // that each thread writes 16-byte vectors instead of 2-byte values: the
    // row belongs to this wave's query, and the LDS accesses of one wave
    // take effect in order, so no barrier is needed (compiler barriers keep
    // the order of the accesses). fp32 values are stored directly.
    constexpr int SROW = kRMAX * 4 / (int)sizeof(T); // staging row, elements
    const bool vec_att = sizeof(T) == 2 && (K * (int)sizeof(T)) % 16 == 0 && K <= SROW &&
                         (reinterpret_cast<uintptr_t>(p.attention) & 15) == 0;
    T *stg = reinterpret_cast<T *>(smem + L.o_tag) + q * SROW;
    auto store_att = [&](int h, const float *w) {
        T *ab = att + (((int64_t)b * H + h) * A + a0) * K;
        if (vec_att) {
            __asm__ volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < SPL; ++i)
                if (jq + TQ * i < K)
                    stg[jq + TQ * i] = from_f<T>(w[i]);
            __asm__ volatile("" ::: "memory");
            if (qin)
                for (int c = jq * E; c < K; c += TQ * E)
                    st_off<uint4>(ab, (uint32_t)(q * K + c) * (uint32_t)sizeof(T),
                                  *reinterpret_cast<const uint4 *>(stg + c));
            __asm__ volatile("" ::: "memory");
            return;
        }
        if (!qin)
            return;
        // one per-thread offset; the slot's stride goes into the (uniform)
        // base. The offset is opaque here, so the compiler forms each address
        // at its store (scalar base + offset) instead of keeping 64-bit
        // addresses of every head and slot live across the block, which
        // spilled them.
        uint32_t ao = (uint32_t)(q * K + jq) * (uint32_t)sizeof(T);
        __asm__ volatile("" : "+v"(ao));
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (jq + TQ * i < K)
                st_off<T>(ab + TQ * i, ao, from_f<T>(w[i]));
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
            for (int c = jq; c < HD; c += TQ)
                og[nrow * HD + c] = from_f<T>(0.0f);
        return;
    }

    const int jal = s_lo & ~7; // band start, aligned for the transposed V rows
    const int span = jhi + 1 - jal;
    const int nch = (span + kRMAX - 1) / kRMAX;
    if (p.wide && nch > kWideChunks) {
        // scattered key ids: the band grows with their spread, not with K;
        // the gather kernel takes this block
        if (tid == 0)
            p.wide[1 + atomicAdd(p.wide, 1)] = wg;
        return;
    }
    const float scale = p.inv_sqrt_d;
    float *twave = tile + hsl * kQB * L.sp; // this wave's head tile
    // Unique writer of each probability cell (query, key row): every
    // allowed slot writes its slot index into the tag tile and the one
    // whose index survives writes the cell with a plain store; the others
    // (repeated key ids in a row) add their weights with LDS atomics after
    // a barrier. A wide band (several chunks) adds every weight atomically.
    // The tags are written here and read after the first barrier of the
    // score phase.
    int *tag = reinterpret_cast<int *>(smem + L.o_tag);
    bool win[SPL];
    int lose_any = 1;
#pragma unroll
    for (int i = 0; i < SPL; ++i)
        win[i] = false;
    if (nch == 1) {
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (rel[i] >= 0)
                tag[q * kRMAX + rel[i] - jal] = jq + TQ * i;
    }

    // V operands (B of P V) of the band chunk starting at key row c0, k
    // chunks kc0 .. kc0+VG-1 of its nkc, for head hw: chunk kc, output block
    // t holds rows c0 + kc*KC + g*QU .. +E-1 of channel hw*DK + t*16 + l16.
    // Chunks past the last re-read it; rows past the batch's last atom are
    // the zero padding of the transposed rows (at most 31 past A). All VG
    // chunks are in flight together.
    auto load_v = [&](uint4 (&dst)[VG][NDBW], int c0, int kc0, int nkc, int hw, int t0) {
        const int hc = min(hw, H - 1);
        const T *vrow = vtg + ((int64_t)b * HD + hc * DK) * vtp;
#pragma unroll
        for (int j = 0; j < VG; ++j) {
            const int r = c0 + min(kc0 + j, nkc - 1) * KC + g * QU;
#pragma unroll
            for (int t = 0; t < NDBW; ++t)
                dst[j][t] = ld_off<uint4>(vrow, (uint32_t)(((t0 + t) * 16 + l16) * vtp + r) * (uint32_t)sizeof(T));
        }
    };
    for (int hg = 0; hg < H; hg += kHG) {
        const int hw = hg + hsl; // this wave's head in the S and P V products
        const bool hv = hw < H;
        // Q fragments (A operand of S): query row l16, fp32
        uint4 qf[NKQ];
        {
            const int aq = a0 + l16;
#pragma unroll
            for (int kc = 0; kc < NKQ; ++kc) {
                qf[kc] = make_uint4(0, 0, 0, 0);
                if (hv && aq < A)
                    qf[kc] = ld_off<uint4>(qg + row0 * HD, (uint32_t)(l16 * HD + hw * DK + kc * 16 + g * 4) * 4u);
            }
        }
        // lg: the pair bias until a slot's logit is added to it (each slot
        // lies in exactly one chunk), then the logit, then the weight
        float (&lg)[SPL][kHG] = beta;
        if (hg > 0) { // only ESMFold2 has more than 4 heads, and no pair bias
#pragma unroll
            for (int i = 0; i < SPL; ++i)
#pragma unroll
                for (int hh = 0; hh < kHG; ++hh)
                    lg[i][hh] = 0.0f;
        }

        for (int c = 0; c < nch; ++c) {
            const int c0 = jal + c * kRMAX;
            const int rows = min(kRMAX, jhi + 1 - c0);
            const int ncb = (rows + 15) / 16;
            if (hv) {
                for (int cb0 = hsub * CBG; cb0 < ncb; cb0 += NSUB * CBG) {
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
                                kb[t][kc] = ld_off<uint4>(kg + (bA + c0) * HD,
                                                          (uint32_t)(r * HD + hw * DK + kc * 16 + g * 4) * 4u);
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
                                twave[acc16_row(v, lane) * L.sp + (cb0 + t) * 16 + acc16_col(lane)] = acc[t][v];
                }
            }
            __syncthreads(); // score tiles (and the tags) written
            if (hg == 0 && c == 0 && nch == 1) {
                lose_any = 0;
                // all tag reads first (unconditional, in range), then the
                // tests: one LDS wait instead of one per slot
                int tv[SPL];
#pragma unroll
                for (int i = 0; i < SPL; ++i)
                    tv[i] = tag[q * kRMAX + (rel[i] >= 0 ? rel[i] - jal : 0)];
#pragma unroll
                for (int i = 0; i < SPL; ++i) {
                    win[i] = rel[i] >= 0 && tv[i] == jq + TQ * i;
                    lose_any |= (rel[i] >= 0 && !win[i]) ? 1 : 0;
                }
            }
            // logits of the slots in this chunk: every tile read issued
            // unconditionally (clamped into the row), then added where the
            // slot is allowed, in the chunk and its head exists
            {
                float sv[kHG][SPL];
#pragma unroll
                for (int hh = 0; hh < kHG; ++hh) {
                    const float *sh = tile + (hh * kQB + q) * L.sp;
#pragma unroll
                    for (int i = 0; i < SPL; ++i)
                        sv[hh][i] = sh[min(max(rel[i] - c0, 0), kRMAX - 1)];
                }
#pragma unroll
                for (int hh = 0; hh < kHG; ++hh)
#pragma unroll
                    for (int i = 0; i < SPL; ++i) {
                        const int r = rel[i] - c0;
                        if (hg + hh < H && rel[i] >= 0 && r >= 0 && r < rows)
                            lg[i][hh] = fmaf(sv[hh][i], scale, lg[i][hh]);
                    }
            }
            // score tiles read; the next chunk or P may reuse them
            if (hg == 0 && c == nch - 1)
                lose_any = __syncthreads_or(lose_any);
            else
                __syncthreads();
        }
        // the tiles become the (zeroed) probability tiles
        for (int i = tid; i < kHG * kQB * L.sp / 4; i += NT)
            reinterpret_cast<float4 *>(tile)[i] = make_float4(0.f, 0.f, 0.f, 0.f);

        // masked softmax per head over the row: TQ lanes per query
#pragma unroll
        for (int hh = 0; hh < kHG; ++hh) {
            if (hg + hh >= H)
                break;
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < SPL; ++i)
                if (rel[i] >= 0)
                    m = fmaxf(m, lg[i][hh]);
            m = TQ == 32 ? fmaxf(max16(m), __shfl_xor(max16(m), 16)) : max16(m);
            float w[SPL];
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                w[i] = rel[i] >= 0 ? __expf(lg[i][hh] - m) : 0.0f;
                sum += w[i];
            }
            sum = sum16(sum);
            if (TQ == 32)
                sum += __shfl_xor(sum, 16);
            const float inv = sum > 0.0f ? __builtin_amdgcn_rcpf(sum) : 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                w[i] *= inv;
                lg[i][hh] = w[i];
            }
            store_att(hg + hh, w);
        }
        __syncthreads(); // probability tiles zero

        // o = P V per head; P scattered by key id (repeats add up)
        // this wave's output blocks of o: t0 .. t0 + NDBW - 1 (none past NDB)
        const int t0 = hsub * NDBW;
        const bool pv = hv && t0 < NDB;
        f32x4_t oacc[NDBW];
#pragma unroll
        for (int t = 0; t < NDBW; ++t)
            oacc[t] = zero4();
        for (int c = 0; c < nch; ++c) {
            const int c0 = jal + c * kRMAX;
            const int rows = min(kRMAX, jhi + 1 - c0);
            const int nkc = (rows + 31) / 32 * 32 / KC;
#pragma unroll
            for (int hh = 0; hh < kHG; ++hh) {
                if (hg + hh >= H)
                    break;
                float *ph = tile + (hh * kQB + q) * L.sp;
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
                    float *ph = tile + (hh * kQB + q) * L.sp;
#pragma unroll
                    for (int i = 0; i < SPL; ++i) {
                        const int r = rel[i] - c0;
                        if (rel[i] >= 0 && !win[i] && r >= 0 && r < rows)
                            atomicAdd(&ph[r], lg[i][hh]);
                    }
                }
            }
            __syncthreads();
            if (pv) {
                const float *prow = twave + l16 * L.sp + g * QU;
                for (int kc0 = 0; kc0 < nkc; kc0 += VG) {
                    uint4 vb[VG][NDBW];
                    load_v(vb, c0, kc0, nkc, hw, t0);
#pragma unroll
                    for (int j = 0; j < VG; ++j) {
                        if (kc0 + j < nkc) {
                            const uint4 av = p_chunk<T>(prow + (kc0 + j) * KC);
#pragma unroll
                            for (int t = 0; t < NDBW; ++t)
                                Mma16<T>::mma(oacc[t], av, vb[j][t]);
                        }
                    }
                }
            }
            if (c + 1 < nch || hg + kHG < H)
                __syncthreads(); // P read: the next chunk or head group may rewrite the tiles
            if (c + 1 < nch) {
                // the next chunk's probability tiles start from zero
                for (int i = tid; i < kHG * kQB * L.sp / 4; i += NT)
                    reinterpret_cast<float4 *>(tile)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                __syncthreads();
            }
        }
        if (pv) {
            // the block's rows of o: a uniform base and one opaque 32-bit
            // lane offset (formed here, not hoisted and kept per element)
            T *ob = og + (bA + a0) * HD + hw * DK + t0 * 16;
            uint32_t oo = (uint32_t)(acc16_row(0, lane) * HD + acc16_col(lane)) * (uint32_t)sizeof(T);
            __asm__ volatile("" : "+v"(oo));
#pragma unroll
            for (int t = 0; t < NDBW; ++t) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = acc16_row(v, lane);
                    if (a0 + r < A)
                        st_off<T>(ob + v * HD + t * 16, oo, from_f<T>(oacc[t][v]));
                }
            }
        }
    }
}

// Kernel of one style/dtype family for the given slots-per-thread, head
// width and pair vectors per row (defined in the instantiating units).
const void *pick_slot_af3_f32(int spl, int D, int nv);
const void *pick_slot_af3_bf16(int spl, int D, int nv);
const void *pick_slot_esm(int dtype, int spl, int D, int tq);
const void *pick_slot_af3_pre(int dtype, int spl, int D);

template <typename T, int STYLE, int NV, int TQ, int S1, int S2, int S3>
const void *pick_slot_tq(int spl, int D) {
    switch (spl) {
    case S1:
        switch (D) {
        case 16: return (const void *)k_slot<T, STYLE, S1, 16, NV, TQ>;
        case 32: return (const void *)k_slot<T, STYLE, S1, 32, NV, TQ>;
        case 64: return (const void *)k_slot<T, STYLE, S1, 64, NV, TQ>;
        default: return (const void *)k_slot<T, STYLE, S1, 128, NV, TQ>;
        }
    case S2:
        switch (D) {
        case 16: return (const void *)k_slot<T, STYLE, S2, 16, NV, TQ>;
        case 32: return (const void *)k_slot<T, STYLE, S2, 32, NV, TQ>;
        case 64: return (const void *)k_slot<T, STYLE, S2, 64, NV, TQ>;
        default: return (const void *)k_slot<T, STYLE, S2, 128, NV, TQ>;
        }
    default:
        switch (D) {
        case 16: return (const void *)k_slot<T, STYLE, S3, 16, NV, TQ>;
        case 32: return (const void *)k_slot<T, STYLE, S3, 32, NV, TQ>;
        case 64: return (const void *)k_slot<T, STYLE, S3, 64, NV, TQ>;
        default: return (const void *)k_slot<T, STYLE, S3, 128, NV, TQ>;
        }
    }
}

// Kernel for slots per thread spl (slot_spl(K, TQ)) and head width D.
template <typename T, int STYLE, int NV, int TQ>
const void *pick_slot_sd(int spl, int D) {
    if constexpr (TQ == 32)
        return pick_slot_tq<T, STYLE, NV, 32, 1, 4, 8>(spl, D);
    else
        return pick_slot_tq<T, STYLE, NV, 16, 1, 8, 16>(spl, D);
}

} // namespace waa
