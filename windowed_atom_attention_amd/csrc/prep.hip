// prep.hip -- entry state, conditioning and Q/K/V/gate projections.
//
// k_token_proj (decoder): tokproj[B*T, C] = select(token_valid, token, 0)
//   @ w_token, fp32, one 32-token tile per workgroup.
// k_prep: one 32-atom tile per workgroup (4 waves). Steps, as in
//   "windowed_atom_attention" (Required behavior):
//   usability; sanitised entry state x0 (decoder: + gathered token
//   projection) and condition c; AF3: q_in = A_0(x0), kv_in = A_1(x0) with
//   A_j(z) = LN(z)*sigmoid(cj@w_scale[j]+b_scale[j]) + cj@w_shift[j],
//   cj = LN(c)*cond_scale[j]; ESMFold2: in = RMS(x0)*(1+m1)+m0 with
//   m = SiLU(c)@w_mod; then Q (+b_q for AF3), K, V and G = sigmoid(q_in @
//   w_value_gate); ESMFold2 also RMS-normalises Q and K per head and
//   applies the half-split rotary before they are stored, so the slot
//   kernel gathers pre-rotated keys. Q and K are stored in fp32 (they set
//   the softmax logits), V and G in the storage dtype; for bf16 storage the
//   computed MFMA operands are split into bf16 hi + lo parts.
//   Matrix products run on MFMA (32x32 tiles, A operand from LDS, packed
//   weights from L2); norms and epilogues are fp32 VALU work on the tile.
//   The kernel also zero-fills token_output (encoder) and the status word,
//   so that the pool kernel only writes non-empty tokens.
// k_masks: the usable/allowed masks alone.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace waa {

// Copy one row of n elements (n*sizeof(T) a multiple of 16 bytes) from
// global memory into an LDS operand row, or zero it; 8 threads per row.
template <typename T>
__device__ __forceinline__ void copy_row(T *dst, const T *src, int n, bool ok,
                                         int sub) {
    // groups of 8 vectors per thread, all loads of a group issued
    // (unconditionally, clamped into the row) before any is stored; rows
    // that are not ok are stored as zeros
    constexpr int E = 16 / sizeof(T), RG = 8;
    const int nv = n / E;
    for (int v0 = sub; v0 < nv; v0 += 8 * RG) {
        uint4 val[RG];
#pragma unroll
        for (int j = 0; j < RG; ++j)
            val[j] = *reinterpret_cast<const uint4 *>(src + min(v0 + 8 * j, nv - 1) * E);
#pragma unroll
        for (int j = 0; j < RG; ++j)
            if (v0 + 8 * j < nv)
                *reinterpret_cast<uint4 *>(dst + (v0 + 8 * j) * E) =
                    ok ? val[j] : make_uint4(0, 0, 0, 0);
    }
}

// --------------------------------------------------------------- K0

template <typename T>
__global__ __launch_bounds__(256) void k_token_proj(BlockArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Dims d = p.d;
    const int rows = d.B * d.T;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = tid >> 3, sub = tid & 7;
    const int r0 = blockIdx.x * 32;
    const int ldU = d.U + pad16<T>();
    T *opA = reinterpret_cast<T *>(smem);
    {
        const int r = r0 + row;
        const int rc = r < rows ? r : 0; // rows past the end read row 0
        const uint8_t tv = p.token_valid[rc];
        const bool ok = r < rows && tv;
        copy_row<T>(opA + row * ldU, reinterpret_cast<const T *>(p.token) + (int64_t)rc * d.U,
                    d.U, ok, sub);
    }
    __syncthreads();
    const int nkc = d.U / Mma32<T>::KC;
    for (int nb = wave; nb < d.C / 32; nb += 4) {
        f32x16_t acc = zero16();
        // (8 chunks in flight: this kernel's grid is small and its registers are free)
        gemm1<T, false, 8>(acc, opA, nullptr, ldU, nkc, p.pk + p.off.w_token + (int64_t)nb * nkc * 64);
        const int c = nb * 32 + acc32_col(lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = r0 + acc32_row(v, lane);
            if (r < rows)
                p.tokproj[(int64_t)r * d.C + c] = acc[v];
        }
    }
}

size_t token_proj_lds_bytes(const Dims &d, int dtype) {
    const size_t e = dtype ? 2 : 4;
    return 32 * (d.U * e + 16);
}

hipError_t launch_token_proj(const BlockArgs &a, int dtype, hipStream_t s) {
    const int rows = a.d.B * a.d.T;
    const int grid = (rows + 31) / 32;
    const size_t lds = token_proj_lds_bytes(a.d, dtype);
    if (dtype == 0) {
        allow_lds((const void *)k_token_proj<float>, lds);
        hipLaunchKernelGGL(k_token_proj<float>, dim3(grid), dim3(256), lds, s, a);
    } else {
        allow_lds((const void *)k_token_proj<bf16_t>, lds);
        hipLaunchKernelGGL(k_token_proj<bf16_t>, dim3(grid), dim3(256), lds, s, a);
    }
    return hipGetLastError();
}

// --------------------------------------------------------------- K1

// LDS of one 32-atom tile. Operand tiles that hold computed fp32 values
// (c_j or SiLU(c), q_in, kv_in) are split into hi + lo parts for bf16 so
// that the logits path keeps ~16 mantissa bits; fp32 tiles are single.
struct PrepLayout {
    int hp, ldS, ldC;
    size_t o_xh, o_xl, o_st, o_us, o_rb, o_cr, o_opA, o_opAl, o_hb, o_opQ, o_opQl, total;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// LDS of one 32-row tile:
//  x0 in the storage type (exact for an encoder: x0 is the atom row; a bf16
//  decoder keeps the rest of the fp32 sum atom + token projection in a
//  second tile); row statistics, usability, atom/batch index per row; the
//  raw condition (AF3 but the bf16 decoder: LN(c) * cond_scale[j] is built
//  twice); the A operand
//  tile (hi + lo in bf16), which ESMFold2 reuses as the fp32 staging tile
//  of its Q/K projections; the Q/K/V/G input tile (hi + lo in bf16).
// AF3 keeps the raw condition tile except in the bf16 decoder, whose x0
// needs a second tile: there the condition rows are read again from global
// memory (L2) where needed, so that three workgroups fit a CU.
__host__ __device__ constexpr bool prep_keeps_c(int esz, int style, int stage) {
    return style == STYLE_AF3 && !(esz == 2 && stage == STAGE_DECODER);
}

__host__ __device__ inline PrepLayout prep_layout(const Dims &d, int esz, int style, int stage) {
    PrepLayout L;
    const bool split = esz == 2;
    L.hp = d.H * d.D + 4;
    L.ldS = d.S + 16 / esz;
    L.ldC = d.C + 16 / esz;
    const size_t tS = align16(32 * (size_t)L.ldS * esz), tC = align16(32 * (size_t)L.ldC * esz);
    size_t o = 0;
    L.o_xh = o; o += tC;
    L.o_xl = o;
    if (split && stage == STAGE_DECODER)
        o += tC;
    L.o_st = o; o += 32 * 4 * 4;
    L.o_us = o; o += 32;
    L.o_rb = o; o += 64 * 4; // per row: atom index within its batch, then batch
    L.o_cr = o;
    if (prep_keeps_c(esz, style, stage))
        o += tS;
    L.o_opA = L.o_hb = o;
    L.o_opAl = o + tS;
    size_t ra = (split ? 2 : 1) * tS;
    if (style == STYLE_ESM && 32 * (size_t)L.hp * 4 > ra)
        ra = 32 * (size_t)L.hp * 4;
    o = align16(o + ra);
    L.o_opQ = o; o += tC;
    L.o_opQl = o;
    if (split)
        o += tC;
    L.total = o;
    return L;
}

size_t prep_lds_bytes(const Dims &d, int dtype, int style, int stage) {
    return prep_layout(d, dtype ? 2 : 4, style, stage).total;
}

// Per-head RMS normalisation and half-split rotary of the 32 x H*D tile in
// hb (fp32), stored to dst (fp32). TPR threads per row; for each head a
// thread takes consecutive coordinate pairs (e, e + D/2), so the rotation
// needs no other thread and the sum of squares one TPR-lane reduction:
//   y = x * rsqrt(mean(x^2) + eps),
//   out[e] = y[e] cos[e] - y[e+D/2] sin[e],
//   out[e+D/2] = y[e+D/2] cos[e+D/2] + y[e] sin[e+D/2].
// Rotary factors of one row for a thread with at most 2 of the head's
// (e, e + D/2) pairs: cos and sin of both members, loaded together.
struct RopeRow {
    float c[2][2], s[2][2];
};
template <typename T, int TPR>
__device__ __forceinline__ RopeRow rope_row(const BlockArgs &p, int n0) {
    const Dims d = p.d;
    const int N = d.B * d.A, D = d.D, half = d.D / 2;
    const int pp = (half + TPR - 1) / TPR;
    const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    // the tile's first row as a uniform base, 32-bit offsets; clamped
    const T *csb = reinterpret_cast<const T *>(p.rope_cos) + (int64_t)n0 * D;
    const T *snb = reinterpret_cast<const T *>(p.rope_sin) + (int64_t)n0 * D;
    const uint32_t ro = (uint32_t)((n0 + row < N ? row : 0) * D);
    RopeRow rr;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t e = (uint32_t)max(min(sub * pp + min(i, pp - 1), half - 1), 0);
        rr.c[i][0] = to_f(ld_off<T>(csb, (ro + e) * (uint32_t)sizeof(T)));
        rr.c[i][1] = to_f(ld_off<T>(csb, (ro + e + half) * (uint32_t)sizeof(T)));
        rr.s[i][0] = to_f(ld_off<T>(snb, (ro + e) * (uint32_t)sizeof(T)));
        rr.s[i][1] = to_f(ld_off<T>(snb, (ro + e + half) * (uint32_t)sizeof(T)));
    }
    return rr;
}

// Per-head RMS norm and rotary embedding of the 32 rows in hb (fp32, pitch
// hp) into dst (fp32 [N][HD]); rr holds the row's factors when a thread
// has at most 2 pairs (D <= 4 * TPR), wider heads read them per head.
template <typename T, int TPR>
__device__ void head_rms_rotary(const BlockArgs &p, const float *hb, int hp,
                                int n0, float *dst, const RopeRow &rr) {
    const Dims d = p.d;
    const int N = d.B * d.A, HD = d.H * d.D, D = d.D, half = d.D / 2;
    const int pp = (half + TPR - 1) / TPR; // pairs per thread
    const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    const int n = n0 + row;
    const bool ok = n < N;
    const T *cs = reinterpret_cast<const T *>(p.rope_cos) + (int64_t)(ok ? n : 0) * D;
    const T *sn = reinterpret_cast<const T *>(p.rope_sin) + (int64_t)(ok ? n : 0) * D;
    const float invD = 1.0f / (float)D;
    constexpr int PPM = 2;
    const bool few = pp <= PPM;
    for (int h = 0; h < d.H; ++h) {
        const float *x = hb + row * hp + h * D;
        float ss = 0.0f;
        for (int i = 0; i < pp; ++i) {
            const int e = sub * pp + i;
            if (e < half) {
                ss = fmaf(x[e], x[e], ss);
                ss = fmaf(x[e + half], x[e + half], ss);
            }
        }
        ss = row_sum<TPR>(ss);
        const float rs = rsqrtf(ss * invD + p.eps);
        if (!ok)
            continue;
        float *out = dst + (int64_t)n * HD + h * D;
        if (few) {
#pragma unroll
            for (int i = 0; i < PPM; ++i) {
                const int e = sub * pp + i;
                if (i < pp && e < half) {
                    const float y1 = x[e] * rs, y2 = x[e + half] * rs;
                    out[e] = y1 * rr.c[i][0] - y2 * rr.s[i][0];
                    out[e + half] = y2 * rr.c[i][1] + y1 * rr.s[i][1];
                }
            }
            continue;
        }
        for (int i = 0; i < pp; ++i) {
            const int e = sub * pp + i;
            if (e >= half)
                break;
            const float y1 = x[e] * rs, y2 = x[e + half] * rs;
            out[e] = y1 * to_f(cs[e]) - y2 * to_f(sn[e]);
            out[e + half] = y2 * to_f(cs[e + half]) + y1 * to_f(sn[e + half]);
        }
    }
}

// Workgroups per CU the LDS layout allows: three for bf16, two for fp32.
template <typename T, int STYLE, int STAGE>
constexpr int prep_wgs() {
    return sizeof(T) == 2 ? 3 : 2;
}

// Pair-bias workgroup (AF3, extra workgroups of k_prep placed on compute
// units its tiles leave idle): the bias of heads 0..3 of every slot of
// [B*A*K], one pair row of NV 16-byte vectors per slot. Workgroup w of
// nw takes chunks w, w + nw, ... of NT*RB consecutive slots (NT threads, RB
// rows per thread in flight at once, at most LIM vectors: a register
// budget). Slot kernels that read pbias skip the pair rows.
template <typename T, int NV, int LIM, int NT>
__device__ __forceinline__ void pair_bias_wg(const BlockArgs &p, int w, int nw, unsigned char *smem) {
    constexpr int E = 16 / sizeof(T), VV = NV * E;
    constexpr int RB0 = LIM / NV < 8 ? LIM / NV : 8;
    constexpr int CG = RB0 < 4 ? RB0 : 4;       // slots per reduction (temporaries)
    constexpr int RB = RB0 / CG * CG;           // slots per thread and chunk, a multiple of CG
    float *w4 = reinterpret_cast<float *>(smem);
    float *wpart = w4 + VV * 4;
    pair_weights<T>(reinterpret_cast<const T *>(p.pair_scale),
                    reinterpret_cast<const T *>(p.w_pair), VV, p.d.H, w4, wpart);
    __syncthreads();
    const float4 wsum = pair_wsum(wpart);
    const int64_t total = (int64_t)p.d.B * p.d.A * p.d.K;
    const int64_t nchunk = (total + NT * RB - 1) / (NT * RB);
    const T *pair = reinterpret_cast<const T *>(p.pair);
    float4 *out = reinterpret_cast<float4 *>(p.pbias);
    for (int64_t c = w; c < nchunk; c += nw) {
        const int64_t s0 = c * NT * RB + threadIdx.x;
        uint4 rows[RB][NV];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int64_t sl = min(s0 + (int64_t)i * NT, total - 1);
#pragma unroll
            for (int pt = 0; pt < NV; ++pt)
                rows[i][pt] = *reinterpret_cast<const uint4 *>(pair + sl * VV + pt * E);
        }
#pragma unroll
        for (int j = 0; j < RB; j += CG) {
            // the weight reads stay inside each group (hoisting all of them
            // out of the loops would hold V float4 registers throughout)
            __asm__ volatile("" ::: "memory");
            uint4 grp[CG][NV];
#pragma unroll
            for (int i = 0; i < CG; ++i)
#pragma unroll
                for (int pt = 0; pt < NV; ++pt)
                    grp[i][pt] = rows[j + i][pt];
            float bb[CG][4];
            pair_bias_rows<T, NV, CG>(grp, reinterpret_cast<const float4 *>(w4), wsum, p.eps, bb);
#pragma unroll
            for (int i = 0; i < CG; ++i) {
                const int64_t sl = s0 + (int64_t)(j + i) * NT;
                if (sl < total)
                    out[sl] = make_float4(bb[i][0], bb[i][1], bb[i][2], bb[i][3]);
            }
        }
    }
}

// NW waves (4: 32x32 output blocks, several workgroups per CU; 8: 32x16
// strips, two waves per SIMD, for grids of at most one tile per CU), TPR =
// 64*NW/32 threads per tile row. Workgroups past the tiles (AF3, pbias set)
// compute the pair bias.
template <typename T, int STYLE, int STAGE, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : (prep_wgs<T, STYLE, STAGE>())) void k_prep(BlockArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NT = 64 * NW, TPR = NT / 32;
    using G = typename std::conditional<NW == 8, Blk16<T>, Blk32<T>>::type;
    constexpr int BW = G::BW;
    constexpr int WGS = NW == 8 ? 1 : prep_wgs<T, STYLE, STAGE>(); // workgroups per CU
    // GEMM pipeline depth: 2 where three workgroups share a CU (registers)
    constexpr int PP = WGS == 3 ? 2 : 4;
    const Dims d = p.d;
    const int N = d.B * d.A, C = d.C, S = d.S, HD = d.H * d.D;
    const int tid = threadIdx.x, lane = tid & 63;
    const int row = tid / TPR, sub = tid % TPR;
    const int n0 = blockIdx.x * 32;
    const int n = n0 + row;
    const bool inb = n < N;
    constexpr int E = 16 / sizeof(T);
    constexpr bool SPLIT = sizeof(T) == 2;
    constexpr bool XLO = SPLIT && STAGE == STAGE_DECODER; // x0 kept as hi + lo
    constexpr bool KEEPC = prep_keeps_c(sizeof(T), STYLE, STAGE); // raw condition tile
    const int ntile = (N + 31) / 32;
    if (STYLE == STYLE_AF3 && (int)blockIdx.x >= ntile) {
        const int w = blockIdx.x - ntile, nw = gridDim.x - ntile;
        // pair rows of up to 32 bytes (bf16) or 64 bytes (fp32); wider
        // bf16 rows keep the bias in the slot kernel (registers)
        constexpr int LIM = WGS == 3 ? 16 : 32;
        const int nv = d.V * (int)sizeof(T) / 16;
        if constexpr (sizeof(T) == 2) {
            if (nv == 1)
                pair_bias_wg<T, 1, LIM, NT>(p, w, nw, smem);
            else
                pair_bias_wg<T, 2, LIM, NT>(p, w, nw, smem);
        } else {
            if (nv == 2)
                pair_bias_wg<T, 2, LIM, NT>(p, w, nw, smem);
            else
                pair_bias_wg<T, 4, LIM, NT>(p, w, nw, smem);
        }
        return;
    }

    if (STAGE == STAGE_ENCODER) {
        T *to = reinterpret_cast<T *>(p.token_output);
        const int64_t total = (int64_t)d.B * d.T * d.U;
        for (int64_t i = (int64_t)blockIdx.x * NT + tid; i < total;
             i += (int64_t)ntile * NT)
            to[i] = from_f<T>(0.0f);
    }
    if (p.status != nullptr && blockIdx.x == 0 && tid == 0)
        p.status[0] = 0;
    zero_vt_pad<T>(reinterpret_cast<T *>(p.v), d.B, HD, d.A, blockIdx.x, ntile);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.wide)
        p.wide[0] = 0; // the slot step's queue of wide blocks starts empty

    const PrepLayout L = prep_layout(d, sizeof(T), STYLE, STAGE);
    T *xh = reinterpret_cast<T *>(smem + L.o_xh);
    T *xl = XLO ? reinterpret_cast<T *>(smem + L.o_xl) : nullptr;
    float *st = reinterpret_cast<float *>(smem + L.o_st);
    uint8_t *us = smem + L.o_us;
    int *rb = reinterpret_cast<int *>(smem + L.o_rb);
    T *crs = reinterpret_cast<T *>(smem + L.o_cr);
    T *opA = reinterpret_cast<T *>(smem + L.o_opA);
    T *opAl = SPLIT ? reinterpret_cast<T *>(smem + L.o_opAl) : nullptr;
    float *hb = reinterpret_cast<float *>(smem + L.o_hb);
    T *opQ = reinterpret_cast<T *>(smem + L.o_opQ);
    T *opQl = SPLIT ? reinterpret_cast<T *>(smem + L.o_opQl) : nullptr;
    // x0 of tile element (r, c)
    auto x0 = [&](int r, int c) -> float {
        float v = to_f(xh[r * L.ldC + c]);
        if (XLO)
            v += to_f(xl[r * L.ldC + c]);
        return v;
    };
    // x0 of the 16-byte piece vi of row r (one LDS read per tile instead of
    // one per element)
    auto x0vec = [&](int r, int vi, float (&out)[E]) {
        unpack16<T>(*reinterpret_cast<const uint4 *>(xh + r * L.ldC + vi * E), out);
        if (XLO) {
            float lo[E];
            unpack16<T>(*reinterpret_cast<const uint4 *>(xl + r * L.ldC + vi * E), lo);
#pragma unroll
            for (int e = 0; e < E; ++e)
                out[e] += lo[e];
        }
    };

    // Loads first, all unconditional (rows past the end read row 0; values
    // of unusable atoms are replaced by zeros: selected, never multiplied):
    // the atom's token and validity, the atom and condition rows, then the
    // token's validity and (decoder) its projection row at the clamped
    // token index. Two dependent steps, with the rows in flight meanwhile.
    const int64_t nc = inb ? n : 0;
    const int64_t tk = p.atom_to_token[nc];
    const uint8_t vld = p.valid[nc];
    const T *ar = reinterpret_cast<const T *>(p.atom) + nc * C;
    const T *cr = reinterpret_cast<const T *>(p.condition) + nc * S;
    const int nvC = C / E, nvS = S / E, nvmax = nvC > nvS ? nvC : nvS;
    constexpr int RV = sizeof(T) == 2 ? 2 : 4; // vectors per array and thread in one round
    uint4 va[RV], vc[RV];
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        const int vi = sub + j * TPR;
        va[j] = *reinterpret_cast<const uint4 *>(ar + min(vi, nvC - 1) * E);
        vc[j] = *reinterpret_cast<const uint4 *>(cr + min(vi, nvS - 1) * E);
    }
    const int b = inb ? n / d.A : 0;
    const int64_t tkc = tk >= 0 && tk < d.T ? tk : 0;
    const uint8_t tvl = p.token_valid[(int64_t)b * d.T + tkc];
    const float *tp = p.tokproj + ((int64_t)b * d.T + tkc) * C;
    float4 tpv[STAGE == STAGE_DECODER ? RV * E / 4 : 1]; // first round's projection values
    if (STAGE == STAGE_DECODER) {
#pragma unroll
        for (int j = 0; j < RV; ++j)
#pragma unroll
            for (int t = 0; t < E / 4; ++t)
                tpv[j * (E / 4) + t] =
                    *reinterpret_cast<const float4 *>(tp + min(sub + j * TPR, nvC - 1) * E + 4 * t);
    }
    const bool u = inb && vld && tk >= 0 && tk < d.T && tvl;
    if (sub == 0) {
        us[row] = u;
        rb[row] = inb ? n - b * d.A : 0; // atom index within its batch
        rb[32 + row] = b;
        if (inb)
            p.usable[n] = u;
    }
    float xsum = 0.0f, csum = 0.0f;
    for (int base = sub; base < nvmax; base += RV * TPR) {
        if (base != sub) { // later rounds (wide C or S)
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                const int vi = base + j * TPR;
                va[j] = *reinterpret_cast<const uint4 *>(ar + min(vi, nvC - 1) * E);
                vc[j] = *reinterpret_cast<const uint4 *>(cr + min(vi, nvS - 1) * E);
            }
        }
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            const int vi = base + j * TPR;
            if (vi < nvC) {
                float xv[E];
                unpack16<T>(va[j], xv);
                if (STAGE == STAGE_DECODER) {
#pragma unroll
                    for (int t = 0; t < E / 4; ++t) {
                        const float4 f = base == sub ? tpv[j * (E / 4) + t]
                                                     : *reinterpret_cast<const float4 *>(tp + vi * E + 4 * t);
                        xv[4 * t + 0] += f.x; xv[4 * t + 1] += f.y;
                        xv[4 * t + 2] += f.z; xv[4 * t + 3] += f.w;
                    }
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = u ? xv[e] : 0.0f;
                    if (XLO)
                        put_split<T>(xh, xl, row * L.ldC + vi * E + e, x);
                    else
                        xh[row * L.ldC + vi * E + e] = from_f<T>(x); // exact
                    xsum += x;
                }
            }
            if (vi < nvS) {
                const uint4 cvv = u ? vc[j] : make_uint4(0, 0, 0, 0);
                float cv[E];
                unpack16<T>(cvv, cv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    csum += cv[e];
                    if (STYLE == STYLE_ESM) // A operand of the modulation: SiLU(c)
                        put_split<T>(opA, opAl, row * L.ldS + vi * E + e, silu_f(cv[e]));
                }
                if (KEEPC)
                    *reinterpret_cast<uint4 *>(crs + row * L.ldS + vi * E) = cvv;
            }
        }
    }
    // 16 bytes vi of this row's sanitised condition: from the tile, or read
    // again (L2) where the tile is not kept
    auto c_vec = [&](int vi) -> uint4 {
        if constexpr (KEEPC)
            return *reinterpret_cast<const uint4 *>(crs + row * L.ldS + vi * E);
        else { // unconditional load, then the selection (a load in a branch waits alone)
            const uint4 v = *reinterpret_cast<const uint4 *>(cr + vi * E);
            return u ? v : make_uint4(0, 0, 0, 0);
        }
    };
    const bool c1 = nvS <= RV * TPR; // the condition row took one round: vc holds it
    // row statistics of x0 (and of c for AF3), each thread over its own
    // entries of the tiles (written above by the same thread)
    {
        if (STYLE == STYLE_AF3) {
            const float mean = row_sum<TPR>(xsum) / (float)C;
            float q = 0.0f;
#pragma unroll 2
            for (int vi = sub; vi < nvC; vi += TPR) {
                float xv[E];
                x0vec(row, vi, xv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float t = xv[e] - mean;
                    q += t * t;
                }
            }
            const float rstd = 1.0f / sqrtf(row_sum<TPR>(q) / (float)C + p.eps);
            const float mc = row_sum<TPR>(csum) / (float)S;
            float q2 = 0.0f;
            if (c1) {
#pragma unroll
                for (int j = 0; j < RV; ++j)
                    if (sub + j * TPR < nvS) {
                        float cv[E];
                        unpack16<T>(u ? vc[j] : make_uint4(0, 0, 0, 0), cv);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const float t = cv[e] - mc;
                            q2 += t * t;
                        }
                    }
            } else {
                for (int vi = sub; vi < nvS; vi += TPR) {
                    float cv[E];
                    unpack16<T>(c_vec(vi), cv);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float t = cv[e] - mc;
                        q2 += t * t;
                    }
                }
            }
            const float rc = 1.0f / sqrtf(row_sum<TPR>(q2) / (float)S + p.eps);
            if (sub == 0) {
                st[row * 4 + 0] = mean; st[row * 4 + 1] = rstd;
                st[row * 4 + 2] = mc;   st[row * 4 + 3] = rc;
            }
        } else {
            float q = 0.0f;
#pragma unroll 2
            for (int vi = sub; vi < nvC; vi += TPR) {
                float xv[E];
                x0vec(row, vi, xv);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    q += xv[e] * xv[e];
            }
            const float rstd = 1.0f / sqrtf(row_sum<TPR>(q) / (float)C + p.eps);
            if (sub == 0) {
                st[row * 4 + 0] = 0.0f;
                st[row * 4 + 1] = rstd;
            }
        }
    }

    const int nkS = S / G::KC, nkC = C / G::KC;
    // Q/K/V/G projections. Q and K (the logit operands) are stored in fp32,
    // V and G in the storage dtype.
    float *qo = reinterpret_cast<float *>(p.q);
    float *ko = reinterpret_cast<float *>(p.k);
    T *vo = reinterpret_cast<T *>(p.v);
    T *go = reinterpret_cast<T *>(p.g);
    const int vtp = vt_pitch(d.A);
    // transposed V position of (atom row r of this tile, channel c)
    auto vt_at = [&](int r, int c) -> int64_t {
        return ((int64_t)rb[32 + r] * HD + c) * vtp + rb[r];
    };
    // V rows r .. r+3 (r a multiple of 4) of channel c into the transposed
    // copy: one 4-element vector store when the four atoms are consecutive
    // there (A a multiple of 4: same batch, aligned), else element by element
    const bool vt_vec = d.A % 4 == 0;
    auto store_v4 = [&](int r, int c, float v0, float v1, float v2, float v3) {
        if (vt_vec && n0 + r + 3 < N) {
            T *dst = vo + vt_at(r, c);
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            } else {
                *reinterpret_cast<float4 *>(dst) = make_float4(v0, v1, v2, v3);
            }
        } else {
            const float v[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n0 + r + j < N)
                    vo[vt_at(r + j, c)] = from_f<T>(v[j]);
        }
    };
    if (STYLE == STYLE_AF3) {
        // A_j(x0) = LN(x0) * sigmoid(a_j @ w_scale[j] + b_scale[j]) + a_j @ w_shift[j]
        // with a_j = LN(c) * cond_scale[j]; A_0 feeds Q and G, A_1 K and V.
        // Order: a_0 | A_0 | Q, G and a_1 | A_1 | K, V (one operand tile for
        // both A_j).
        const T *cscale = reinterpret_cast<const T *>(p.cond_scale);
        const T *bscale = reinterpret_cast<const T *>(p.b_scale);
        const T *bq = reinterpret_cast<const T *>(p.b_q);
        auto build_a = [&](int j) {
            const float mc = st[row * 4 + 2], rc = st[row * 4 + 3];
            if (c1) { // one round: every load issued before any is used
                uint4 cvv[RV], scv[RV];
#pragma unroll
                for (int jj = 0; jj < RV; ++jj) {
                    const int vi = min(sub + jj * TPR, nvS - 1);
                    cvv[jj] = c_vec(vi);
                    scv[jj] = *reinterpret_cast<const uint4 *>(cscale + j * S + vi * E);
                }
#pragma unroll
                for (int jj = 0; jj < RV; ++jj) {
                    const int vi = sub + jj * TPR;
                    if (vi < nvS) {
                        float cv[E], sc[E];
                        unpack16<T>(cvv[jj], cv);
                        unpack16<T>(scv[jj], sc);
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            put_split<T>(opA, opAl, row * L.ldS + vi * E + e, (cv[e] - mc) * rc * sc[e]);
                    }
                }
                return;
            }
            for (int vi = sub; vi < nvS; vi += TPR) {
                float cv[E], sc[E];
                unpack16<T>(c_vec(vi), cv);
                unpack16<T>(*reinterpret_cast<const uint4 *>(cscale + j * S + vi * E), sc);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    put_split<T>(opA, opAl, row * L.ldS + vi * E + e, (cv[e] - mc) * rc * sc[e]);
            }
        };
        auto adaln = [&](int j) {
            gemm_stage_cv<G, T, true, SPLIT, PP>(
                C / BW, opA, opAl, L.ldS, nkS, p.pk + p.off.w_scale[j], (int64_t)nkS * 64,
                opA, opAl, L.ldS, nkS, p.pk + p.off.w_shift[j], (int64_t)nkS * 64,
                [&](int c) { return to_f(bscale[j * C + c]); },
                [&](int r, int c, float x1, float x2, float bs) {
                    const float ln = (x0(r, c) - st[r * 4 + 0]) * st[r * 4 + 1];
                    put_split<T>(opQ, opQl, r * L.ldC + c, ln * sigmoid_f(x1 + bs) + x2);
                });
        };
        __syncthreads(); // statistics of every row
        build_a(0);
        __syncthreads();
        adaln(0);
        __syncthreads();
        gemm_stage_cv<G, T, true, SPLIT, PP>(
            HD / BW, opQ, opQl, L.ldC, nkC, p.pk + p.off.w_q, (int64_t)nkC * 64,
            opQ, opQl, L.ldC, nkC, p.pk + p.off.w_vg, (int64_t)nkC * 64,
            [&](int c) { return to_f(bq[c]); },
            [&](int r, int c, float x1, float x2, float bqc) {
                const int nn = n0 + r;
                if (nn < N) {
                    qo[(int64_t)nn * HD + c] = x1 + bqc;
                    go[(int64_t)nn * HD + c] = from_f<T>(sigmoid_f(x2));
                }
            });
        build_a(1); // the A tile is free once A_0 is formed
        __syncthreads();
        adaln(1);
        __syncthreads();
        gemm_stage_blk<G, T, true, SPLIT, PP>(
            HD / BW, opQ, opQl, L.ldC, nkC, p.pk + p.off.w_k, (int64_t)nkC * 64,
            opQ, opQl, L.ldC, nkC, p.pk + p.off.w_v, (int64_t)nkC * 64,
            [&](int nb, const typename G::Acc &x1, const typename G::Acc &x2) {
                const int c = nb * BW + G::col(lane);
#pragma unroll
                for (int i = 0; i < G::NE; i += 4) {
                    const int r = G::row(i, lane);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (n0 + r + j < N)
                            ko[(int64_t)(n0 + r + j) * HD + c] = G::at(x1, i + j);
                    store_v4(r, c, G::at(x2, i), G::at(x2, i + 1), G::at(x2, i + 2), G::at(x2, i + 3));
                }
            });
    } else {
        // in = RMS(x0) * (1 + m1) + m0, m = SiLU(c) @ w_mod[0..1]
        __syncthreads(); // statistics and SiLU(c) of every row
        gemm_stage<G, T, true, SPLIT, PP>(
            C / BW, opA, opAl, L.ldS, nkS, p.pk + p.off.w_mod[0], (int64_t)nkS * 64,
            opA, opAl, L.ldS, nkS, p.pk + p.off.w_mod[1], (int64_t)nkS * 64,
            [&](int r, int c, float x1, float x2) {
                const float rm = x0(r, c) * st[r * 4 + 1];
                put_split<T>(opQ, opQl, r * L.ldC + c, rm * (1.0f + x2) + x1);
            });
        __syncthreads(); // the A tile becomes the projection staging tile hb
        const RopeRow rr = rope_row<T, TPR>(p, n0); // in flight during the projections
        for (int pass = 0; pass < 2; ++pass) {
            const int64_t off1 = pass == 0 ? p.off.w_q : p.off.w_k;
            const int64_t off2 = pass == 0 ? p.off.w_vg : p.off.w_v;
            gemm_stage_blk<G, T, true, SPLIT, PP>(
                HD / BW, opQ, opQl, L.ldC, nkC, p.pk + off1, (int64_t)nkC * 64,
                opQ, opQl, L.ldC, nkC, p.pk + off2, (int64_t)nkC * 64,
                [&](int nb, const typename G::Acc &x1, const typename G::Acc &x2) {
                    const int c = nb * BW + G::col(lane);
#pragma unroll
                    for (int i = 0; i < G::NE; i += 4) {
                        const int r = G::row(i, lane);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            hb[(r + j) * L.hp + c] = G::at(x1, i + j);
                            if (pass == 0 && n0 + r + j < N)
                                go[(int64_t)(n0 + r + j) * HD + c] = from_f<T>(sigmoid_f(G::at(x2, i + j)));
                        }
                        if (pass == 1)
                            store_v4(r, c, G::at(x2, i), G::at(x2, i + 1), G::at(x2, i + 2), G::at(x2, i + 3));
                    }
                });
            __syncthreads();
            head_rms_rotary<T, TPR>(p, hb, L.hp, n0, pass == 0 ? qo : ko, rr);
            __syncthreads();
        }
    }
}

// Pair-bias workgroups: one per compute unit the tiles leave idle.
static int pair_bias_wgs(const Dims &d) {
    const int64_t ntile = ((int64_t)d.B * d.A + 31) / 32;
    return ntile < device_cus() ? device_cus() - (int)ntile : 0;
}

bool prep_hosts_pair_bias(const Dims &d, int dtype, int style, int stage) {
    (void)stage;
    if (style != STYLE_AF3 || (dtype == 1 && d.V > 16))
        return false;
    return pair_bias_wgs(d) * 4 >= device_cus(); // a quarter of the GPU or more is idle
}

hipError_t launch_prep(const BlockArgs &a, int dtype, int style, int stage,
                       hipStream_t s) {
    const int N = a.d.B * a.d.A;
    const int grid = (N + 31) / 32 + (a.pbias != nullptr ? pair_bias_wgs(a.d) : 0);
    const size_t lds = prep_lds_bytes(a.d, dtype, style, stage);
    const void *fn = nullptr;
#define WAA_PICK(T, ST, SG) fn = a.nw8 ? (const void *)k_prep<T, ST, SG, 8> : (const void *)k_prep<T, ST, SG, 4>
    if (dtype == 0) {
        if (style == STYLE_AF3) { if (stage == STAGE_ENCODER) WAA_PICK(float, 0, 0); else WAA_PICK(float, 0, 1); }
        else { if (stage == STAGE_ENCODER) WAA_PICK(float, 1, 0); else WAA_PICK(float, 1, 1); }
    } else {
        if (style == STYLE_AF3) { if (stage == STAGE_ENCODER) WAA_PICK(bf16_t, 0, 0); else WAA_PICK(bf16_t, 0, 1); }
        else { if (stage == STAGE_ENCODER) WAA_PICK(bf16_t, 1, 0); else WAA_PICK(bf16_t, 1, 1); }
    }
#undef WAA_PICK
    allow_lds(fn, lds);
    void *args[] = {(void *)&a};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(a.nw8 ? 512 : 256), args, lds, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

// --------------------------------------------------------------- masks

// x[0 .. n) = value (a kernel rather than a memset, so that a captured
// graph replays it like any other launch)
__global__ __launch_bounds__(256) void k_fill_i32(int32_t *x, int64_t n, int32_t value) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        x[i] = value;
}

__global__ __launch_bounds__(256) void k_masks(Dims d, const uint8_t *valid,
                                               const uint8_t *token_valid,
                                               const uint8_t *window_mask,
                                               const int64_t *a2t,
                                               const int64_t *key_index,
                                               int64_t radius, uint8_t *usable,
                                               uint8_t *allowed, int32_t *token_count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t N = (int64_t)d.B * d.A;
    auto usable_of = [&](int64_t m) -> bool {
        const int64_t t = a2t[m];
        return valid[m] && t >= 0 && t < d.T && token_valid[(m / d.A) * d.T + t];
    };
    if (i < N) {
        const bool u = usable_of(i);
        if (usable)
            usable[i] = u;
        // usable atoms per token: integer additions, so the count does not
        // depend on their order
        if (token_count && u)
            atomicAdd(&token_count[(i / d.A) * d.T + a2t[i]], 1);
    }
    if (i < N * d.K && allowed) {
        const int64_t n = i / d.K;
        const int64_t a = n % d.A, b = n / d.A;
        const int64_t j = key_index[i];
        bool ok = usable_of(n) && j >= 0 && j < d.A && window_mask[i] &&
                  usable_of(b * d.A + j);
        if (ok && radius >= 0)
            ok = (j > a ? j - a : a - j) <= radius;
        allowed[i] = ok;
    }
}

hipError_t launch_masks(const Dims &d, const uint8_t *valid,
                        const uint8_t *token_valid, const uint8_t *window_mask,
                        const int64_t *atom_to_token, const int64_t *key_index,
                        int64_t radius, uint8_t *usable, uint8_t *allowed,
                        int32_t *token_count, hipStream_t s) {
    if (token_count) {
        const int64_t nt = (int64_t)d.B * d.T;
        hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s,
                           token_count, nt, 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t work = (int64_t)d.B * d.A * d.K;
    const int64_t grid = (work + 255) / 256;
    hipLaunchKernelGGL(k_masks, dim3((unsigned)grid), dim3(256), 0, s, d, valid,
                       token_valid, window_mask, atom_to_token, key_index,
                       radius, usable, allowed, token_count);
    return hipGetLastError();
}

} // namespace waa
