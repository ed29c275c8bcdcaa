// pair_s2p.hip -- single-to-pair features ("ESMFold Single-to-Pair
// Features", Required behavior): for tokens x [B,N,C] with presence mask
// [B,N],
//   y = (LN(x) * norm_scale + norm_bias) @ weight + bias, q = y[:H], k = y[H:]
//   pair_features[b,i,j] = [k_i * q_j, q_j - k_i]                    (2H)
//   output[b,i,j] = pair_features[b,i,j] @ out_weight + out_bias      (D)
//                   then, when output_norm, LN(.) * output_scale + output_bias
// both tensors zero unless tokens i and j are present; absent tokens'
// payloads are never read into arithmetic (select, not multiply).
//
// k_s2p_tok: one workgroup per TT tokens: the rows in LDS (fp32), their
//   population statistics, the affine norm and the projection (VALU, fp32),
//   written as fp32 [B,N,2H] rows (q then k) to the workspace.
// k_s2p_pair: one workgroup per tile of 32 key tokens j and kIG query tokens
//   i; NW = D/32 waves, wave w owns output columns 32w..32w+31. The A
//   operand of the pair head is the pair-feature row itself, formed chunk by
//   chunk in registers from q_j (fp32, registers) and k_i (fp32, LDS) and rounded
//   to the storage type -- exactly the values stored as pair_features, so
//   output = stored features @ out_weight on the matrix cores (32x32 MFMA,
//   fp32 accumulation). Each wave stores the feature chunks kc = w (mod NW);
//   the output tile goes through LDS (bias, optional LayerNorm with
//   cross-wave row sums, mask) and leaves as 16-byte row vectors.
#include <cmath>
#include <cstring>

#include "../../include/atom_attn.h"
#include "common.hpp"
#include "kernels.hpp"

namespace waa {

namespace {

constexpr int kTT = 4;   // tokens per workgroup of the token kernel
constexpr int kTokThreads = 1024;  // threads per workgroup of the token kernel
constexpr int kIG = 8;   // query tokens per workgroup of the pair kernel

template <typename T>
__global__ __launch_bounds__(kTokThreads) void k_s2p_tok(S2PArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NWV = kTokThreads / 64;
    const int C = p.C, H2 = 2 * p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kTT;
    const int64_t ntok = (int64_t)p.B * p.N;
    float *xs = reinterpret_cast<float *>(smem);   // [kTT][C]
    float *st = xs + kTT * C;                       // [kTT][2] mean, rstd
    float *red = st + 2 * kTT;                      // [NWV][kTT][2H] partial sums
    const T *x = reinterpret_cast<const T *>(p.x);
    const int nel = kTT * C;
    // the norm parameters of this thread's elements e0 + u * kTokThreads (the
    // first group: every later group repeats its channels when C divides
    // the thread count, else they are read again below), requested first
    const T *ns = reinterpret_cast<const T *>(p.norm_scale);
    const T *nb = reinterpret_cast<const T *>(p.norm_bias);
    const bool prm_once = kTokThreads % C == 0;
    T sv0[4], bv0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = min(tid + u * kTokThreads, nel - 1);
        const int c = e - (e / C) * C;
        sv0[u] = ns[c];
        bv0[u] = nb[c];
    }
    // rows in LDS: the row and presence loads of four elements are issued
    // together from clamped indices, absent or missing tokens are selected to
    // zeros (their payloads never enter arithmetic)
    for (int e0 = tid; e0 < nel; e0 += 4 * kTokThreads) {
        T v[4];
        uint8_t m[4];
        bool in[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = min(e0 + u * kTokThreads, nel - 1);
            const int r = e / C;
            const int64_t t = min(t0 + r, ntok - 1);
            in[u] = t0 + r < ntok;
            m[u] = p.mask[t];
            v[u] = x[t * C + (e - r * C)];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * kTokThreads;
            if (e < nel)
                xs[e] = in[u] && m[u] != 0 ? to_f(v[u]) : 0.0f;
        }
    }
    __syncthreads();
    // population mean and variance (two passes over LDS), one row per wave,
    // 16-byte reads with several in flight (C is a multiple of 32)
    for (int r = wave; r < kTT; r += NWV) {
        float s = 0.0f;
#pragma unroll 4
        for (int c = 4 * lane; c < C; c += 256) {
            const float4 v = *reinterpret_cast<const float4 *>(xs + r * C + c);
            s += (v.x + v.y) + (v.z + v.w);
        }
        s = group_sum<64>(s);
        const float mean = s / (float)C;
        float q = 0.0f;
#pragma unroll 4
        for (int c = 4 * lane; c < C; c += 256) {
            const float4 v = *reinterpret_cast<const float4 *>(xs + r * C + c);
            const float d0 = v.x - mean, d1 = v.y - mean, d2 = v.z - mean, d3 = v.w - mean;
            q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
        }
        q = group_sum<64>(q);
        if (lane == 0) {
            st[2 * r] = mean;
            st[2 * r + 1] = 1.0f / sqrtf(q / (float)C + p.eps);
        }
    }
    __syncthreads();
    for (int e0 = tid; e0 < nel; e0 += 4 * kTokThreads) {
        T sv[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sv[u] = sv0[u];
            bv[u] = bv0[u];
        }
        if (!prm_once || e0 != tid) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = min(e0 + u * kTokThreads, nel - 1);
                const int c = e - (e / C) * C;
                sv[u] = ns[c];
                bv[u] = nb[c];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * kTokThreads;
            if (e < nel) {
                const int r = e / C;
                xs[e] = (xs[e] - st[2 * r]) * st[2 * r + 1] * to_f(sv[u]) + to_f(bv[u]);
            }
        }
    }
    __syncthreads();
    // projection: thread -> (group of E consecutive output columns, one of
    // P parts of the C range). One 16-byte weight load feeds kTT x E FMAs;
    // eight loads are in flight at a time. The parts of a wave reduce with
    // lane exchanges, the waves' partial sums through LDS in wave order.
    constexpr int E = 16 / sizeof(T);
    const int ng = H2 / E, P = kTokThreads / ng;   // ng divides 64 (2H a power of 2)
    const int og = tid % ng, part = tid / ng;
    const int clo = (int)((int64_t)part * C / P), chi = (int)((int64_t)(part + 1) * C / P);
    const T *w = reinterpret_cast<const T *>(p.weight) + og * E;
    float acc[kTT][E];
#pragma unroll
    for (int rr = 0; rr < kTT; ++rr)
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[rr][e] = 0.0f;
    for (int c = clo; c < chi; c += 8) {
        uint4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            wv[u] = *reinterpret_cast<const uint4 *>(w + (int64_t)min(c + u, chi - 1) * H2);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (c + u < chi) {
                float wf[E];
                unpack16<T>(wv[u], wf);
#pragma unroll
                for (int rr = 0; rr < kTT; ++rr) {
                    const float xv = xs[rr * C + c + u];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        acc[rr][e] = fmaf(xv, wf[e], acc[rr][e]);
                }
            }
        }
    }
    for (int o = ng; o < 64; o <<= 1)
#pragma unroll
        for (int rr = 0; rr < kTT; ++rr)
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[rr][e] += __shfl_xor(acc[rr][e], o);
    if (lane < ng)
#pragma unroll
        for (int rr = 0; rr < kTT; ++rr)
#pragma unroll
            for (int e = 0; e < E; ++e)
                red[(wave * kTT + rr) * H2 + og * E + e] = acc[rr][e];
    __syncthreads();
    const T *bias = reinterpret_cast<const T *>(p.bias);
    for (int idx = tid; idx < kTT * H2; idx += kTokThreads) {
        const int rr = idx / H2, oo = idx - rr * H2;
        float v = to_f(bias[oo]);
#pragma unroll
        for (int q = 0; q < NWV; ++q)
            v += red[(q * kTT + rr) * H2 + oo];
        const int64_t t = t0 + rr;
        if (t < ntok)
            p.qk[t * H2 + oo] = v;
    }
}

// NW = D/32 waves, HH = H (q and k width). A workgroup owns one tile of 32
// key tokens j and kIG query tokens i. Each lane owns one row r = lane%32 of
// the tile and the lane half hh = lane/32 of every A chunk: feature indices
// kc*KC + hh*HALF + e. Chunks kc < H/KC are products k_i*q_j, the rest
// differences q_j - k_i of the same q indices, so a lane keeps H/2 values of
// q_j in registers for the whole workgroup. Everything the loop over i reads
// (q_j, the masks, k_i, the weight fragments) is loaded before it, so the
// loop issues only stores and LDS traffic: a global load inside it would
// make each tile wait for the stores issued before it.
template <typename T, int HH, int NW, bool NORM>
__global__ __launch_bounds__(64 * NW) void k_s2p_pair(S2PArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KC = Mma32<T>::KC, HALF = Mma32<T>::HALF, E = 16 / sizeof(T);
    constexpr int H2 = 2 * HH, NKC = H2 / KC, NQC = HH / KC, D = NW * 32;
    const int N = p.N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntile = (N + 31) / 32;
    const int nig = (N + kIG - 1) / kIG;
    const int t = blockIdx.x % ntile;              // key tile
    const int64_t bg = blockIdx.x / ntile;         // b * nig + query group
    const int64_t b = bg / nig;
    const int i0 = (int)(bg % nig) * kIG;
    const int j0 = t * 32;
    const int ni = min(kIG, N - i0);
    constexpr int SP = D + 4;                     // LDS row pitch of the output tile (fp32)
    float *ki = reinterpret_cast<float *>(smem);  // [kIG][H] k_i
    float *ot = ki + kIG * HH;                    // [32][SP] output tile
    float *red = ot + 32 * SP;                    // [NW][32] row partial sums
    int *mi = reinterpret_cast<int *>(red + NW * 32);  // [kIG] query presence
    int *mj = mi + kIG;                           // [32] key presence
    constexpr int FP = H2 + E;                    // LDS row pitch of the feature tile
    T *ft = reinterpret_cast<T *>(mj + 32);       // [32][FP] feature tile
    const float *qk = p.qk + b * (int64_t)N * H2;
    const uint8_t *mrow = p.mask + b * N;
    for (int e = tid; e < kIG * HH; e += 64 * NW) {
        const int ii = e / HH;
        ki[e] = p.qk[(b * N + i0 + min(ii, ni - 1)) * H2 + HH + (e - ii * HH)];
    }
    if (tid < kIG)
        mi[tid] = tid < ni ? mrow[i0 + tid] : 0;
    if (tid < 32)
        mj[tid] = j0 + tid < N ? mrow[j0 + tid] : 0;
    // B fragments of this wave's 32 output columns over all 2H feature rows,
    // from the packed copy of out_weight (one 16-byte load per chunk)
    const int col = wave * 32 + (lane & 31), hh = lane >> 5;
    uint4 bfrag[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        bfrag[kc] = p.wo_packed[((int64_t)wave * NKC + kc) * 64 + lane];
    const float bias_c = to_f(reinterpret_cast<const T *>(p.out_bias)[col]);
    float osc = 1.0f, osh = 0.0f;
    if (NORM) {
        osc = to_f(reinterpret_cast<const T *>(p.output_scale)[col]);
        osh = to_f(reinterpret_cast<const T *>(p.output_bias)[col]);
    }
    // this lane's q_j values (indices qc*KC + hh*HALF + e, qc < H/KC)
    const int r = lane & 31;
    const int jr = min(j0 + r, N - 1);            // clamped row of this lane
    float qv[NQC][HALF];
#pragma unroll
    for (int qc = 0; qc < NQC; ++qc)
#pragma unroll
        for (int e = 0; e < HALF; e += 4) {
            const float4 f = *reinterpret_cast<const float4 *>(
                qk + (int64_t)jr * H2 + qc * KC + hh * HALF + e);
            qv[qc][e] = f.x; qv[qc][e + 1] = f.y; qv[qc][e + 2] = f.z; qv[qc][e + 3] = f.w;
        }
    const bool jlive = j0 + r < N && mrow[jr] != 0;
    __syncthreads();
    constexpr int VPF = H2 / E, VPO = D / E;      // 16-byte vectors per row
    const int rows = min(32, N - j0);
    for (int ii = 0; ii < ni; ++ii) {
        const int64_t bi = b * N + i0 + ii;
        T *pf = reinterpret_cast<T *>(p.pair_features) + (bi * N + j0) * (int64_t)H2;
        T *out = reinterpret_cast<T *>(p.output) + (bi * N + j0) * (int64_t)D;
        if (mi[ii] == 0) {
            // absent query token: its rows of both tensors are zeros
            const uint4 z = make_uint4(0, 0, 0, 0);
            for (int idx = tid; idx < rows * VPF; idx += 64 * NW)
                reinterpret_cast<uint4 *>(pf)[idx] = z;
            for (int idx = tid; idx < rows * VPO; idx += 64 * NW)
                reinterpret_cast<uint4 *>(out)[idx] = z;
            continue;
        }
        const float *kis = ki + ii * HH;
        f32x16_t acc = zero16();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const int qc = kc % NQC, k0 = kc * KC + hh * HALF;
            const int m0 = qc * KC + hh * HALF;       // index into q_j and k_i
            float f[HALF];
#pragma unroll
            for (int e = 0; e < HALF; ++e)
                f[e] = kc < NQC ? kis[m0 + e] * qv[qc][e] : qv[qc][e] - kis[m0 + e];
            const uint4 a = pack16<T>(f);
            Mma32<T>::mma(acc, a, bfrag[kc]);
            // this wave puts feature chunks kc = wave (mod NW) into the
            // feature tile; absent pairs are zeros
            if (kc % NW == wave)
                *reinterpret_cast<uint4 *>(ft + r * FP + k0) = jlive ? a : make_uint4(0, 0, 0, 0);
        }
        // bias, then the optional LayerNorm over the D columns (rows are
        // split over the NW waves: sums over a wave's 32 lanes, then partial
        // sums across waves in LDS; two passes, mean then variance)
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            v[e] = acc[e] + bias_c;
        if (NORM) {
            float s[16];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                s[e] = group_sum<32>(v[e]);
            if (r == 0)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    red[wave * 32 + acc32_row(e, lane)] = s[e];
            __syncthreads();
            float mean[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float m = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    m += red[w * 32 + acc32_row(e, lane)];
                mean[e] = m / (float)D;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < 16; ++e)
                s[e] = group_sum<32>((v[e] - mean[e]) * (v[e] - mean[e]));
            if (r == 0)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    red[wave * 32 + acc32_row(e, lane)] = s[e];
            __syncthreads();
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float q = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    q += red[w * 32 + acc32_row(e, lane)];
                v[e] = (v[e] - mean[e]) / sqrtf(q / (float)D + p.eps) * osc + osh;
            }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
            ot[acc32_row(e, lane) * SP + col] = v[e];
        __syncthreads();
        // both tiles leave as whole rows of 16-byte vectors; absent pairs
        // as zeros
        for (int idx = tid; idx < rows * VPF; idx += 64 * NW) {
            const int rr = idx / VPF, c0 = (idx - rr * VPF) * E;
            *reinterpret_cast<uint4 *>(pf + (int64_t)rr * H2 + c0) =
                *reinterpret_cast<const uint4 *>(ft + rr * FP + c0);
        }
        for (int idx = tid; idx < rows * VPO; idx += 64 * NW) {
            const int rr = idx / VPO, c0 = (idx - rr * VPO) * E;
            *reinterpret_cast<uint4 *>(out + (int64_t)rr * D + c0) =
                mj[rr] != 0 ? pack16<T>(ot + rr * SP + c0) : make_uint4(0, 0, 0, 0);
        }
        __syncthreads(); // the tile and the partial sums are rewritten next
    }
}

} // namespace

size_t s2p_tok_lds(int C, int H) {
    return ((size_t)kTT * C + kTT * 2 + (size_t)(kTokThreads / 64) * kTT * 2 * H) * 4;
}
size_t s2p_pair_lds(int H, int D, int esz) {
    return ((size_t)kIG * H + 32 * (size_t)(D + 4) + (size_t)(D / 32) * 32) * 4 +
           (size_t)(kIG + 32) * 4 + (size_t)32 * (2 * H + 16 / esz) * esz;
}

int s2p_supported(int64_t C, int64_t H, int64_t D, int dtype) {
    const bool h_ok = H == 32 || H == 64 || (H == 128 && dtype == 1);
    return C >= 1 && C <= 4096 && h_ok && (D == 64 || D == 128 || D == 256);
}

template <typename T, int HH>
const void *pick_s2p(int nw, int norm) {
    switch (nw) {
    case 2: return norm ? (const void *)k_s2p_pair<T, HH, 2, true> : (const void *)k_s2p_pair<T, HH, 2, false>;
    case 4: return norm ? (const void *)k_s2p_pair<T, HH, 4, true> : (const void *)k_s2p_pair<T, HH, 4, false>;
    default: return norm ? (const void *)k_s2p_pair<T, HH, 8, true> : (const void *)k_s2p_pair<T, HH, 8, false>;
    }
}

hipError_t launch_s2p(const S2PArgs &a, int dtype, int output_norm, hipStream_t s) {
    const int64_t ntok = (int64_t)a.B * a.N;
    {
        // out_weight [2H, D] into MFMA B-fragment order (32-column blocks)
        PackArgs pa;
        std::memset(&pa, 0, sizeof(pa));
        pa.job[0] = PackJob{a.out_weight, a.D, 2 * a.H, a.D, 0, 0};
        pa.njobs = 1;
        pa.total = packed_units(2 * a.H, a.D, dtype ? 2 : 4);
        pa.out = const_cast<uint4 *>(a.wo_packed);
        hipError_t e = launch_pack(pa, dtype, s);
        if (e != hipSuccess)
            return e;
    }
    const size_t lt = s2p_tok_lds(a.C, a.H);
    const void *ft = dtype ? (const void *)k_s2p_tok<bf16_t> : (const void *)k_s2p_tok<float>;
    allow_lds(ft, lt);
    S2PArgs pa = a;
    void *args[] = {(void *)&pa};
    ProfSpan sp = prof_begin(KN_S2P_TOK, s);
    hipError_t e = hipLaunchKernel(ft, dim3((unsigned)((ntok + kTT - 1) / kTT)), dim3(kTokThreads), args,
                                   lt, s);
    prof_end(sp, s);
    if (e != hipSuccess)
        return e;
    const int nw = a.D / 32;
    const int ntile = (a.N + 31) / 32;
    const int64_t grid = (int64_t)a.B * ((a.N + kIG - 1) / kIG) * ntile;
    const void *fp;
    if (dtype)
        fp = a.H == 32 ? pick_s2p<bf16_t, 32>(nw, output_norm)
                       : (a.H == 64 ? pick_s2p<bf16_t, 64>(nw, output_norm)
                                    : pick_s2p<bf16_t, 128>(nw, output_norm));
    else
        fp = a.H == 32 ? pick_s2p<float, 32>(nw, output_norm) : pick_s2p<float, 64>(nw, output_norm);
    const size_t lp = s2p_pair_lds(a.H, a.D, dtype ? 2 : 4);
    allow_lds(fp, lp);
    sp = prof_begin(KN_S2P_PAIR, s);
    e = hipLaunchKernel(fp, dim3((unsigned)grid), dim3(64 * nw), args, lp, s);
    prof_end(sp, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

} // namespace waa

// ------------------------------------------------------------- C ABI

namespace {
bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
int s2p_check(const atom_attn_s2p_dims *d, int dtype) {
    if (!d || d->B < 1 || d->N < 1 || d->C < 1 || d->H < 1 || d->D < 1 ||
        (dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16))
        return ATOM_ATTN_EINVAL;
    if (!waa::s2p_supported(d->C, d->H, d->D, dtype) || d->B * d->N > ((int64_t)1 << 24) ||
        d->B * d->N * d->N * 2 * d->H > ((int64_t)1 << 40))
        return ATOM_ATTN_EUNSUPPORTED;
    return ATOM_ATTN_OK;
}
} // namespace

extern "C" {

int atom_attn_single_to_pair_workspace_bytes(const atom_attn_s2p_dims *dims, int dtype,
                                             size_t *bytes) {
    int rc = s2p_check(dims, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!bytes)
        return ATOM_ATTN_EINVAL;
    const size_t esz = dtype == ATOM_ATTN_BF16 ? 2 : 4;
    *bytes = (((size_t)(dims->B * dims->N * 2 * dims->H) * 4 + 255) & ~(size_t)255) +
             (size_t)(2 * dims->H * dims->D) * esz;
    return ATOM_ATTN_OK;
}

int atom_attn_single_to_pair(const atom_attn_s2p_dims *dims, int dtype, double eps,
                             int output_norm, const void *x, const uint8_t *mask,
                             const void *weight, const void *bias, const void *norm_scale,
                             const void *norm_bias, const void *out_weight,
                             const void *out_bias, const void *output_scale,
                             const void *output_bias, void *pair_features, void *output,
                             void *workspace, size_t workspace_bytes, void *stream) {
    int rc = s2p_check(dims, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const float fe = (float)eps;
    if (!(eps > 0.0) || !(fe > 0.0f) || !std::isfinite(fe) || !x || !mask || !weight ||
        !bias || !norm_scale || !norm_bias || !out_weight || !out_bias ||
        (output_norm && (!output_scale || !output_bias)) || !pair_features || !output ||
        !al16(pair_features) || !al16(output) || !al16(weight))
        return ATOM_ATTN_EINVAL;
    size_t need = 0;
    atom_attn_single_to_pair_workspace_bytes(dims, dtype, &need);
    if (!workspace || !al16(workspace) || workspace_bytes < need)
        return ATOM_ATTN_EWORKSPACE;
    waa::S2PArgs a;
    a.B = (int)dims->B; a.N = (int)dims->N; a.C = (int)dims->C; a.H = (int)dims->H;
    a.D = (int)dims->D;
    a.eps = fe;
    a.x = x; a.mask = mask; a.weight = weight; a.bias = bias; a.norm_scale = norm_scale;
    a.norm_bias = norm_bias; a.out_weight = out_weight; a.out_bias = out_bias;
    a.output_scale = output_scale; a.output_bias = output_bias;
    a.qk = (float *)workspace;
    a.wo_packed = (const uint4 *)((char *)workspace +
                                  ((((size_t)(dims->B * dims->N * 2 * dims->H) * 4) + 255) &
                                   ~(size_t)255));
    a.pair_features = pair_features; a.output = output;
    return waa::launch_s2p(a, dtype == ATOM_ATTN_BF16 ? 1 : 0, output_norm ? 1 : 0,
                           (hipStream_t)stream) == hipSuccess
               ? ATOM_ATTN_OK
               : ATOM_ATTN_ELAUNCH;
}

} // extern "C"
