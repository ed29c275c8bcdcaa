// pair_tied.hip -- tied pair row attention ("Tied Pair Row Attention",
// Required behavior and Worked example). For a pair grid F [B,L,L,C] and
// bias features Fb [B,L,L,Cb], with both pair axes exchanged first
// (X[s][i] = F[i][s], Xb[i][j] = Fb[j][i]):
//   xn = LN(X) * norm_scale + norm_bias,  q, k, v = xn @ w_q, w_k, w_v,
//   g = sigmoid(xn @ w_gate)  (all bias-free, [C, H*D]),
//   beta[h][i][j] = (LN(Xb[i][j]) * bias_norm_scale + bias_norm_bias) @ w_bias[:, h]
//   A[h][i][j] = softmax_j( sum_{s,d} q[s][i][h][d] k[s][j][h][d] / sqrt(L*D)
//                           + beta[h][i][j] )
//   U[i][k][h][d] = sum_j A[h][i][j] v[k][j][h][d]     (query i, anchor k)
//   update[i][k] = (g[i][k] * U[i][k]) @ w_out + b_out, axes exchanged back:
//   out[k][i] = update[i][k], i.e. out[a][c] = (g(F[a][c]) * U[c][a]) @ w_out + b_out.
// No residual is added.
//
// Kernels (all on the caller's stream, workspace laid out by tied_layout):
//  k_pack (pack.hip)  w_q, w_k, w_v, w_gate, w_out into MFMA B-fragment order
//  k_tied_bias        beta, eight threads per (b, i, j), fp32 (only when Cb is
//                     not a multiple of 8 or exceeds 256; else k_tied_proj
//                     forms beta)
//  k_tied_proj        one workgroup per 32 entries F[j0..j0+31][kcol] of a
//                     grid column: affine LayerNorm (fp32) into an LDS
//                     operand tile (and, for the bias, the LayerNorm of
//                     Fb[j][kcol] times w_bias, written as beta[h][kcol][j]),
//                     then q|k and v|gate on MFMA (32x32
//                     blocks, one head per block since D = 32). q and k
//                     (rows: grid row, reduction index: grid column*D + d)
//                     and v (rows: anchor*D + d, reduction index: key) are
//                     stored in operand-fragment order (frag_base below),
//                     G as G[row][col][h*D + d], so that each later product
//                     loads a wave's operand as one contiguous kilobyte.
//                     Entries outside the L x L grid (the grid is padded to
//                     Lp = L rounded up to 32) are zeros.
//  k_tied_logits      kKS workgroups per (b, h, 32 rows i, 32 columns j):
//                     S = Qh Kh^T over the Lp*D reduction (split over the
//                     kKS workgroups and their 4 waves; the waves' parts are
//                     summed in LDS, each workgroup writes its partial tile),
//                     scaled by 1/sqrt(L*D); the softmax adds the partials
// bf16 storage keeps five roundings in a chain (LayerNorm output, q/k/v/g,
// the weights, the gated U, the output), enough to reach the 2e-2 bound on
// large grids; so the LayerNorm output and the gated U go into the matrix
// products as hi + lo bf16 pairs, and q and k are stored as hi + lo pairs
// whose logits take three bf16 products (hi.hi + hi.lo + lo.hi).
//  k_tied_softmax     one wave per row: + beta, softmax over j < L (zeros
//                     past L), A in the storage type
//  k_tied_out         one workgroup per (b, 32 queries i, NA anchors k):
//                     per head U = A Vt^T on MFMA, times the gate, into an
//                     LDS tile; the output projection on MFMA (w_out packed),
//                     + b_out, rows out[b][k][i0..i0+31] as 16-byte vectors.
#include <cmath>
#include <type_traits>
#include <cstring>

#include "../../include/atom_attn.h"
#include "common.hpp"
#include "kernels.hpp"

namespace waa {

namespace {

constexpr int kTD = 32;  // head width

__host__ __device__ inline size_t tal16(size_t x) { return (x + 15) & ~(size_t)15; }
constexpr int kNA = 4;   // anchors per workgroup of k_tied_out
constexpr int kKS = 4;   // workgroups sharing one logit tile's reduction

struct TiedArgs {
    int B, L, Lp, C, Cb, H;
    float eps, scale;                 // scale = 1/sqrt(L*D)
    const void *f, *fb;               // features [B,L,L,C], bias features [B,L,L,Cb]
    const void *ns, *nb, *bns, *bnb;  // LayerNorm affine parameters
    const void *w_bias, *b_out;       // [Cb,H], [C]
    const uint4 *pk;                  // packed w_q, w_k, w_v, w_gate, w_out
    int64_t off_q, off_k, off_v, off_g, off_o;
    void *qh, *kh, *vt, *g, *amat;    // storage type
    void *qlo, *klo;                  // bf16: the rest of q and k (q = qh + qlo), else null
    float *beta, *s;                  // fp32 [B][H][Lp][Lp]
    void *out;                        // [B,L,L,C]
    int fuse_bias;                    // beta formed by k_tied_proj (Cb % 8 == 0, Cb <= 256)
    int vec_f, vec_fb;                // rows of F / Fb read as 16-byte vectors
};

// Operand-fragment order of the intermediates read by the matrix products
// (q, k, their low parts, v, A). A [rows][Kd] matrix of matrix mat is stored
// as 1 KB fragments, one per (row tile rt of 32 rows, k chunk kc of KC):
// lane l = r + 32*hf holds k = kc*KC + hf*HALF + e of row rt*32 + r at
// element offset (((mat*ntiles + rt)*nkc + kc)*64 + l)*HALF + e, i.e. exactly
// the 16 bytes that lane passes to the 32x32 MFMA, so a wave's operand load
// is one contiguous kilobyte. frag_base gives the offset of fragment (rt, 0);
// ntiles*32 = rows (Lp for q, k, A; Lp anchors of 32 columns for v) and
// nkc*KC = Kd, so every matrix holds Lp*Lp*32 or Lp*Lp elements as before.
template <typename T>
__device__ __forceinline__ int64_t frag_base(int64_t mat, int rt, int nkc, int ntiles) {
    return ((mat * ntiles + rt) * (int64_t)nkc) * 64 * Mma32<T>::HALF;
}

__device__ __forceinline__ float f4_get(const float4 &f, int c) {
    return c == 0 ? f.x : c == 1 ? f.y : c == 2 ? f.z : f.w;
}

// Channels [0, per) of one eighth of a row (per <= 32) into x, zeros past per
// and for rows that are not valid. The loads are issued together from
// clamped offsets before any value is used: 16-byte vectors when vec (the
// row part 16-byte aligned), else single elements.
template <typename T>
__device__ __forceinline__ void load_part(const T *row, int per, bool vec, bool valid,
                                          float (&x)[32]) {
    constexpr int E = 16 / sizeof(T);
    if (vec) {
        uint4 v[32 / E];
#pragma unroll
        for (int u = 0; u < 32 / E; ++u)
            v[u] = *reinterpret_cast<const uint4 *>(row + min(u * E, per - E));
#pragma unroll
        for (int u = 0; u < 32 / E; ++u) {
            float f[E];
            unpack16<T>(v[u], f);
#pragma unroll
            for (int e = 0; e < E; ++e)
                x[u * E + e] = valid && u * E + e < per ? f[e] : 0.0f;
        }
    } else {
        T v[32];
#pragma unroll
        for (int e = 0; e < 32; ++e)
            v[e] = row[min(e, per - 1)];
#pragma unroll
        for (int e = 0; e < 32; ++e)
            x[e] = valid && e < per ? to_f(v[e]) : 0.0f;
    }
}

// ---------------------------------------------------------------- bias
// 8 threads per (b, i, j) entry, each a strided eighth of the Cb channels;
// the row statistics and the H head sums reduce over the 8 lanes.
template <typename T>
__global__ __launch_bounds__(256) void k_tied_bias(TiedArgs p) {
    const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
    const int sub = threadIdx.x & 7;
    const int64_t LL = (int64_t)p.L * p.L;
    const bool live = t < (int64_t)p.B * LL;          // uniform over the 8 lanes of an entry
    const int64_t tc = live ? t : 0;
    const int64_t b = tc / LL;
    const int i = (int)((tc - b * LL) / p.L), j = (int)(tc - b * LL - (int64_t)i * p.L);
    // exchanged axes: the bias of (query i, key j) comes from Fb[j][i]
    const T *row = reinterpret_cast<const T *>(p.fb) + ((b * p.L + j) * p.L + i) * p.Cb;
    const T *sc = reinterpret_cast<const T *>(p.bns);
    const T *sh = reinterpret_cast<const T *>(p.bnb);
    const T *wb = reinterpret_cast<const T *>(p.w_bias);
    const int Cb = p.Cb;
    float s = 0.0f;
    for (int c = sub; c < Cb; c += 8)
        s += to_f(row[c]);
    const float mean = sum8(s) / (float)Cb;
    float q = 0.0f;
    for (int c = sub; c < Cb; c += 8) {
        const float d = to_f(row[c]) - mean;
        q += d * d;
    }
    const float rstd = 1.0f / sqrtf(sum8(q) / (float)Cb + p.eps);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = sub; c < Cb; c += 8) {
        const float xn = (to_f(row[c]) - mean) * rstd * to_f(sc[c]) + to_f(sh[c]);
#pragma unroll
        for (int h = 0; h < 8; ++h)
            if (h < p.H)
                acc[h] = fmaf(xn, to_f(wb[c * p.H + h]), acc[h]);
    }
#pragma unroll
    for (int h = 0; h < 8; ++h)
        acc[h] = sum8(acc[h]);
    const int64_t LpLp = (int64_t)p.Lp * p.Lp;
    if (live && sub < p.H) {
        float v = acc[0];
#pragma unroll
        for (int h = 1; h < 8; ++h)
            if (sub == h)
                v = acc[h];
        p.beta[(b * p.H + sub) * LpLp + (int64_t)i * p.Lp + j] = v;
    }
}

// ---------------------------------------------------------- projections
// PB: bias-row channels per thread fixed at compile time (16: bias width
// 128), or 0 for any width.
template <typename T, int PB>
__global__ __launch_bounds__(256) void k_tied_proj(TiedArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int E = 16 / sizeof(T);
    const int C = p.C, H = p.H, HD = H * kTD, L = p.L, Lp = p.Lp;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int njb = Lp / 32;
    const int64_t tile = blockIdx.x;
    const int64_t b = tile / ((int64_t)Lp * njb);
    const int kcol = (int)((tile / njb) % Lp);
    const int j0 = (int)(tile % njb) * 32;
    constexpr bool SPLIT = sizeof(T) == 2;        // bf16: operands as hi + lo pairs
    const int lda = C + E;                        // operand tile pitch (elements)
    T *opA = reinterpret_cast<T *>(smem);         // [32][lda]
    T *opAlo = opA + 32 * lda;                    // [32][lda] (bf16 only)
    float *stg = reinterpret_cast<float *>(smem + tal16((size_t)(SPLIT ? 2 : 1) * 32 * lda * sizeof(T)));
    float *ws = stg + wave * 32 * 33;             // this wave's 32x32 staging block
    // LayerNorm parameters (and, when beta is formed here, the bias
    // LayerNorm's and w_bias) into LDS; rows: 8 threads per entry, each an
    // eighth of the channels, all loads issued before the first use.
    // Channel c of a vector sits at c + c / per (per = channels per thread),
    // w_bias row c at (c + c / perb) * H: the 8 threads of an entry read
    // channels per apart, and the padding puts them in 8 different LDS
    // banks (unpadded, a stride of 16 or 64 floats sent all 8 to one bank).
    const int Cb = p.Cb;
    const bool fb = p.fuse_bias != 0;
    const int per = C / 8, perb = PB > 0 ? PB : Cb / 8;
    const int HP = H <= 4 ? 4 : 8;                // w_bias rows padded to HP heads (zeros past H)
    float *prm = stg + 4 * 32 * 33;               // ns, nb [C + 8]; bns, bnb [Cb + 8]; w_bias [Cb + 8][HP]
    float *pns = prm, *pnb = prm + (C + 8);
    float *pbs = prm + 2 * (C + 8), *pbh = pbs + (Cb + 8), *pwb = pbh + (Cb + 8);
    const int nprm = 2 * C + (fb ? Cb * (2 + HP) : 0);
    {
        for (int e0 = tid; e0 < nprm; e0 += 4 * 256) {
            T v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = min(e0 + u * 256, nprm - 1);
                const void *src = e < C ? p.ns : e < 2 * C ? p.nb
                                : e < 2 * C + Cb ? p.bns : e < 2 * C + 2 * Cb ? p.bnb : p.w_bias;
                int idx;
                if (e < 2 * C + 2 * Cb) {
                    idx = e - (e < C ? 0 : e < 2 * C ? C : e < 2 * C + Cb ? 2 * C : 2 * C + Cb);
                } else { // w_bias entry (c, h) of the padded rows; h >= H reads (c, H - 1), unused
                    const int k = e - 2 * C - 2 * Cb, c = k / HP;
                    idx = c * H + min(k - c * HP, H - 1);
                }
                v[u] = reinterpret_cast<const T *>(src)[idx];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * 256;
                if (e >= nprm)
                    continue;
                float *dst;
                if (e < 2 * C) {
                    const int c = e < C ? e : e - C;
                    dst = (e < C ? pns : pnb) + c + c / per;
                } else if (e < 2 * C + 2 * Cb) {
                    const int c = e < 2 * C + Cb ? e - 2 * C : e - 2 * C - Cb;
                    dst = (e < 2 * C + Cb ? pbs : pbh) + c + c / perb;
                } else {
                    const int k = e - 2 * C - 2 * Cb, c = k / HP, h = k - c * HP;
                    dst = pwb + (c + c / perb) * HP + h;
                    if (h >= H)
                        v[u] = T{};
                }
                *dst = to_f(v[u]);
            }
        }
    }
    const int r = tid >> 3, sub = tid & 7;
    const int j = j0 + r;
    const bool valid = j < L && kcol < L;
    const int64_t ent = (b * L + min(j, L - 1)) * L + min(kcol, L - 1);
    float x[32], xb[32];
    load_part<T>(reinterpret_cast<const T *>(p.f) + ent * C + sub * per, per, p.vec_f != 0, valid, x);
    if (fb)
        load_part<T>(reinterpret_cast<const T *>(p.fb) + ent * Cb + sub * perb, perb,
                     p.vec_fb != 0, valid, xb);
    __syncthreads();
    {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e)
            s += x[e];
        const float mean = sum8(s) / (float)C;
        float q = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const float d = e < per ? x[e] - mean : 0.0f;
            q += d * d;
        }
        const float rstd = 1.0f / sqrtf(sum8(q) / (float)C + p.eps);
        // (padded parameter index of channel sub * per + e: + sub)
        if (per % E == 0) {
            // whole 16-byte pieces of the row (16-byte aligned: the tile
            // pitch and sub * per * sizeof(T) are multiples of 16 bytes)
#pragma unroll
            for (int u = 0; u < 32 / E; ++u) {
                if (u * E < per) {
                    float hv[E], lv[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int c = sub * per + u * E + e;
                        const float v = (x[u * E + e] - mean) * rstd * pns[c + sub] + pnb[c + sub];
                        hv[e] = v;
                        lv[e] = v - to_f(from_f<T>(v));
                    }
                    const int off = r * lda + sub * per + u * E;
                    *reinterpret_cast<uint4 *>(opA + off) = pack16<T>(hv);
                    if (SPLIT)
                        *reinterpret_cast<uint4 *>(opAlo + off) = pack16<T>(lv);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                if (e < per) {
                    const int c = sub * per + e;
                    put_split<T>(opA, SPLIT ? opAlo : nullptr, r * lda + c,
                                 (x[e] - mean) * rstd * pns[c + sub] + pnb[c + sub]);
                }
            }
        }
    }
    if (fb) {
        // beta[h][kcol][j] of this entry: the bias row is Fb[j][kcol], the
        // entry (query kcol, key j) once both axes are exchanged
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e)
            s += xb[e];
        const float mean = sum8(s) / (float)Cb;
        float q = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const float d = e < perb ? xb[e] - mean : 0.0f;
            q += d * d;
        }
        const float rstd = 1.0f / sqrtf(sum8(q) / (float)Cb + p.eps);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // one or two 16-byte reads of the padded weight row per channel, no
        // branch inside the channel loop (a fixed PB unrolls it whole)
        auto bias_sum = [&](auto hp8) {
            constexpr bool H8 = decltype(hp8)::value;
            constexpr int NP = H8 ? 8 : 4;
#pragma unroll
            for (int e = 0; e < (PB > 0 ? PB : 32); ++e) {
                if (PB > 0 || e < perb) {
                    const int c = sub * perb + e + sub; // padded index
                    const float xn = (xb[e] - mean) * rstd * pbs[c] + pbh[c];
                    const float4 w0 = *reinterpret_cast<const float4 *>(pwb + c * NP);
                    acc[0] = fmaf(xn, w0.x, acc[0]);
                    acc[1] = fmaf(xn, w0.y, acc[1]);
                    acc[2] = fmaf(xn, w0.z, acc[2]);
                    acc[3] = fmaf(xn, w0.w, acc[3]);
                    if (H8) {
                        const float4 w1 = *reinterpret_cast<const float4 *>(pwb + c * NP + 4);
                        acc[4] = fmaf(xn, w1.x, acc[4]);
                        acc[5] = fmaf(xn, w1.y, acc[5]);
                        acc[6] = fmaf(xn, w1.z, acc[6]);
                        acc[7] = fmaf(xn, w1.w, acc[7]);
                    }
                }
            }
        };
        if (HP == 8)
            bias_sum(std::true_type{});
        else
            bias_sum(std::false_type{});
#pragma unroll
        for (int h = 0; h < 8; ++h)
            acc[h] = sum8(acc[h]);
        if (valid && sub < H) {
            float v = acc[0];
#pragma unroll
            for (int h = 1; h < 8; ++h)
                if (sub == h)
                    v = acc[h];
            p.beta[((b * H + sub) * Lp + kcol) * (int64_t)Lp + j] = v;
        }
    }
    __syncthreads();
    T *qh = reinterpret_cast<T *>(p.qh), *kh = reinterpret_cast<T *>(p.kh);
    T *vt = reinterpret_cast<T *>(p.vt), *gg = reinterpret_cast<T *>(p.g);
    const int nkc = C / Mma32<T>::KC;
    // stage a 32x32 block (rows = entries, cols = d) of this wave, then store
    // it with 16-byte vectors in the layout of `which`
    auto put = [&](const f32x16_t &acc, int h, int which) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int rr = acc32_row(e, lane), cc = lane & 31;
            float v = acc[e];
            if (which == 3)
                v = sigmoid_f(v);
            ws[rr * 33 + cc] = (j0 + rr < L && kcol < L) ? v : 0.0f;
        }
        __asm__ volatile("" ::: "memory");
        // (one wave's LDS accesses take effect in order)
        constexpr int KC = Mma32<T>::KC, HALF = Mma32<T>::HALF;   // HALF == E
        if (which == 3) {
            // G[row][col][h*D + d]: rows of the block, 16-byte vectors
            for (int idx = lane; idx < 32 * 32 / E; idx += 64) {
                const int a = idx / (32 / E), c0 = (idx % (32 / E)) * E;
                float v[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[e] = ws[a * 33 + c0 + e];
                *reinterpret_cast<uint4 *>(gg + ((b * Lp + j0 + a) * (int64_t)Lp + kcol) * HD +
                                           h * kTD + c0) = pack16<T>(v);
            }
        } else {
            // operand-fragment order (see frag_base): each step of 64 lanes
            // writes one 1 KB fragment. q, k: A fragments of rows j0 + r
            // (row tile j0/32), k index kcol*D + d; v: B fragments of anchor
            // kcol, column d, k index j0 + r.
            for (int idx = lane; idx < 32 * 32 / E; idx += 64) {
                const int kcl = idx >> 6, ln = idx & 63;
                const int rr = ln & 31, k0 = kcl * KC + (ln >> 5) * HALF;
                float v[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[e] = which == 2 ? ws[(k0 + e) * 33 + rr] : ws[rr * 33 + k0 + e];
                const uint4 pv = pack16<T>(v);
                if (which == 2) {
                    *reinterpret_cast<uint4 *>(vt + frag_base<T>(b * H + h, kcol, Lp / KC, Lp) +
                                               ((int64_t)(j0 / KC + kcl) * 64 + ln) * E) = pv;
                } else {
                    const int64_t qo = frag_base<T>(b * H + h, j0 / 32, Lp * kTD / KC, Lp / 32) +
                                       ((int64_t)(kcol * (kTD / KC) + kcl) * 64 + ln) * E;
                    *reinterpret_cast<uint4 *>((which == 0 ? qh : kh) + qo) = pv;
                    if (SPLIT) {
                        // the remainder after rounding, so that hi + lo keeps
                        // about 16 significant bits of the fp32 value
                        float lo[E];
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            lo[e] = v[e] - to_f(from_f<T>(v[e]));
                        *reinterpret_cast<uint4 *>(reinterpret_cast<T *>(which == 0 ? p.qlo : p.klo) + qo) =
                            pack16<T>(lo);
                    }
                }
            }
        }
        __asm__ volatile("" ::: "memory");
    };
    T *lo = SPLIT ? opAlo : nullptr;
    gemm_stage_blk<Blk32<T>, T, true, SPLIT, 4>(
        H, opA, lo, lda, nkc, p.pk + p.off_q, (int64_t)nkc * 64, opA, lo, lda, nkc,
        p.pk + p.off_k, (int64_t)nkc * 64, [&](int nb, const auto &a1, const auto &a2) {
            put(a1.a, nb, 0);
            put(a2.a, nb, 1);
        });
    gemm_stage_blk<Blk32<T>, T, true, SPLIT, 4>(
        H, opA, lo, lda, nkc, p.pk + p.off_v, (int64_t)nkc * 64, opA, lo, lda, nkc,
        p.pk + p.off_g, (int64_t)nkc * 64, [&](int nb, const auto &a1, const auto &a2) {
            put(a1.a, nb, 2);
            put(a2.a, nb, 3);
        });
}

// --------------------------------------------------------------- logits
template <typename T>
__global__ __launch_bounds__(256) void k_tied_logits(TiedArgs p) {
    __shared__ float red[4][32][33];
    constexpr int KC = Mma32<T>::KC, HALF = Mma32<T>::HALF;
    const int Lp = p.Lp, H = p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = Lp / 32;
    // logical block order (b, h, ks, ib, jb), dealt to the XCDs in
    // contiguous runs, so that the tiles reading one K range of one head's
    // q and k rows share an L2
    int64_t t = xcd_remap(blockIdx.x, gridDim.x);
    const int jb = (int)(t % nb); t /= nb;
    const int ib = (int)(t % nb); t /= nb;
    const int ks = (int)(t % kKS); t /= kKS;
    const int h = (int)(t % H);
    const int64_t b = t / H;
    const int64_t K = (int64_t)Lp * kTD;
    // chunks per wave: Lp*D/KC is a multiple of 4*kKS*U (Lp a multiple of 32)
    const int nkc = (int)(K / KC), per = nkc / (4 * kKS);
    const int c0 = (ks * 4 + wave) * per;
    // q and k in operand-fragment order: chunk c of a row tile is the
    // kilobyte at c*64*HALF, this lane's 16 bytes at lane*HALF
    const T *qa = reinterpret_cast<const T *>(p.qh) + frag_base<T>(b * H + h, ib, nkc, nb) + lane * HALF;
    const T *kb = reinterpret_cast<const T *>(p.kh) + frag_base<T>(b * H + h, jb, nkc, nb) + lane * HALF;
    f32x16_t acc = zero16();
    // two register stages: the chunks of the next step are requested before
    // the products of this one (clamped at the end, so every load is
    // unconditional)
    constexpr int U = 4;
    if constexpr (sizeof(T) == 2) {
        // q.k = qh.kh + qh.klo + qlo.kh (the qlo.klo term is below the
        // rounding of the sum)
        const int64_t dl = reinterpret_cast<const T *>(p.qlo) - reinterpret_cast<const T *>(p.qh);
        const int64_t dk = reinterpret_cast<const T *>(p.klo) - reinterpret_cast<const T *>(p.kh);
        uint4 av[U], bv[U], al[U], bl[U];
        auto ld = [&](int kc) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = (int64_t)(c0 + kc + u) * 64 * HALF;
                av[u] = *reinterpret_cast<const uint4 *>(qa + o);
                bv[u] = *reinterpret_cast<const uint4 *>(kb + o);
                al[u] = *reinterpret_cast<const uint4 *>(qa + dl + o);
                bl[u] = *reinterpret_cast<const uint4 *>(kb + dk + o);
            }
        };
        ld(0);
        for (int kc = 0; kc < per; kc += U) {
            uint4 ca[U], cb[U], cal[U], cbl[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ca[u] = av[u]; cb[u] = bv[u]; cal[u] = al[u]; cbl[u] = bl[u];
            }
            ld(min(kc + U, per - U));
#pragma unroll
            for (int u = 0; u < U; ++u) {
                Mma32<T>::mma(acc, ca[u], cb[u]);
                Mma32<T>::mma(acc, ca[u], cbl[u]);
                Mma32<T>::mma(acc, cal[u], cb[u]);
            }
        }
    } else {
        uint4 av[U], bv[U];
        auto ld = [&](int kc) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = (int64_t)(c0 + kc + u) * 64 * HALF;
                av[u] = *reinterpret_cast<const uint4 *>(qa + o);
                bv[u] = *reinterpret_cast<const uint4 *>(kb + o);
            }
        };
        ld(0);
        for (int kc = 0; kc < per; kc += U) {
            uint4 ca[U], cb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ca[u] = av[u]; cb[u] = bv[u];
            }
            ld(min(kc + U, per - U));
#pragma unroll
            for (int u = 0; u < U; ++u)
                Mma32<T>::mma(acc, ca[u], cb[u]);
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
        red[wave][acc32_row(e, lane)][lane & 31] = acc[e];
    __syncthreads();
    // partial tile ks of the logits: S[ks][b][h][i][j]
    float *srow = p.s + (int64_t)ks * p.B * H * Lp * Lp + ((b * H + h) * (int64_t)Lp + ib * 32) * Lp +
                  jb * 32;
    for (int idx = tid; idx < 32 * 32; idx += 256) {
        const int rr = idx >> 5, cc = idx & 31;
        srow[(int64_t)rr * Lp + cc] =
            (red[0][rr][cc] + red[1][rr][cc] + red[2][rr][cc] + red[3][rr][cc]) * p.scale;
    }
}

// -------------------------------------------------------------- softmax
template <typename T>
__global__ __launch_bounds__(256) void k_tied_softmax(TiedArgs p) {
    constexpr int KC = Mma32<T>::KC, HALF = Mma32<T>::HALF, NU = 16 / HALF;
    const int Lp = p.Lp, L = p.L;
    const int lane = threadIdx.x & 63;
    const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*H + h)*Lp + i
    const int64_t nrow = (int64_t)p.B * p.H * Lp;
    if (rowid >= nrow)
        return;
    const int i = (int)(rowid % Lp);
    // A in operand-fragment order (row tile i/32, k index j): the HALF
    // consecutive j of one step of this lane are one 16-byte piece
    T *am = reinterpret_cast<T *>(p.amat) + frag_base<T>(rowid / Lp, i / 32, Lp / KC, Lp / 32);
    auto put = [&](int jj, const float *v) {
        const int kc = jj / KC, hf = (jj % KC) / HALF;
        *reinterpret_cast<uint4 *>(am + ((int64_t)kc * 64 + (i & 31) + 32 * hf) * HALF) = pack16<T>(v);
    };
    float v[NU][HALF];
    if (i >= L) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int e = 0; e < HALF; ++e)
                v[u][e] = 0.0f;
            const int jj = (u * 64 + lane) * HALF;
            if (jj < Lp)
                put(jj, v[u]);
        }
        return;
    }
    const float *srow = p.s + rowid * Lp;
    const int64_t pstride = (int64_t)p.B * p.H * Lp * Lp;  // between partial logit tiles
    const float *brow = p.beta + rowid * Lp;
    // this lane's j = (u*64 + lane)*HALF + e: loads of clamped offsets, all
    // issued before the first use
    float4 bq[NU][HALF / 4], sq[kKS][NU][HALF / 4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int jj = min((u * 64 + lane) * HALF, Lp - HALF);
#pragma unroll
        for (int q = 0; q < HALF / 4; ++q) {
            bq[u][q] = *reinterpret_cast<const float4 *>(brow + jj + 4 * q);
#pragma unroll
            for (int k = 0; k < kKS; ++k)
                sq[k][u][q] = *reinterpret_cast<const float4 *>(srow + k * pstride + jj + 4 * q);
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < HALF; ++e) {
            const int j = (u * 64 + lane) * HALF + e;
            float x = f4_get(bq[u][e / 4], e % 4);
#pragma unroll
            for (int k = 0; k < kKS; ++k)
                x += f4_get(sq[k][u][e / 4], e % 4);
            v[u][e] = j < L ? x : -INFINITY;
            m = fmaxf(m, v[u][e]);
        }
    m = group_max<64>(m);
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < HALF; ++e) {
            const int j = (u * 64 + lane) * HALF + e;
            v[u][e] = j < L ? expf(v[u][e] - m) : 0.0f;
            sum += v[u][e];
        }
    sum = group_sum<64>(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int e = 0; e < HALF; ++e)
            v[u][e] *= inv;
        const int jj = (u * 64 + lane) * HALF;
        if (jj < Lp)
            put(jj, v[u]);
    }
}

// ---------------------------------------------------- U, gate, output
template <typename T>
__global__ __launch_bounds__(256) void k_tied_out(TiedArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KC = Mma32<T>::KC, HALF = Mma32<T>::HALF, E = 16 / sizeof(T);
    const int Lp = p.Lp, L = p.L, H = p.H, HD = H * kTD, C = p.C;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nib = Lp / 32, nag = (L + kNA - 1) / kNA;
    int64_t t = blockIdx.x;
    const int ag = (int)(t % nag); t /= nag;
    const int ib = (int)(t % nib);
    const int64_t b = t / nib;
    const int i0 = ib * 32;
    constexpr bool SPLIT = sizeof(T) == 2;  // bf16: the gated U tile as hi + lo
    const int ldu = HD + E;
    T *ut = reinterpret_cast<T *>(smem);                                  // [32][ldu]
    T *utlo = ut + 32 * ldu;                                              // [32][ldu] (bf16)
    float *ot = reinterpret_cast<float *>(smem + tal16((size_t)(SPLIT ? 2 : 1) * 32 * ldu * sizeof(T)));  // [32][C+4]
    const int ldo = C + 4;
    const T *amat = reinterpret_cast<const T *>(p.amat);
    const T *vt = reinterpret_cast<const T *>(p.vt);
    const T *gg = reinterpret_cast<const T *>(p.g);
    const T *bo = reinterpret_cast<const T *>(p.b_out);
    T *out = reinterpret_cast<T *>(p.out);
    const int nkc = Lp / KC;
    const int r = lane & 31;
    for (int a = ag * kNA; a < min(L, ag * kNA + kNA); ++a) {
        // U[i][a] of each head this wave takes, times the gate g(F[a][i])
        for (int h = wave; h < H; h += 4) {
            // A (row tile i0/32) and v (anchor a) in operand-fragment order:
            // chunk k is the kilobyte at k*64*HALF
            const T *ar = amat + frag_base<T>(b * H + h, i0 / 32, nkc, nib) + lane * HALF;
            const T *vr = vt + frag_base<T>(b * H + h, a, nkc, Lp) + lane * HALF;
            f32x16_t acc = zero16();
            constexpr int U = 4;
            for (int kc = 0; kc < nkc; kc += U) {
                uint4 av[U], bv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = min(kc + u, nkc - 1);
                    av[u] = *reinterpret_cast<const uint4 *>(ar + (int64_t)k * 64 * HALF);
                    bv[u] = *reinterpret_cast<const uint4 *>(vr + (int64_t)k * 64 * HALF);
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (kc + u < nkc)
                        Mma32<T>::mma(acc, av[u], bv[u]);
            }
            // element e: query row acc32_row(e), channel d = lane % 32
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int rr = acc32_row(e, lane);
                const int ic = min(i0 + rr, Lp - 1);
                const float gv = to_f(gg[((b * Lp + a) * (int64_t)Lp + ic) * HD + h * kTD + r]);
                put_split<T>(ut, SPLIT ? utlo : nullptr, rr * ldu + h * kTD + r, acc[e] * gv);
            }
        }
        __syncthreads();
        // output projection of the 32 rows: [32 x HD] @ w_out [HD x C]
        const int nkh = HD / KC;
        gemm_stage<Blk32<T>, T, false, SPLIT, 4>(
            C / 32, ut, SPLIT ? utlo : nullptr, ldu, nkh, p.pk + p.off_o, (int64_t)nkh * 64, ut,
            SPLIT ? utlo : nullptr, ldu, 0,
            p.pk + p.off_o, 0, [&](int rr, int c, float x1, float) {
                ot[rr * ldo + c] = x1 + to_f(bo[c]);
            });
        __syncthreads();
        // out[b][a][i0 + rr][:] rows as 16-byte vectors
        const int vpr = C / E;
        for (int idx = tid; idx < 32 * vpr; idx += 256) {
            const int rr = idx / vpr, c0 = (idx - rr * vpr) * E;
            if (i0 + rr < L)
                *reinterpret_cast<uint4 *>(out + ((b * L + a) * (int64_t)L + i0 + rr) * C + c0) =
                    pack16<T>(ot + rr * ldo + c0);
        }
        __syncthreads(); // the LDS tiles are rewritten for the next anchor
    }
}

} // namespace

// Workspace layout of one call.
struct TiedLayout {
    size_t packed, qh, kh, qlo, klo, vt, g, amat, beta, s, total;
    int64_t units_qkvg, units_o;
};

static size_t up256t(size_t x) { return (x + 255) & ~(size_t)255; }

TiedLayout tied_layout(int64_t B, int64_t L, int64_t C, int64_t H, int esz) {
    TiedLayout Lo;
    const int64_t Lp = (L + 31) / 32 * 32, HD = H * kTD;
    Lo.units_qkvg = packed_units((int)C, (int)HD, esz);
    Lo.units_o = packed_units((int)HD, (int)C, esz);
    size_t o = 0;
    Lo.packed = o; o = up256t(o + (size_t)(4 * Lo.units_qkvg + Lo.units_o) * 16);
    const size_t big = (size_t)(B * H * Lp * Lp * kTD) * esz;
    Lo.qh = o; o = up256t(o + big);
    Lo.kh = o; o = up256t(o + big);
    Lo.qlo = Lo.klo = o;
    if (esz == 2) {
        Lo.qlo = o; o = up256t(o + big);
        Lo.klo = o; o = up256t(o + big);
    }
    Lo.vt = o; o = up256t(o + big);
    Lo.g = o; o = up256t(o + big);
    Lo.amat = o; o = up256t(o + (size_t)(B * H * Lp * Lp) * esz);
    Lo.beta = o; o = up256t(o + (size_t)(B * H * Lp * Lp) * 4);
    Lo.s = o; o = up256t(o + (size_t)kKS * (B * H * Lp * Lp) * 4);
    Lo.total = o;
    return Lo;
}

static bool tied_fuse_bias(int64_t Cb) { return Cb % 8 == 0 && Cb <= 256; }
static size_t tied_proj_lds(int64_t C, int64_t Cb, int64_t H, int esz) {
    return tal16((size_t)(esz == 2 ? 2 : 1) * 32 * (C + 16 / esz) * esz) + (size_t)4 * 32 * 33 * 4 +
           (size_t)(2 * (C + 8) + (tied_fuse_bias(Cb) ? (Cb + 8) * (2 + (H <= 4 ? 4 : 8)) : 0)) * 4;
}
static size_t tied_out_lds(int64_t C, int64_t H, int esz) {
    return tal16((size_t)(esz == 2 ? 2 : 1) * 32 * (H * kTD + 16 / esz) * esz) +
           (size_t)32 * (C + 4) * 4;
}

int tied_supported(int64_t B, int64_t L, int64_t C, int64_t Cb, int64_t H, int64_t D) {
    return D == kTD && H >= 1 && H <= 8 && C >= 32 && C <= 256 && C % 32 == 0 && Cb >= 1 &&
           Cb <= 1024 && L >= 1 && L <= 1024 && B >= 1 && B * L * L <= ((int64_t)1 << 26);
}

} // namespace waa

// ------------------------------------------------------------- C ABI

extern "C" {

int atom_attn_tied_row_attention_workspace_bytes(const atom_attn_tied_dims *d, int dtype,
                                                 size_t *bytes) {
    if (!d || !bytes || (dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16) || d->B < 1 ||
        d->L < 1 || d->C < 1 || d->CB < 1 || d->H < 1 || d->D < 1)
        return ATOM_ATTN_EINVAL;
    if (!waa::tied_supported(d->B, d->L, d->C, d->CB, d->H, d->D))
        return ATOM_ATTN_EUNSUPPORTED;
    *bytes = waa::tied_layout(d->B, d->L, d->C, d->H, dtype == ATOM_ATTN_BF16 ? 2 : 4).total;
    return ATOM_ATTN_OK;
}

int atom_attn_tied_row_attention(const atom_attn_tied_dims *d, int dtype, double eps,
                                 const void *features, const void *bias_features,
                                 const void *norm_scale, const void *norm_bias,
                                 const void *bias_norm_scale, const void *bias_norm_bias,
                                 const void *w_q, const void *w_k, const void *w_v,
                                 const void *w_bias, const void *w_gate, const void *w_out,
                                 const void *b_out, void *output, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    using namespace waa;
    size_t need = 0;
    int rc = atom_attn_tied_row_attention_workspace_bytes(d, dtype, &need);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const float fe = (float)eps;
    const void *ptrs[] = {features, bias_features, norm_scale, norm_bias, bias_norm_scale,
                          bias_norm_bias, w_q, w_k, w_v, w_bias, w_gate, w_out, b_out, output};
    for (const void *q : ptrs)
        if (!q)
            return ATOM_ATTN_EINVAL;
    if (!(eps > 0.0) || !(fe > 0.0f) || !std::isfinite(fe) || ((uintptr_t)output & 15) != 0 ||
        ((uintptr_t)features & 15) != 0)
        return ATOM_ATTN_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 15) != 0 || workspace_bytes < need)
        return ATOM_ATTN_EWORKSPACE;
    const int esz = dtype == ATOM_ATTN_BF16 ? 2 : 4, dt = esz == 2 ? 1 : 0;
    const TiedLayout Lo = tied_layout(d->B, d->L, d->C, d->H, esz);
    char *ws = (char *)workspace;
    hipStream_t s = (hipStream_t)stream;
    const int C = (int)d->C, HD = (int)(d->H * kTD);
    // pack the five matrices into B-fragment order (32-column blocks)
    PackArgs pa;
    std::memset(&pa, 0, sizeof(pa));
    const void *mats[5] = {w_q, w_k, w_v, w_gate, w_out};
    int64_t off = 0;
    for (int m = 0; m < 5; ++m) {
        const int kd = m < 4 ? C : HD, n = m < 4 ? HD : C;
        pa.job[m] = PackJob{mats[m], n, kd, n, off, 0};
        off += packed_units(kd, n, esz);
    }
    pa.njobs = 5;
    pa.total = off;
    pa.out = (uint4 *)(ws + Lo.packed);
    TiedArgs a;
    std::memset(&a, 0, sizeof(a));
    a.B = (int)d->B; a.L = (int)d->L; a.Lp = (int)((d->L + 31) / 32 * 32); a.C = C;
    a.Cb = (int)d->CB; a.H = (int)d->H;
    a.eps = fe;
    a.scale = (float)(1.0 / std::sqrt((double)d->L * kTD));
    a.f = features; a.fb = bias_features; a.ns = norm_scale; a.nb = norm_bias;
    a.bns = bias_norm_scale; a.bnb = bias_norm_bias; a.w_bias = w_bias; a.b_out = b_out;
    a.pk = (const uint4 *)(ws + Lo.packed);
    a.off_q = 0; a.off_k = Lo.units_qkvg; a.off_v = 2 * Lo.units_qkvg;
    a.off_g = 3 * Lo.units_qkvg; a.off_o = 4 * Lo.units_qkvg;
    a.qh = ws + Lo.qh; a.kh = ws + Lo.kh; a.vt = ws + Lo.vt; a.g = ws + Lo.g;
    a.qlo = esz == 2 ? ws + Lo.qlo : nullptr;
    a.klo = esz == 2 ? ws + Lo.klo : nullptr;
    a.amat = ws + Lo.amat; a.beta = (float *)(ws + Lo.beta); a.s = (float *)(ws + Lo.s);
    a.out = output;
    a.fuse_bias = tied_fuse_bias(d->CB) ? 1 : 0;
    a.vec_f = (C / 8 * esz) % 16 == 0;
    a.vec_fb = a.fuse_bias && (d->CB / 8 * esz) % 16 == 0 && ((uintptr_t)bias_features & 15) == 0;
    void *args[] = {(void *)&a};
    const int64_t Lp = a.Lp;
    hipError_t e = launch_pack(pa, dt, s);
    if (e != hipSuccess)
        return ATOM_ATTN_ELAUNCH;
    auto go = [&](int id, const void *fn, int64_t grid, size_t lds) -> bool {
        allow_lds(fn, lds);
        ProfSpan sp = prof_begin(id, s);
        hipError_t r = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, lds, s);
        prof_end(sp, s);
        return r == hipSuccess;
    };
    const int64_t nb32 = Lp / 32;
    const bool ok =
        (a.fuse_bias ||
         go(KN_TIED_BIAS, dt ? (const void *)k_tied_bias<bf16_t> : (const void *)k_tied_bias<float>,
            (a.B * (int64_t)a.L * a.L * 8 + 255) / 256, 0)) &&
        go(KN_TIED_PROJ,
           a.fuse_bias && d->CB == 128
               ? (dt ? (const void *)k_tied_proj<bf16_t, 16> : (const void *)k_tied_proj<float, 16>)
               : (dt ? (const void *)k_tied_proj<bf16_t, 0> : (const void *)k_tied_proj<float, 0>),
           a.B * Lp * nb32, tied_proj_lds(C, d->CB, d->H, esz)) &&
        go(KN_TIED_LOGITS,
           dt ? (const void *)k_tied_logits<bf16_t> : (const void *)k_tied_logits<float>,
           a.B * (int64_t)a.H * nb32 * nb32 * kKS, 0) &&
        go(KN_TIED_SOFTMAX,
           dt ? (const void *)k_tied_softmax<bf16_t> : (const void *)k_tied_softmax<float>,
           (a.B * (int64_t)a.H * Lp + 3) / 4, 0) &&
        go(KN_TIED_OUT, dt ? (const void *)k_tied_out<bf16_t> : (const void *)k_tied_out<float>,
           a.B * nb32 * ((a.L + kNA - 1) / kNA), tied_out_lds(C, a.H, esz));
    if (!ok || hipGetLastError() != hipSuccess)
        return ATOM_ATTN_ELAUNCH;
    return ATOM_ATTN_OK;
}

} // extern "C"
