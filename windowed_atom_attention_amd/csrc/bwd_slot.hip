// bwd_slot.hip -- the slot-attention step of the backward pass
// ("windowed_atom_attention", Required behavior: masked softmax over each
// query's allowed slots of Q.K/sqrt(D) (+ the AF3 pair bias), o = sum of
// weights times the selected V rows; a key chosen by several slots, of one
// query or of many, receives the sum of their gradients).
//
// Forward (fp32, weights kept): one wave per query atom. The wave marks its
// allowed slots, computes the AF3 pair bias of each, then per head the
// logits (lane = slot), the masked softmax (wave reductions) and o (lane =
// channel, lane groups over slots).
//
// Backward, query side (one wave per query atom), per head h:
//   dW_s = dA_s + dO_h . V[key_s]_h,   dS_s = P_s (dW_s - sum_t P_t dW_t),
//   dQ_h = sum_s dS_s K[key_s]_h / sqrt(D);
// AF3: dS_s is also the gradient of the slot's pair bias, which flows back
// through LN(pair) * pair_scale @ w_pair to the pair row, pair_scale and
// w_pair (per-workgroup partial sums, reduced in a fixed order).
// The query side writes each slot's dS and P (every head) at the slot's
// place in the reverse index of the slot -> key map (per key, its (query,
// slot) entries in ascending order), so that on the key side one wave per
// key sums
//   dK_j = sum dS Q_query / sqrt(D),  dV_j = sum P dO_query
// over every selection of key j reading them contiguously, with no
// floating-point atomics in global memory.
//
// Block forms (large grids, K <= 128, H <= 4, D >= 16): the forward and the
// query side per block of 16 queries whose allowed keys lie in a band of at
// most 128 rows, with the band products (Q.K^T, P.V, dO.V^T, dS.K) on the
// matrix cores and each band row read once per block; blocks with a wider
// band are queued for the per-query kernels.
#include "bwd.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace waa {
namespace bwd {

namespace {

constexpr int kMaxK = 512, kMaxH = 8, kMaxHD = 256;
constexpr int kPairV = 16, kPairH = 4; // AF3 pair-bias gradient bounds
static_assert(kSlotPairRecord == kPairV + kPairV * kPairH, "record layout");

struct SK {
    SlotBwdArgs a;
    float inv_sqrt_d;
};

// LDS floats per wave: key ids [K], per-slot values [K*H], one head's slot
// values [K], one query row [HD], the weights of every head [K*H] (query
// side of the backward).
__host__ __device__ inline int wave_floats(int K, int H, int HD) { return K + K * H + K + HD + K * H; }

// Channels 4 qv .. 4 qv + 3 of pair row `row` (zeros past V): one 8- or
// 16-byte load when V is a multiple of 4, else element loads.
template <typename TP>
__device__ __forceinline__ void load_pair_piece(const TP *pair, int64_t row, int V, int qv,
                                                float (&x)[4]) {
    const TP *p = pair + row * V + 4 * qv;
    if (V % 4 == 0) {
        if (4 * qv < V) {
            if constexpr (sizeof(TP) == 4) {
                const float4 t = *reinterpret_cast<const float4 *>(p);
                x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
            } else {
                const uint2 t = *reinterpret_cast<const uint2 *>(p);
                x[0] = __uint_as_float(t.x << 16);
                x[1] = __uint_as_float(t.x & 0xffff0000u);
                x[2] = __uint_as_float(t.y << 16);
                x[3] = __uint_as_float(t.y & 0xffff0000u);
            }
        } else {
            x[0] = x[1] = x[2] = x[3] = 0.0f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = 4 * qv + i < V ? to_f(p[i]) : 0.0f;
    }
}

// sum over the four lanes of a slot (lanes 4 k .. 4 k + 3)
__device__ __forceinline__ float sum4(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    return v;
}

// LN of a pair row held as four 4-channel pieces by the slot's four lanes
// (x = 0 past V): xhat in place, returns 1/sqrt(var + eps).
__device__ __forceinline__ float pair_ln4(float (&x)[4], int V, int qv, float eps) {
    const float m = sum4(x[0] + x[1] + x[2] + x[3]) / (float)V;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float d = 4 * qv + i < V ? x[i] - m : 0.0f;
        x[i] = d;
        q += d * d;
    }
    const float r = 1.0f / sqrtf(sum4(q) / (float)V + eps);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        x[i] *= r;
    return r;
}

// sum over slots s (in order within each lane group) of w[s] times the
// D channels at rows[kid[s] * HD + off ..]: lane group g = lane / (D/4)
// takes slots g, g + 256/D, ...; its lanes hold one float4 of channels each
// and issue four slots' loads before using them. The groups' partial sums
// are added by lane exchanges; every lane returns its float4 of the total
// (channels 4 * (lane % (D/4)) ..).
template <int D>
__device__ __forceinline__ float4 slot_rowsum(const float *w, const int *kid, int K,
                                              const float *rows, int HD, int off, int lane) {
    constexpr int L4 = D / 4, SP = 64 / L4;
    const int g = lane / L4, q = lane - g * L4;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = 0; s0 < K; s0 += 4 * SP) {
        float4 r[4];
        float ww[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + u * SP + g;
            ww[u] = s < K ? w[s] : 0.0f;
            r[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (ww[u] != 0.0f)
                r[u] = *reinterpret_cast<const float4 *>(rows + (int64_t)kid[s] * HD + off + q * 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc.x += ww[u] * r[u].x;
            acc.y += ww[u] * r[u].y;
            acc.z += ww[u] * r[u].z;
            acc.w += ww[u] * r[u].w;
        }
    }
#pragma unroll
    for (int o = L4; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o);
        acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o);
        acc.w += __shfl_xor(acc.w, o);
    }
    return acc;
}

// dot of the D channels at row[0..D) (global, 16-byte aligned) with v[0..D)
// (LDS), all loads issued first.
template <int D>
__device__ __forceinline__ float row_dot(const float *row, const float *v) {
    float4 r[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
        r[i] = reinterpret_cast<const float4 *>(row)[i];
    float x = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
        x += v[4 * i] * r[i].x + v[4 * i + 1] * r[i].y + v[4 * i + 2] * r[i].z + v[4 * i + 3] * r[i].w;
    return x;
}

// Slot ownership of the per-slot values (logits, weights, gradients):
// slot s = 64 c + sl(lane) of chunk c, sl(lane) = (lane % (D/4)) * (256/D)
// + lane / (D/4) -- the order in which group_dots produces the slots.
template <int D> __device__ __forceinline__ int slot_of_lane(int lane) {
    constexpr int L4 = D / 4, G = 64 / L4;
    return (lane % L4) * G + lane / L4;
}

// Dots of v[0..D) (LDS) with the rows rows[kid[s] * HD + off ..] of slots s
// of chunks c < NC (kid < 0: 0): lane groups of D/4 lanes read one row per
// load (one 16-byte piece per lane, so a load instruction touches 256/D
// rows, not one row per lane), four rows per group in flight; each group's
// partial dots are added by lane exchanges and the lane that owns the slot
// (slot_of_lane) keeps it in out[c].
template <int D, int NC>
__device__ __forceinline__ void group_dots(const float *v, const int *kid, int K,
                                           const float *rows, int HD, int off, int lane,
                                           float (&out)[NC]) {
    constexpr int L4 = D / 4, G = 64 / L4;
    const int g = lane / L4, q = lane - g * L4;
    const float4 vv = reinterpret_cast<const float4 *>(v)[q];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        out[c] = 0.0f;
        if (c * 64 >= K)
            continue;
#pragma unroll
        for (int i0 = 0; i0 < L4; i0 += 4) {
            float4 r[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = c * 64 + (i0 + u) * G + g;
                const int id = (i0 + u < L4 && s < K) ? kid[s] : -1;
                r[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (id >= 0)
                    r[u] = *reinterpret_cast<const float4 *>(rows + (int64_t)id * HD + off + q * 4);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (i0 + u >= L4)
                    break;
                float x = vv.x * r[u].x + vv.y * r[u].y + vv.z * r[u].z + vv.w * r[u].w;
#pragma unroll
                for (int o = 1; o < L4; o <<= 1)
                    x += __shfl_xor(x, o);
                if (q == i0 + u)
                    out[c] = x;
            }
        }
    }
}

template <typename TP, bool AF3, int D>
__global__ __launch_bounds__(256) void k_slot_fwd(SK p) {
    extern __shared__ float smem[];
    const SlotBwdArgs &a = p.a;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int K = a.K, H = a.H, HD = H * D;
    float *base = smem + w * wave_floats(K, H, HD);
    int *skid = reinterpret_cast<int *>(base);
    float *sbeta = base + K;
    float *sP = sbeta + K * H;
    float *sq = sP + K;
    const int64_t N = (int64_t)a.B * a.A;
    // neighbouring queries (which share key rows) on one XCD
    int64_t n = (int64_t)xcd_remap((int)blockIdx.x, (int)gridDim.x) * 4 + w;
    bool live = n < N;
    if (a.wide) {
        // queue mode: four workgroups per queued 16-query block
        const int qi = (int)blockIdx.x >> 2;
        if (qi >= a.wide[0])
            return;
        const int blk = a.wide[1 + qi], nqb = (a.A + 15) / 16;
        const int qa0 = (blk % nqb) * 16 + ((int)blockIdx.x & 3) * 4 + w;
        live = qa0 < a.A;
        n = (int64_t)(blk / nqb) * a.A + qa0;
    }
    const int64_t nn = live ? n : 0;
    const int64_t b = nn / a.A, qa = nn - b * a.A;
    const bool qu = live && a.usable[nn];

    for (int s = lane; s < K; s += 64) {
        const int64_t e = nn * K + s;
        const int64_t j = a.key_index[e];
        bool ok = qu && j >= 0 && j < a.A && a.window_mask[e];
        if (ok)
            ok = a.usable[b * a.A + j] && (a.radius < 0 || (j > qa ? j - qa : qa - j) <= a.radius);
        const int id = ok ? (int)(b * a.A + j) : -1;
        skid[s] = id;
        if (live)
            a.kid[e] = id;
    }
    if constexpr (AF3) {
        // pair bias (LN(pair row) * pair_scale) @ w_pair: four lanes per
        // slot, lane quarter qv holding channels 4 qv .. 4 qv + 3 (16
        // slots per pass, whole rows per load); lane qv writes head qv
        const int V = a.V, qv = lane & 3, sg4 = lane >> 2;
        float wv[4][kPairH];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = 4 * qv + i;
            const float ps = v < V ? a.ps[v] : 0.0f;
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                wv[i][h] = (v < V && h < H) ? ps * a.wp[v * H + h] : 0.0f;
        }
        for (int s0 = 0; s0 < K; s0 += 16) {
            const int s = s0 + sg4;
            const bool in = s < K;
            const bool ok = in && skid[s] >= 0;
            float x[4];
            load_pair_piece(reinterpret_cast<const TP *>(a.pair), nn * K + (in ? s : 0), V, qv, x);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x[i] = ok ? x[i] : 0.0f; // rows of slots not allowed may hold junk
            pair_ln4(x, V, qv, a.eps);
            float bh[kPairH];
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                bh[h] = sum4(x[0] * wv[0][h] + x[1] * wv[1][h] + x[2] * wv[2][h] + x[3] * wv[3][h]);
            float mine = bh[0];
#pragma unroll
            for (int h = 1; h < kPairH; ++h)
                mine = qv == h ? bh[h] : mine;
            if (in && qv < H)
                sbeta[s * H + qv] = ok ? mine : 0.0f;
        }
    }
    for (int i = lane; i < HD; i += 64)
        sq[i] = a.q[nn * HD + i];
    __syncthreads();

    const int sl = slot_of_lane<D>(lane);
    for (int h = 0; h < H; ++h) {
        float l[kMaxK / 64];
        group_dots<D, kMaxK / 64>(sq + h * D, skid, K, a.k, HD, h * D, lane, l);
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < kMaxK / 64; ++c) {
            const int s = sl + 64 * c;
            if (s < K && skid[s] >= 0) {
                l[c] = l[c] * p.inv_sqrt_d + (AF3 ? sbeta[s * H + h] : 0.0f);
                mx = fmaxf(mx, l[c]);
            } else {
                l[c] = -INFINITY;
            }
        }
        mx = group_max<64>(mx);
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxK / 64; ++c) {
            const int s = sl + 64 * c;
            if (s < K && skid[s] >= 0) {
                l[c] = expf(l[c] - mx);
                sum += l[c];
            }
        }
        sum = group_sum<64>(sum);
        const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxK / 64; ++c) {
            const int s = sl + 64 * c;
            if (s < K) {
                const float pw = skid[s] >= 0 ? l[c] * inv : 0.0f;
                sP[s] = pw;
                if (live)
                    a.P[((b * H + h) * a.A + qa) * K + s] = pw;
            }
        }
        __syncthreads();
        const float4 acc = slot_rowsum<D>(sP, skid, K, a.v, HD, h * D, lane);
        if (live && lane < D / 4)
            *reinterpret_cast<float4 *>(a.o + nn * HD + h * D + lane * 4) = acc;
        __syncthreads();
    }
}

template <typename TP, bool AF3, int D>
__global__ __launch_bounds__(256) void k_slot_bwd_q(SK p) {
    extern __shared__ float smem[];
    __shared__ float wred[4][kPairV + kPairV * kPairH];
    const SlotBwdArgs &a = p.a;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int K = a.K, H = a.H, HD = H * D;
    float *base = smem + w * wave_floats(K, H, HD);
    int *skid = reinterpret_cast<int *>(base);
    float *sdl = base + K;
    float *sP = sdl + K * H;
    float *sdo = sP + K;
    float *spa = sdo + HD;
    const int64_t N = (int64_t)a.B * a.A;
    // neighbouring queries (which share key rows) on one XCD
    int64_t n = (int64_t)xcd_remap((int)blockIdx.x, (int)gridDim.x) * 4 + w;
    bool live = n < N;
    // pair-parameter partial record: by workgroup, or in queue mode by the
    // queued block's id (fixed places whatever the queue order; the block
    // kernel zeroes the four records of every block it completes)
    int rec = a.rec0 + (int)blockIdx.x;
    if (a.wide) {
        // queue mode: four workgroups per queued 16-query block
        const int qi = (int)blockIdx.x >> 2;
        if (qi >= a.wide[0])
            return;
        const int blk = a.wide[1 + qi], nqb = (a.A + 15) / 16;
        rec = a.rec0 + blk * 4 + ((int)blockIdx.x & 3);
        const int qa0 = (blk % nqb) * 16 + ((int)blockIdx.x & 3) * 4 + w;
        live = qa0 < a.A;
        n = (int64_t)(blk / nqb) * a.A + qa0;
    }
    const int64_t nn = live ? n : 0;
    const int64_t b = nn / a.A, qa = nn - b * a.A;

    for (int s = lane; s < K; s += 64)
        skid[s] = live ? a.kid[nn * K + s] : -1;
    for (int i = lane; i < HD; i += 64)
        sdo[i] = a.d_o[nn * HD + i];
    __syncthreads();

    const int sl = slot_of_lane<D>(lane);
    for (int h = 0; h < H; ++h) {
        const int64_t rowbase = ((b * H + h) * a.A + qa) * K;
        float pw[kMaxK / 64], dw[kMaxK / 64], vd[kMaxK / 64];
        group_dots<D, kMaxK / 64>(sdo + h * D, skid, K, a.v, HD, h * D, lane, vd);
        float dsum = 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxK / 64; ++c) {
            const int s = sl + 64 * c;
            pw[c] = 0.0f;
            dw[c] = 0.0f;
            if (s < K && skid[s] >= 0) {
                pw[c] = a.P[rowbase + s];
                spa[s * H + h] = pw[c];
                const float x = (a.d_att ? a.d_att[rowbase + s] : 0.0f) + vd[c];
                dw[c] = x;
                dsum += pw[c] * x;
            }
        }
        dsum = group_sum<64>(dsum);
#pragma unroll
        for (int c = 0; c < kMaxK / 64; ++c) {
            const int s = sl + 64 * c;
            if (s < K) {
                const float dl = pw[c] * (dw[c] - dsum);
                sP[s] = dl;
                sdl[s * H + h] = dl;
            }
        }
        __syncthreads();
        float4 acc = slot_rowsum<D>(sP, skid, K, a.k, HD, h * D, lane);
        if (live && lane < D / 4) {
            acc.x *= p.inv_sqrt_d;
            acc.y *= p.inv_sqrt_d;
            acc.z *= p.inv_sqrt_d;
            acc.w *= p.inv_sqrt_d;
            *reinterpret_cast<float4 *>(a.dq + nn * HD + h * D + lane * 4) = acc;
        }
        __syncthreads();
    }

    // every head's dS and P of an allowed slot go to the slot's place in the
    // reverse index (key-major), H values together
    for (int s = lane; s < K; s += 64) {
        const int pos = (live && skid[s] >= 0) ? a.inv[nn * K + s] : -1;
        if (pos < 0)
            continue;
        float *dd = a.dS + (int64_t)pos * H;
        float *pp = a.Pk + (int64_t)pos * H;
        if (H % 4 == 0) { // 16-byte global stores (LDS read element-wise: K may be odd)
            for (int h = 0; h < H; h += 4) {
                const float *x = sdl + s * H + h, *y = spa + s * H + h;
                *reinterpret_cast<float4 *>(dd + h) = make_float4(x[0], x[1], x[2], x[3]);
                *reinterpret_cast<float4 *>(pp + h) = make_float4(y[0], y[1], y[2], y[3]);
            }
        } else {
            for (int h = 0; h < H; ++h) {
                dd[h] = sdl[s * H + h];
                pp[h] = spa[s * H + h];
            }
        }
    }

    if constexpr (AF3) {
        // pair bias beta_h = sum_v xhat_v ps_v wp[v][h]: its gradient dS
        // flows to the pair row, pair_scale and w_pair. Four lanes per slot,
        // lane quarter qv holding channels 4 qv .. 4 qv + 3 (16 slots per
        // pass, whole rows per load and store).
        const int V = a.V, qv = lane & 3, sg4 = lane >> 2;
        float psv[4], wpv[4][kPairH];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = 4 * qv + i;
            psv[i] = v < V ? a.ps[v] : 0.0f;
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                wpv[i][h] = (v < V && h < H) ? a.wp[v * H + h] : 0.0f;
        }
        float gps[4], gwp[4][kPairH];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gps[i] = 0.0f;
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                gwp[i][h] = 0.0f;
        }
        for (int s0 = 0; s0 < K; s0 += 16) {
            const int s = s0 + sg4;
            const bool in = s < K;
            const bool ok = in && skid[s] >= 0;
            const int64_t e = nn * K + (in ? s : 0);
            float x[4];
            load_pair_piece(reinterpret_cast<const TP *>(a.pair), e, V, qv, x);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x[i] = ok ? x[i] : 0.0f; // rows of slots not allowed may hold junk
            const float r = pair_ln4(x, V, qv, a.eps);
            float db[kPairH];
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                db[h] = (ok && h < H) ? sdl[s * H + h] : 0.0f;
            float y[4];
            float my = 0.0f, myx = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float dpn = 0.0f;
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    dpn += db[h] * wpv[i][h];
                gps[i] += dpn * x[i];
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    gwp[i][h] += x[i] * psv[i] * db[h];
                y[i] = dpn * psv[i];
                my += y[i];
                myx += y[i] * x[i];
            }
            my = sum4(my) / (float)V;
            myx = sum4(myx) / (float)V;
            if (a.d_pair && live && in) {
                float dp[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dp[i] = ok ? r * (y[i] - my - x[i] * myx) : 0.0f;
                float *dst = a.d_pair + e * V + 4 * qv;
                if (V % 4 == 0) {
                    if (4 * qv < V)
                        *reinterpret_cast<float4 *>(dst) = make_float4(dp[0], dp[1], dp[2], dp[3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * qv + i < V)
                            dst[i] = dp[i];
                }
            }
        }
        // sums over the wave's 16 slot groups (lanes of one channel quarter)
#pragma unroll
        for (int o = 4; o < 64; o <<= 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gps[i] += __shfl_xor(gps[i], o);
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    gwp[i][h] += __shfl_xor(gwp[i][h], o);
            }
        }
        if (lane < 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = 4 * lane + i;
                wred[w][v] = gps[i];
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    wred[w][kPairV + v * kPairH + h] = gwp[i][h];
            }
        }
        // then the workgroup's four waves in order
        __syncthreads();
        constexpr int W = kPairV + kPairV * kPairH;
        for (int i = threadIdx.x; i < W; i += 256)
            a.pw_partial[(int64_t)rec * W + i] =
                ((wred[0][i] + wred[1][i]) + wred[2][i]) + wred[3][i];
    }
}

// ---------------------------------------------------------------------
// Block form of the query side (K <= 128, H <= 4, D >= 16): one workgroup
// per block of 16 consecutive query atoms whose allowed key ids lie in a
// band of at most kBandRows rows. The two products over the band run on
// the matrix cores with each band row read once per block instead of once
// per slot: G = dO_block . V_band^T (per head a 16 x band tile in LDS,
// read by each slot at its key), then dS per slot (16 threads per query,
// slot jq + 16 i), scattered by key into the tile (repeated keys add), and
// dQ = dS_tile . K_band. Blocks with a wider band go to a queue that the
// per-query kernel takes.
constexpr int kBandRows = 128, kBandPitch = kBandRows + 4;
constexpr int kBlockMinBlocks = 768; // grids from which the block form is used

// (at fewer blocks than about three per CU the per-query kernels' finer
// grid is faster: config 1, 288 blocks, query side 74 against 107 us)
inline bool block_form(const SlotBwdArgs &a, int nblocks) {
    return a.K <= 128 && a.H <= kPairH && a.D >= 16 && a.wide && nblocks >= kBlockMinBlocks;
}

__host__ __device__ inline int block_lds_floats() { return kPairH * 16 * kBandPitch; }

template <typename TP, bool AF3, int D>
__global__ __launch_bounds__(256) void k_slot_bwd_qb(SK p) {
    extern __shared__ __align__(16) float smem[];
    __shared__ int s_lo, s_hi;
    __shared__ float wred[4][kPairV + kPairV * kPairH];
    constexpr int SPL = 8, NKC = D / 16, W = kPairV + kPairV * kPairH;
    const SlotBwdArgs &a = p.a;
    const int K = a.K, H = a.H, HD = H * D, A = a.A;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q = tid >> 4, jq = tid & 15;    // query of the block, its thread
    const int l16 = lane & 15, g4 = lane >> 4; // matrix-core lane coordinates
    const int nqb = (A + 15) / 16;
    // neighbouring blocks (overlapping key bands) on one XCD
    const int wg = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int b = wg / nqb, a0 = (wg - b * nqb) * 16;
    const int64_t bA = (int64_t)b * A;
    const bool live = a0 + q < A;
    const int64_t n = bA + a0 + (live ? q : 0);
    float *tile = smem; // [head][16][kBandPitch]

    // allowed key ids of this thread's slots, relative to the batch
    int rel[SPL];
    int lo = INT_MAX, hi = -1;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int sl = jq + 16 * i;
        rel[i] = -1;
        if (live && sl < K) {
            const int id = a.kid[n * K + sl];
            rel[i] = id >= 0 ? (int)(id - bA) : -1;
        }
        if (rel[i] >= 0) {
            lo = min(lo, rel[i]);
            hi = max(hi, rel[i]);
        }
    }
    if (tid == 0) {
        s_lo = INT_MAX;
        s_hi = -1;
    }
    __syncthreads();
    lo = wave_min_i(lo);
    hi = wave_max_i(hi);
    if (lane == 0) {
        atomicMin(&s_lo, lo);
        atomicMax(&s_hi, hi);
    }
    __syncthreads();
    const int bhi = s_hi, blo = bhi >= 0 ? s_lo : 0;
    const bool any = bhi >= 0;
    const int rows = any ? bhi + 1 - blo : 0;
    if (rows > kBandRows) {
        // scattered ids: the per-query kernel takes this block
        if (tid == 0)
            a.wide[1 + atomicAdd(a.wide, 1)] = wg;
        if constexpr (AF3)
            for (int i = tid; i < W; i += 256)
                a.pw_partial[(int64_t)wg * W + i] = 0.0f;
        return;
    }
    const int ncb = (rows + 15) / 16;
    const int hw = w; // this wave's head in the two products
    const bool hv = hw < H && any;

    // ---- G = dO . V_band^T: query l16, band row 16 cb + l16
    if (hv) {
        uint4 af[NKC];
        const bool qin = a0 + l16 < A;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            af[kc] = make_uint4(0, 0, 0, 0);
            if (qin)
                af[kc] = *reinterpret_cast<const uint4 *>(a.d_o + (bA + a0 + l16) * HD + hw * D + kc * 16 + g4 * 4);
        }
        for (int cb0 = 0; cb0 < ncb; cb0 += 4) {
            uint4 vb[4][NKC];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = (cb0 + t) * 16 + l16;
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    vb[t][kc] = make_uint4(0, 0, 0, 0);
                    if (r < rows)
                        vb[t][kc] = *reinterpret_cast<const uint4 *>(a.v + (bA + blo + r) * HD + hw * D + kc * 16 + g4 * 4);
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (cb0 + t >= ncb)
                    break;
                f32x4_t acc = zero4();
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
                    Mma16<float>::mma(acc, af[kc], vb[t][kc]);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    tile[(hw * 16 + acc16_row(v, lane)) * kBandPitch + (cb0 + t) * 16 + acc16_col(lane)] = acc[v];
            }
        }
    }
    __syncthreads();

    // ---- dS per slot and head: dW = dA + G[key], dS = P (dW - sum P dW)
    float dsv[SPL][kPairH], pv[SPL][kPairH];
#pragma unroll
    for (int h = 0; h < kPairH; ++h) {
        float dsum = 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            dsv[i][h] = 0.0f;
            pv[i][h] = 0.0f;
            if (h < H && rel[i] >= 0) {
                const int64_t at = (((int64_t)b * H + h) * A + a0 + q) * K + jq + 16 * i;
                const float P = a.P[at];
                const float x = (a.d_att ? a.d_att[at] : 0.0f) + tile[(h * 16 + q) * kBandPitch + rel[i] - blo];
                pv[i][h] = P;
                dsv[i][h] = x;
                dsum += P * x;
            }
        }
        dsum = sum16(dsum);
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            dsv[i][h] = pv[i][h] * (dsv[i][h] - dsum);
    }
    __syncthreads(); // G read
    for (int i = tid; i < block_lds_floats() / 4; i += 256)
        reinterpret_cast<float4 *>(tile)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
    // dS into the tile by key (a query's repeated keys add, in slot order)
#pragma unroll
    for (int h = 0; h < kPairH; ++h)
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (h < H && rel[i] >= 0)
                atomicAdd(&tile[(h * 16 + q) * kBandPitch + rel[i] - blo], dsv[i][h]);
    __syncthreads();

    // ---- dQ = dS_tile . K_band / sqrt(D): query l16, channel 16 db + l16
    if (hw < H) {
        f32x4_t acc[NKC];
#pragma unroll
        for (int db = 0; db < NKC; ++db)
            acc[db] = zero4();
        for (int kc = 0; kc < ncb; ++kc) {
            const uint4 av = *reinterpret_cast<const uint4 *>(tile + (hw * 16 + l16) * kBandPitch + kc * 16 + g4 * 4);
            float kv[NKC][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = kc * 16 + g4 * 4 + t;
#pragma unroll
                for (int db = 0; db < NKC; ++db)
                    kv[db][t] = r < rows ? a.k[(bA + blo + r) * HD + hw * D + db * 16 + l16] : 0.0f;
            }
#pragma unroll
            for (int db = 0; db < NKC; ++db)
                Mma16<float>::mma(acc[db], av, make_uint4(__float_as_uint(kv[db][0]), __float_as_uint(kv[db][1]),
                                                          __float_as_uint(kv[db][2]), __float_as_uint(kv[db][3])));
        }
#pragma unroll
        for (int db = 0; db < NKC; ++db)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = acc16_row(v, lane);
                if (a0 + r < A)
                    a.dq[(bA + a0 + r) * HD + hw * D + db * 16 + acc16_col(lane)] = acc[db][v] * p.inv_sqrt_d;
            }
    }

    // ---- every head's dS and P of an allowed slot at its place in the
    // reverse index (key-major)
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        if (rel[i] < 0)
            continue;
        const int pos = a.inv[n * K + jq + 16 * i];
        float *dd = a.dS + (int64_t)pos * H;
        float *pp = a.Pk + (int64_t)pos * H;
        if (H == 4) {
            *reinterpret_cast<float4 *>(dd) = make_float4(dsv[i][0], dsv[i][1], dsv[i][2], dsv[i][3]);
            *reinterpret_cast<float4 *>(pp) = make_float4(pv[i][0], pv[i][1], pv[i][2], pv[i][3]);
        } else {
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                if (h < H) {
                    dd[h] = dsv[i][h];
                    pp[h] = pv[i][h];
                }
        }
    }

    if constexpr (AF3) {
        // pair-bias gradients as in the per-query kernel, over the block's
        // 16 K slots: four lanes per slot (channel quarter qv), 64 slots per
        // pass; the slots' dS from LDS
        __syncthreads(); // dQ read the tile
        float *sdl = smem; // [16][K][H]
#pragma unroll
        for (int h = 0; h < kPairH; ++h)
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const int sl = jq + 16 * i;
                if (h < H && sl < K)
                    sdl[(q * K + sl) * H + h] = dsv[i][h];
            }
        __syncthreads();
        const int V = a.V, qv = lane & 3, sg4 = tid >> 2;
        float psv[4], wpv[4][kPairH];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = 4 * qv + i;
            psv[i] = v < V ? a.ps[v] : 0.0f;
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                wpv[i][h] = (v < V && h < H) ? a.wp[v * H + h] : 0.0f;
        }
        float gps[4], gwp[4][kPairH];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gps[i] = 0.0f;
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                gwp[i][h] = 0.0f;
        }
        for (int e0 = 0; e0 < 16 * K; e0 += 64) {
            const int idx = e0 + sg4;
            const int qq = idx / K, sl = idx - qq * K;
            const bool in = idx < 16 * K && a0 + qq < A;
            const int64_t e = (bA + a0 + (in ? qq : 0)) * K + (in ? sl : 0);
            const bool ok = in && a.kid[e] >= 0;
            float x[4];
            load_pair_piece(reinterpret_cast<const TP *>(a.pair), e, V, qv, x);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x[i] = ok ? x[i] : 0.0f; // rows of slots not allowed may hold junk
            const float r = pair_ln4(x, V, qv, a.eps);
            float db[kPairH];
#pragma unroll
            for (int h = 0; h < kPairH; ++h)
                db[h] = (ok && h < H) ? sdl[(qq * K + sl) * H + h] : 0.0f;
            float y[4];
            float my = 0.0f, myx = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float dpn = 0.0f;
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    dpn += db[h] * wpv[i][h];
                gps[i] += dpn * x[i];
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    gwp[i][h] += x[i] * psv[i] * db[h];
                y[i] = dpn * psv[i];
                my += y[i];
                myx += y[i] * x[i];
            }
            my = sum4(my) / (float)V;
            myx = sum4(myx) / (float)V;
            if (a.d_pair && in) {
                float dp[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dp[i] = ok ? r * (y[i] - my - x[i] * myx) : 0.0f;
                float *dst = a.d_pair + e * V + 4 * qv;
                if (V % 4 == 0) {
                    if (4 * qv < V)
                        *reinterpret_cast<float4 *>(dst) = make_float4(dp[0], dp[1], dp[2], dp[3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * qv + i < V)
                            dst[i] = dp[i];
                }
            }
        }
#pragma unroll
        for (int o = 4; o < 64; o <<= 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gps[i] += __shfl_xor(gps[i], o);
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    gwp[i][h] += __shfl_xor(gwp[i][h], o);
            }
        }
        if (lane < 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = 4 * lane + i;
                wred[w][v] = gps[i];
#pragma unroll
                for (int h = 0; h < kPairH; ++h)
                    wred[w][kPairV + v * kPairH + h] = gwp[i][h];
            }
        }
        __syncthreads();
        for (int i = tid; i < W; i += 256)
            a.pw_partial[(int64_t)wg * W + i] = ((wred[0][i] + wred[1][i]) + wred[2][i]) + wred[3][i];
        // this block's four records of the queue-mode kernel stay zero
        const int nblocks = a.B * nqb;
        for (int i = tid; i < 4 * W; i += 256)
            a.pw_partial[((int64_t)nblocks + 4 * wg) * W + i] = 0.0f;
    }
}

// Block form of the forward step (same conditions as the query side's):
// per 16-query block, S = Q . K_band^T on the matrix cores into a per-head
// tile, each thread's slots take their logits from it (plus the AF3 pair
// bias of the slot's row), the masked softmax runs over the query's 16
// threads, and o = P_tile . V_band, with P scattered by key (repeated keys
// add). Blocks with a wide key band are queued for the per-query kernel.
template <typename TP, bool AF3, int D>
__global__ __launch_bounds__(256) void k_slot_fwd_b(SK p) {
    extern __shared__ __align__(16) float smem[];
    __shared__ int s_lo, s_hi;
    __shared__ float sw[kPairV * kPairH]; // pair_scale[v] * w_pair[v][h]
    constexpr int SPL = 8, NKC = D / 16;
    const SlotBwdArgs &a = p.a;
    const int K = a.K, H = a.H, HD = H * D, A = a.A;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q = tid >> 4, jq = tid & 15;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nqb = (A + 15) / 16;
    // neighbouring blocks (overlapping key bands) on one XCD
    const int wg = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int b = wg / nqb, a0 = (wg - b * nqb) * 16;
    const int64_t bA = (int64_t)b * A;
    const bool live = a0 + q < A;
    const int64_t n = bA + a0 + (live ? q : 0);
    const bool qu = live && a.usable[n];
    float *tile = smem; // [head][16][kBandPitch]

    int rel[SPL];
    int lo = INT_MAX, hi = -1;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int sl = jq + 16 * i;
        rel[i] = -1;
        if (live && sl < K) {
            const int64_t e = n * K + sl;
            const int64_t j = a.key_index[e];
            bool ok = qu && j >= 0 && j < A && a.window_mask[e];
            if (ok) {
                const int64_t dq = j > a0 + q ? j - (a0 + q) : (a0 + q) - j;
                ok = a.usable[bA + j] && (a.radius < 0 || dq <= a.radius);
            }
            rel[i] = ok ? (int)j : -1;
            a.kid[e] = ok ? (int)(bA + j) : -1;
        }
        if (rel[i] >= 0) {
            lo = min(lo, rel[i]);
            hi = max(hi, rel[i]);
        }
    }
    if (tid == 0) {
        s_lo = INT_MAX;
        s_hi = -1;
    }
    if (AF3 && tid < kPairV * kPairH) {
        const int v = tid / kPairH, h = tid - v * kPairH;
        sw[tid] = (v < a.V && h < H) ? a.ps[v] * a.wp[v * H + h] : 0.0f;
    }
    __syncthreads();
    lo = wave_min_i(lo);
    hi = wave_max_i(hi);
    if (lane == 0) {
        atomicMin(&s_lo, lo);
        atomicMax(&s_hi, hi);
    }
    __syncthreads();
    const int bhi = s_hi, blo = bhi >= 0 ? s_lo : 0;
    const bool any = bhi >= 0;
    const int rows = any ? bhi + 1 - blo : 0;
    if (rows > kBandRows) {
        if (tid == 0)
            a.wide[1 + atomicAdd(a.wide, 1)] = wg;
        return;
    }
    const int ncb = (rows + 15) / 16;
    const int hw = w;

    // pair bias of the thread's slots (whole rows, 16-byte pieces)
    float lg[SPL][kPairH]; // the bias, then the logit, then the weight
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
        for (int h = 0; h < kPairH; ++h)
            lg[i][h] = 0.0f;
    if constexpr (AF3) {
        const int V = a.V;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            if (rel[i] < 0)
                continue;
            const int64_t e = n * K + jq + 16 * i;
            float x[kPairV];
#pragma unroll
            for (int qv = 0; qv < kPairV / 4; ++qv) {
                float x4[4];
                load_pair_piece(reinterpret_cast<const TP *>(a.pair), e, V, qv, x4);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    x[4 * qv + t] = x4[t];
            }
            float m = 0.0f;
#pragma unroll
            for (int v = 0; v < kPairV; ++v)
                m += x[v];
            m /= (float)V;
            float var = 0.0f;
#pragma unroll
            for (int v = 0; v < kPairV; ++v) {
                const float d = v < V ? x[v] - m : 0.0f;
                x[v] = d;
                var += d * d;
            }
            const float r = 1.0f / sqrtf(var / (float)V + a.eps);
#pragma unroll
            for (int h = 0; h < kPairH; ++h) {
                float acc = 0.0f;
#pragma unroll
                for (int v = 0; v < kPairV; ++v)
                    acc += x[v] * sw[v * kPairH + h];
                lg[i][h] = acc * r;
            }
        }
    }

    // ---- S = Q . K_band^T: query l16, band row 16 cb + l16
    if (hw < H && any) {
        uint4 af[NKC];
        const bool qin = a0 + l16 < A;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            af[kc] = make_uint4(0, 0, 0, 0);
            if (qin)
                af[kc] = *reinterpret_cast<const uint4 *>(a.q + (bA + a0 + l16) * HD + hw * D + kc * 16 + g4 * 4);
        }
        for (int cb0 = 0; cb0 < ncb; cb0 += 4) {
            uint4 kb[4][NKC];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = (cb0 + t) * 16 + l16;
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    kb[t][kc] = make_uint4(0, 0, 0, 0);
                    if (r < rows)
                        kb[t][kc] = *reinterpret_cast<const uint4 *>(a.k + (bA + blo + r) * HD + hw * D + kc * 16 + g4 * 4);
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (cb0 + t >= ncb)
                    break;
                f32x4_t acc = zero4();
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
                    Mma16<float>::mma(acc, af[kc], kb[t][kc]);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    tile[(hw * 16 + acc16_row(v, lane)) * kBandPitch + (cb0 + t) * 16 + acc16_col(lane)] = acc[v];
            }
        }
    }
    __syncthreads();

    // ---- masked softmax over the query's allowed slots
#pragma unroll
    for (int h = 0; h < kPairH; ++h) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            if (h < H && rel[i] >= 0) {
                lg[i][h] += tile[(h * 16 + q) * kBandPitch + rel[i] - blo] * p.inv_sqrt_d;
                mx = fmaxf(mx, lg[i][h]);
            }
        }
        mx = max16(mx);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            lg[i][h] = (h < H && rel[i] >= 0) ? expf(lg[i][h] - mx) : 0.0f;
            sum += lg[i][h];
        }
        sum = sum16(sum);
        const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            lg[i][h] *= inv;
            const int sl = jq + 16 * i;
            if (h < H && live && sl < K)
                a.P[(((int64_t)b * H + h) * A + a0 + q) * K + sl] = lg[i][h];
        }
    }
    __syncthreads(); // S read
    for (int i = tid; i < block_lds_floats() / 4; i += 256)
        reinterpret_cast<float4 *>(tile)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kPairH; ++h)
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (h < H && rel[i] >= 0)
                atomicAdd(&tile[(h * 16 + q) * kBandPitch + rel[i] - blo], lg[i][h]);
    __syncthreads();

    // ---- o = P_tile . V_band: query l16, channel 16 db + l16
    if (hw < H) {
        f32x4_t acc[NKC];
#pragma unroll
        for (int db = 0; db < NKC; ++db)
            acc[db] = zero4();
        for (int kc = 0; kc < ncb; ++kc) {
            const uint4 av = *reinterpret_cast<const uint4 *>(tile + (hw * 16 + l16) * kBandPitch + kc * 16 + g4 * 4);
            float vv[NKC][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = kc * 16 + g4 * 4 + t;
#pragma unroll
                for (int db = 0; db < NKC; ++db)
                    vv[db][t] = r < rows ? a.v[(bA + blo + r) * HD + hw * D + db * 16 + l16] : 0.0f;
            }
#pragma unroll
            for (int db = 0; db < NKC; ++db)
                Mma16<float>::mma(acc[db], av, make_uint4(__float_as_uint(vv[db][0]), __float_as_uint(vv[db][1]),
                                                          __float_as_uint(vv[db][2]), __float_as_uint(vv[db][3])));
        }
#pragma unroll
        for (int db = 0; db < NKC; ++db)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = acc16_row(v, lane);
                if (a0 + r < A)
                    a.o[(bA + a0 + r) * HD + hw * D + db * 16 + acc16_col(lane)] = acc[db][v];
            }
    }
}

// One wave per key atom, over its list of (query, slot) entries in order.
// A lane holds one float4 of the H*D channels (all in one head); the wave
// takes EPP = 64 / (HD/4) entries per pass (one per lane group) and four
// passes' loads are issued before they are used. The groups' sums are
// added in group order at the end.
__global__ __launch_bounds__(256) void k_slot_bwd_kv(SK p) {
    const SlotBwdArgs &a = p.a;
    const int lane = threadIdx.x & 63;
    const int64_t N = (int64_t)a.B * a.A;
    // neighbouring keys (selected by the same queries) on one XCD
    const int64_t j = (int64_t)xcd_remap((int)blockIdx.x, (int)gridDim.x) * 4 + (threadIdx.x >> 6);
    if (j >= N)
        return;
    const int K = a.K, H = a.H, D = a.D, HD = H * D;
    const int LPE = HD / 4, EPP = 64 / LPE;
    const int g = lane / LPE, q = lane - g * LPE;
    const bool act = g < EPP;
    const int h = (q * 4) / D;
    float4 ak = make_float4(0.0f, 0.0f, 0.0f, 0.0f), av = ak;
    const int beg = a.offset[j], end = a.offset[j + 1];
    for (int base = beg; base < end; base += 64) {
        const int cnt = min(64, end - base);
        const int le = lane < cnt ? a.list[base + lane] : 0;
        for (int u0 = 0; u0 < cnt; u0 += 4 * EPP) {
            float4 rq[4], ro[4];
            float ws[4], wp[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int idx = u0 + u * EPP + g;
                const int64_t e = __shfl(le, idx < 64 ? idx : 0);
                ws[u] = wp[u] = 0.0f;
                rq[u] = ro[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (act && idx < cnt) {
                    const int64_t n = e / K;
                    const int64_t at = (int64_t)(base + idx) * H + h; // key-major
                    ws[u] = a.dS[at];
                    wp[u] = a.Pk[at];
                    rq[u] = *reinterpret_cast<const float4 *>(a.q + n * HD + q * 4);
                    ro[u] = *reinterpret_cast<const float4 *>(a.d_o + n * HD + q * 4);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ak.x += ws[u] * rq[u].x; ak.y += ws[u] * rq[u].y;
                ak.z += ws[u] * rq[u].z; ak.w += ws[u] * rq[u].w;
                av.x += wp[u] * ro[u].x; av.y += wp[u] * ro[u].y;
                av.z += wp[u] * ro[u].z; av.w += wp[u] * ro[u].w;
            }
        }
    }
    // groups' sums in group order, into the lanes of group 0
    float4 tk = make_float4(0.0f, 0.0f, 0.0f, 0.0f), tv = tk;
    for (int gg = 0; gg < EPP; ++gg) {
        const int src = gg * LPE + q;
        tk.x += __shfl(ak.x, src); tk.y += __shfl(ak.y, src);
        tk.z += __shfl(ak.z, src); tk.w += __shfl(ak.w, src);
        tv.x += __shfl(av.x, src); tv.y += __shfl(av.y, src);
        tv.z += __shfl(av.z, src); tv.w += __shfl(av.w, src);
    }
    if (g == 0) {
        tk.x *= p.inv_sqrt_d; tk.y *= p.inv_sqrt_d; tk.z *= p.inv_sqrt_d; tk.w *= p.inv_sqrt_d;
        *reinterpret_cast<float4 *>(a.dk + j * HD + q * 4) = tk;
        *reinterpret_cast<float4 *>(a.dv + j * HD + q * 4) = tv;
    }
}

inline unsigned nblk(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

template <typename Fn> void set_lds(Fn fn, size_t bytes) {
    allow_lds(reinterpret_cast<const void *>(fn), bytes);
}

} // namespace

int slot_bwd_supported(int K, int H, int D, int V, int style) {
    if (K < 1 || K > kMaxK || H < 1 || H > kMaxH)
        return 0;
    if (D != 8 && D != 16 && D != 32 && D != 64)
        return 0;
    if (H * D > kMaxHD)
        return 0;
    if (style == STYLE_AF3 && (V < 1 || V > kPairV || H > kPairH))
        return 0;
    return 1;
}

int slot_bwd_records(const SlotBwdArgs &a) {
    const int nblocks = a.B * ((a.A + 15) / 16);
    return block_form(a, nblocks) ? 5 * nblocks : (int)nblk((int64_t)a.B * a.A, 4);
}

size_t slot_bwd_partial_floats(int64_t B, int64_t A, int V, int H) {
    (void)V;
    (void)H;
    // the per-query kernel over every query (one record per 4 queries), or
    // the block kernel (one per 16-query block) followed by the per-query
    // kernel in queue mode (four per block)
    const int64_t blocks = B * ((A + 15) / 16);
    return (size_t)std::max<int64_t>(nblk(B * A, 4), 5 * blocks) * (kPairV + kPairV * kPairH) + 256;
}

int64_t slot_bwd_queue_ints(int64_t B, int64_t A) { return 1 + B * ((A + 15) / 16); }

template <int D>
void launch_fwd(const SK &p, int style, size_t lds, dim3 grid, hipStream_t s) {
    if (style == STYLE_AF3) {
        if (p.a.pair_dtype == 1) {
            set_lds(k_slot_fwd<bf16_t, true, D>, lds);
            hipLaunchKernelGGL((k_slot_fwd<bf16_t, true, D>), grid, dim3(256), lds, s, p);
        } else {
            set_lds(k_slot_fwd<float, true, D>, lds);
            hipLaunchKernelGGL((k_slot_fwd<float, true, D>), grid, dim3(256), lds, s, p);
        }
    } else {
        set_lds(k_slot_fwd<float, false, D>, lds);
        hipLaunchKernelGGL((k_slot_fwd<float, false, D>), grid, dim3(256), lds, s, p);
    }
}

template <int D>
void launch_fwd_b(const SK &p, int style, size_t lds, dim3 grid, hipStream_t s) {
    if (style == STYLE_AF3) {
        if (p.a.pair_dtype == 1) {
            set_lds(k_slot_fwd_b<bf16_t, true, D>, lds);
            hipLaunchKernelGGL((k_slot_fwd_b<bf16_t, true, D>), grid, dim3(256), lds, s, p);
        } else {
            set_lds(k_slot_fwd_b<float, true, D>, lds);
            hipLaunchKernelGGL((k_slot_fwd_b<float, true, D>), grid, dim3(256), lds, s, p);
        }
    } else {
        set_lds(k_slot_fwd_b<float, false, D>, lds);
        hipLaunchKernelGGL((k_slot_fwd_b<float, false, D>), grid, dim3(256), lds, s, p);
    }
}

template <int D>
void launch_bwd_qb(const SK &p, int style, size_t lds, dim3 grid, hipStream_t s) {
    if (style == STYLE_AF3) {
        if (p.a.pair_dtype == 1) {
            set_lds(k_slot_bwd_qb<bf16_t, true, D>, lds);
            hipLaunchKernelGGL((k_slot_bwd_qb<bf16_t, true, D>), grid, dim3(256), lds, s, p);
        } else {
            set_lds(k_slot_bwd_qb<float, true, D>, lds);
            hipLaunchKernelGGL((k_slot_bwd_qb<float, true, D>), grid, dim3(256), lds, s, p);
        }
    } else {
        set_lds(k_slot_bwd_qb<float, false, D>, lds);
        hipLaunchKernelGGL((k_slot_bwd_qb<float, false, D>), grid, dim3(256), lds, s, p);
    }
}

template <int D>
void launch_bwd_q(const SK &p, int style, size_t lds, dim3 grid, hipStream_t s) {
    if (style == STYLE_AF3) {
        if (p.a.pair_dtype == 1) {
            set_lds(k_slot_bwd_q<bf16_t, true, D>, lds);
            hipLaunchKernelGGL((k_slot_bwd_q<bf16_t, true, D>), grid, dim3(256), lds, s, p);
        } else {
            set_lds(k_slot_bwd_q<float, true, D>, lds);
            hipLaunchKernelGGL((k_slot_bwd_q<float, true, D>), grid, dim3(256), lds, s, p);
        }
    } else {
        set_lds(k_slot_bwd_q<float, false, D>, lds);
        hipLaunchKernelGGL((k_slot_bwd_q<float, false, D>), grid, dim3(256), lds, s, p);
    }
}

hipError_t slot_fwd(const SlotBwdArgs &a, int style, hipStream_t s) {
    const int64_t N = (int64_t)a.B * a.A;
    if (N <= 0)
        return hipSuccess;
    SK p{a, 1.0f / sqrtf((float)a.D)};
    const size_t lds = 4 * sizeof(float) * (size_t)wave_floats(a.K, a.H, a.H * a.D);
    dim3 grid(nblk(N, 4));
    // block form where it applies (as the query side's), then the
    // per-query kernel for the queued blocks; else the per-query kernel
    const int nblocks = a.B * ((a.A + 15) / 16);
    SK pq = p;
    pq.a.wide = nullptr;
    if (block_form(a, nblocks)) {
        hipError_t e1 = fill_int(a.wide, 1, 0, s);
        if (e1 != hipSuccess)
            return e1;
        const size_t blds = sizeof(float) * (size_t)block_lds_floats();
        switch (a.D) {
        case 16: launch_fwd_b<16>(p, style, blds, dim3((unsigned)nblocks), s); break;
        case 32: launch_fwd_b<32>(p, style, blds, dim3((unsigned)nblocks), s); break;
        case 64: launch_fwd_b<64>(p, style, blds, dim3((unsigned)nblocks), s); break;
        default: return hipErrorInvalidValue;
        }
        pq.a.wide = a.wide;
        grid = dim3((unsigned)(4 * nblocks));
    }
    switch (a.D) {
    case 8: launch_fwd<8>(pq, style, lds, grid, s); break;
    case 16: launch_fwd<16>(pq, style, lds, grid, s); break;
    case 32: launch_fwd<32>(pq, style, lds, grid, s); break;
    case 64: launch_fwd<64>(pq, style, lds, grid, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t slot_bwd(const SlotBwdArgs &a, int style, float *d_pair_scale, float *d_w_pair,
                    hipStream_t s) {
    const int64_t N = (int64_t)a.B * a.A;
    if (N <= 0)
        return hipSuccess;
    SK p{a, 1.0f / sqrtf((float)a.D)};
    const size_t lds = 4 * sizeof(float) * (size_t)wave_floats(a.K, a.H, a.H * a.D);
    const dim3 grid(nblk(N, 4));
    // reverse index of the slot -> key map and each entry's place in it
    ProfSpan sp = prof_begin(KN_BWD_SLOT_KV, s);
    {
        const hipError_t e0 =
            reverse_index(a.kid, N * a.K, (int)N, a.count, a.offset, a.list, s, a.inv);
        if (e0 != hipSuccess)
            return e0;
    }
    prof_end(sp, s);
    sp = prof_begin(KN_BWD_SLOT_Q, s);
    // block form where it applies (blocks with a wide key band are queued
    // for the per-query kernel), else the per-query kernel over every query
    const int nblocks = a.B * ((a.A + 15) / 16);
    const bool block = block_form(a, nblocks);
    int records = (int)grid.x;
    SK pq = p;
    pq.a.wide = nullptr;
    pq.a.rec0 = 0;
    dim3 gq = grid;
    if (block) {
        hipError_t e1 = fill_int(a.wide, 1, 0, s);
        if (e1 != hipSuccess)
            return e1;
        const size_t blds = sizeof(float) * (size_t)block_lds_floats();
        switch (a.D) {
        case 16: launch_bwd_qb<16>(p, style, blds, dim3((unsigned)nblocks), s); break;
        case 32: launch_bwd_qb<32>(p, style, blds, dim3((unsigned)nblocks), s); break;
        case 64: launch_bwd_qb<64>(p, style, blds, dim3((unsigned)nblocks), s); break;
        default: return hipErrorInvalidValue;
        }
        pq.a.wide = a.wide;
        pq.a.rec0 = nblocks;
        gq = dim3((unsigned)(4 * nblocks));
        records = 5 * nblocks;
    }
    switch (a.D) {
    case 8: launch_bwd_q<8>(pq, style, lds, gq, s); break;
    case 16: launch_bwd_q<16>(pq, style, lds, gq, s); break;
    case 32: launch_bwd_q<32>(pq, style, lds, gq, s); break;
    case 64: launch_bwd_q<64>(pq, style, lds, gq, s); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    prof_end(sp, s);
    if (style == STYLE_AF3 && (d_pair_scale || d_w_pair)) {
        // sum the per-workgroup partials in workgroup order, then pick the
        // [V] and [V][H] blocks out of the padded record
        constexpr int W = kPairV + kPairV * kPairH;
        const int rows = records;
        float *sums = a.pw_partial + (size_t)rows * W;
        e = colsum(rows, W, view(a.pw_partial, W), View{nullptr, 0}, sums, 0.0f, a.sc, s);
        if (e == hipSuccess && d_pair_scale)
            e = ew(EW_COPY, 1, a.V, View{d_pair_scale, a.V}, view(sums, kPairV), View{nullptr, 0},
                   View{nullptr, 0}, nullptr, nullptr, 0, s);
        if (e == hipSuccess && d_w_pair)
            e = ew(EW_COPY, a.V, a.H, View{d_w_pair, a.H}, view(sums + kPairV, kPairH),
                   View{nullptr, 0}, View{nullptr, 0}, nullptr, nullptr, 0, s);
        if (e != hipSuccess)
            return e;
    }
    sp = prof_begin(KN_BWD_SLOT_KV, s);
    hipLaunchKernelGGL(k_slot_bwd_kv, grid, dim3(256), 0, s, p);
    prof_end(sp, s);
    return hipGetLastError();
}

} // namespace bwd
} // namespace waa
