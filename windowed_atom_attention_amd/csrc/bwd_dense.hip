// bwd_dense.hip -- the dense and row kernels of the block's backward pass:
// an fp32 matrix-core product for any operand strides (split-k for long
// reductions; grouped launches of independent products), column sums, the
// elementwise steps of the chain rule (grouped launches, 16-byte accesses
// where aligned), row normalisation and its backward,
// the ESMFold2 head RMS + rotary and its backward, sanitising, the pooling
// backward, and the reverse index that turns "entry -> key" maps into
// per-key lists without floating-point atomics.
#include <algorithm>

#include "bwd.hpp"
#include "common.hpp"

namespace waa {
namespace bwd {

namespace {

// ------------------------------------------------------------------ product

struct GemmK {
    const float *A;
    int64_t ars, acs;
    const float *B;
    int64_t brs, bcs;
    float *C;
    int64_t ldc;
    const float *bias;
    float beta;
    int M, N, K, kchunk, splits;
    int avec, bvec;  // 16-byte loads along the operand's contiguous axis
    float *partial;  // split mode: partial[z][M][N]
};

constexpr int kKS = 32; // k depth of one LDS stage

// Eight consecutive elements of a row (stride 1) starting at `idx` of a
// length-`lim` axis: two 16-byte loads when allowed and whole, else
// guarded scalar loads.
__device__ __forceinline__ void load8(const float *p, int idx, int lim, bool vec, float *r) {
    if (vec && idx + 7 < lim) {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = idx + i < lim ? p[i] : 0.0f;
    }
}

// One operand pair of a product: A [M, K] (element (m, k) at
// A[m * ars + k * acs]), B [K, N] likewise.
struct SegK {
    const float *A;
    int64_t ars, acs;
    const float *B;
    int64_t brs, bcs;
    int K;
    int avec, bvec; // 16-byte loads along the operand's contiguous axis
};

// 64x64 output tile per workgroup, four waves of 32x32 (v_mfma_f32_32x32x2_f32):
// acc += A[m0.., kb..ke) B[kb..ke, n0..). k advances in 32-deep stages
// staged through LDS; the next stage's operand tiles are loaded into
// registers while the current one is multiplied. Each thread moves 8
// consecutive elements of an operand's contiguous axis. Every stage starts
// with a barrier, so consecutive calls may reuse As/Bs.
__device__ __forceinline__ void tile_product(const SegK &g, int M, int N, int m0, int n0, int kb,
                                             int ke, float (&As)[kKS][68], float (&Bs)[kKS][68],
                                             f32x16_t &acc) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const bool a_k = g.acs == 1;
    const bool b_n = g.bcs == 1;
    float ra[8], rb[8];
    auto load = [&](int k0) {
        if (a_k) {
            // row m, 8 consecutive k
            const int m = t >> 2, kq = (t & 3) * 8;
            const int gm = m0 + m, gk = k0 + kq;
            if (gm < M)
                load8(g.A + (int64_t)gm * g.ars + gk, gk, ke, g.avec, ra);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) ra[i] = 0.0f;
        } else {
            // column k, 8 consecutive m (stride ars)
            const int k = t >> 3, mq = (t & 7) * 8;
            const int gk = k0 + k, gm = m0 + mq;
            if (gk < ke) {
                if (g.ars == 1)
                    load8(g.A + (int64_t)gk * g.acs + gm, gm, M, g.avec, ra);
                else
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        ra[i] = gm + i < M ? g.A[(int64_t)(gm + i) * g.ars + (int64_t)gk * g.acs] : 0.0f;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) ra[i] = 0.0f;
            }
        }
        if (b_n) {
            // row k, 8 consecutive n
            const int k = t >> 3, nq = (t & 7) * 8;
            const int gk = k0 + k, gn = n0 + nq;
            if (gk < ke)
                load8(g.B + (int64_t)gk * g.brs + gn, gn, N, g.bvec, rb);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) rb[i] = 0.0f;
        } else {
            // column n, 8 consecutive k (stride brs)
            const int n = t >> 2, kq = (t & 3) * 8;
            const int gn = n0 + n, gk = k0 + kq;
            if (gn < N) {
                if (g.brs == 1)
                    load8(g.B + (int64_t)gn * g.bcs + gk, gk, ke, g.bvec, rb);
                else
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        rb[i] = gk + i < ke ? g.B[(int64_t)(gk + i) * g.brs + (int64_t)gn * g.bcs] : 0.0f;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) rb[i] = 0.0f;
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (a_k)
                As[(t & 3) * 8 + i][t >> 2] = ra[i];
            else
                As[t >> 3][(t & 7) * 8 + i] = ra[i];
            if (b_n)
                Bs[t >> 3][(t & 7) * 8 + i] = rb[i];
            else
                Bs[(t & 3) * 8 + i][t >> 2] = rb[i];
        }
    };
    const int wm = (w & 1) * 32, wn = (w >> 1) * 32;
    const int half = lane >> 5, l32 = lane & 31;
    if (kb < ke)
        load(kb);
    for (int k0 = kb; k0 < ke; k0 += kKS) {
        __syncthreads();
        store();
        __syncthreads();
        if (k0 + kKS < ke)
            load(k0 + kKS);
#pragma unroll
        for (int kk = 0; kk < kKS / 2; ++kk) {
            const float a = As[kk * 2 + half][wm + l32];
            const float b = Bs[kk * 2 + half][wn + l32];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
    }
}

// Split k: every workgroup writes its partial tile; k_gemm_reduce sums
// them in split order.
__global__ __launch_bounds__(256) void k_gemm(GemmK g) {
    __shared__ float As[kKS][68];
    __shared__ float Bs[kKS][68];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int kb = blockIdx.z * g.kchunk;
    const int ke = min(g.K, kb + g.kchunk);
    const SegK sg{g.A, g.ars, g.acs, g.B, g.brs, g.bcs, g.K, g.avec, g.bvec};
    f32x16_t acc = zero16();
    tile_product(sg, g.M, g.N, m0, n0, kb, ke, As, Bs, acc);
    const int wm = (w & 1) * 32, wn = (w >> 1) * 32;
    const int c = n0 + wn + (lane & 31);
    if (g.splits == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = m0 + wm + acc32_row(v, lane);
            if (r >= g.M || c >= g.N)
                continue;
            float x = acc[v];
            if (g.bias)
                x += g.bias[c];
            float *dst = g.C + (int64_t)r * g.ldc + c;
            *dst = g.beta != 0.0f ? *dst + x : x;
        }
        return;
    }
    const int64_t MN = (int64_t)g.M * g.N;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm + acc32_row(v, lane);
        if (r < g.M && c < g.N)
            g.partial[(int64_t)blockIdx.z * MN + (int64_t)r * g.N + c] = acc[v];
    }
}

// Independent products in one launch: workgroups tile0[j] .. tile0[j+1]-1
// take job j's 64x64 tiles (row-major over its tile grid).
struct GemmJobK {
    SegK seg[kGroupSegs];
    int nseg, M, N, epi;
    float *C;
    int64_t ldc;
    const float *bias;
    float beta;
    int tiles_n, tile0;
};
struct GemmGroupK {
    GemmJobK job[kGroupJobs];
    int n;
};

__global__ __launch_bounds__(256) void k_gemm_group(GemmGroupK G) {
    __shared__ float As[kKS][68];
    __shared__ float Bs[kKS][68];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // consecutive tiles (the column tiles of one row block) on one XCD, so
    // the second read of a row block's A comes from that XCD's L2
    const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    int j = 0;
    while (j + 1 < G.n && bid >= G.job[j + 1].tile0)
        ++j;
    const GemmJobK &g = G.job[j];
    const int tl = bid - g.tile0;
    const int m0 = (tl / g.tiles_n) * 64, n0 = (tl % g.tiles_n) * 64;
    f32x16_t acc = zero16();
    for (int i = 0; i < g.nseg; ++i)
        tile_product(g.seg[i], g.M, g.N, m0, n0, 0, g.seg[i].K, As, Bs, acc);
    const int wm = (w & 1) * 32, wn = (w >> 1) * 32;
    const int c = n0 + wn + (lane & 31);
    if (c >= g.N)
        return;
    const float bc = g.bias ? g.bias[c] : 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm + acc32_row(v, lane);
        if (r >= g.M)
            continue;
        float x = acc[v] + bc;
        if (g.epi == GEMM_SIGMOID)
            x = sigmoid_f(x);
        float *dst = g.C + (int64_t)r * g.ldc + c;
        *dst = g.beta != 0.0f ? *dst + x : x;
    }
}

// C = beta*C + bias + sum over splits (a kernel of its own: the partial
// tiles of other workgroups become visible at the launch boundary, with no
// device-wide fence inside a kernel). Eight lanes per output element: lane
// l of the group sums splits l, l+8, ... in order, then the eight sums are
// added by a fixed butterfly -- the same order on every call.
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmK g) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
    const int sub = threadIdx.x & 7;
    const int64_t MN = (int64_t)g.M * g.N;
    const bool live = i < MN;
    float x = 0.0f;
    if (live)
        for (int z = sub; z < g.splits; z += 8)
            x += g.partial[(int64_t)z * MN + i];
    x += __shfl_xor(x, 1, 8);
    x += __shfl_xor(x, 2, 8);
    x += __shfl_xor(x, 4, 8);
    if (!live || sub != 0)
        return;
    const int r = (int)(i / g.N), c = (int)(i - (int64_t)r * g.N);
    if (g.bias)
        x += g.bias[c];
    float *dst = g.C + (int64_t)r * g.ldc + c;
    *dst = g.beta != 0.0f ? *dst + x : x;
}

// ------------------------------------------------------------- column sums

__global__ __launch_bounds__(256) void k_colsum(int rows, int W, const float *X, int64_t ldx,
                                                const float *Y, int64_t ldy, float *partial,
                                                int rows_per) {
    __shared__ float red[4][64];
    const int t = threadIdx.x, grp = t >> 6;
    const int col = blockIdx.x * 64 + (t & 63);
    const int r0 = blockIdx.y * rows_per, r1 = min(rows, r0 + rows_per);
    float acc = 0.0f;
    if (col < W)
        for (int r = r0 + grp; r < r1; r += 4) {
            float x = X[(int64_t)r * ldx + col];
            if (Y)
                x *= Y[(int64_t)r * ldy + col];
            acc += x;
        }
    red[grp][t & 63] = acc;
    __syncthreads();
    if (grp == 0 && col < W)
        partial[(int64_t)blockIdx.y * W + col] =
            ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
}

// One wave per column: lane l sums splits l, l+64, ... in order, then a
// fixed butterfly adds the lanes.
__global__ __launch_bounds__(256) void k_colsum_reduce(int W, int splits, const float *partial,
                                                       float *out, float beta) {
    const int col = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (col >= W)
        return;
    float x = 0.0f;
    for (int z = lane; z < splits; z += 64)
        x += partial[(int64_t)z * W + col];
    x = group_sum<64>(x);
    if (lane == 0)
        out[col] = beta != 0.0f ? out[col] + x : x;
}

// --------------------------------------------------- parameter-gradient leaves

// Up to kLeafJobs parameter-gradient leaves in two launches: split partial
// sums, then their fixed-order reduction. A leaf is a product C = A B whose
// long reduction axis K is split over workgroups (64x64 tiles, as k_gemm),
// or a column sum out[c] = sum_r X[r, c] (* Y[r, c]) whose rows are split.
struct LeafK {
    int kind; // 0 product, 1 column sum
    SegK seg; // product operands; column sum: A = X (ars = ld), B = Y or null (brs = ld)
    int M, N, kchunk, splits, tiles_n, units;
    float *out;
    int64_t ldo;
    float *partial; // [splits][M][N] (column sum: [splits][N])
    int unit0, red0;
};
struct LeafGroupK {
    LeafK job[kLeafJobs];
    int n;
};

__global__ __launch_bounds__(256) void k_leaf_split(LeafGroupK G) {
    __shared__ float As[kKS][68];
    __shared__ float Bs[kKS][68];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int j = 0;
    while (j + 1 < G.n && (int)blockIdx.x >= G.job[j + 1].unit0)
        ++j;
    const LeafK &g = G.job[j];
    const int u = (int)blockIdx.x - g.unit0;
    if (g.kind == 0) {
        const int tiles = (g.units / g.splits);
        const int z = u / tiles, tl = u - z * tiles;
        const int m0 = (tl / g.tiles_n) * 64, n0 = (tl % g.tiles_n) * 64;
        const int kb = z * g.kchunk, ke = min(g.seg.K, kb + g.kchunk);
        f32x16_t acc = zero16();
        tile_product(g.seg, g.M, g.N, m0, n0, kb, ke, As, Bs, acc);
        const int wm = (w & 1) * 32, wn = (w >> 1) * 32;
        const int c = n0 + wn + (lane & 31);
        const int64_t MN = (int64_t)g.M * g.N;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = m0 + wm + acc32_row(v, lane);
            if (r < g.M && c < g.N)
                g.partial[(int64_t)z * MN + (int64_t)r * g.N + c] = acc[v];
        }
        return;
    }
    // column sum: 64 columns per workgroup, rows split in `splits` ranges
    const int nb = (g.N + 63) / 64;
    const int z = u / nb, cb = u - z * nb;
    const int col = cb * 64 + lane;
    const int rows = g.seg.K, per = g.kchunk;
    const int r0 = z * per, r1 = min(rows, r0 + per);
    float acc = 0.0f;
    if (col < g.N)
        for (int r = r0 + w; r < r1; r += 4) {
            float x = g.seg.A[(int64_t)r * g.seg.ars + col];
            if (g.seg.B)
                x *= g.seg.B[(int64_t)r * g.seg.brs + col];
            acc += x;
        }
    float *red = &As[0][0];
    red[w * 64 + lane] = acc;
    __syncthreads();
    if (w == 0 && col < g.N)
        g.partial[(int64_t)z * g.N + col] = ((red[lane] + red[64 + lane]) + red[128 + lane]) + red[192 + lane];
}

// 8 lanes per output element: lane l of the group sums splits l, l+8, ...
// in order, then a fixed butterfly
__global__ __launch_bounds__(256) void k_leaf_reduce(LeafGroupK G) {
    int j = 0;
    while (j + 1 < G.n && (int)blockIdx.x >= G.job[j + 1].red0)
        ++j;
    const LeafK &g = G.job[j];
    const int64_t i = ((int64_t)((int)blockIdx.x - g.red0) * 256 + threadIdx.x) >> 3;
    const int sub = threadIdx.x & 7;
    const int64_t MN = (int64_t)g.M * g.N;
    const bool live = i < MN;
    float x = 0.0f;
    if (live)
        for (int z = sub; z < g.splits; z += 8)
            x += g.partial[(int64_t)z * MN + i];
    x += __shfl_xor(x, 1, 8);
    x += __shfl_xor(x, 2, 8);
    x += __shfl_xor(x, 4, 8);
    if (!live || sub != 0)
        return;
    const int r = (int)(i / g.N), c = (int)(i - (int64_t)r * g.N);
    g.out[(int64_t)r * g.ldo + c] = x;
}

// ------------------------------------------------------------- elementwise

__device__ __forceinline__ float dsilu_f(float z) {
    const float s = sigmoid_f(z);
    return s * (1.0f + z * (1.0f - s));
}

struct EwK {
    int op, rows, W, acc;
    float *o;
    int64_t ldo;
    const float *a, *b, *c, *d;
    int64_t lda, ldb, ldc, ldd;
    const float *vec, *vec2, *vec3;
    const uint8_t *mask;
    int blk0; // first workgroup of the job in a group launch
    int v4;   // four consecutive columns per thread (16-byte accesses)
};
struct EwGroupK {
    EwK job[kGroupJobs];
    int n;
};

__device__ __forceinline__ float ew_op(int op, float a, float b, float c, float d, float vc,
                                       float vc2, float vc3) {
    switch (op) {
    case EW_COPY: return a;
    case EW_ADD: return a + b;
    case EW_MUL: return a * b;
    case EW_MUL_VEC: return a * vc;
    case EW_AFFINE: return a * b + c;
    case EW_AFFINE1: return a * (1.0f + b) + c;
    case EW_MUL1: return a * (1.0f + b);
    case EW_SIGMOID: return sigmoid_f(a);
    case EW_SIGMOID_VEC: return sigmoid_f(a + vc);
    case EW_SILU: return silu_f(a);
    case EW_SWIGLU: return silu_f(a) * b;
    case EW_RESID: return a + b * c;
    case EW_RESID_MASK: return a + b * c;
    case EW_MASK: return a;
    case EW_DSIG: return a * b * (1.0f - b);
    case EW_DGATE: return a * b * c * (1.0f - c);
    case EW_DSWIGLU_A: return a * c * dsilu_f(b);
    case EW_DSWIGLU_B: return a * silu_f(b);
    case EW_DSILU: return a * dsilu_f(b);
    case EW_ADD_VEC: return a + vc;
    case EW_ZERO: return 0.0f;
    case EW_FMA2: return a * b + c * d;
    case EW_MUL_VEC3: return a * vc + b * vc2 + c * vc3;
    default: return 0.0f;
    }
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

__global__ __launch_bounds__(256) void k_ew(EwGroupK G) {
    int j = 0;
    while (j + 1 < G.n && (int)blockIdx.x >= G.job[j + 1].blk0)
        ++j;
    const EwK &e = G.job[j];
    const int64_t i = (int64_t)((int)blockIdx.x - e.blk0) * 256 + threadIdx.x;
    if (e.v4) {
        const int W4 = e.W >> 2;
        if (i >= (int64_t)e.rows * W4)
            return;
        const int r = (int)(i / W4), col = (int)(i - (int64_t)r * W4) * 4;
        const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float4 a = e.a ? ld4(e.a + (int64_t)r * e.lda + col) : z;
        const float4 b = e.b ? ld4(e.b + (int64_t)r * e.ldb + col) : z;
        const float4 c = e.c ? ld4(e.c + (int64_t)r * e.ldc + col) : z;
        const float4 d = e.d ? ld4(e.d + (int64_t)r * e.ldd + col) : z;
        const float4 v1 = e.vec ? ld4(e.vec + col) : z;
        const float4 v2 = e.vec2 ? ld4(e.vec2 + col) : z;
        const float4 v3 = e.vec3 ? ld4(e.vec3 + col) : z;
        const bool m = e.mask ? e.mask[r] != 0 : true;
        float4 x;
        x.x = ew_op(e.op, a.x, b.x, c.x, d.x, v1.x, v2.x, v3.x);
        x.y = ew_op(e.op, a.y, b.y, c.y, d.y, v1.y, v2.y, v3.y);
        x.z = ew_op(e.op, a.z, b.z, c.z, d.z, v1.z, v2.z, v3.z);
        x.w = ew_op(e.op, a.w, b.w, c.w, d.w, v1.w, v2.w, v3.w);
        if (!m)
            x = z;
        float4 *dst = reinterpret_cast<float4 *>(e.o + (int64_t)r * e.ldo + col);
        if (e.acc) {
            const float4 o = *dst;
            x.x += o.x;
            x.y += o.y;
            x.z += o.z;
            x.w += o.w;
        }
        *dst = x;
        return;
    }
    if (i >= (int64_t)e.rows * e.W)
        return;
    const int r = (int)(i / e.W), col = (int)(i - (int64_t)r * e.W);
    const float a = e.a ? e.a[(int64_t)r * e.lda + col] : 0.0f;
    const float b = e.b ? e.b[(int64_t)r * e.ldb + col] : 0.0f;
    const float c = e.c ? e.c[(int64_t)r * e.ldc + col] : 0.0f;
    const float d = e.d ? e.d[(int64_t)r * e.ldd + col] : 0.0f;
    const float vc = e.vec ? e.vec[col] : 0.0f;
    const float vc2 = e.vec2 ? e.vec2[col] : 0.0f;
    const float vc3 = e.vec3 ? e.vec3[col] : 0.0f;
    const bool m = e.mask ? e.mask[r] != 0 : true;
    float x = ew_op(e.op, a, b, c, d, vc, vc2, vc3);
    if (!m)
        x = 0.0f;
    float *dst = e.o + (int64_t)r * e.ldo + col;
    *dst = e.acc ? *dst + x : x;
}

// --------------------------------------------------------- normalisation

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__global__ __launch_bounds__(256) void k_norm_rows(int mode, int rows, int W, float eps,
                                                   const float *x, int64_t ldx, float *xh,
                                                   int64_t ldh, float *rstd) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const float *xr = x + (int64_t)row * ldx;
    float mean = 0.0f;
    if (mode == 0) {
        float s = 0.0f;
        for (int i = lane; i < W; i += 64)
            s += xr[i];
        mean = wave_sum(s) / (float)W;
    }
    float q = 0.0f;
    for (int i = lane; i < W; i += 64) {
        const float d = xr[i] - mean;
        q += d * d;
    }
    const float r = 1.0f / sqrtf(wave_sum(q) / (float)W + eps);
    float *hr = xh + (int64_t)row * ldh;
    for (int i = lane; i < W; i += 64)
        hr[i] = (xr[i] - mean) * r;
    if (lane == 0)
        rstd[row] = r;
}

__global__ __launch_bounds__(256) void k_norm_rows_bwd(int mode, int rows, int W,
                                                       const float *xh, int64_t ldh,
                                                       const float *rstd, const float *g,
                                                       int64_t ldg, float *o, int64_t ldo,
                                                       int acc) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const float *hr = xh + (int64_t)row * ldh;
    const float *gr = g + (int64_t)row * ldg;
    float sg = 0.0f, sgx = 0.0f;
    for (int i = lane; i < W; i += 64) {
        sg += gr[i];
        sgx += gr[i] * hr[i];
    }
    const float mg = mode == 0 ? wave_sum(sg) / (float)W : 0.0f;
    const float mgx = wave_sum(sgx) / (float)W;
    const float r = rstd[row];
    float *orow = o + (int64_t)row * ldo;
    for (int i = lane; i < W; i += 64) {
        const float d = r * (gr[i] - mg - hr[i] * mgx);
        orow[i] = acc ? orow[i] + d : d;
    }
}

// ------------------------------------------------------------ conversions

template <typename T>
__global__ __launch_bounds__(256) void k_to_f32(const T *src, int64_t rows, int W, int64_t lds,
                                                float *dst, const uint8_t *mask) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * W)
        return;
    const int64_t r = i / W;
    const int col = (int)(i - r * W);
    dst[i] = (!mask || mask[r]) ? to_f(src[r * lds + col]) : 0.0f;
}

template <typename T>
__global__ __launch_bounds__(256) void k_sanitize_x(int B, int A, int T_, int C, const T *atom,
                                                    const uint8_t *usable, const int64_t *a2t,
                                                    const float *tokproj, float *x0) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)B * A * C)
        return;
    const int64_t n = i / C;
    const int col = (int)(i - n * C);
    float x = 0.0f;
    if (usable[n]) {
        x = to_f(atom[i]);
        if (tokproj) {
            const int64_t b = n / A;
            x += tokproj[(b * T_ + a2t[n]) * C + col];
        }
    }
    x0[i] = x;
}

// ------------------------------------------------------ head RMS + rotary

// One thread per (row, channel i of a head); the D threads of a row's head
// are an aligned lane group, so head sums and the rotary partner i ^ D/2
// are lane exchanges.
template <int D>
__global__ __launch_bounds__(256) void k_head_rope(int rows, int H, float eps, const float *qraw,
                                                   const float *kraw, const float *cs,
                                                   const float *sn, float *q, float *k) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / D;
    const int i = (int)(t % D);
    const bool live = row < rows;
    const int64_t rr = live ? row : 0;
    const float c = cs[rr * D + i], s = sn[rr * D + i];
    const int HD = H * D;
    for (int which = 0; which < 2; ++which) {
        const float *src = which ? kraw : qraw;
        float *dst = which ? k : q;
        for (int h = 0; h < H; ++h) {
            const float x = src[rr * HD + h * D + i];
            const float r = 1.0f / sqrtf(group_sum<D>(x * x) / (float)D + eps);
            const float y = x * r;
            const float yp = __shfl_xor(y, D / 2, D);
            const float rot = i < D / 2 ? -yp : yp;
            if (live)
                dst[rr * HD + h * D + i] = y * c + rot * s;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_head_rope_bwd(int rows, int H, float eps,
                                                       const float *qraw, const float *kraw,
                                                       const float *cs, const float *sn,
                                                       float *dq, float *dk, float *dcos,
                                                       float *dsin) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / D;
    const int i = (int)(t % D);
    const bool live = row < rows;
    const int64_t rr = live ? row : 0;
    const float c = cs[rr * D + i], s = sn[rr * D + i];
    const int HD = H * D;
    float gc = 0.0f, gs = 0.0f;
    for (int which = 0; which < 2; ++which) {
        const float *src = which ? kraw : qraw;
        float *g = which ? dk : dq;
        for (int h = 0; h < H; ++h) {
            const int64_t at = rr * HD + h * D + i;
            const float x = src[at];
            const float r = 1.0f / sqrtf(group_sum<D>(x * x) / (float)D + eps);
            const float y = x * r;
            const float yp = __shfl_xor(y, D / 2, D);
            const float rot = i < D / 2 ? -yp : yp;
            const float go = live ? g[at] : 0.0f;
            gc += go * y;
            gs += go * rot;
            // through the rotation: dy = cos*go + R^T (sin*go)
            const float zp = __shfl_xor(s * go, D / 2, D);
            const float dy = c * go + (i < D / 2 ? zp : -zp);
            // through the RMS: dx = r * (dy - y * mean(dy * y))
            const float m = group_sum<D>(dy * y) / (float)D;
            if (live)
                g[at] = r * (dy - y * m);
        }
    }
    if (live) {
        if (dcos)
            dcos[rr * D + i] = gc;
        if (dsin)
            dsin[rr * D + i] = gs;
    }
}

// ------------------------------------------------------------ pooling

__global__ __launch_bounds__(256) void k_pool_bwd(int B, int A, int T_, int U,
                                                  const uint8_t *usable, const int64_t *a2t,
                                                  const int32_t *count, const float *dto,
                                                  const float *proj, float *dp) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)B * A * U)
        return;
    const int64_t n = i / U;
    const int col = (int)(i - n * U);
    float x = 0.0f;
    if (usable[n] && proj[i] > 0.0f) {
        const int64_t tok = (n / A) * T_ + a2t[n];
        x = dto[tok * U + col] / (float)count[tok];
    }
    dp[i] = x;
}

__global__ __launch_bounds__(256) void k_token_keys(int B, int A, int T_, const uint8_t *usable,
                                                    const int64_t *a2t, int32_t *key_of) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= (int64_t)B * A)
        return;
    key_of[n] = usable[n] ? (int32_t)((n / A) * T_ + a2t[n]) : -1;
}

// ------------------------------------------------------- reverse index

__global__ __launch_bounds__(256) void k_fill_int(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = v;
}

__global__ __launch_bounds__(256) void k_ri_count(const int32_t *key_of, int64_t n,
                                                  int32_t *count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const int k = key_of[i];
    if (k >= 0)
        atomicAdd(&count[k], 1);
}

// Exclusive scan of count into offset[0..nkeys] in three launches: each
// workgroup scans a tile of kScanTile keys (8 consecutive per thread, wave
// scans by lane exchanges) and writes the tile's total to bsum; one
// workgroup scans the totals; then every offset gets its tile's prefix.
constexpr int kScanTile = 2048;

__global__ __launch_bounds__(256) void k_ri_scan_local(const int32_t *count, int nkeys,
                                                       int32_t *offset, int32_t *bsum) {
    __shared__ int32_t wsum[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t base = (int64_t)blockIdx.x * kScanTile + t * 8;
    int32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = base + i < nkeys ? count[base + i] : 0;
    int32_t tot = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int32_t c = v[i];
        v[i] = tot;
        tot += c;
    }
    int32_t x = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        wsum[w] = x;
    __syncthreads();
    int32_t pre = 0;
    for (int ww = 0; ww < w; ++ww)
        pre += wsum[ww];
    const int32_t excl = pre + x - tot;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (base + i < nkeys)
            offset[base + i] = excl + v[i];
    if (t == 0)
        bsum[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// bsum[0..nb) -> exclusive prefix, bsum[nb] = total (one workgroup, chunks
// of 1024 with a carried sum)
__global__ __launch_bounds__(1024) void k_ri_scan_top(int32_t *bsum, int nb) {
    __shared__ int32_t sh[1024];
    const int t = threadIdx.x;
    int32_t carry = 0;
    for (int c0 = 0; c0 < nb; c0 += 1024) {
        const int i = c0 + t;
        const int32_t v = i < nb ? bsum[i] : 0;
        sh[t] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t y = t >= off ? sh[t - off] : 0;
            __syncthreads();
            sh[t] += y;
            __syncthreads();
        }
        if (i < nb)
            bsum[i] = carry + sh[t] - v;
        carry += sh[1023];
        __syncthreads();
    }
    if (t == 0)
        bsum[nb] = carry;
}

// offset[i] += its tile's prefix; count[i] = 0 (the fill's cursor)
__global__ __launch_bounds__(256) void k_ri_scan_add(int32_t *offset, int32_t *count, int nkeys,
                                                     const int32_t *bsum, int nb) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i == 0)
        offset[nkeys] = bsum[nb];
    if (i >= nkeys)
        return;
    offset[i] += bsum[i / kScanTile];
    count[i] = 0;
}

__global__ __launch_bounds__(256) void k_ri_fill(const int32_t *key_of, int64_t n,
                                                 const int32_t *offset, int32_t *cursor,
                                                 int32_t *list) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const int k = key_of[i];
    if (k >= 0)
        list[offset[k] + atomicAdd(&cursor[k], 1)] = (int32_t)i;
}

// Sort every list of at most kSortCap entries ascending, one wave per key:
// an entry's place is the number of smaller entries in its list (entries
// are distinct), counted over lane exchanges (<= 64) or an LDS copy. With
// inv, every listed entry's final place is also written there (lists of
// one entry and lists longer than kSortCap keep their order).
__global__ __launch_bounds__(256) void k_ri_sort(const int32_t *offset, int nkeys,
                                                 int32_t *list, int32_t *inv) {
    __shared__ int32_t sh[4][kSortCap];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int key = blockIdx.x * 4 + w;
    int o = 0, L = 0;
    if (key < nkeys) {
        o = offset[key];
        L = offset[key + 1] - o;
    }
    const bool small = L > 1 && L <= 64;
    const bool mid = L > 64 && L <= kSortCap;
    if (inv && (L == 1 || L > kSortCap))
        for (int i = lane; i < L; i += 64)
            inv[list[o + i]] = o + i;
    if (small) {
        const int32_t x = lane < L ? list[o + lane] : 0x7fffffff;
        int rank = 0;
        for (int m = 0; m < L; ++m)
            rank += __shfl(x, m) < x ? 1 : 0;
        if (lane < L) {
            list[o + rank] = x;
            if (inv)
                inv[x] = o + rank;
        }
    }
    if (mid)
        for (int i = lane; i < L; i += 64)
            sh[w][i] = list[o + i];
    __syncthreads();
    if (mid)
        for (int i = lane; i < L; i += 64) {
            const int32_t x = sh[w][i];
            int rank = 0;
            for (int m = 0; m < L; ++m)
                rank += sh[w][m] < x ? 1 : 0;
            list[o + rank] = x;
            if (inv)
                inv[x] = o + rank;
        }
}

__global__ __launch_bounds__(256) void k_segment_sum(int nkeys, int W, const int32_t *offset,
                                                     const int32_t *list, const float *X,
                                                     float *out) {
    const int lane = threadIdx.x & 63;
    const int key = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (key >= nkeys)
        return;
    const int b = offset[key], e = offset[key + 1];
    for (int c0 = 0; c0 < W; c0 += 64) {
        const int col = c0 + lane;
        float acc = 0.0f;
        if (col < W)
            for (int i = b; i < e; ++i)
                acc += X[(int64_t)list[i] * W + col];
        if (col < W)
            out[(int64_t)key * W + col] = acc;
    }
}

inline unsigned nblk(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

} // namespace

hipError_t gemm(int M, int N, int K, Mat A, Mat B, View C, float beta, const float *bias,
                Scratch sc, hipStream_t s) {
    if (M <= 0 || N <= 0)
        return hipSuccess;
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
    GemmK g{A.p, A.rs, A.cs, B.p, B.rs, B.cs, C.p, C.ld, bias, beta, M, N, K, 0, 1, 0, 0,
            nullptr};
    // 16-byte loads: contiguous axis stride 1, base and the other stride
    // 16-byte aligned
    g.avec = al16(A.p) && ((A.cs == 1 && A.rs % 4 == 0) || (A.rs == 1 && A.cs % 4 == 0));
    g.bvec = al16(B.p) && ((B.cs == 1 && B.rs % 4 == 0) || (B.rs == 1 && B.cs % 4 == 0));
    const int64_t tiles = (int64_t)nblk(M, 64) * nblk(N, 64);
    // split only long reductions (parameter gradients over every atom)
    int64_t splits = 1;
    if (sc.partial && tiles < 256 && K >= 1024) {
        splits = std::min<int64_t>((512 + tiles - 1) / tiles, K / 128);
        splits = std::min<int64_t>(splits, (int64_t)(sc.cap / ((size_t)M * N)));
        if (splits < 2)
            splits = 1;
    }
    int64_t kchunk = std::max<int64_t>(1, (K + splits - 1) / splits);
    kchunk = (kchunk + kKS - 1) / kKS * kKS;
    splits = K > 0 ? (K + kchunk - 1) / kchunk : 1;
    g.kchunk = (int)kchunk;
    g.splits = (int)splits;
    if (splits > 1)
        g.partial = sc.partial;
    hipLaunchKernelGGL(k_gemm, dim3(nblk(N, 64), nblk(M, 64), (unsigned)splits), dim3(256), 0,
                       s, g);
    if (splits > 1)
        hipLaunchKernelGGL(k_gemm_reduce, dim3(nblk((int64_t)M * N * 8, 256)), dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t gemm_group(const GemmJob *jobs, int n, hipStream_t s) {
    if (n < 1 || n > kGroupJobs)
        return hipErrorInvalidValue;
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
    auto vec_ok = [&](const Mat &x) {
        return al16(x.p) && ((x.cs == 1 && x.rs % 4 == 0) || (x.rs == 1 && x.cs % 4 == 0));
    };
    GemmGroupK G{};
    int tiles = 0, m = 0;
    for (int j = 0; j < n; ++j) {
        const GemmJob &x = jobs[j];
        if (x.M <= 0 || x.N <= 0)
            continue;
        if (x.nseg < 1 || x.nseg > kGroupSegs)
            return hipErrorInvalidValue;
        GemmJobK &k = G.job[m];
        for (int i = 0; i < x.nseg; ++i) {
            const GemmSeg &sg = x.seg[i];
            k.seg[i] = SegK{sg.A.p, sg.A.rs, sg.A.cs, sg.B.p, sg.B.rs, sg.B.cs, sg.K,
                            vec_ok(sg.A) ? 1 : 0, vec_ok(sg.B) ? 1 : 0};
        }
        k.nseg = x.nseg;
        k.M = x.M;
        k.N = x.N;
        k.epi = x.epi;
        k.C = x.C.p;
        k.ldc = x.C.ld;
        k.bias = x.bias;
        k.beta = x.beta;
        k.tiles_n = (int)nblk(x.N, 64);
        k.tile0 = tiles;
        tiles += (int)nblk(x.M, 64) * k.tiles_n;
        ++m;
    }
    if (m == 0)
        return hipSuccess;
    G.n = m;
    hipLaunchKernelGGL(k_gemm_group, dim3((unsigned)tiles), dim3(256), 0, s, G);
    return hipGetLastError();
}

hipError_t leaf_group(const LeafJob *jobs, int n, Scratch sc, hipStream_t s) {
    if (n < 1 || n > kLeafJobs)
        return hipErrorInvalidValue;
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
    LeafGroupK G{};
    // splits: about 512 workgroups per product (chunks of at least 128 rows)
    // and rows / 128 (at most 1024) per column sum, scaled down together if
    // the partial sums would not fit the scratch
    int64_t want[kLeafJobs], outs[kLeafJobs], need = 0;
    int m = 0;
    for (int j = 0; j < n; ++j) {
        const LeafJob &x = jobs[j];
        if (!x.out || x.N <= 0 || (x.kind == 0 && x.M <= 0))
            continue;
        const int64_t K = x.K;
        if (x.kind == 0) {
            const int64_t tiles = (int64_t)nblk(x.M, 64) * nblk(x.N, 64);
            want[m] = std::max<int64_t>(1, std::min<int64_t>((512 + tiles - 1) / tiles, K / 128));
            outs[m] = (int64_t)x.M * x.N;
        } else {
            want[m] = std::max<int64_t>(1, std::min<int64_t>((K + 127) / 128, 1024));
            outs[m] = x.N;
        }
        need += want[m] * outs[m];
        G.job[m].kind = x.kind;
        ++m;
    }
    if (m == 0)
        return hipSuccess;
    const double scale = need > (int64_t)sc.cap ? (double)sc.cap / (double)need : 1.0;
    int units = 0, reds = 0, jj = 0;
    size_t off = 0;
    for (int j = 0; j < n; ++j) {
        const LeafJob &x = jobs[j];
        if (!x.out || x.N <= 0 || (x.kind == 0 && x.M <= 0))
            continue;
        LeafK &k = G.job[jj];
        int64_t splits = std::max<int64_t>(1, (int64_t)(want[jj] * scale));
        const int64_t K = x.K;
        if (x.kind == 0) {
            int64_t kchunk = (K + splits - 1) / splits;
            kchunk = (kchunk + kKS - 1) / kKS * kKS;
            splits = K > 0 ? (K + kchunk - 1) / kchunk : 1;
            k.kchunk = (int)kchunk;
            k.seg = SegK{x.A.p, x.A.rs, x.A.cs, x.B.p, x.B.rs, x.B.cs, (int)K,
                         (al16(x.A.p) && ((x.A.cs == 1 && x.A.rs % 4 == 0) || (x.A.rs == 1 && x.A.cs % 4 == 0))) ? 1 : 0,
                         (al16(x.B.p) && ((x.B.cs == 1 && x.B.rs % 4 == 0) || (x.B.rs == 1 && x.B.cs % 4 == 0))) ? 1 : 0};
            k.M = x.M;
            k.tiles_n = (int)nblk(x.N, 64);
            k.units = (int)(nblk(x.M, 64) * k.tiles_n * splits);
        } else {
            const int64_t per = std::max<int64_t>(1, (K + splits - 1) / splits);
            splits = K > 0 ? (K + per - 1) / per : 1;
            k.kchunk = (int)per;
            k.seg = SegK{x.A.p, x.A.rs, 1, x.B.p, x.B.rs, 1, (int)K, 0, 0};
            k.M = 1;
            k.tiles_n = 1;
            k.units = (int)(nblk(x.N, 64) * splits);
        }
        k.N = x.N;
        k.splits = (int)splits;
        k.out = x.out;
        k.ldo = x.ldo;
        k.partial = sc.partial + off;
        off += (size_t)splits * (size_t)k.M * (size_t)x.N;
        if (off > sc.cap)
            return hipErrorInvalidValue;
        k.unit0 = units;
        units += k.units;
        k.red0 = reds;
        reds += (int)nblk((int64_t)k.M * x.N * 8, 256);
        ++jj;
    }
    G.n = jj;
    hipLaunchKernelGGL(k_leaf_split, dim3((unsigned)units), dim3(256), 0, s, G);
    hipLaunchKernelGGL(k_leaf_reduce, dim3((unsigned)reds), dim3(256), 0, s, G);
    return hipGetLastError();
}

hipError_t colsum(int rows, int W, View X, View Y, float *out, float beta, Scratch sc,
                  hipStream_t s) {
    if (W <= 0)
        return hipSuccess;
    int64_t splits = std::max<int64_t>(1, std::min<int64_t>((rows + 127) / 128, 1024));
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, (int64_t)(sc.cap / (size_t)W)));
    const int rows_per = std::max(1, (int)((rows + splits - 1) / splits));
    splits = rows > 0 ? (rows + rows_per - 1) / rows_per : 1;
    hipLaunchKernelGGL(k_colsum, dim3(nblk(W, 64), (unsigned)splits), dim3(256), 0, s, rows, W,
                       (const float *)X.p, X.ld, (const float *)Y.p, Y.ld, sc.partial, rows_per);
    hipLaunchKernelGGL(k_colsum_reduce, dim3(nblk(W, 4)), dim3(256), 0, s, W, (int)splits,
                       (const float *)sc.partial, out, beta);
    return hipGetLastError();
}

hipError_t ew_group(const EwJob *jobs, int n, hipStream_t s) {
    if (n < 1 || n > kGroupJobs)
        return hipErrorInvalidValue;
    EwGroupK G{};
    int blk = 0, m = 0;
    for (int j = 0; j < n; ++j) {
        const EwJob &x = jobs[j];
        const int64_t cnt = (int64_t)x.rows * x.W;
        if (cnt <= 0)
            continue;
        // 16-byte accesses when every row of every operand starts aligned
        auto ok4 = [](const float *p, int64_t ld) {
            return !p || (((uintptr_t)p & 15u) == 0 && ld % 4 == 0);
        };
        auto okv = [](const float *p) { return !p || ((uintptr_t)p & 15u) == 0; };
        const int v4 = (x.W % 4 == 0 && ok4(x.o.p, x.o.ld) && ok4(x.a.p, x.a.ld) &&
                        ok4(x.b.p, x.b.ld) && ok4(x.c.p, x.c.ld) && ok4(x.d.p, x.d.ld) &&
                        okv(x.vec) && okv(x.vec2) && okv(x.vec3)) ? 1 : 0;
        G.job[m] = EwK{(int)x.op, x.rows, x.W, x.acc, x.o.p, x.o.ld, x.a.p, x.b.p, x.c.p, x.d.p,
                       x.a.ld, x.b.ld, x.c.ld, x.d.ld, x.vec, x.vec2, x.vec3, x.mask, blk, v4};
        blk += (int)nblk(v4 ? cnt / 4 : cnt, 256);
        ++m;
    }
    if (m == 0)
        return hipSuccess;
    G.n = m;
    hipLaunchKernelGGL(k_ew, dim3((unsigned)blk), dim3(256), 0, s, G);
    return hipGetLastError();
}

hipError_t ew(EwOp op, int rows, int W, View o, View a, View b, View c, const float *vec,
              const uint8_t *mask, int acc, hipStream_t s) {
    EwJob j{op, rows, W, o, a, b, c, View{nullptr, 0}, vec, nullptr, nullptr, mask, acc};
    return ew_group(&j, 1, s);
}

hipError_t norm_rows(int mode, int rows, int W, float eps, View x, View xhat, float *rstd,
                     hipStream_t s) {
    if (rows <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_norm_rows, dim3(nblk(rows, 4)), dim3(256), 0, s, mode, rows, W, eps,
                       (const float *)x.p, x.ld, xhat.p, xhat.ld, rstd);
    return hipGetLastError();
}

hipError_t norm_rows_bwd(int mode, int rows, int W, View xhat, const float *rstd, View g,
                         View o, int acc, hipStream_t s) {
    if (rows <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_norm_rows_bwd, dim3(nblk(rows, 4)), dim3(256), 0, s, mode, rows, W,
                       (const float *)xhat.p, xhat.ld, rstd, (const float *)g.p, g.ld, o.p,
                       o.ld, acc);
    return hipGetLastError();
}

hipError_t to_f32(const void *src, int dtype, int64_t rows, int W, int64_t lds, float *dst,
                  const uint8_t *mask, hipStream_t s) {
    const int64_t n = rows * W;
    if (n <= 0)
        return hipSuccess;
    if (dtype == 1)
        hipLaunchKernelGGL(k_to_f32<bf16_t>, dim3(nblk(n, 256)), dim3(256), 0, s,
                           (const bf16_t *)src, rows, W, lds, dst, mask);
    else
        hipLaunchKernelGGL(k_to_f32<float>, dim3(nblk(n, 256)), dim3(256), 0, s,
                           (const float *)src, rows, W, lds, dst, mask);
    return hipGetLastError();
}

hipError_t head_rope(int rows, int H, int D, float eps, const float *qraw, const float *kraw,
                     const float *cs, const float *sn, float *q, float *k, hipStream_t s) {
    const dim3 grid(nblk((int64_t)rows * D, 256));
    switch (D) {
    case 8: hipLaunchKernelGGL(k_head_rope<8>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, q, k); break;
    case 16: hipLaunchKernelGGL(k_head_rope<16>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, q, k); break;
    case 32: hipLaunchKernelGGL(k_head_rope<32>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, q, k); break;
    case 64: hipLaunchKernelGGL(k_head_rope<64>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, q, k); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t head_rope_bwd(int rows, int H, int D, float eps, const float *qraw,
                         const float *kraw, const float *cs, const float *sn, float *dq,
                         float *dk, float *dcos, float *dsin, hipStream_t s) {
    const dim3 grid(nblk((int64_t)rows * D, 256));
    switch (D) {
    case 8: hipLaunchKernelGGL(k_head_rope_bwd<8>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, dq, dk, dcos, dsin); break;
    case 16: hipLaunchKernelGGL(k_head_rope_bwd<16>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, dq, dk, dcos, dsin); break;
    case 32: hipLaunchKernelGGL(k_head_rope_bwd<32>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, dq, dk, dcos, dsin); break;
    case 64: hipLaunchKernelGGL(k_head_rope_bwd<64>, grid, dim3(256), 0, s, rows, H, eps, qraw, kraw, cs, sn, dq, dk, dcos, dsin); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t sanitize(int B, int A, int T, int C, int S, int dtype, const void *atom,
                    const void *cond, const uint8_t *usable, const int64_t *a2t,
                    const float *tokproj, float *x0, float *c, hipStream_t s) {
    const int64_t n = (int64_t)B * A * C;
    if (dtype == 1)
        hipLaunchKernelGGL(k_sanitize_x<bf16_t>, dim3(nblk(n, 256)), dim3(256), 0, s, B, A, T, C,
                           (const bf16_t *)atom, usable, a2t, tokproj, x0);
    else
        hipLaunchKernelGGL(k_sanitize_x<float>, dim3(nblk(n, 256)), dim3(256), 0, s, B, A, T, C,
                           (const float *)atom, usable, a2t, tokproj, x0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return to_f32(cond, dtype, (int64_t)B * A, S, S, c, usable, s);
}

hipError_t pool_bwd(int B, int A, int T, int U, const uint8_t *usable, const int64_t *a2t,
                    const int32_t *count, const float *dto, const float *proj, float *dp,
                    hipStream_t s) {
    const int64_t n = (int64_t)B * A * U;
    hipLaunchKernelGGL(k_pool_bwd, dim3(nblk(n, 256)), dim3(256), 0, s, B, A, T, U, usable, a2t,
                       count, dto, proj, dp);
    return hipGetLastError();
}

hipError_t token_keys(int B, int A, int T, const uint8_t *usable, const int64_t *a2t,
                      int32_t *key_of, hipStream_t s) {
    hipLaunchKernelGGL(k_token_keys, dim3(nblk((int64_t)B * A, 256)), dim3(256), 0, s, B, A, T,
                       usable, a2t, key_of);
    return hipGetLastError();
}

hipError_t reverse_index(const int32_t *key_of, int64_t n, int nkeys, int32_t *count,
                         int32_t *offset, int32_t *list, hipStream_t s, int32_t *inv) {
    hipLaunchKernelGGL(k_fill_int, dim3(nblk(nkeys, 256)), dim3(256), 0, s, count,
                       (int64_t)nkeys, 0);
    if (n > 0)
        hipLaunchKernelGGL(k_ri_count, dim3(nblk(n, 256)), dim3(256), 0, s, key_of, n, count);
    // tile totals after the nkeys counts (the caller sizes count with
    // reverse_index_count_ints)
    const int nb = (int)nblk(nkeys, kScanTile);
    int32_t *bsum = count + nkeys;
    if (nb > 0)
        hipLaunchKernelGGL(k_ri_scan_local, dim3((unsigned)nb), dim3(256), 0, s,
                           (const int32_t *)count, nkeys, offset, bsum);
    hipLaunchKernelGGL(k_ri_scan_top, dim3(1), dim3(1024), 0, s, bsum, nb);
    hipLaunchKernelGGL(k_ri_scan_add, dim3(nblk(nkeys + 1, 256)), dim3(256), 0, s, offset, count,
                       nkeys, (const int32_t *)bsum, nb);
    if (n > 0)
        hipLaunchKernelGGL(k_ri_fill, dim3(nblk(n, 256)), dim3(256), 0, s, key_of, n,
                           (const int32_t *)offset, count, list);
    hipLaunchKernelGGL(k_ri_sort, dim3(nblk(nkeys, 4)), dim3(256), 0, s,
                       (const int32_t *)offset, nkeys, list, inv);
    return hipGetLastError();
}

hipError_t fill_int(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_fill_int, dim3(nblk(n, 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t segment_sum(int nkeys, int W, const int32_t *offset, const int32_t *list,
                       const float *X, float *out, hipStream_t s) {
    if (nkeys <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_segment_sum, dim3(nblk(nkeys, 4)), dim3(256), 0, s, nkeys, W, offset,
                       list, X, out);
    return hipGetLastError();
}

} // namespace bwd
} // namespace waa
