// bwd.hpp -- kernels and launchers of the block's backward pass (internal).
//
// The backward pass works in fp32 throughout: inputs stored as bf16 are
// widened once, every intermediate the chain rule needs is recomputed from
// the inputs by the same kernels (dense products on the matrix cores, row
// and elementwise kernels, a slot-attention step that keeps its softmax
// weights), and gradients are fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace waa {
namespace bwd {

// A row-major fp32 matrix view: element (r, c) at p[r * ld + c].
struct View {
    float *p;
    int64_t ld;
};
inline View view(float *p, int64_t ld) { return View{p, ld}; }
inline View view(const float *p, int64_t ld) { return View{const_cast<float *>(p), ld}; }

// Operand of a product: element (r, c) at p[r * rs + c * cs] (a transposed
// operand is the same memory with the strides exchanged).
struct Mat {
    const float *p;
    int64_t rs, cs;
};
inline Mat mat(const float *p, int64_t ld) { return Mat{p, ld, 1}; }
inline Mat mat_t(const float *p, int64_t ld) { return Mat{p, 1, ld}; }

// Scratch of the products and column sums: `partial` (cap floats) for
// split reductions.
struct Scratch {
    float *partial;
    size_t cap;
};
constexpr size_t kGemmPartialFloats = (size_t)8 << 20;

// C[M, N] = beta * C + A[M, K] B[K, N] (+ bias[N]); beta is 0 or 1. Long
// reductions are split over workgroups and summed in a fixed order, so
// results are deterministic.
hipError_t gemm(int M, int N, int K, Mat A, Mat B, View C, float beta, const float *bias,
                Scratch sc, hipStream_t s);

// Independent products in one launch (no split k): job j computes
//   C_j (+)= sum over its segments i of A_i[M, K_i] B_i[K_i, N] (+ bias[N]),
// then applies its epilogue (GEMM_SIGMOID: sigmoid of the sum). Segments of
// one job are accumulated in order; every output element is written by one
// workgroup, so results do not depend on the grouping.
constexpr int kGroupJobs = 8, kGroupSegs = 4;
enum GemmEpi { GEMM_NONE, GEMM_SIGMOID };
struct GemmSeg {
    Mat A, B;
    int K;
};
struct GemmJob {
    int M, N;
    int nseg;
    GemmSeg seg[kGroupSegs];
    View C;
    float beta;
    const float *bias;
    int epi;
};
hipError_t gemm_group(const GemmJob *jobs, int n, hipStream_t s);

// Parameter-gradient leaves, up to kLeafJobs in two launches (split partial
// sums, then their reduction in a fixed order; results overwrite `out`):
//   kind 0: out[M][N] = A[M][K] B[K][N] (K the long axis, split);
//   kind 1: out[c] = sum over K rows r of A[r][c] (* B[r][c] when B.p), c < N
//           (A = mat(X, ldx), B = mat(Y, ldy) or a null pointer).
constexpr int kLeafJobs = 8;
struct LeafJob {
    int kind;
    int M, N, K;
    Mat A, B;
    float *out;
    int64_t ldo;
};
hipError_t leaf_group(const LeafJob *jobs, int n, Scratch sc, hipStream_t s);

// out[c] = beta * out[c] + sum_r X[r, c] (* Y[r, c] when Y.p), c < W.
hipError_t colsum(int rows, int W, View X, View Y, float *out, float beta, Scratch sc,
                  hipStream_t s);

// Elementwise operations over rows x W (o = op, or o += op when acc).
enum EwOp {
    EW_COPY,        // a
    EW_ADD,         // a + b
    EW_MUL,         // a * b
    EW_MUL_VEC,     // a * vec[c]
    EW_AFFINE,      // a * b + c
    EW_AFFINE1,     // a * (1 + b) + c
    EW_MUL1,        // a * (1 + b)
    EW_SIGMOID,     // sigmoid(a)
    EW_SIGMOID_VEC, // sigmoid(a + vec[c])
    EW_SILU,        // silu(a)
    EW_SWIGLU,      // silu(a) * b
    EW_RESID,       // a + b * c
    EW_RESID_MASK,  // mask[r] ? a + b * c : 0
    EW_MASK,        // mask[r] ? a : 0
    EW_DSIG,        // a * b * (1 - b)          (b = sigmoid output)
    EW_DGATE,       // a * b * c * (1 - c)      (c = sigmoid output)
    EW_DSWIGLU_A,   // a * c * silu'(b)
    EW_DSWIGLU_B,   // a * silu(b)
    EW_DSILU,       // a * silu'(b)
    EW_ADD_VEC,     // a + vec[c]
    EW_ZERO,        // 0
    EW_FMA2,        // a * b + c * d
    EW_MUL_VEC3,    // a * vec[c] + b * vec2[c] + c * vec3[c]
};
// A mask (one byte per row) zeroes the result of every row whose byte is 0.
hipError_t ew(EwOp op, int rows, int W, View o, View a, View b, View c, const float *vec,
              const uint8_t *mask, int acc, hipStream_t s);
// Independent elementwise jobs in one launch.
struct EwJob {
    EwOp op;
    int rows, W;
    View o, a, b, c, d;
    const float *vec, *vec2, *vec3;
    const uint8_t *mask;
    int acc;
};
hipError_t ew_group(const EwJob *jobs, int n, hipStream_t s);

// p[0..n) = v
hipError_t fill_int(int32_t *p, int64_t n, int32_t v, hipStream_t s);

// Row normalisation without affine terms (mode 0 LayerNorm, 1 RMS): xhat
// and the row's 1/sqrt(var + eps) (resp. 1/sqrt(mean x^2 + eps)).
hipError_t norm_rows(int mode, int rows, int W, float eps, View x, View xhat, float *rstd,
                     hipStream_t s);
// Its backward: given g = dL/dxhat, o (+)= dL/dx = rstd * (g - mean(g)
// - xhat * mean(g * xhat)) (LayerNorm) or rstd * (g - xhat * mean(g * xhat))
// (RMS).
hipError_t norm_rows_bwd(int mode, int rows, int W, View xhat, const float *rstd, View g,
                         View o, int acc, hipStream_t s);

// Storage dtype (0 fp32, 1 bf16) -> fp32, n elements; rows of width W with
// source row stride lds (W == lds for a flat copy); a row whose mask byte
// is 0 is written as zeros (mask may be null).
hipError_t to_f32(const void *src, int dtype, int64_t rows, int W, int64_t lds, float *dst,
                  const uint8_t *mask, hipStream_t s);

// ESMFold2 per-head RMS + rotary of Q and K rows (raw -> rotated), and its
// backward (rotated-row gradients -> raw-row gradients, plus the gradients
// of the rotary tables, summed over heads and over Q and K).
hipError_t head_rope(int rows, int H, int D, float eps, const float *qraw, const float *kraw,
                     const float *cs, const float *sn, float *q, float *k, hipStream_t s);
hipError_t head_rope_bwd(int rows, int H, int D, float eps, const float *qraw,
                         const float *kraw, const float *cs, const float *sn, float *dq,
                         float *dk, float *dcos, float *dsin, hipStream_t s);

// Decoder entry and sanitising: x0 = usable ? atom (+ tokproj[b, t]) : 0,
// c = usable ? condition : 0 (storage dtype -> fp32).
hipError_t sanitize(int B, int A, int T, int C, int S, int dtype, const void *atom,
                    const void *cond, const uint8_t *usable, const int64_t *a2t,
                    const float *tokproj, float *x0, float *c, hipStream_t s);

// Encoder pooling backward: dP = usable ? d_token_output[b, t] / count[b, t]
// * (proj > 0) : 0.
hipError_t pool_bwd(int B, int A, int T, int U, const uint8_t *usable, const int64_t *a2t,
                    const int32_t *count, const float *dto, const float *proj, float *dp,
                    hipStream_t s);

// Reverse index: for entries e < n with key_of[e] >= 0, list holds the
// entries of key k at offset[k] .. offset[k+1]-1, in ascending entry order
// for every key with at most kSortCap entries (longer lists keep their fill
// order).
// count/cursor: nkeys ints plus the scan's tile totals
// (reverse_index_count_ints(nkeys) ints in all).
constexpr int kSortCap = 2048;
inline int64_t reverse_index_count_ints(int64_t nkeys) { return nkeys + nkeys / 2048 + 2; }
// With inv (n ints), inv[e] = the position of entry e in list, for every
// listed entry (others are left as they were).
hipError_t reverse_index(const int32_t *key_of, int64_t n, int nkeys, int32_t *count,
                         int32_t *offset, int32_t *list, hipStream_t s, int32_t *inv = nullptr);

// out[k, :] = sum over list entries e of key k (in list order) of X[e, :].
hipError_t segment_sum(int nkeys, int W, const int32_t *offset, const int32_t *list,
                       const float *X, float *out, hipStream_t s);

// Token id b*T + t of each usable atom (else -1).
hipError_t token_keys(int B, int A, int T, const uint8_t *usable, const int64_t *a2t,
                      int32_t *key_of, hipStream_t s);

// Slot attention in fp32 with the softmax weights kept: P [B,H,A,K] (0 on
// slots that are not allowed), o [B*A, H*D], kid [B*A*K] = b*A + key for an
// allowed slot, else -1. AF3: pair [B,A,K,V] in the storage dtype, ps [V],
// wp [V,H] fp32.
struct SlotBwdArgs {
    int B, A, K, H, D, V;
    float eps;
    int64_t radius;
    int pair_dtype;
    const uint8_t *usable, *window_mask;
    const int64_t *key_index;
    const float *q, *k, *v;
    const void *pair;
    const float *ps, *wp;
    // forward results / backward inputs
    float *P, *o;
    int32_t *kid;
    // backward
    const float *d_att, *d_o; // d_att may be null
    // the logits' gradients and the weights in the key-major order of the
    // reverse index: [list position][H]
    float *dS, *Pk;
    int32_t *inv;             // [B*A*K]: list position of each allowed slot entry
    int32_t *wide;            // queue of 16-query blocks with a wide key band
                              // (count, then block ids; null: no block form)
    int rec0;                 // first pair-parameter record of a launch
    float *dq, *dk, *dv;      // [B*A, H*D]
    float *d_pair;            // [B,A,K,V] or null
    float *pw_partial;        // per-workgroup sums for d_pair_scale / d_w_pair
    int32_t *count, *offset, *list;
    Scratch sc;               // column-sum scratch
};
int slot_bwd_supported(int K, int H, int D, int V, int style);
hipError_t slot_fwd(const SlotBwdArgs &a, int style, hipStream_t s);
// The reverse index of kid; the query side: dS, dq, d_pair and the
// pair-parameter partial sums; then the key side: dk, dv.
hipError_t slot_bwd(const SlotBwdArgs &a, int style, float *d_pair_scale, float *d_w_pair,
                    hipStream_t s);
// Floats of pair-parameter partial sums slot_bwd uses for B batches of A
// query rows, and the ints of its queue of wide blocks.
size_t slot_bwd_partial_floats(int64_t B, int64_t A, int V, int H);
int64_t slot_bwd_queue_ints(int64_t B, int64_t A);
// Pair-parameter partial records slot_bwd writes (rows of
// kSlotPairRecord floats: [16] pair_scale sums, then [16][4] w_pair sums).
constexpr int kSlotPairRecord = 16 + 16 * 4;
int slot_bwd_records(const SlotBwdArgs &a);

} // namespace bwd
} // namespace waa
