// kernels.hpp -- argument blocks and host launchers of the libatomattn
// kernels (internal to the library; the public ABI is include/atom_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace waa {

enum { STYLE_AF3 = 0, STYLE_ESM = 1 };
enum { STAGE_ENCODER = 0, STAGE_DECODER = 1 };

struct Dims {
    int B, A, T, K, C, S, H, D, V, M, U;
};

// V is stored transposed per batch, [B][H*D][vt_pitch(A)], so that the slot
// kernel's P V product reads 8 (bf16) or 4 (fp32) consecutive key rows of one
// channel as one 16-byte vector. Columns A .. pitch-1 hold zeros (written by
// the kernel that writes V): a 32-row P V chunk of a band that ends at the
// batch's last atom then reads whole vectors, zeros past the end.
__host__ __device__ inline int vt_pitch(int A) { return ((A + 7) & ~7) + 32; }

// Offsets, in 16-byte units, of each packed weight matrix inside the packed
// area of the workspace (-1 = absent).
struct PackedOffsets {
    int64_t w_scale[3], w_shift[3], w_rg[2], w_mod[6];
    int64_t w_q, w_k, w_v, w_vg, w_ao, ff_gate, ff_up, ff_out, w_pool, w_token;
};

// Everything the projection, post and pool kernels read or write.
struct BlockArgs {
    Dims d;
    float eps;
    int64_t radius;
    // inputs
    const void *atom, *condition, *pair, *token, *rope_cos, *rope_sin;
    const uint8_t *valid, *token_valid, *window_mask;
    const int64_t *atom_to_token, *key_index;
    // vector parameters (read directly, storage dtype)
    const void *cond_scale, *b_scale, *b_rg, *b_q, *readout_scale,
        *readout_bias, *w_readout;
    // packed matrices
    const uint4 *pk;
    PackedOffsets off;
    // workspace
    void *q, *k, *v, *g, *o;
    uint8_t *usable;
    float *tokproj;
    // encoder pooling records, one per 32-row tile: first / last segment
    // sums [tile][2][U] and [tile][8] ints (segments, first key, first
    // count, last key, last count)
    float *pool_sum;
    int *pool_int;
    // post kernel: stream the whole transition width in one pass (set by
    // its launcher)
    int post_wide;
    // grid of at most one tile per CU: the projection and post kernels run
    // eight waves per workgroup with 32x16 output strips, and their
    // matrices are packed in the strip layout
    int nw8;
    // AF3 pair bias computed by extra workgroups of the projection kernel
    // (when its tiles leave most of the GPU idle): pbias[slot][4] fp32, the
    // bias of heads 0..3 of every slot (b, a, k); null when the slot kernel
    // computes it from the pair rows itself
    const void *pair_scale, *w_pair;
    float *pbias;
    // the slot step's queue of wide query blocks (wide[0] = count, set to 0
    // by the projection kernel)
    int *wide;
    // outputs
    void *hidden, *attention, *token_output, *position_update;
    int32_t *status;
};

// The slot-attention kernel's arguments.
struct SlotArgs {
    int B, A, K, H, D, V;  // v is transposed: [B][H*D][vt_pitch(A)]
    float eps, inv_sqrt_d;
    int64_t radius;
    const uint8_t *usable, *window_mask;
    const int64_t *key_index;
    const void *q, *k, *v, *pair, *pair_scale, *w_pair;
    // AF3: the pair bias of every slot, [B*A*K][4] fp32, when precomputed
    // (then pair, pair_scale and w_pair are not read); null otherwise
    const float *pbias;
    void *attention, *o;
    // query blocks whose key band spans more than kWideChunks chunks are
    // queued here (wide[0] = count, zeroed before the slot kernel; wide[1..]
    // = block ids) and computed by k_slot_gather from row-major V rows
    // vrows; null: every block stays in the slot kernel. vrows_out (may be
    // null): the slot kernel writes each block's 16 V rows there, row-major,
    // from the transposed copy (vrows then points to the same buffer).
    int *wide;
    const void *vrows;
    void *vrows_out;
};
constexpr int kWideChunks = 8;

// Kernel timing with HIP events for the library's profiling mode (a no-op
// unless atom_attn_profile_enable is on): prof_begin before a launch and
// prof_end after it, on the launch stream. Ids past the block's kernels:
enum { KN_S2P_TOK = 7, KN_S2P_PAIR = 8, KN_WINDOW = 9, KN_TIED_BIAS = 10, KN_TIED_PROJ = 11,
       KN_TIED_LOGITS = 12, KN_TIED_SOFTMAX = 13, KN_TIED_OUT = 14,
       // backward pass: forward recomputation, its slot step, the slot
       // backward (query side, reverse index + key side), the dense chain
       KN_BWD_RECOMPUTE = 15, KN_BWD_SLOT_FWD = 16, KN_BWD_SLOT_Q = 17, KN_BWD_SLOT_KV = 18,
       KN_BWD_CHAIN = 19, KN_SLOT_GATHER = 20 };
struct ProfSpan {
    int kernel = -1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
};
ProfSpan prof_begin(int kernel, hipStream_t s);
void prof_end(const ProfSpan &sp, hipStream_t s);

// Single-to-pair features (pair_s2p.hip): tokens x [B,N,C], mask [B,N];
// weight [C,2H], bias [2H], norm_scale/norm_bias [C], out_weight [2H,D],
// out_bias [D], output_scale/output_bias [D]; outputs pair_features
// [B,N,N,2H], output [B,N,N,D]; qk: workspace, fp32 [B,N,2H] (q then k).
struct S2PArgs {
    int B, N, C, H, D;
    float eps;
    const void *x;
    const uint8_t *mask;
    const void *weight, *bias, *norm_scale, *norm_bias, *out_weight, *out_bias,
        *output_scale, *output_bias;
    float *qk;
    const uint4 *wo_packed; // workspace: out_weight in MFMA B-fragment order
    void *pair_features, *output;
};
hipError_t launch_s2p(const S2PArgs &a, int dtype, int output_norm, hipStream_t s);
int s2p_supported(int64_t C, int64_t H, int64_t D, int dtype);
size_t s2p_tok_lds(int C, int H);
size_t s2p_pair_lds(int H, int D, int esz);

// One matrix to pack: src[r*ld + c] for r < kd, c < n (storage dtype).
struct PackJob {
    const void *src;
    int64_t ld;
    int32_t kd, n;
    int64_t dst; // offset in 16-byte units
    int32_t strip; // 1: 16-column strip layout (8-wave kernels), 0: 32-column blocks
};
constexpr int kMaxPackJobs = 32;
struct PackArgs {
    PackJob job[kMaxPackJobs];
    int njobs;
    int64_t total; // 16-byte units over all jobs
    uint4 *out;
};

// 16-byte units a packed [kd x n] matrix takes (kd, n multiples of 32).
inline int64_t packed_units(int kd, int n, int dtype_bytes) {
    return (int64_t)kd * n * dtype_bytes / 16;
}

// Whether the projection kernel also computes the AF3 pair bias (fp32, or
// bf16 pair rows of at most 16 channels): when its tiles leave a quarter of
// the compute units or more idle, extra workgroups (one per idle unit)
// compute the bias there and the slot kernel's pair-row phase disappears.
bool prep_hosts_pair_bias(const Dims &d, int dtype, int style, int stage);

// Host launchers; dtype 0 = fp32, 1 = bf16.
hipError_t launch_pack(const PackArgs &a, int dtype, hipStream_t s);
hipError_t launch_token_proj(const BlockArgs &a, int dtype, hipStream_t s);
hipError_t launch_prep(const BlockArgs &a, int dtype, int style, int stage,
                       hipStream_t s);
hipError_t launch_post(const BlockArgs &a, int dtype, int style, int stage,
                       hipStream_t s);
hipError_t launch_pool(const BlockArgs &a, int dtype, hipStream_t s);
hipError_t launch_slot(const SlotArgs &a, int dtype, int style, hipStream_t s);
// the queued wide blocks of the last launch_slot (exits at once when none)
hipError_t launch_slot_gather(const SlotArgs &a, int dtype, int style, hipStream_t s);
size_t slot_gather_lds_bytes(int K, int H, int D);
// transposed copy of v for the standalone slot step; also sets wide[0] = 0
// when wide is not null
hipError_t launch_vt(const void *v, const uint8_t *usable, void *vt, int B, int A,
                     int HD, int dtype, int *wide, hipStream_t s);
hipError_t launch_masks(const Dims &d, const uint8_t *valid,
                        const uint8_t *token_valid, const uint8_t *window_mask,
                        const int64_t *atom_to_token, const int64_t *key_index,
                        int64_t radius, uint8_t *usable, uint8_t *allowed,
                        int32_t *token_count, hipStream_t s);

// LDS bytes each kernel needs for these sizes (host-side shape checks).
size_t prep_lds_bytes(const Dims &d, int dtype, int style, int stage);
size_t post_lds_bytes(const Dims &d, int dtype, int style);
size_t token_proj_lds_bytes(const Dims &d, int dtype);
size_t slot_lds_bytes(const Dims &d, int dtype, int style);
int slot_supported(const Dims &d, int dtype, int style);

constexpr size_t kMaxLds = 160 * 1024;

// Raise a kernel's dynamic-LDS limit to `bytes` if it is lower (the runtime
// call is made only when a launch needs more than any launch before).
void allow_lds(const void *fn, size_t bytes);

// Compute units of the current device (cached per device).
int device_cus();

} // namespace waa
