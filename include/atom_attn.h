/*
 * atom_attn.h -- C ABI of libatomattn.so, the windowed atom-attention block
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the page "windowed_atom_attention -- Local atom
 * attention, encoder pooling and decoder skip/readout" defines (Required
 * behavior), with its two encoder special cases on the pages "AlphaFold 3
 * Atom Attention Encoder" and "ESMFold 2 Atom Attention Encoder": each atom
 * attends over its supplied key slots under usability, window_mask and an
 * optional index radius; AF3 style uses adaptive LayerNorm, a pair-logit
 * bias and sigmoid residual gates, ESMFold2 style uses SiLU(condition)@w_mod
 * RMS modulation, per-head Q/K RMS norm, half-split rotary and raw gates;
 * then the gated transition, and either encoder mean-pooling to tokens or
 * the decoder token-gather skip with a coordinate-update readout.
 *
 * Conventions shared by every entry point:
 *  - Pointers to tensors are DEVICE pointers to caller-owned, contiguous,
 *    row-major buffers. Float tensors all have the dtype given by `dtype`
 *    (ATOM_ATTN_F32: IEEE fp32; ATOM_ATTN_BF16: bfloat16 storage; arithmetic
 *    is fp32 in both). Index tensors are int64, masks one byte per element
 *    (0 = False, anything else = True).
 *  - Parameter matrices are stored [in][out] (a projection is x @ W).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work; outputs are valid once the stream has run it.
 *    No call synchronises the host, allocates or frees memory, or writes
 *    any input.
 *  - Scratch memory comes from the caller's `workspace`, sized by
 *    atom_attn_workspace_bytes(); it must stay untouched until the stream
 *    has finished the call. Two calls that run concurrently need separate
 *    workspaces.
 *  - Every call returns an int status (never throws): ATOM_ATTN_OK or a
 *    negative code below. Argument and shape checks happen on the host
 *    before anything is enqueued. Data values are never errors: NaN/Inf
 *    payloads of unusable atoms, missing (-1 or out-of-range) key ids and
 *    all-missing rows are part of the semantics.
 */
#ifndef ATOM_ATTN_H
#define ATOM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ATOM_ATTN_OK 0
#define ATOM_ATTN_EINVAL (-1)       /* bad enum, dim < 1, NULL pointer the
                                       style/stage needs, eps not finite and
                                       > 0 in the dtype, radius < -1 */
#define ATOM_ATTN_EODD_HEAD (-2)    /* ESMFold2 with odd head width D */
#define ATOM_ATTN_EWORKSPACE (-3)   /* workspace NULL or too small */
#define ATOM_ATTN_ELAUNCH (-4)      /* the HIP runtime refused a launch */
#define ATOM_ATTN_EUNSUPPORTED (-5) /* shape outside the kernels' supported
                                       set (see atom_attn_error_string) */

enum { ATOM_ATTN_AF3 = 0, ATOM_ATTN_ESMFOLD2 = 1 };
enum { ATOM_ATTN_F32 = 0, ATOM_ATTN_BF16 = 1 };
enum { ATOM_ATTN_ENCODER = 0, ATOM_ATTN_DECODER = 1 };

/* Sizes (all >= 1): B batches, A atoms per batch, T tokens per batch,
 * K key slots per atom, C atom width, S condition width, H heads, D head
 * width, V pair width (AF3; ignored for ESMFold2), M transition width,
 * U token width (encoder output width, decoder input width).
 * Supported set of the kernels: C, S, H*D, M, U multiples of 32 and at most
 * 512; D one of 16, 32, 64, 128; K <= 256; AF3: V a multiple of 8
 * with V*sizeof(dtype) <= 64 bytes, H <= 8, and H <= 4 when K > 128.
 * Float pointers and the workspace must be 16-byte aligned. */
typedef struct {
    int64_t B, A, T, K, C, S, H, D, V, M, U;
} atom_attn_dims;

/* Inputs ("activations", "masks" and "structure" on the pages).
 *  atom [B,A,C], condition [B,A,S]; pair [B,A,K,V] (AF3 only, per-slot
 *  descriptors); token [B,T,U] (decoder only); rope_cos / rope_sin [B,A,D]
 *  (ESMFold2 only, full-width, shared by every head); valid [B,A];
 *  token_valid [B,T]; window_mask [B,A,K]; atom_to_token [B,A];
 *  key_index [B,A,K] (within-batch atom ids; ids outside [0,A) are
 *  missing). Unused pointers may be NULL. */
typedef struct {
    const void *atom, *condition, *pair, *token, *rope_cos, *rope_sin;
    const uint8_t *valid, *token_valid, *window_mask;
    const int64_t *atom_to_token, *key_index;
} atom_attn_inputs;

/* Parameters (names as on the pages; w_q/w_k/w_v are the Q/K/V weights).
 *  AF3:     cond_scale [3,S], w_scale [3,S,C], b_scale [3,C],
 *           w_shift [3,S,C], w_residual_gate [2,S,C], b_residual_gate [2,C],
 *           b_q [H*D], pair_scale [V], w_pair [V,H]
 *  ESMFold2: w_mod [S,6,C] (attention shift, scale, gate; transition
 *           shift, scale, gate)
 *  both:    w_q, w_k, w_v, w_value_gate [C,H*D], w_attention_out [H*D,C],
 *           w_ff_gate, w_ff_up [C,M], w_ff_out [M,C]
 *  encoder: w_pool [C,U]
 *  decoder: w_token [U,C], readout_scale [C], readout_bias [C] (ESMFold2),
 *           w_readout [C,3]
 * The value gate is per channel: sigmoid(query-side input @ w_value_gate)
 * multiplies each head's D coordinates elementwise. */
typedef struct {
    const void *cond_scale, *w_scale, *b_scale, *w_shift, *w_residual_gate,
        *b_residual_gate;
    const void *w_mod;
    const void *w_q, *b_q, *w_k, *w_v, *pair_scale, *w_pair, *w_value_gate,
        *w_attention_out;
    const void *w_ff_gate, *w_ff_up, *w_ff_out;
    const void *w_pool, *w_token, *readout_scale, *readout_bias, *w_readout;
} atom_attn_params;

/* Outputs: hidden [B,A,C], attention [B,H,A,K], token_output [B,T,U]
 * (encoder) or position_update [B,A,3] (decoder), in the float dtype.
 * status (optional, device int32, may be NULL): set to 0 by the call, and
 * to 1 if the encoder's usable atoms are not sorted by atom_to_token within
 * a batch -- the pooling kernel's precondition; token_output is then
 * unspecified (no fault, no other output affected). */
typedef struct {
    void *hidden, *attention, *token_output, *position_update;
    int32_t *status;
} atom_attn_outputs;

/* Workspace bytes a call with these sizes needs (host-only, no GPU work). */
int atom_attn_workspace_bytes(const atom_attn_dims *dims, int style,
                              int stage, int dtype, size_t *bytes);

/* Encoder stage of the block (token_output = exact per-token mean of
 * ReLU(hidden @ w_pool) over usable assigned atoms; empty tokens 0).
 * eps > 0 is the stabiliser inside every LayerNorm / RMS root (used in
 * fp32); radius >= 0 additionally requires |key id - query id| <= radius,
 * radius == -1 disables that index window. */
int atom_attn_encoder(const atom_attn_dims *dims, int style, int dtype,
                      const atom_attn_inputs *in, const atom_attn_params *par,
                      double eps, int64_t radius, atom_attn_outputs *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Decoder stage (entry state atom + gather(token @ w_token, atom_to_token);
 * position_update = masked (LN(hidden) * readout_scale [+ readout_bias])
 * @ w_readout, a coordinate update). Same arguments as the encoder. */
int atom_attn_decoder(const atom_attn_dims *dims, int style, int dtype,
                      const atom_attn_inputs *in, const atom_attn_params *par,
                      double eps, int64_t radius, atom_attn_outputs *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Masks alone, as the block uses them ("windowed_atom_attention", Required
 * behavior): usable [B,A] = valid and 0 <= atom_to_token < T and that
 * token valid; allowed [B,A,K] = key id in [0,A), query and key usable,
 * window_mask, and the radius window. Uses dims B, A, T, K only. */
int atom_attn_masks(const atom_attn_dims *dims, const atom_attn_inputs *in,
                    int64_t radius, uint8_t *usable, uint8_t *allowed,
                    void *stream);

/* The slot-attention step alone, on caller-supplied per-atom rows q, k, v
 * [B,A,H*D] (head-major; for ESMFold2 already RMS-normalised and rotated)
 * and usable [B,A]. q and k are fp32 whatever `dtype` is (the block keeps
 * the logit operands in fp32); v, pair, pair_scale, w_pair, attention and
 * o use `dtype`. Computes logits q.k/sqrt(D) (+ AF3 pair bias
 * (LN(pair) * pair_scale) @ w_pair), the softmax over the allowed slots
 * with exact-zero empty rows, attention [B,H,A,K] and o [B,A,H*D] = sum of
 * weights times v rows -- with the same kernel as the full block, after a
 * copy of v into the transposed layout that kernel reads (in `workspace`,
 * atom_attn_slot_workspace_bytes() bytes). Uses dims B, A, K, H, D, V; eps
 * is used by the pair LayerNorm. */
int atom_attn_slot_workspace_bytes(const atom_attn_dims *dims, int dtype,
                                   size_t *bytes);
int atom_attn_slot_attention(const atom_attn_dims *dims, int style, int dtype,
                             double eps, int64_t radius, const uint8_t *usable,
                             const void *q, const void *k, const void *v,
                             const int64_t *key_index,
                             const uint8_t *window_mask, const void *pair,
                             const void *pair_scale, const void *w_pair,
                             void *attention, void *o, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Where a block call with these sizes computes the AF3 pair bias on the
 * current device (host-only, no GPU work; the compute-unit count of the
 * current device decides): *split = 1 when extra workgroups of the
 * projection kernel compute it on compute units its 32-atom tiles leave
 * idle and the slot kernel reads it back (16 bytes per slot, in the
 * workspace); 0 when the slot kernel computes it from the pair rows
 * (always 0 for ESMFold2, which has no pair input). The results are the
 * same either way. Status codes as atom_attn_workspace_bytes. */
int atom_attn_pair_bias_split(const atom_attn_dims *dims, int style, int stage,
                              int dtype, int *split);

/* Static description of a status code (never NULL). */
const char *atom_attn_error_string(int code);

/* Library ABI version (incremented on any signature change). */
int atom_attn_version(void);

/* Kernel timing with HIP events, for benchmarks. While enabled, every
 * kernel a call enqueues is bracketed by two events on the caller's stream.
 * atom_attn_profile_read() waits for the recorded events, writes up to
 * `max` per-kernel totals (name, summed milliseconds, launch count) and
 * clears them; it returns the number of kernels written or a negative
 * status. Not thread-safe; meant for single-threaded benchmark drivers. */
int atom_attn_profile_enable(int on);
int atom_attn_profile_read(const char **names, double *total_ms,
                           int64_t *launches, int max);

#ifdef __cplusplus
}
#endif
#endif
