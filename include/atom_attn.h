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
#define ATOM_ATTN_ESCRATCH (-6)     /* atom_attn_block_noalloc: the sizes
                                       need more scratch than its static
                                       buffer holds */

enum { ATOM_ATTN_AF3 = 0, ATOM_ATTN_ESMFOLD2 = 1 };
enum { ATOM_ATTN_F32 = 0, ATOM_ATTN_BF16 = 1 };
enum { ATOM_ATTN_ENCODER = 0, ATOM_ATTN_DECODER = 1 };

/* Sizes (all >= 1): B batches, A atoms per batch, T tokens per batch,
 * K key slots per atom, C atom width, S condition width, H heads, D head
 * width, V pair width (AF3; ignored for ESMFold2), M transition width,
 * U token width (encoder output width, decoder input width).
 * Supported set of the kernels: C, S, H*D, M, U multiples of 32 and at most
 * 512; D one of 16, 32, 64, 128; K <= 256; AF3: V a multiple of 8
 * with V*sizeof(dtype) <= 64 bytes and H <= 4; D*(A+39)*sizeof(dtype) <
 * 2^31 (the slot kernel's 32-bit offsets into one head's transposed value
 * rows). Float pointers and the workspace must be 16-byte aligned. */
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
    /* Optional: the weight matrices packed beforehand by
     * atom_attn_pack_params for calls with the same C, S, H*D, M, U, style,
     * stage and dtype (NULL = pack them in the call, into the workspace).
     * The other parameter pointers above are still required and read. */
    const void *packed;
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

/* Encoder stage of the block. Defined by "windowed_atom_attention -- Local
 * atom attention, encoder pooling and decoder skip/readout", Required
 * behavior (stage 'encoder': the encoder starts from the sanitised atom
 * features; token_output is the exact per-token mean of ReLU(hidden @
 * w_pool) over usable assigned atoms, empty tokens 0), and by the pages
 * "AlphaFold 3 Atom Attention Encoder" and "ESMFold 2 Atom Attention
 * Encoder" (Required behavior, Worked example) for the two styles.
 * eps > 0 is the stabiliser inside every LayerNorm / RMS root (used in
 * fp32); radius >= 0 additionally requires |key id - query id| <= radius,
 * radius == -1 disables that index window.
 * Outputs: hidden, attention, token_output (position_update unused).
 * Errors: the status codes above, all detected before any launch. */
int atom_attn_encoder(const atom_attn_dims *dims, int style, int dtype,
                      const atom_attn_inputs *in, const atom_attn_params *par,
                      double eps, int64_t radius, atom_attn_outputs *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Decoder stage. Defined by "windowed_atom_attention -- Local atom
 * attention, encoder pooling and decoder skip/readout", Required behavior
 * (stage 'decoder', the default there: entry state atom (skip) +
 * gather(token @ w_token, atom_to_token), bias-free, zero for unusable
 * atoms; position_update = (LN(hidden) * readout_scale [+ readout_bias for
 * ESMFold2]) @ w_readout, masked to zero, a coordinate update).
 * Same arguments as the encoder; outputs hidden, attention,
 * position_update (token_output unused). */
int atom_attn_decoder(const atom_attn_dims *dims, int style, int dtype,
                      const atom_attn_inputs *in, const atom_attn_params *par,
                      double eps, int64_t radius, atom_attn_outputs *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Masks alone, as the block uses them ("windowed_atom_attention", Required
 * behavior: the usability, slot-permission and radius bullets; the pooling
 * bullet for the counts): usable [B,A] = valid and 0 <= atom_to_token < T
 * and that token valid; allowed [B,A,K] = key id in [0,A), query and key
 * usable, window_mask, and the radius window; token_count [B,T] (int32) =
 * number of usable atoms assigned to each token, the denominator of the
 * encoder's token mean. Any of the three outputs may be NULL (not all).
 * Uses dims B, A, T, K and the inputs valid, token_valid, window_mask,
 * atom_to_token, key_index only. Errors: EINVAL for a bad argument,
 * EUNSUPPORTED for A > 2^30 or B*T >= 2^31. */
int atom_attn_masks(const atom_attn_dims *dims, const atom_attn_inputs *in,
                    int64_t radius, uint8_t *usable, uint8_t *allowed,
                    int32_t *token_count, void *stream);

/* The slot-attention step alone ("windowed_atom_attention", Required
 * behavior: the slot-permission, radius, pair-bias and attention-logit
 * bullets), on caller-supplied per-atom rows q, k, v [B,A,H*D] (head-major;
 * for ESMFold2 already RMS-normalised and rotated) and usable [B,A]. q and k
 * are fp32 whatever `dtype` is (the block keeps the logit operands in
 * fp32); v, pair, pair_scale, w_pair, attention and o use `dtype`. Computes
 * logits q.k/sqrt(D) (+ AF3 pair bias (LN(pair) * pair_scale) @ w_pair),
 * the softmax over the allowed slots with exact-zero empty rows, attention
 * [B,H,A,K] and o [B,A,H*D] = sum of weights times v rows -- with the same
 * kernel as the full block, after a copy of v into the transposed layout
 * that kernel reads (in `workspace`, atom_attn_slot_workspace_bytes()
 * bytes; rows of unusable atoms are copied as zeros, so their payload may
 * be NaN/Inf). Uses dims B, A, K, H, D, V; eps is used by the pair
 * LayerNorm. Errors: as the block, EUNSUPPORTED outside the slot kernel's
 * supported set. */
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

/* ---------------------------------------------------------------- backward
 * Gradients of the block ("windowed_atom_attention", Required behavior: the
 * block's steps, and the rule that a key atom selected by several slots --
 * of one query or of many -- receives the sum of the gradients of all those
 * selections; "AlphaFold 3 Atom Attention Encoder" / "ESMFold 2 Atom
 * Attention Encoder", Starter code: outputs are graded on values, shapes and
 * gradients). For upstream gradients g_hidden, g_attention, g_token_output
 * (encoder) or g_position_update (decoder), the call writes the derivative
 * of sum <output, g> with respect to every float input and parameter.
 *
 * All gradient buffers (upstream and written) are fp32, row-major, in the
 * shapes of the tensors they belong to, whatever `dtype` the inputs use;
 * every write overwrites (nothing is accumulated into caller buffers).
 * Upstream: hidden [B,A,C] (NULL = zero), attention [B,H,A,K], token_output
 * [B,T,U], position_update [B,A,3] (each NULL = zero). Written gradients:
 * any pointer may be NULL (not computed). Entries of unusable atoms, of
 * slots that are not allowed and of invalid tokens get exact zeros: their
 * payloads never enter the arithmetic. rope_cos / rope_sin receive the sum
 * over heads of Q's and K's rotary terms (ESMFold2).
 *
 * The call recomputes the forward in fp32 from the inputs (its own kernels;
 * results may differ from the forward call's in the last bits), then runs
 * the chain rule on the device. Sums over atoms (parameter gradients) and
 * over selections of a key (key and value rows) are taken in a fixed order
 * with no floating-point atomics, so repeated calls give identical bits --
 * except that a key atom selected by more than 2048 slots sums them in the
 * order the reverse index was filled.
 *
 * Supported set: K <= 512; H <= 8; D one of 8, 16, 32, 64; H*D <= 256;
 * AF3: V <= 16 and H <= 4; C, S, M, U <= 4096; B*A < 2^30;
 * B*A*K*max(H, V) < 2^31; B*A*max(6C, S, M, U, H*D) <= 2^34. Otherwise
 * EUNSUPPORTED. Status codes as the block
 * call; workspace (256-byte aligned) of atom_attn_backward_workspace_bytes()
 * bytes. Asynchronous on `stream`. */
typedef struct {
    const float *hidden, *attention, *token_output, *position_update;
} atom_attn_grad_outputs;
typedef struct {
    float *atom, *condition, *pair, *token, *rope_cos, *rope_sin;
} atom_attn_input_grads;
typedef struct {
    float *cond_scale, *w_scale, *b_scale, *w_shift, *w_residual_gate,
        *b_residual_gate;
    float *w_mod;
    float *w_q, *b_q, *w_k, *w_v, *pair_scale, *w_pair, *w_value_gate,
        *w_attention_out;
    float *w_ff_gate, *w_ff_up, *w_ff_out;
    float *w_pool, *w_token, *readout_scale, *readout_bias, *w_readout;
} atom_attn_param_grads;
int atom_attn_backward_workspace_bytes(const atom_attn_dims *dims, int style,
                                       int stage, int dtype, size_t *bytes);
int atom_attn_backward(const atom_attn_dims *dims, int style, int stage,
                       int dtype, const atom_attn_inputs *in,
                       const atom_attn_params *par, double eps, int64_t radius,
                       const atom_attn_grad_outputs *grad_out,
                       atom_attn_input_grads *grad_in,
                       atom_attn_param_grads *grad_par, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Gradients of the slot-attention step alone ("windowed_atom_attention",
 * Required behavior: the slot-permission, radius, pair-bias, logit and
 * repeated-selection bullets), in fp32: q, k, v [B,A,H*D] fp32 (16-byte
 * aligned), usable [B,A], key_index / window_mask [B,A,K]; AF3 pair
 * [B,A,K,V], pair_scale [V], w_pair [V,H] in `dtype`. Upstream d_o
 * [B,A,H*D] and d_attention [B,H,A,K] (NULL = zero), fp32. Writes dq, dk,
 * dv [B,A,H*D] and, AF3, d_pair [B,A,K,V], d_pair_scale [V], d_w_pair [V,H]
 * (each NULL = not computed); attention [B,H,A,K] and o [B,A,H*D] receive
 * the recomputed fp32 forward when not NULL. Supported set and ordering of
 * sums as atom_attn_backward (dims T, C, S, M, U are not read). */
int atom_attn_slot_backward_workspace_bytes(const atom_attn_dims *dims,
                                            int style, size_t *bytes);
int atom_attn_slot_attention_backward(
    const atom_attn_dims *dims, int style, int dtype, double eps,
    int64_t radius, const uint8_t *usable, const float *q, const float *k,
    const float *v, const int64_t *key_index, const uint8_t *window_mask,
    const void *pair, const void *pair_scale, const void *w_pair,
    const float *d_attention, const float *d_o, float *attention, float *o,
    float *dq, float *dk, float *dv, float *d_pair, float *d_pair_scale,
    float *d_w_pair, void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the block
 * call of atom_attn_encoder (stage ATOM_ATTN_ENCODER) or atom_attn_decoder
 * (stage ATOM_ATTN_DECODER) with the same arguments, results and status
 * codes, minus the workspace. Its scratch memory is a static array inside
 * the library, atom_attn_noalloc_max_bytes() bytes (64 MiB) per device,
 * which each GPU the library runs on holds from its first such call until
 * the process ends. The call allocates and frees nothing. Sizes whose
 * atom_attn_workspace_bytes() exceeds that maximum are rejected with
 * ATOM_ATTN_ESCRATCH before anything is enqueued. Every call on a device
 * shares that device's array (nothing in it is assumed to start at zero):
 * calls that may overlap on one GPU -- on different streams, or from
 * different host threads -- race and must be serialised by the caller. */
size_t atom_attn_noalloc_max_bytes(void);
int atom_attn_block_noalloc(const atom_attn_dims *dims, int style, int stage,
                            int dtype, const atom_attn_inputs *in,
                            const atom_attn_params *par, double eps,
                            int64_t radius, atom_attn_outputs *out,
                            void *stream);

/* The windowed slot table on the device (the layout of local windows the
 * block's key_index input describes; "windowed_atom_attention", Required
 * behavior, takes key ids as supplied data, this builds such data): for
 * every batch and query atom a, key_index[b,a,k] = q0 - (K-block)/2 + k with
 * q0 = block*floor(a/block), i.e. each block of `block` consecutive queries
 * sees the K consecutive ids centred on it. Ids outside [0, A) and, for
 * radius >= 0, ids with |id - a| > radius are written as -1 (missing slots
 * either way, so a block call gives the same results with or without
 * them). Writes [B,A,K] ids of index_bytes = 8 (int64, the block's
 * key_index type) or 4 (int32) into caller-owned device memory on
 * `stream`. Errors: EINVAL for a size < 1, radius < -1, an index size
 * other than 4 or 8 or a NULL output; EUNSUPPORTED for A > 2^29 or
 * B*A*K >= 2^31. */
int atom_attn_window_table(int64_t B, int64_t A, int64_t K, int64_t block,
                           int64_t radius, int index_bytes, void *key_index,
                           void *stream);

/* Single-to-pair features ("ESMFold Single-to-Pair Features", Required
 * behavior and Worked example). Tokens x [B,N,C] with presence mask [B,N]
 * (one byte, 0 = absent; absent payloads may be NaN/Inf and are never read
 * into arithmetic): y = (LN(x) * norm_scale + norm_bias) @ weight + bias
 * (population LayerNorm, eps inside the root; weight [C,2H] stored
 * [in][out], bias [2H], norm_scale/norm_bias [C]); q = y[:H], k = y[H:];
 * pair_features[b,i,j] = [k_i * q_j, q_j - k_i] ([B,N,N,2H]);
 * output[b,i,j] = pair_features[b,i,j] @ out_weight + out_bias
 * (out_weight [2H,D], out_bias [D]), then, if output_norm, LN(.) *
 * output_scale + output_bias ([D] each, may be NULL otherwise); both
 * outputs are zero unless tokens i and j are both present. Float tensors
 * share `dtype` (arithmetic fp32; for bf16 the features are rounded to
 * bf16 once and the output is computed from those rounded values). Output
 * pointers and `weight` 16-byte aligned. Supported: H in {32, 64} (and 128 for bf16),
 * D in {64, 128, 256}, C <= 4096, B*N <= 2^24. Workspace: fp32 q|k rows,
 * atom_attn_single_to_pair_workspace_bytes() bytes. Errors: EINVAL,
 * EWORKSPACE, EUNSUPPORTED, ELAUNCH as for the block. */
typedef struct {
    int64_t B, N, C, H, D;
} atom_attn_s2p_dims;
int atom_attn_single_to_pair_workspace_bytes(const atom_attn_s2p_dims *dims,
                                             int dtype, size_t *bytes);
int atom_attn_single_to_pair(const atom_attn_s2p_dims *dims, int dtype,
                             double eps, int output_norm, const void *x,
                             const uint8_t *mask, const void *weight,
                             const void *bias, const void *norm_scale,
                             const void *norm_bias, const void *out_weight,
                             const void *out_bias, const void *output_scale,
                             const void *output_bias, void *pair_features,
                             void *output, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Tied pair row attention ("Tied Pair Row Attention", Required behavior
 * and Worked example). features [B,L,L,C] and bias_features [B,L,L,CB]
 * (a pair grid and its bias features); both pair axes are exchanged first
 * and the update's axes exchanged back, so that for output position (a, c)
 *   A[h][i][j] = softmax_j( sum_{s,d} q(F[i][s])[h,d] k(F[j][s])[h,d]
 *                           / sqrt(L*D) + beta_h(Fb[j][i]) )
 *   out[a][c] = (g(F[a][c]) * sum_j A[h][c][j] v(F[j][a])) @ w_out + b_out
 * with F normalised by affine population LayerNorm (norm_scale, norm_bias
 * [C]; eps inside the root), q, k, v = . @ w_q, w_k, w_v and the value gate
 * g = sigmoid(. @ w_gate) (all [C,H*D], bias-free), beta_h = (LN(Fb) *
 * bias_norm_scale + bias_norm_bias) @ w_bias[:, h] (w_bias [CB,H]), w_out
 * [H*D,C], b_out [C]. The update is written to `output` [B,L,L,C]; no
 * residual is added. Float tensors share `dtype` (arithmetic fp32; bf16
 * keeps q, k, v, the gate and the attention weights in bf16 between
 * kernels). Supported: D = 32, H <= 8, C a multiple of 32 <= 256,
 * CB <= 1024, L <= 1024, B*L*L <= 2^26; features and output 16-byte
 * aligned. Workspace: atom_attn_tied_row_attention_workspace_bytes(). */
typedef struct {
    int64_t B, L, C, CB, H, D;
} atom_attn_tied_dims;
int atom_attn_tied_row_attention_workspace_bytes(const atom_attn_tied_dims *dims,
                                                 int dtype, size_t *bytes);
int atom_attn_tied_row_attention(const atom_attn_tied_dims *dims, int dtype,
                                 double eps, const void *features,
                                 const void *bias_features,
                                 const void *norm_scale, const void *norm_bias,
                                 const void *bias_norm_scale,
                                 const void *bias_norm_bias, const void *w_q,
                                 const void *w_k, const void *w_v,
                                 const void *w_bias, const void *w_gate,
                                 const void *w_out, const void *b_out,
                                 void *output, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Weight packing ahead of time (not a step of the method: the block
 * reorders its weight matrices into the matrix cores' operand order, and a
 * caller that keeps one parameter set across calls can do that once).
 * atom_attn_packed_bytes gives the size of the packed copy of the matrices
 * a call with these sizes reads (host-only); atom_attn_pack_params writes it
 * into `packed` (device, 16-byte aligned, caller-owned) on `stream`, for
 * every grid size: both operand layouts the projection kernels use. Pass
 * it as atom_attn_params.packed to block calls with the same C, S, H*D, M,
 * U, style, stage and dtype; it stays valid until the caller changes the
 * matrices. Errors as atom_attn_workspace_bytes, EINVAL for a missing or
 * misaligned matrix, EWORKSPACE for a missing or small `packed`. */
int atom_attn_packed_bytes(const atom_attn_dims *dims, int style, int stage,
                           int dtype, size_t *bytes);
int atom_attn_pack_params(const atom_attn_dims *dims, int style, int stage,
                          int dtype, const atom_attn_params *par, void *packed,
                          size_t packed_bytes, void *stream);

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
