/*
 * oracle.h -- plain fp64 CPU oracle of the windowed atom-attention block.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library includes,
 * links or calls this file; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it. It shares no code, header,
 * table or helper with the HIP implementation.
 *
 * What it computes follows the pages "windowed_atom_attention -- Local atom
 * attention, encoder pooling and decoder skip/readout" (Required behavior),
 * "AlphaFold 3 Atom Attention Encoder" (Required behavior, Worked example)
 * and "ESMFold 2 Atom Attention Encoder" (Required behavior, Worked example).
 *
 * Every float array is fp64, contiguous, row-major, on the host. Index
 * arrays are int64, mask arrays are one byte per element (0 = False).
 * Matrices are stored [in][out], so a projection is y = x @ W.
 */
#ifndef WAA_ORACLE_H
#define WAA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_AF3 = 0, ORC_ESMFOLD2 = 1 };
enum { ORC_ENCODER = 0, ORC_DECODER = 1 };

/* B batches, A atoms, T tokens, K key slots, C atom width, S condition
 * width, H heads, D head width, V pair width, M transition width, U token
 * width. */
typedef struct {
    int64_t B, A, T, K, C, S, H, D, V, M, U;
} orc_dims;

typedef struct {
    const double *atom;        /* [B,A,C] */
    const double *condition;   /* [B,A,S] */
    const double *pair;        /* [B,A,K,V]  AF3 only */
    const double *token;       /* [B,T,U]    decoder only */
    const double *rope_cos;    /* [B,A,D]    ESMFold2 only */
    const double *rope_sin;    /* [B,A,D]    ESMFold2 only */
    const uint8_t *valid;       /* [B,A] */
    const uint8_t *token_valid; /* [B,T] */
    const uint8_t *window_mask; /* [B,A,K] */
    const int64_t *atom_to_token; /* [B,A] */
    const int64_t *key_index;     /* [B,A,K] */
} orc_inputs;

typedef struct {
    /* AF3 conditioning */
    const double *cond_scale;      /* [3,S] */
    const double *w_scale;         /* [3,S,C] */
    const double *b_scale;         /* [3,C] */
    const double *w_shift;         /* [3,S,C] */
    const double *w_residual_gate; /* [2,S,C] */
    const double *b_residual_gate; /* [2,C] */
    /* ESMFold2 conditioning */
    const double *w_mod;           /* [S,6,C] */
    /* attention */
    const double *w_q;             /* [C,H*D] */
    const double *b_q;             /* [H*D]   AF3 only */
    const double *w_k;             /* [C,H*D] */
    const double *w_v;             /* [C,H*D] */
    const double *pair_scale;      /* [V]     AF3 only */
    const double *w_pair;          /* [V,H]   AF3 only */
    const double *w_value_gate;    /* [C,H*D] */
    const double *w_attention_out; /* [H*D,C] */
    /* transition */
    const double *w_ff_gate;       /* [C,M] */
    const double *w_ff_up;         /* [C,M] */
    const double *w_ff_out;        /* [M,C] */
    /* stage boundary */
    const double *w_pool;          /* [C,U]  encoder */
    const double *w_token;         /* [U,C]  decoder */
    const double *readout_scale;   /* [C]    decoder */
    const double *readout_bias;    /* [C]    decoder, ESMFold2 only */
    const double *w_readout;       /* [C,3]  decoder */
} orc_params;

typedef struct {
    /* block outputs (required) */
    double *hidden;          /* [B,A,C] */
    double *attention;       /* [B,H,A,K] */
    double *token_output;    /* [B,T,U]  encoder */
    double *position_update; /* [B,A,3]  decoder */
    /* optional intermediates (NULL = not wanted) */
    uint8_t *usable;   /* [B,A] */
    uint8_t *allowed;  /* [B,A,K] */
    double *x0;        /* [B,A,C]   sanitised entry state (decoder: + token gather) */
    double *q_in;      /* [B,A,C]   query-side normalised input */
    double *kv_in;     /* [B,A,C]   key/value-side normalised input */
    double *q;         /* [B,A,H*D] after head RMS + rotary (ESMFold2) */
    double *k;         /* [B,A,H*D] */
    double *v;         /* [B,A,H*D] */
    double *g;         /* [B,A,H*D] sigmoid value gate */
    double *o;         /* [B,A,H*D] attention-weighted values, before gating */
    double *x1;        /* [B,A,C]   state after the attention residual */
    /* which outputs were computed when a selection is given */
    uint8_t *done_atom;  /* [B,A] */
    uint8_t *done_token; /* [B,T] */
} orc_outputs;

/* Whole block. `select` ([B,A], may be NULL = every atom) restricts the work
 * to the chosen atoms: hidden/attention/position_update rows are computed
 * for them (plus, for the encoder, every usable atom sharing a token with a
 * chosen usable atom, so that those tokens' means are complete). Rows that
 * were not computed are left untouched; done_atom/done_token report which
 * were. nthreads <= 0 means the OpenMP default.
 * Returns 0, or -1 on an argument error (bad style/stage, dims < 1, eps not
 * finite and positive, radius < -1, odd D for ESMFold2, missing pointer). */
int orc_block(const orc_dims *dims, int style, int stage, double eps,
              int64_t radius, const orc_inputs *in, const orc_params *par,
              const uint8_t *select, orc_outputs *out, int nthreads);

/* Slot-attention step alone, from supplied per-atom Q/K/V rows ([B,A,H*D],
 * head-major) and the usability mask. AF3 adds the pair-logit bias (pass
 * pair/pair_scale/w_pair), ESMFold2 passes NULL for them. Writes
 * attention [B,H,A,K], o [B,A,H*D] and (if not NULL) allowed [B,A,K]. */
int orc_slot_attention(const orc_dims *dims, int style, double eps,
                       int64_t radius, const uint8_t *usable,
                       const double *q, const double *k, const double *v,
                       const int64_t *key_index, const uint8_t *window_mask,
                       const double *pair, const double *pair_scale,
                       const double *w_pair, double *attention, double *o,
                       uint8_t *allowed, int nthreads);

/* Number of OpenMP threads a parallel region would use with `nthreads`. */
int orc_threads(int nthreads);

#ifdef __cplusplus
}
#endif
#endif
