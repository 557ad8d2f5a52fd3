/*
 * hstu.h -- C ABI of the MI355X (gfx950) HSTU pointwise aggregated attention
 * library (libhstu.so).
 *
 * What the library computes (per head h, for a jagged batch of user-action
 * sequences):
 *
 *   S_ij = <Q_i, K_j> + rab_pos[pb(i, j)] + rab_time[tb(i, j)]
 *   O_i  = alpha * sum_{j visible from i} SiLU(S_ij) * V_j          (no softmax)
 *   Y_i  = LayerNorm(concat_h O_i) (.) U_i                         (optional)
 *
 * following the layer described on the pages
 *   "生成式推荐（一）：HSTU" (sections "高性能自注意力Encoder：HSTU" and
 *   "Pointwise aggregated attention": SiLU activations, LayerNorm, the
 *   Norm(A(X)V(X)) (.) U(X) gate, rab^{p,t} from position and time),
 *   "Meta HSTU: как действия пользователя стали основой большой
 *   рекомендательной модели" (section "Что меняется внутри HSTU по сравнению
 *   с обычным Transformer": Q, K, V, U built together, position and time
 *   biases, normalise-then-gate, residual) and
 *   "行动胜于言语：万亿参数序列转导器用于生成式推荐" (section "7. 模型细节":
 *   normalised attention without softmax; section "2.3 M-FALCON算法").
 *
 * Definitions used throughout (row r of sequence b is buffer row
 * seq_offsets[b] + r; L_b rows; n_b = L_b - num_candidates[b] history rows):
 *   visible(i, j): i < n_b: j <= i (causal, the diagonal included);
 *                  i >= n_b (a ranking candidate): j < n_b or j == i.
 *   position p(i) = min(i, n_b)       (every candidate sits just after the
 *                                      history, as a single appended target)
 *   pb(i, j) = min(p(i) - p(j), num_pos_buckets - 1)
 *   tb(i, j) = min(num_time_buckets - 1, bit_length(|t_i - t_j|)),
 *              t in int64 seconds, bit_length(0) = 0.
 *
 * Conventions
 *   - All data pointers are DEVICE pointers unless stated otherwise.  The
 *     caller owns every buffer; the library never allocates or frees device
 *     memory.  Scratch memory is a caller-provided workspace whose size is
 *     returned by the matching *_workspace_bytes() query -- except for
 *     hstu_attn_fwd_noalloc, whose scratch is a fixed device array of the
 *     library (loaded with it on each GPU).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every entry point
 *     checks its arguments synchronously, then enqueues its kernels on
 *     `stream` and returns without synchronising.  Device-side faults surface
 *     at the caller's next synchronisation.
 *   - Strides are in ELEMENTS between consecutive rows.  Head h of row r of Q
 *     starts at q + r * q_stride + h * d_qk (same for K; V, O with d_v).
 *   - On any error no kernel has been launched; hstu_last_error() returns a
 *     thread-local message for the last failing call on that thread.
 *   - Device data (offsets, lengths, candidate counts) is trusted: it must
 *     satisfy 0 <= seq_offsets[b] <= seq_offsets[b+1] <= num_rows,
 *     0 <= L_b <= max_seq_len, 0 <= num_candidates[b] <= L_b; violating it is
 *     undefined behaviour unless it is checked: hstu_validate_offsets() checks
 *     it on the device, and with the environment variable HSTU_VALIDATE=1
 *     hstu_attn_fwd, mfalcon_score, the layer calls (forward and gradients,
 *     with or without saved activations; for these also the packed layout,
 *     seq_offsets[0] = 0 and seq_offsets[B] = num_rows) and hstu_attn_bwd run
 *     that check before launching anything (synchronising the stream: a debug
 *     aid, not for timed runs).
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 11

/* ------------------------------------------------------------------ status */
typedef int32_t hstu_status;
#define HSTU_OK 0
#define HSTU_ERR_ARG (-1)          /* invalid argument (NULL, bad size, ...) */
#define HSTU_ERR_UNSUPPORTED (-2)  /* valid, but no kernel for this shape/dtype */
#define HSTU_ERR_WORKSPACE (-3)    /* workspace NULL or smaller than required */
#define HSTU_ERR_DEVICE (-4)       /* a HIP call or kernel launch failed */

/* ------------------------------------------------------------------- enums */
#define HSTU_F32 0   /* float32 Q/K/V/U/O/Y, fp32 arithmetic */
#define HSTU_BF16 1  /* bfloat16 Q/K/V/U/O/Y, bf16 MFMA with fp32 accumulation */

#define HSTU_ACT_SILU 0      /* the method's activation */
#define HSTU_ACT_IDENTITY 1  /* test mode: A = S (no activation) */

/* Shapes compiled into this build:
 *   HSTU_BF16: d_qk = d_v = 128, any H >= 1.
 *   HSTU_F32:  d_qk = d_v in {32, 64}, any H >= 1.
 *   max_seq_len <= 65536; num_pos_buckets in [1, 8192]; num_time_buckets >= 1.
 *   bf16 buffers need 16-byte aligned row starts (pointer and stride*2). */

/* ------------------------------------------------------- attention (core) */
typedef struct hstu_attn_args {
    uint32_t struct_size;          /* = sizeof(hstu_attn_args) */
    int32_t B;                     /* sequences, >= 0 */
    int32_t H;                     /* heads, >= 1 */
    int32_t d_qk, d_v;             /* head dims */
    int32_t max_seq_len;           /* upper bound on every L_b */
    int64_t num_rows;              /* rows in the jagged buffers (>= seq_offsets[B]) */
    const int32_t* seq_offsets;    /* [B+1] first row of each sequence */
    const int32_t* seq_lengths;    /* [B] L_b, or NULL: L_b = offsets[b+1]-offsets[b].
                                      Rows offsets[b]+L_b .. offsets[b+1]-1 are padding:
                                      never read, never written. */
    const int32_t* num_candidates; /* [B] candidates at the end of each sequence
                                      (M-FALCON), or NULL: all rows are history */
    int32_t dtype;                 /* HSTU_F32 | HSTU_BF16 (Q, K, V, U, O, Y) */
    int32_t act;                   /* HSTU_ACT_SILU | HSTU_ACT_IDENTITY */
    const void* q; int64_t q_stride;
    const void* k; int64_t k_stride;
    const void* v; int64_t v_stride;
    const int64_t* timestamps;     /* [num_rows] seconds */
    const float* rab_pos;          /* [num_pos_buckets] (+ h*rab_pos_head_stride) */
    int32_t num_pos_buckets;
    int32_t rab_pos_head_stride;   /* 0: one table shared by all heads */
    const float* rab_time;         /* [num_time_buckets] (+ h*rab_time_head_stride) */
    int32_t num_time_buckets;
    int32_t rab_time_head_stride;
    float alpha;                   /* output scale (1/n), finite */
    void* o; int64_t o_stride;     /* out: [rows, H*d_v] attention output O */
    /* optional epilogue Y = LayerNorm(O_row) (.) U_row over all H*d_v values */
    const void* u; int64_t u_stride;   /* [rows, H*d_v]; required when y != NULL */
    void* y; int64_t y_stride;         /* out, or NULL to skip the epilogue */
    float ln_eps;                      /* > 0, added to the variance */
    /* optional hipEvent_t stamped with the start / end of the attention-core
       kernel itself (they travel with its launch on `stream`, adding no
       packets between kernels); for timing that kernel alone; NULL = none */
    void* ev_core_begin;
    void* ev_core_end;
    /* optional hipEvent_t stamped with the start / end of the epilogue kernel
       (LayerNorm (.) U, when y != NULL) in the same way; NULL = none */
    void* ev_epi_begin;
    void* ev_epi_end;
} hstu_attn_args;

/* Version of this ABI (HSTU_ABI_VERSION). */
int hstu_abi_version(void);

/* Static description of a status code; never NULL. */
const char* hstu_status_string(hstu_status s);

/* Thread-local detail of the last error on this thread ("" if none). */
const char* hstu_last_error(void);

/* Workspace bytes needed by hstu_attn_fwd for these arguments (0 on invalid
 * arguments; call hstu_attn_fwd to get the reason).  Depends only on B,
 * max_seq_len, dtype and, for HSTU_BF16, H and d_v (fp32 partial sums of
 * row blocks split over their key tiles, at most 1024 slots of 128 x d_v)
 * and num_rows (a 4-byte timestamp code and a 4-byte split-map entry per
 * row). */
size_t hstu_attn_workspace_bytes(const hstu_attn_args* args);

/* Pointwise aggregated attention over a jagged batch.  Builds the jagged
 * tile work list (skipping fully masked tiles) on the device, runs the
 * attention core into `o`, then (if y != NULL) the LayerNorm(O) (.) U
 * epilogue into `y`.  `o` must not alias any input.
 * Errors: HSTU_ERR_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE,
 * HSTU_ERR_DEVICE. */
hstu_status hstu_attn_fwd(const hstu_attn_args* args, void* workspace, size_t workspace_bytes,
                          void* stream);

/* hstu_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results, but no workspace: the work list,
 * timestamp codes and split-block partial sums live in a scratch buffer the
 * library holds on every GPU it runs on (hstu_attn_noalloc_scratch_bytes()
 * bytes, 32 MiB, from module load to the end of the process).  The call
 * allocates and frees nothing; it may use fewer split-block partial slots
 * than hstu_attn_fwd (rows then match to rounding, not bit for bit).  Calls
 * on one GPU share its buffer: calls that may overlap on one GPU (streams
 * with no ordering between them) race.  Errors: as hstu_attn_fwd, and
 * HSTU_ERR_WORKSPACE (before any launch) when the call needs more scratch
 * than the buffer holds. */
hstu_status hstu_attn_fwd_noalloc(const hstu_attn_args* args, void* stream);

/* Bytes of the library-held scratch buffer of hstu_attn_fwd_noalloc. */
size_t hstu_attn_noalloc_scratch_bytes(void);

/* --------------------------------------------------- M-FALCON ranking pass */
/* One forward pass scoring b_m candidates per user against the shared
 * history: "行动胜于言语：万亿参数序列转导器用于生成式推荐", section
 * "2.3 M-FALCON算法"; "生成式推荐（一）：HSTU", section "M-FALCON"; "Meta HSTU",
 * section "M-FALCON переиспользует историю между кандидатами".
 *   scores[b * score_stride + c] = < Y[n_b + c, :], w >,
 * Y = LayerNorm(O) (.) U as in hstu_attn_fwd, for c < num_candidates[b].
 * A candidate row's output depends on the history rows' keys and values only,
 * never on their outputs, so with candidates_only set (and attn.y == NULL)
 * just the query tiles that hold candidate rows are computed: the O rows of
 * history outside those tiles are left unwritten, and the scores are
 * bit-identical to those of the full pass. */
typedef struct hstu_mfalcon_args {
    uint32_t struct_size;     /* = sizeof(hstu_mfalcon_args) */
    hstu_attn_args attn;      /* num_candidates and u are required; attn.y may be
                                 NULL (Y not stored) or a buffer for Y */
    const float* w;           /* [H*d_v] score vector */
    float* scores;            /* out: [B * score_stride] fp32 */
    int32_t score_stride;     /* >= max candidates per sequence */
    int32_t candidates_only;  /* nonzero: only the query tiles holding candidate
                                 rows (requires attn.y == NULL) */
} hstu_mfalcon_args;

size_t hstu_mfalcon_workspace_bytes(const hstu_mfalcon_args* args);

hstu_status mfalcon_score(const hstu_mfalcon_args* args, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ----------------------------------- M-FALCON against a history KV cache */
/* Scores of many candidates per user against a cached history: M-FALCON at
 * scale ("行动胜于言语：万亿参数序列转导器用于生成式推荐", section "2.3 M-FALCON
 * 算法": candidates in microbatches, the history's keys and values computed
 * once and cached).  Each candidate c of user b sees the user's n_b history
 * keys and itself, at position n_b -- exactly the rows of mfalcon_score for
 * the sequence [history | candidates] -- so, without a softmax, its output is
 * a sum over the cached history plus its own term:
 *   O_c = alpha (sum_{j<n_b} SiLU(S_cj) V_j + SiLU(q_c.k_c + rab_pos[0]
 *         + rab_time[0]) v_c),   S_cj = q_c.K_j + rab_pos[min(n_b - j, P-1)]
 *         + rab_time[tb(t_c, t_j)],
 *   scores[b * score_stride + c] = < LN(O_c) (.) U_c, w >.
 * Any number of candidates per call (a call is one or many microbatches);
 * candidate timestamps are given per candidate.  bf16, d = 128.
 * Errors: HSTU_ERR_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE, HSTU_ERR_DEVICE. */
typedef struct hstu_mfalcon_cached_args {
    uint32_t struct_size;          /* = sizeof(hstu_mfalcon_cached_args) */
    int32_t B, H, d;               /* users, heads, head dim (128) */
    int32_t max_hist_len;          /* >= every n_b */
    int32_t max_cands;             /* >= every candidate count */
    const int32_t* hist_offsets;   /* [B+1] device: rows of the history cache */
    int64_t num_hist_rows;
    const void* k_hist; int64_t k_hist_stride;   /* [hist rows, H*d] bf16 cached keys */
    const void* v_hist; int64_t v_hist_stride;   /* cached values */
    const int64_t* ts_hist;        /* [hist rows] seconds */
    const int32_t* cand_offsets;   /* [B+1] device: rows of the candidates */
    int64_t num_cand_rows;
    const void* q; int64_t q_stride;   /* [cand rows, H*d] bf16, the candidates' */
    const void* k; int64_t k_stride;
    const void* v; int64_t v_stride;
    const void* u; int64_t u_stride;
    const int64_t* ts_cand;        /* [cand rows] */
    const float* rab_pos; int32_t num_pos_buckets; int32_t rab_pos_head_stride;
    const float* rab_time; int32_t num_time_buckets; int32_t rab_time_head_stride;
    float alpha;
    float ln_eps;
    const float* w;                /* [H*d] */
    float* scores;                 /* out [B * score_stride] */
    int32_t score_stride;          /* >= max_cands */
    void* o; int64_t o_stride;     /* out: candidates' O [cand rows, H*d] bf16, or NULL */
    void* ev_core_begin;           /* optional hipEvent_t around the attention core */
    void* ev_core_end;
} hstu_mfalcon_cached_args;

size_t hstu_mfalcon_cached_workspace_bytes(const hstu_mfalcon_cached_args* args);

hstu_status mfalcon_score_cached(const hstu_mfalcon_cached_args* args, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ HSTU layer */
/* One HSTU layer over a packed jagged batch (bf16, d = 128):
 *   Z = SiLU(X W1^T + b1)  split by columns into U | V | Q | K (H*d each,
 *                          head h at sub-columns h*d .. h*d+d-1)
 *   O = attention(Q, K, V) as hstu_attn_fwd (causal, or M-FALCON)
 *   Y = LayerNorm(O) (.) U
 *   X_out = X + Y W2^T + b2
 * ("生成式推荐（一）：HSTU", section "高性能自注意力Encoder：HSTU": pointwise
 * projection f1 with SiLU, spatial aggregation, pointwise transformation
 * with f2; residual between identical layers.) */
typedef struct hstu_layer_args {
    uint32_t struct_size;          /* = sizeof(hstu_layer_args) */
    int32_t B, H, d, D;            /* d must be 128; D (model width) % 64 == 0 */
    int32_t max_seq_len;
    int64_t num_rows;              /* = seq_offsets[B] (packed layout) */
    const int32_t* seq_offsets;    /* [B+1] */
    const int32_t* num_candidates; /* [B] or NULL */
    const void* x;                 /* [num_rows, D] bf16 */
    const void* w1;                /* [4*H*d, D] bf16 (out x in) */
    const float* b1;               /* [4*H*d] or NULL */
    const void* w2;                /* [D, H*d] bf16 (out x in) */
    const float* b2;               /* [D] or NULL */
    const int64_t* timestamps;     /* [num_rows] */
    const float* rab_pos; int32_t num_pos_buckets;
    const float* rab_time; int32_t num_time_buckets;
    float alpha;
    float ln_eps;
    void* x_out;                   /* [num_rows, D] bf16; may alias x */
} hstu_layer_args;

size_t hstu_layer_workspace_bytes(const hstu_layer_args* args);

hstu_status hstu_layer_fwd(const hstu_layer_args* args, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The last layer of an M-FALCON stack, candidate rows only ("生成式推荐（一）：
 * HSTU", section "M-FALCON"; "行动胜于言语：万亿参数序列转导器用于生成式推荐",
 * section "2.3 M-FALCON 算法": the ranking pass needs the outputs of the
 * candidates alone): Z = SiLU(X W1^T + b1) for every row (the history's K
 * and V are needed), attention, and for each candidate c of sequence b
 *   scores[b * score_stride + c] = < LN(O[n_b + c]) (.) U[n_b + c], w >.
 * With candidates_only the attention computes only the query tiles that
 * hold candidate rows.  layer.w2, layer.b2 and layer.x_out are not used
 * (may be NULL); layer.num_candidates is required.
 * Errors: as hstu_layer_fwd, HSTU_ERR_ARG without candidates, w or scores. */
typedef struct hstu_mfalcon_layer_args {
    uint32_t struct_size;          /* = sizeof(hstu_mfalcon_layer_args) */
    hstu_layer_args layer;
    const float* w;                /* [H*d] */
    float* scores;                 /* out [B * score_stride] */
    int32_t score_stride;          /* >= every candidate count */
    int32_t candidates_only;
} hstu_mfalcon_layer_args;

size_t hstu_mfalcon_layer_workspace_bytes(const hstu_mfalcon_layer_args* args);

hstu_status mfalcon_layer_score(const hstu_mfalcon_layer_args* args, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------- attention (gradients) */
/* Gradients of the attention path for training (bf16, d_qk = d_v = 128):
 * the chain rule through the forward definition of hstu_attn_fwd ("生成式推荐
 * （一）：HSTU", sections "高性能自注意力Encoder：HSTU" and "Pointwise
 * aggregated attention"; training is what the pages' speed-ups are quoted
 * for).  Per head and visible pair (i, j), with S_ij the forward's logit:
 *   dV_j += alpha SiLU(S_ij) dO_i
 *   G_ij  = alpha <dO_i, V_j> SiLU'(S_ij)
 *   dQ_i += G_ij K_j,  dK_j += G_ij Q_i,
 *   drab_pos[pb(i, j)] += G_ij,  drab_time[tb(i, j)] += G_ij.
 * The upstream gradient is either dout = dLoss/dO, or dy = dLoss/dY of the
 * forward's Y = LayerNorm(O) (.) U (then attn.o must hold the forward's O,
 * attn.u its U, attn.ln_eps its eps; dO and, if du != NULL, dU are derived
 * first).  O and Y are not recomputed; S is.
 * Outputs: the valid rows of dq, dk, dv (bf16, [rows, H*128] with strides in
 * elements, 16-byte aligned rows) are overwritten, padding rows untouched;
 * drab_pos / drab_time (fp32, device) are overwritten with the table
 * gradients, shaped like the tables: [num_pos_buckets] summed over heads for
 * a shared table, [H][num_pos_buckets] (dense, stride num_pos_buckets) for
 * per-head tables; NULL skips one.  The table gradients are summed in a
 * fixed order (run-to-run identical).  attn.y, attn.o (without dy) and the
 * attention events are not used.
 * Limits: bf16 with d = 128; num_pos_buckets at most about 5200 (the
 * position table and its padded copies share the dK/dV kernel's LDS with its
 * tile ring); (max_seq_len / 32 + 1) * H * 4096 below 2^31.
 * Errors: HSTU_ERR_ARG, HSTU_ERR_UNSUPPORTED (fp32, d != 128, tables too
 * long), HSTU_ERR_WORKSPACE, HSTU_ERR_DEVICE. */
typedef struct hstu_attn_bwd_args {
    uint32_t struct_size;               /* = sizeof(hstu_attn_bwd_args) */
    hstu_attn_args attn;                /* the forward's arguments */
    const void* dy; int64_t dy_stride;  /* [rows, H*d_v] bf16, or NULL */
    const void* dout; int64_t dout_stride;   /* [rows, H*d_v] bf16 when dy == NULL */
    void* dq; int64_t dq_stride;
    void* dk; int64_t dk_stride;
    void* dv; int64_t dv_stride;
    void* du; int64_t du_stride;        /* with dy: dLoss/dU, or NULL */
    float* drab_pos;
    float* drab_time;
    /* optional hipEvent_t stamped with the start / end of the dQ kernel and of
       the dK/dV kernel (travel with those launches); NULL = none */
    void* ev_dq_begin; void* ev_dq_end;
    void* ev_dkv_begin; void* ev_dkv_end;
} hstu_attn_bwd_args;

/* Workspace bytes for hstu_attn_bwd (0 on invalid arguments): two work lists,
 * the timestamp codes, dO when dy is given (rows x H*128 bf16), one fp32 row
 * of num_pos_buckets + num_time_buckets table-gradient partial sums per
 * (128-row block, head), K of every 32-key tile and head in the dQ kernel's
 * operand order (8 KiB each, B * ceil(max_seq_len / 32) * H of them), and
 * dLoss/dS of every 32 x 32 block holding a visible pair, fp32 (4 KiB per
 * block and head; the count is bounded from B, max_seq_len and the row
 * count: at most (ceil(max_seq_len / 32) + 1) / 2 blocks per 32-row tile).
 * The last grows with the visible pairs: about 4 bytes per pair and head. */
size_t hstu_attn_bwd_workspace_bytes(const hstu_attn_bwd_args* args);

hstu_status hstu_attn_bwd(const hstu_attn_bwd_args* args, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ----------------------------------------------------- layer (gradients) */
/* Gradients of one HSTU layer (hstu_layer_fwd) for training: the chain rule
 * through f2 + residual, the LayerNorm (.) U gate, the attention and
 * f1 + SiLU ("生成式推荐（一）：HSTU", section "高性能自注意力Encoder：HSTU"):
 *   dY = dX_out W2,  dW2 = dX_out^T Y,  db2 = sum_t dX_out,
 *   dO, dU from the gate; dQ, dK, dV and the table gradients as in
 *   hstu_attn_bwd;  dP = (dU | dV | dQ | dK) (.) SiLU'(X W1^T + b1),
 *   dX = dX_out + dP W1,  dW1 = dP^T X,  db1 = sum_t dP.
 * The forward intermediates (Z, O, Y) are recomputed from layer's inputs.
 * Token sums run in a fixed order (run-to-run identical results).
 * Requirements beyond hstu_layer_fwd's: D % 128 == 0, H*d % 128 == 0,
 * num_pos_buckets <= ~5200.
 * Errors: HSTU_ERR_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE, HSTU_ERR_DEVICE. */
typedef struct hstu_layer_bwd_args {
    uint32_t struct_size;      /* = sizeof(hstu_layer_bwd_args) */
    hstu_layer_args layer;     /* the forward's arguments (layer.x_out unused) */
    const void* dx_out;        /* [num_rows, D] bf16: dLoss/dX_out */
    void* dx;                  /* out [num_rows, D] bf16; may alias dx_out */
    float* dw1;                /* out [4*H*d, D] fp32 */
    float* db1;                /* out [4*H*d] fp32, or NULL */
    float* dw2;                /* out [D, H*d] fp32 */
    float* db2;                /* out [D] fp32, or NULL */
    float* drab_pos;           /* out [num_pos_buckets] fp32, or NULL */
    float* drab_time;          /* out [num_time_buckets] fp32, or NULL */
} hstu_layer_bwd_args;

/* Workspace bytes for hstu_layer_bwd (0 on invalid arguments): the
 * recomputed Z, its pre-activation, O, Y (bf16), dY, dZ, transposed weights,
 * the attention's and the weight products' scratch. */
size_t hstu_layer_bwd_workspace_bytes(const hstu_layer_bwd_args* args);

hstu_status hstu_layer_bwd(const hstu_layer_bwd_args* args, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The same layer and gradients with the forward's activations kept instead
 * of recomputed (the section above): hstu_layer_fwd_saved computes what
 * hstu_layer_fwd computes and also writes, into the caller's buffer `saved`
 * (device, 16-byte aligned, hstu_layer_saved_bytes() bytes), Z = SiLU(X W1^T
 * + b1) (U | V | Q | K), the pre-activation X W1^T + b1, O and Y (bf16,
 * num_rows rows each, about 2 * (2 * 4*H*d + 2 * H*d) bytes per row), in
 * that order, row-major with no row padding, each region starting at the
 * next multiple of 256 bytes after the previous one (Z at byte 0);
 * hstu_layer_bwd_saved computes what hstu_layer_bwd computes from them,
 * reading `saved` only, without running f1, the attention or the gate
 * forward again.  Both calls must see the same layer arguments, weights and
 * inputs; X must still hold the forward's input when the gradients run, so
 * hstu_layer_fwd_saved rejects an x_out that overlaps x (unlike
 * hstu_layer_fwd).  Workspaces: hstu_layer_workspace_bytes for the forward,
 * hstu_layer_bwd_saved_workspace_bytes for the gradients (no room for a
 * recomputed forward; any workspace of hstu_layer_bwd_workspace_bytes also
 * fits).  Errors: as hstu_layer_fwd and hstu_layer_bwd; HSTU_ERR_ARG for a
 * NULL `saved` with a non-empty batch or an x_out overlapping x,
 * HSTU_ERR_WORKSPACE for a misaligned or too small buffer. */
size_t hstu_layer_saved_bytes(const hstu_layer_args* args);

/* Workspace bytes for hstu_layer_bwd_saved (0 on invalid arguments): dY, dZ,
 * transposed weights, the attention's and the weight products' scratch. */
size_t hstu_layer_bwd_saved_workspace_bytes(const hstu_layer_bwd_args* args);

hstu_status hstu_layer_fwd_saved(const hstu_layer_args* args, void* saved, size_t saved_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream);

hstu_status hstu_layer_bwd_saved(const hstu_layer_bwd_args* args, const void* saved, size_t saved_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ stochastic length */
/* Stochastic length on the device ("行动胜于言语：万亿参数序列转导器用于生成式
 * 推荐", section "2.1"; the GRs summary page, section 2.1): each sequence
 * longer than its cap is replaced by a random order-preserving subsequence of
 * cap events, and the kept rows of up to 8 row-major tensors are gathered
 * into a packed jagged batch.  Sampler: event j of sequence b gets the top 32
 * bits of the first word of Philox-4x64-10 (Salmon et al., SC'11) for counter
 * (j, b, step, 0) and key (seed, 0x534c); the sequence keeps its
 * min(cap_b, L_b) events with the smallest (key, j), in order (a pure
 * function of its inputs: run-to-run identical; every subset of that size
 * is equally likely).  For the cap of "N^(alpha/2)" with the exponent being
 * swept, pass the caps the host computes.
 * Outputs: out_offsets [B+1] (device) of the kept rows; out_index (device,
 * capacity num_rows) the source row of each kept row, in order; dst[t] row r
 * = src[t] row out_index[r] (row_bytes[t] bytes, a multiple of 4; strides in
 * bytes; 16-byte rows and strides copy 16 bytes at a time).  No workspace.
 * Errors: HSTU_ERR_ARG, HSTU_ERR_DEVICE. */
#define HSTU_SL_MAX_TENSORS 8
typedef struct hstu_sl_args {
    uint32_t struct_size;          /* = sizeof(hstu_sl_args) */
    int32_t B;                     /* sequences, >= 0 */
    int64_t num_rows;              /* rows of the input tensors (>= seq_offsets[B]) */
    const int32_t* seq_offsets;    /* [B+1] device */
    int32_t cap;                   /* cap of every sequence (>= 0) when caps == NULL */
    const int32_t* caps;           /* [B] device per-sequence caps, or NULL */
    uint64_t seed;                 /* Philox key word 0 */
    uint64_t step;                 /* Philox counter word 2 (e.g. the training step) */
    int32_t* out_offsets;          /* out [B+1] device */
    int64_t* out_index;            /* out [num_rows] device */
    int32_t num_tensors;           /* 0 .. HSTU_SL_MAX_TENSORS */
    const void* src[HSTU_SL_MAX_TENSORS];
    int64_t src_stride[HSTU_SL_MAX_TENSORS];
    void* dst[HSTU_SL_MAX_TENSORS];
    int64_t dst_stride[HSTU_SL_MAX_TENSORS];
    int32_t row_bytes[HSTU_SL_MAX_TENSORS];
} hstu_sl_args;

hstu_status hstu_stochastic_length(const hstu_sl_args* args, void* stream);

/* ------------------------------------------------------ scheduler access */
/* Builds only the jagged tile work list into `workspace` (same layout as the
 * one hstu_attn_fwd builds) and copies it to the HOST array `items_out`
 * (capacity `cap` rows of 8 int32 per piece: b, query tile, end of the first
 * key-tile range [0, a_end), second range packed as begin | end << 16, the
 * piece's positions in that tile list packed as p0 | p1 << 16, the row
 * block's first partial slot (-1: not split), the piece index, the number
 * of pieces of the row block).  A row
 * block whose tile list is long next to the work per workgroup is split into
 * pieces over disjoint position ranges.  `count_out` (host) receives the
 * number of pieces.  Synchronises `stream`.  For tests of the scheduler
 * against a brute-force tile enumeration. */
/* ------------------------------------------------------ batch validation */
/* Checks the batch structure the other calls read from device memory without
 * a host copy (the jagged layout of "Meta HSTU: как действия пользователя стали
 * основой большой рекомендательной модели", section "Разная длина истории
 * превращается в выигрыш по ресурсам", and the M-FALCON candidate counts of
 * "生成式推荐（一）：HSTU", section "M-FALCON"): seq_offsets[0] >= 0, the
 * offsets non-decreasing, seq_offsets[B] <= num_rows, 0 <= seq_lengths[b] <=
 * seq_offsets[b+1] - seq_offsets[b] (when given), every L_b <= max_seq_len,
 * 0 <= num_candidates[b] <= L_b (when given).  Only those fields of `args`
 * are read, and only the pointers are checked on the host.  One small kernel
 * on `stream`; synchronises `stream`.  Returns HSTU_OK, or HSTU_ERR_ARG with
 * hstu_last_error() naming the first failing sequence and check
 * (HSTU_ERR_DEVICE if the launch fails).  The result passes through a device
 * variable of the library (one per GPU): calls on one GPU must not overlap. */
hstu_status hstu_validate_offsets(const hstu_attn_args* args, void* stream);

hstu_status hstu_attn_schedule(const hstu_attn_args* args, void* workspace, size_t workspace_bytes,
                               int32_t* items_out, int64_t cap, int64_t* count_out,
                               int32_t* tile_m_out, int32_t* tile_n_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
