/*
 * mtla.h -- C ABI of the Multi-head Temporal Latent Attention (MTLA) hot path
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [Notes] "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
 *           Paper-Notes, NeurIPS 2025), method section: overall framework,
 *           key designs (hyper-network temporal merging, stride-aware causal
 *           mask, decoupled RoPE with temporal compression), hyper-parameters.
 *   [Fig1]  "Multi-head Temporal Latent Attention" (sciencestack.ai), Figure 1.
 *   [Fig2]  same page, Figure 2 (a) incremental inference, (c) training.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer to row-major data in the
 *    storage type named by mtla_dims.dtype (fp32 or bf16), except where a
 *    parameter says otherwise.  Accumulation is always fp32.
 *  - Every device pointer must be 16-byte aligned.
 *  - Linear maps are stored [out, in] (y = x W^T), the nn.Linear layout.
 *  - The caller owns all memory.  The library never allocates, frees or
 *    synchronises: every call only enqueues kernels on `stream` (a
 *    hipStream_t; NULL is the null stream) and returns.  It writes only the
 *    outputs, the cache rows and the workspace its documentation names.
 *  - Errors: argument checks run on the host before anything is enqueued.  On
 *    MTLA_ERR_ARG, MTLA_ERR_CAPACITY or MTLA_ERR_UNSUPPORTED nothing is
 *    written.  MTLA_ERR_HIP reports a failed launch.  No C++ exception crosses
 *    this boundary.  mtla_last_error_detail() describes the last failure of
 *    the calling thread.
 *  - Frame positions are 0-based.  Frame i belongs to slot floor(i/s); slot j
 *    is complete once frame s*j + s - 1 has been merged (the pages count from
 *    1 and call that frame's index a multiple of s).
 *  - Supported shapes: (r, d_hR) in {(256, 32), (512, 64)} (r = 4 d_h and
 *    d_hR = d_h/2 for d_h = 64 or 128), H <= 64 (H <= 32 when r = 512), d a
 *    multiple of 32, s >= 1.
 *    Other shapes return MTLA_ERR_UNSUPPORTED.
 *  - Calls on one stream are ordered; calls on different streams that touch
 *    the same cache or workspace race.
 */
#ifndef MTLA_H
#define MTLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTLA_OK = 0,
  MTLA_ERR_ARG = 1,          /* bad dimension, null or misaligned pointer */
  MTLA_ERR_CAPACITY = 2,     /* a position does not fit the cache or gate table */
  MTLA_ERR_UNSUPPORTED = 3,  /* valid but not implemented shape or dtype */
  MTLA_ERR_HIP = 4           /* a HIP launch failed */
} mtla_status;

typedef enum { MTLA_F32 = 0, MTLA_BF16 = 1 } mtla_dtype;

/* Layer dimensions ([Notes] hyper-parameters: r = 4 d_h, d_hR = d_h / 2,
 * default s = 2). */
typedef struct {
  int32_t d;      /* width of an input frame x_i */
  int32_t H;      /* attention heads */
  int32_t d_h;    /* head width; only sets the default softmax scale */
  int32_t r;      /* latent width of c_i and of a cache slot */
  int32_t d_hR;   /* decoupled-RoPE key width, one key shared by all heads */
  int32_t s;      /* temporal compression ratio: s frames per cache slot */
  float scale;    /* softmax scale; 0 selects 1/sqrt(d_h) ([Notes] Y formula) */
  int32_t dtype;  /* mtla_dtype of all tensor arguments */
} mtla_dims;

/* Weights of one layer (device pointers, storage dtype unless noted). */
typedef struct {
  const void *W_dkv;      /* [r, d]    latent map, c_i = W_dkv x_i ([Notes] overall framework) */
  const void *W_gate;     /* [r, d]    W_hc W_dkv from mtla_gate_content_map: the weight of
                             the hyper-network content branch Linear(c_i) = W_hc c_i + b_hc
                             folded into the latent map, so W_gate x_i = W_hc c_i ... */
  const void *b_hc;       /* [r]       ... and the bias b_hc ([Notes] temporal merging) */
  const float *gate_pos;  /* [gate_pos_rows, r] FP32: Linear(pe_j) for slot j, from
                             mtla_gate_pos_table ([Notes] temporal merging) */
  int32_t gate_pos_rows;  /* rows of gate_pos; every slot index used must be below it */
  const void *A;          /* [H, r, d] absorbed query map: A[h] = (W_Q^(h) W_K^(h)T)^T,
                             q~_h = A[h] x ([Notes] Y formula, [Fig1]) */
  const void *Bvo;        /* [d, H, r] absorbed output map: Bvo[:, h, :] = (W_V^(h) W_O^(h))^T,
                             y = sum_h Bvo[:, h, :] o_h ([Notes] Y formula, [Fig1]) */
} mtla_weights;

/* Compressed cache ([Notes] overall framework: ceil(T/s) slots of r latent
 * values; decoupled RoPE: one compressed RoPE key per slot).  Slot j of
 * sequence b starts at element b*batch_stride + j*(r + d_hR): the merged
 * latent c^_j (r values) followed by the RoPE key k^R_j (d_hR values) of the
 * newest frame merged into it.  16-byte aligned; batch_stride >=
 * max_slots*(r + d_hR) and a multiple of 8 elements. */
typedef struct {
  void *slots;
  int64_t batch_stride;   /* elements between consecutive sequences */
  int32_t max_slots;      /* slots allocated per sequence */
} mtla_cache;

/* Position branch of the hyper-network, evaluated once into a table
 * ([Notes] temporal merging: w_i = Sigmoid(Linear(c_i) * Linear(pe_j))):
 *   table[j, :] = W_hp pe_j + b_hp, fp32, for j < rows.
 * pe [rows, d_pe] and W_hp [r, d_pe], b_hp [r] in storage dtype; d_pe a
 * multiple of 32.  table [rows, r] fp32 (device).  Only dims->r and
 * dims->dtype are read. */
mtla_status mtla_gate_pos_table(const mtla_dims *dims, const void *pe, int32_t rows, int32_t d_pe,
                                const void *W_hp, const void *b_hp, float *table, void *stream);

/* Content branch of the hyper-network folded into the latent map, evaluated
 * once ([Notes] temporal merging: Linear(c_i) with c_i = W_dkv x_i; matrix
 * products are associative, the device the pages use to absorb W_K and W_V):
 *   W_gate[r, d] = W_hc[r, r] W_dkv[r, d], accumulated in fp32 and stored in
 * the storage dtype.  All three device pointers in that dtype; only dims->r,
 * dims->d and dims->dtype are read. */
mtla_status mtla_gate_content_map(const mtla_dims *dims, const void *W_hc, const void *W_dkv,
                                  void *W_gate, void *stream);

/* Decoupled-RoPE inputs ([Notes] decoupled RoPE with temporal compression:
 * the RoPE-carrying parts of the queries and keys), for M frames X [M, d] at
 * absolute positions pos [M] (device int32, >= 0):
 *   QR[m, h] = R(pos[m]) W_QR[h] x_m   (W_QR [H*d_hR, d]: rows of head h)
 *   KR[m]    = R(pos[m]) W_KR x_m      (W_KR [d_hR, d]; one key for all heads)
 * where R(p) turns the adjacent pairs (2k, 2k+1) of a d_hR-wide vector by
 * p * base^(-2k/d_hR) (the standard rotary form, base typically 10000; the
 * pages do not spell the form out).  QR [M, H, d_hR], KR [M, d_hR] in the
 * storage dtype: the inputs every other entry point takes already rotated.
 * Angles are reduced in fp64.  Workspace: mtla_workspace_bytes(op=6, M, 1). */
mtla_status mtla_rope_inputs(const mtla_dims *dims, const void *W_QR, const void *W_KR,
                             const void *X, const int32_t *pos, int32_t M, float base, void *QR,
                             void *KR, void *workspace, size_t ws_bytes, void *stream);

/* Merge-append ([Notes] temporal merging; [Fig2] (a)): for every sequence b
 * with frame position t = pos[b] and j = floor(t/s):
 *   c = W_dkv x_t;  w = Sigmoid((W_gate x_t + b_hc) * gate_pos[j]);  u = w * c
 *   (W_gate x_t = W_hc c, so w = Sigmoid(Linear(c) * Linear(pe_j)))
 *   slot j latent <- u            if t mod s == 0 (t opens slot j)
 *   slot j latent <- slot j + u   otherwise (accumulated in place)
 *   slot j RoPE key <- KR_t[b]
 * X_t [B, d], KR_t [B, d_hR] (already rotated), pos [B] int32 device array.
 * max_pos: host-side upper bound of every pos[b] (the caller's contract);
 * floor(max_pos/s) must be < cache->max_slots and < gate_pos_rows
 * (else MTLA_ERR_CAPACITY).  The device checks the contract as well: a
 * sequence whose pos[b] lies outside [0, max_pos] is dropped (nothing of it
 * is read or written), and the int32 status word at byte 0 of the workspace
 * holds, once the call has completed, the number of dropped sequences (each
 * call clears it first).  Workspace: mtla_workspace_bytes(op=0). */
mtla_status mtla_merge_append(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                              const void *X_t, const void *KR_t, const int32_t *pos, int32_t B,
                              int32_t max_pos, void *workspace, size_t ws_bytes, void *stream);

/* Chunked merge-append ([Notes] temporal merging; [Fig2] (a) applied frame
 * after frame): sequence b merges frames t = pos0[b] .. pos0[b] + n_b - 1 in
 * order, with the result of n_b successive mtla_merge_append calls, where
 * n_b = lens[b] clamped to [0, L], or L when lens is NULL.  A chunk that
 * starts inside a group (pos0[b] mod s != 0) continues the live partial slot
 * floor(pos0[b]/s) from its stored value -- the hand-off from a prefill that
 * ended inside a group, or from earlier chunks; every slot the chunk touches
 * ends holding its group's newest state and the RoPE key of the newest frame
 * merged into it.  No other cache row is read or written.
 * X [B, L, d], KR [B, L, d_hR] (rotated at positions pos0[b] + i), pos0 [B]
 * and lens [B] (nullable) device int32; pos0[b] >= 0.
 * max_pos: host-side upper bound of every pos0[b] + n_b - 1 (the caller's
 *   contract); floor(max_pos/s) must be < cache->max_slots and <
 *   gate_pos_rows (else MTLA_ERR_CAPACITY).  The kernel itself skips slots at
 *   or beyond either bound, so a broken contract drops frames but never
 *   writes outside the cache.
 * Cprime_out (nullable): [B, L, r]; row i of sequence b receives the state of
 *   frame pos0[b] + i's slot right after that frame's merge (the intermediate
 *   state C' of the parallel form); rows i >= n_b are not written.
 * In bf16 storage a slot is rounded once per chunk, where per-frame calls
 * round it once per frame.  L = 0 is a no-op that returns MTLA_OK (X, KR and
 * the workspace may then be NULL).
 * Workspace: mtla_workspace_bytes(op=3, B, L). */
mtla_status mtla_append_chunk(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                              const void *X, const void *KR, const int32_t *pos0,
                              const int32_t *lens, int32_t B, int32_t L, int32_t max_pos,
                              void *Cprime_out, void *workspace, size_t ws_bytes, void *stream);

/* One incremental decoding step ([Notes] stride-aware mask motivation and Y
 * formula; [Fig2] (a)): mtla_merge_append at pos[b], then for every head h
 *   q~_h = A[h] x_t
 *   z_j  = (q~_h . c^_j + QR_t[b, h] . k^R_j) * scale,  j = 0 .. floor(pos[b]/s)
 *   o_h  = sum_j softmax(z)_j c^_j        (the newest slot may be temporary)
 *   Y[b] = sum_h Bvo[:, h, :] o_h
 * QR_t [B, H, d_hR] already rotated; Y [B, d].  Positions follow
 * mtla_merge_append's contract and device check: a sequence whose pos[b] lies
 * outside [0, max_pos] is dropped -- no cache row of it is read or written,
 * Y[b] = 0 -- and counted in the int32 status word at byte 0 of the
 * workspace.  The slot work is balanced over the workgroups from the actual
 * positions (up to 256 sequences).  Results do not depend on the workspace's
 * prior contents, and two calls on the same inputs give identical bits.
 * Workspace: mtla_workspace_bytes(op=1). */
mtla_status mtla_decode_step(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                             const void *X_t, const void *QR_t, const void *KR_t, const int32_t *pos,
                             int32_t B, int32_t max_pos, void *Y, void *workspace, size_t ws_bytes,
                             void *stream);

/* mtla_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as mtla_decode_step minus the workspace: the
 * step runs in a device scratch array of 64 MiB that the library holds per
 * GPU for the life of the process (the LLM-scale step, B = 128, H = 32,
 * r = 512, 16384 slots, needs 40.6 MiB).  A shape whose workspace
 * (mtla_workspace_bytes(op=1)) exceeds it returns MTLA_ERR_CAPACITY and
 * launches nothing.  `stream` must belong to the current device.  Nothing is
 * allocated or freed: the scratch's device address is looked up once per
 * device (hipGetSymbolAddress).  Every call on a GPU shares that GPU's
 * scratch, which keeps the last call's contents (each call clears what must
 * start at zero itself): calls that may overlap on one GPU -- different
 * streams, or host threads -- race; keep them on one stream.  The dropped-
 * frame status word is not readable through this entry point. */
mtla_status mtla_decode_step_noalloc(const mtla_dims *dims, const mtla_weights *w,
                                     const mtla_cache *cache, const void *X_t, const void *QR_t,
                                     const void *KR_t, const int32_t *pos, int32_t B,
                                     int32_t max_pos, void *Y, void *stream);

/* Parallel (prefill / training-forward) form under the stride-aware causal
 * mask ([Notes] stride-aware causal mask and decoupled RoPE; [Fig2] (c)), for
 * frames 0..T-1 of B sequences:
 *   C'_i = sum over the frames i' of i's group with i' <= i of w_i' * c_i'
 *   query m sees column n iff n = m, or n < m and n mod s = s - 1
 *   z = (q~_{m,h} . C'_n + QR[m, h] . KR[n]) * scale over the visible n
 *   Y[m] = sum_h Bvo[:, h, :] sum_n softmax(z)_n C'_n
 * X [B, T, d], QR [B, T, H, d_hR], KR [B, T, d_hR] (rotated at positions
 * 0..T-1), Y [B, T, d].
 * cache_out (nullable): receives slots 0..ceil(T/s)-1 of every sequence; the
 *   last one is partial when T mod s != 0, so decoding can continue at t = T.
 * Cprime_out (nullable): [B, T, r] intermediate states C'.
 * floor((T-1)/s) must be < gate_pos_rows (and < cache_out->max_slots).
 * Workspace: mtla_workspace_bytes(op=2, T). */
mtla_status mtla_prefill_strided(const mtla_dims *dims, const mtla_weights *w, const void *X,
                                 const void *QR, const void *KR, int32_t B, int32_t T, void *Y,
                                 const mtla_cache *cache_out, void *Cprime_out, void *workspace,
                                 size_t ws_bytes, void *stream);

/* Weights of the per-head (unabsorbed) form ([Fig1] (b): the maps W_Q, W_K,
 * W_V, W_O of every head before they are absorbed into A and Bvo).  The
 * hyper-network fields are those of mtla_weights. */
typedef struct {
  const void *W_dkv;      /* [r, d]     latent map */
  const void *W_gate;     /* [r, d]     W_hc W_dkv (mtla_gate_content_map) */
  const void *b_hc;       /* [r]        content-branch bias */
  const float *gate_pos;  /* [gate_pos_rows, r] FP32 position-branch table */
  int32_t gate_pos_rows;
  const void *W_Q;        /* [H*d_h, d] rows h*d_h .. h*d_h+d_h-1 map x_m to the query Q_h[m] */
  const void *W_K;        /* [H*d_h, r] rows of head h map C'_n to its key K_h[n] */
  const void *W_V;        /* [H*d_h, r] rows of head h map C'_n to its value V_h[n] */
  const void *W_O;        /* [d, H*d_h] Y[m] = W_O (o_0; ...; o_{H-1}) */
} mtla_unabsorbed_weights;

/* Parallel forward in the per-head form ([Notes] stride-aware causal mask,
 * decoupled RoPE: training may use the uncompressed RoPE keys; [Fig1] before
 * absorption).  Same frames, gate, intermediate states and optional cache
 * and C' outputs as mtla_prefill_strided; the attention runs at head width:
 *   Q_h[m] = W_Q^(h) x_m,  K_h[n] = W_K^(h) C'_n,  V_h[n] = W_V^(h) C'_n
 *   z = (Q_h[m] . K_h[n] + QR[m, h] . KR[n]) * scale over the visible n
 *   Y[m] = W_O (o_0; ...; o_{H-1}),  o_h = sum_n softmax(z)_n V_h[n]
 * With Wq_h, Wk_h, Wv_h the row blocks of head h of W_Q, W_K, W_V and Wo_h
 * the column block of head h of W_O, the absorbed maps A[h] = Wk_h^T Wq_h
 * and Bvo[:, h, :] = Wo_h Wv_h make this exactly mtla_prefill_strided; the
 * per-head form spends 2 (d_h + d_hR) + 2 d_h flops per visible pair and head
 * on attention instead of 2 (r + d_hR) + 2 r.  Supported: (d_h, d_hR) =
 * (64, 32) or (128, 64) (else MTLA_ERR_UNSUPPORTED), with bf16 storage (MFMA
 * attention) or fp32 storage (a correctness-oriented fp32 attention
 * kernel).  Workspace:
 * mtla_workspace_bytes(op=4, B, T). */
mtla_status mtla_prefill_unabsorbed(const mtla_dims *dims, const mtla_unabsorbed_weights *w,
                                    const void *X, const void *QR, const void *KR, int32_t B,
                                    int32_t T, void *Y, const mtla_cache *cache_out,
                                    void *Cprime_out, void *workspace, size_t ws_bytes,
                                    void *stream);

/* Gradients of the per-head form's weights (device pointers, FP32,
 * overwritten by mtla_prefill_unabsorbed_backward), in the layouts of the
 * weights themselves. */
typedef struct {
  float *dW_dkv;     /* [r, d] */
  float *dW_hc;      /* [r, r]  the content-branch weight W_hc (the pages' parameter) */
  float *db_hc;      /* [r] */
  float *dgate_pos;  /* [gate_pos_rows, r] the position-branch table Linear(pe_j) */
  float *dW_Q;       /* [H*d_h, d] */
  float *dW_K;       /* [H*d_h, r] */
  float *dW_V;       /* [H*d_h, r] */
  float *dW_O;       /* [d, H*d_h] */
} mtla_unabsorbed_grads;

/* Backward of mtla_prefill_unabsorbed ([Notes] stride-aware causal mask: the
 * parallel form is what training runs; [Fig2] (c)): for the loss gradient
 * dY [B, T, d], the gradients of <dY, Y> with respect to the inputs --
 * dX [B, T, d], dQR [B, T, H, d_hR], dKR [B, T, d_hR] (storage dtype) -- and
 * to every weight (FP32, `grads`): through the output map, the masked
 * softmax (scores recomputed), the key, value and query maps, the group sums
 * (a reverse scan inside each group) and the sigmoid gate.  The gate's
 * content branch is differentiated in the pages' form, Linear(c) = W_hc c +
 * b_hc, so W_hc [r, r] (storage dtype) is passed besides the folded W_gate
 * the forward uses; the position branch is differentiated as its table.
 * The forward is recomputed inside.  Supported: (d_h, d_hR) = (64, 32) or
 * (128, 64) (else MTLA_ERR_UNSUPPORTED), with bf16 storage (MFMA kernels)
 * or fp32 storage (correctness-oriented fp32 kernels).  Workspace:
 * mtla_workspace_bytes(op=5, B, T).
 * Reproducibility: every output repeats bit for bit from call to call --
 * the sums over frames and sequences behind the weight gradients, db_hc and
 * dgate_pos add their per-workgroup partials in a fixed order. */
mtla_status mtla_prefill_unabsorbed_backward(const mtla_dims *dims,
                                             const mtla_unabsorbed_weights *w, const void *W_hc,
                                             const void *X, const void *QR, const void *KR,
                                             int32_t B, int32_t T, const void *dY, void *dX,
                                             void *dQR, void *dKR,
                                             const mtla_unabsorbed_grads *grads, void *workspace,
                                             size_t ws_bytes, void *stream);

/* Profiling variants of mtla_decode_step, mtla_prefill_strided and
 * mtla_prefill_unabsorbed: the same
 * computation, and in addition the attention kernel (the split-K decode
 * attention, resp. the strided prefill attention) is launched so that the
 * runtime stamps events[0] with its start and events[1] with its end
 * (hipExtLaunchKernel; no extra marker packets), for hipEventElapsedTime.
 * `events` points to two hipEvent_t handles (created with timing enabled)
 * owned by the caller; a missing handle is MTLA_ERR_ARG. */
mtla_status mtla_decode_step_timed(const mtla_dims *dims, const mtla_weights *w,
                                   const mtla_cache *cache, const void *X_t, const void *QR_t,
                                   const void *KR_t, const int32_t *pos, int32_t B, int32_t max_pos,
                                   void *Y, void *workspace, size_t ws_bytes, void *stream,
                                   void *const *events);
mtla_status mtla_prefill_strided_timed(const mtla_dims *dims, const mtla_weights *w, const void *X,
                                       const void *QR, const void *KR, int32_t B, int32_t T,
                                       void *Y, const mtla_cache *cache_out, void *Cprime_out,
                                       void *workspace, size_t ws_bytes, void *stream,
                                       void *const *events);
mtla_status mtla_prefill_unabsorbed_timed(const mtla_dims *dims, const mtla_unabsorbed_weights *w,
                                          const void *X, const void *QR, const void *KR,
                                          int32_t B, int32_t T, void *Y,
                                          const mtla_cache *cache_out, void *Cprime_out,
                                          void *workspace, size_t ws_bytes, void *stream,
                                          void *const *events);

/* Workspace size in bytes for op 0 (merge-append), 1 (decode step, with
 * T_or_max_pos = max_pos), 2 (prefill, with T_or_max_pos = T), 3 (chunked
 * merge-append, with T_or_max_pos = L), 4 (per-head prefill, with
 * T_or_max_pos = T), 5 (its backward, with T_or_max_pos = T) or 6 (rotary
 * inputs of B * T_or_max_pos frames).  Returns 0 for invalid arguments.
 * Pure host function. */
size_t mtla_workspace_bytes(const mtla_dims *dims, int32_t op, int32_t B, int32_t T_or_max_pos);

/* Static description of a status code.  Pure host function. */
const char *mtla_status_string(mtla_status status);

/* Description of the last failure on the calling thread ("" if none).
 * Pure host function. */
const char *mtla_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* MTLA_H */
