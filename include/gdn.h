/*
 * gdn.h -- C ABI of the gated-delta-rule (GDN) prepare / decode / prefill
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the GDN linear-attention layer of the
 * Qwen3-Next / Qwen3.5 family, as the following pages define them:
 *   [P1] vllm.cpp src/vt/cpu/cpu_ops.cpp
 *   [P2] vllm.cpp src/vllm/model_executor/models/qwen3_5.cpp
 *   [P3] ferrum-kernels 0.8.0 src/ferrum_kernels/backend/cpu.rs
 * (cited below by page and function).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Dimensions: Hk key heads, Hv value heads (Hv a multiple of Hk; value head h
 *   reads key/query head h / (Hv/Hk)), head dims Dk and Dv, conv kernel K.
 *   Cc = 2*Hk*Dk + Hv*Dv conv channels, laid out q | k | v, each head-major
 *   ([P1] GdnConvSplitKernel; [P3] linear_attention_prepare_varlen_f32).
 *   Supported: Dk, Dv in {16, 32, 64, 128, 256}; 1 <= K <= 4.
 * Pointers: "device" pointers must be device memory visible to the stream;
 *   "host" pointers are read synchronously before the call returns.  Device
 *   tensors are dense row-major, 16-byte aligned, except where a row stride
 *   (in elements) is passed; such rows must start on 16-byte boundaries.
 * Ownership: the caller owns every buffer.  The library allocates nothing;
 *   scratch memory is passed in as a workspace whose size a query returns.
 *   Weights (conv weight, A_log, dt_bias) are read in place every call.
 * Streams: `stream` is a hipStream_t (NULL = the null stream).  All device
 *   work is enqueued on it; no call synchronises the host.
 * Errors: every argument is checked on the host before any device work is
 *   enqueued; a failing check returns a non-zero gdn_status, enqueues
 *   nothing and records a message retrievable with gdn_last_error() on the
 *   calling thread.  GDN_ERR_DEVICE reports a failed kernel launch.
 * State pools: the conv history pool is [num_slots, Cc, W] in the
 *   activation dtype, W = dims.conv_state_len taps per channel (0 means
 *   K-1).  gdn_prepare, gdn_decode and gdn_decode_gated use the leading K-1
 *   taps of each row (column j holds the j-th oldest of the last K-1 raw
 *   inputs) and leave the others as they are; a wider row is the one that
 *   speculative decoding keeps (gdn_decode_spec), so both kinds of step can
 *   share one pool ([P1] CausalConv1dUpdateKernel on widened rows,
 *   GdnStateGatherKernel / GdnStateScatterKernel; [P2]
 *   ValidateGdnStateCacheLayout, CopyStateRowsStrided).  The recurrent state
 *   pool is [num_slots, Hv, Dv, Dk] (Dk
 *   contiguous) in f32, bf16 or f16 ([P2] ValidateGdnStateCacheLayout,
 *   ResolveMambaSsmCacheDType).  A call reads a slot's state at its storage
 *   dtype, computes in f32 and stores it back rounded (round to nearest
 *   even) once at the end of the call ([P2] GatherStateF32 /
 *   ScatterStateF32).  Slot indices are int32; a live slot is in
 *   [0, num_slots) and appears at most once per call; -1 marks an inert row
 *   in decode only ([P2] ValidateGdnStateIndices).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_dtype {
  GDN_F32 = 0,
  GDN_BF16 = 1,
  GDN_F16 = 2
} gdn_dtype;

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1, /* null pointer, misaligned pointer, bad flag */
  GDN_ERR_SHAPE = 2,            /* dims, offsets or strides inconsistent     */
  GDN_ERR_INDEX = 3,            /* slot index out of range or duplicated     */
  GDN_ERR_DTYPE = 4,            /* unsupported dtype combination             */
  GDN_ERR_WORKSPACE = 5,        /* workspace missing or too small            */
  GDN_ERR_DEVICE = 6            /* HIP reported an error                     */
} gdn_status;

/* Mamba2 / SSD layer dimensions: H heads of head_dim P, G groups (H a
 * multiple of G; head h uses group h / (H/G)), state_dim N. */
typedef struct gdn_ssm_dims {
  int32_t num_heads;  /* H */
  int32_t head_dim;   /* P */
  int32_t num_groups; /* G */
  int32_t state_dim;  /* N */
} gdn_ssm_dims;

/* Mamba2 step-size processing: dt = clamp(softplus(dt_raw + dt_bias[h]),
 * dt_min, dt_max), the softplus when `softplus` is non-zero (the identity
 * above 20); dt_bias may be NULL. */
typedef struct gdn_ssm_dt {
  const float* dt_bias; /* device f32 [H] or NULL */
  int32_t softplus;
  float dt_min, dt_max;
} gdn_ssm_dt;

typedef struct gdn_dims {
  int32_t num_k_heads; /* Hk */
  int32_t num_v_heads; /* Hv, a multiple of Hk */
  int32_t head_k_dim;  /* Dk */
  int32_t head_v_dim;  /* Dv */
  int32_t conv_kernel; /* K */
  int32_t conv_state_len; /* W, taps per conv-history row: 0 (= K-1) or K-1 <= W <= 1024 */
} gdn_dims;

/*
 * gdn_prepare -- varlen prepare step (conv + SiLU, split, L2 norm, gates).
 *
 * Defined by [P1] CausalConv1dFwdKernel, GdnPostConvKernel, L2NormKernel,
 * GdnGBetaKernel and [P3] linear_attention_prepare_varlen_f32.
 * For every sequence s (tokens cu[s] .. cu[s+1]-1, each sequence non-empty),
 * channel c and token t:
 *   y[t,c] = silu( sum_j w[c,j] * x_s(t-(K-1)+j) ),
 * where x_s(p) is mixed_qkv[p, c] inside the sequence and, before its start,
 * the conv history row of the sequence's slot (when has_initial_state[s] is
 * non-zero) or zero.  Then q = y[:, q block], k = y[:, k block], v = y[:, v
 * block]; when apply_qk_l2norm is non-zero, q and k are scaled per (token,
 * key head) by 1/sqrt(sum of squares + 1e-6).  Per (token, value head):
 *   g    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 *   beta = sigmoid(b[t,h]).
 * Finally the history row of each sequence's slot is replaced by the
 * sequence's last K-1 raw inputs (a sequence shorter than K-1 keeps the
 * tail of the old history in front of them).
 *
 * Arguments:
 *   dims                  layer dimensions (see above).
 *   num_seqs, total_tokens N >= 1 sequences, T = cu[N] tokens (N = T = 0 is a no-op).
 *   cu_seqlens_host       host int32 [N+1], cu[0] = 0, strictly increasing, cu[N] = T.
 *   cu_seqlens_dev        device copy of the same offsets.
 *   mixed_qkv             device [T, mixed_row_stride] in act_dtype; the first Cc columns are used.
 *   a_raw, b_raw          device [T, row stride] in act_dtype; the first Hv columns are used.
 *   act_dtype             GDN_F32 or GDN_BF16; also the dtype of conv_weight and of the history pool.
 *   conv_weight           device [Cc, K] in act_dtype.
 *   A_log, dt_bias        device f32 [Hv].
 *   conv_state_pool       device [num_slots, Cc, W] in act_dtype, read and written in place
 *                         (may be NULL when K = 1).
 *   slot_idx_host/_dev    int32 [N] slot of each sequence; both NULL means slot s for sequence s.
 *   has_initial_state_dev device uint8 [N], or NULL for "every sequence continues its slot".
 *   q_out, k_out          device [T, Hk, Dk] in qkv_dtype (GDN_F32 or GDN_BF16).
 *   v_out                 device [T, Hv, Dv] in qkv_dtype.
 *   g_out, beta_out       device f32 [T, Hv].
 */
gdn_status gdn_prepare(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                       const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                       const void* mixed_qkv, int64_t mixed_row_stride, const void* a_raw,
                       int64_t a_row_stride, const void* b_raw, int64_t b_row_stride,
                       gdn_dtype act_dtype, const void* conv_weight, const float* A_log,
                       const float* dt_bias, void* conv_state_pool, int32_t num_slots,
                       const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                       const uint8_t* has_initial_state_dev, int32_t apply_qk_l2norm,
                       void* q_out, void* k_out, void* v_out, gdn_dtype qkv_dtype,
                       float* g_out, float* beta_out, void* stream);

/*
 * gdn_decode -- fused single-token step for a batch of rows against the
 * slot-indexed pools: the prepare step of one token (conv against the slot's
 * history, which is then shifted left by one and appended with the raw
 * input; SiLU; q/k L2 norm, always applied; gates) followed by one step of
 * the gated delta rule per value head h with key head kh = h/(Hv/Hk):
 *   S <- exp(g) S;  u = S k;  delta = beta (v - u);  S <- S + delta k^T;
 *   o = S (scale q)
 * on the [Dv, Dk] state of the row's slot, in place.
 *
 * Defined by [P1] CausalConv1dUpdateKernel, GdnPackedDecodeKernel,
 * GdnDecodeKernel, GdnHeadTokenStep and [P3]
 * linear_attention_decode_prepare_f32, recurrent_gated_delta_rule_batch_f32.
 * A row whose slot is -1 gets a zero output and touches neither pool
 * ([P1] GdnDecodeKernel, CausalConv1dUpdateKernel).
 *
 * Arguments:
 *   batch                 B >= 0 rows (B = 0 is a no-op).
 *   mixed_qkv, a_raw, b_raw, act_dtype, conv_weight, A_log, dt_bias: as gdn_prepare, with B rows.
 *   conv_state_pool       device [num_slots, Cc, W] in act_dtype, in place.
 *   ssm_state_pool        device [num_slots, Hv, Dv, Dk] in state_dtype, in place.
 *   slot_idx_dev          device int32 [B]; -1 = inert row.
 *   slot_idx_host         host copy for validation (range, -1 only negative, no duplicate live slot),
 *                         or NULL to skip it; the kernel then treats any slot outside
 *                         [0, num_slots) as inert, and duplicated live slots race.
 *   scale                 query scale (1/sqrt(Dk) in the Qwen3-Next layer).
 *   out                   device [B, Hv, Dv] in act_dtype.
 */
gdn_status gdn_decode(const gdn_dims* dims, int32_t batch, const void* mixed_qkv,
                      int64_t mixed_row_stride, const void* a_raw, int64_t a_row_stride,
                      const void* b_raw, int64_t b_row_stride, gdn_dtype act_dtype,
                      const void* conv_weight, const float* A_log, const float* dt_bias,
                      void* conv_state_pool, void* ssm_state_pool, gdn_dtype state_dtype,
                      int32_t num_slots, const int32_t* slot_idx_dev,
                      const int32_t* slot_idx_host, float scale, void* out, void* stream);

/*
 * gdn_decode_gated -- gdn_decode with the layer's output epilogue fused (the
 * gated RMS norm of gdn_gated_rmsnorm, below): equal to gdn_decode followed
 * by gdn_gated_rmsnorm on the same rows, including the rounding of o to
 * act_dtype that storing and reloading it would make.  The fusion is
 * possible because one workgroup of the decode kernel owns every value row
 * of its heads.  [P1] RmsNormGatedKernel; [P3] gated_rms_norm_f32.
 *
 * Arguments: those of gdn_decode, plus
 *   z, z_row_stride       device gate in act_dtype: row b, value head h, element j at
 *                         z[b * z_row_stride + h * Dv + j]; z_row_stride >= Hv * Dv, so z may be
 *                         the z columns of a packed [q | k | v | z] projection row.
 *   norm_weight           device [Dv] in act_dtype.
 *   eps                   finite, >= 0 (inside the square root, next to the mean of squares).
 *   sigmoid_gate          0: silu gate; 1: logistic gate.
 *   out                   device [B, Hv, Dv] in act_dtype: the gated, normalised output.
 * Errors: those of gdn_decode; a null z or norm_weight, a short z_row_stride or a bad eps or
 * sigmoid_gate is GDN_ERR_INVALID_ARGUMENT / GDN_ERR_SHAPE.
 */
gdn_status gdn_decode_gated(const gdn_dims* dims, int32_t batch, const void* mixed_qkv,
                            int64_t mixed_row_stride, const void* a_raw, int64_t a_row_stride,
                            const void* b_raw, int64_t b_row_stride, gdn_dtype act_dtype,
                            const void* conv_weight, const float* A_log, const float* dt_bias,
                            void* conv_state_pool, void* ssm_state_pool, gdn_dtype state_dtype,
                            int32_t num_slots, const int32_t* slot_idx_dev,
                            const int32_t* slot_idx_host, float scale, const void* z,
                            int64_t z_row_stride, const void* norm_weight, float eps,
                            int32_t sigmoid_gate, void* out, void* stream);

/*
 * gdn_decode_spec -- speculative multi-token decode: each request carries up
 * to C = num_cols tokens (the last accepted token and the draft tokens after
 * it) and a row of C state slots, and every token's state is kept so that
 * the next step can resume after whichever token was accepted last.
 * Defined by [P1] CausalConv1dSpecUpdateKernel and GdnSpecDecodeKernel, with
 * the metadata rules of the speculative part of [P2]
 * ValidateGdnAttentionMetadata.
 *
 * Request i has tokens cu[i] .. cu[i+1]-1 (1 <= L_i <= C of them), slot row
 * state_idx[i, 0..C-1] and n_i = num_accepted[i] in [1, C].
 *   Conv: the request's conv-history row is that of slot state_idx[i, 0],
 *     widened to W >= (K-1) + (C-1) taps.  With off = n_i - 1, the conv reads
 *     the K-1 taps of the row starting at tap off followed by the L_i raw
 *     inputs (a tap past the row's end reads as zero); token t's output is
 *     silu of the K-tap product at stream positions t .. t+K-1.  The row then
 *     becomes its taps off+1 .. off+W-L_i followed by the L_i inputs, so that
 *     the next step's offset selects the window ending at its last accepted
 *     token.
 *   Recurrence: starts from the state in slot state_idx[i, n_i - 1] (the state
 *     after the last accepted token of the previous step); q/k L2 norm, gates
 *     and the token step are those of gdn_decode.  After token t the state is
 *     stored into slot state_idx[i, t], rounded to state_dtype (the running
 *     state is not rounded); a -1 column skips only that store.
 *   A request whose slot state_idx[i, n_i - 1] is -1 is padding: zero output,
 *     neither pool touched.
 * The pages leave open which slot holds a request's conv row; column 0 is
 * taken (the row is shifted in place rather than copied per token, so it
 * needs one fixed slot per request).
 *
 * Arguments:
 *   dims                  as gdn_decode; K >= 2; dims.conv_state_len = W >= (K-1) + (C-1).
 *   num_reqs, total_tokens, cu_seqlens_host/_dev: as gdn_prepare (N requests, T tokens), with
 *                         every request's token count at most C.
 *   mixed_qkv, a_raw, b_raw, act_dtype, conv_weight, A_log, dt_bias: as gdn_prepare, T rows.
 *   conv_state_pool       device [num_slots, Cc, W] in act_dtype, in place.
 *   ssm_state_pool        device [num_slots, Hv, Dv, Dk] in state_dtype, in place.
 *   num_cols              C, 1 <= C <= 8.
 *   state_idx_dev         device int32 [N, C].
 *   num_accepted_dev      device int32 [N].
 *   state_idx_host, num_accepted_host  host copies for validation (both or neither): n_i in
 *                         [1, C]; every entry -1 or in [0, num_slots); a live request's column 0
 *                         live; live slots distinct across the whole table.  With neither, the
 *                         kernel treats a request whose n_i, initial slot or column-0 slot is out
 *                         of range as padding and skips stores to out-of-range columns, and
 *                         repeated slots race.
 *   scale                 query scale.
 *   out                   device [T, Hv, Dv] in act_dtype.
 */
gdn_status gdn_decode_spec(const gdn_dims* dims, int32_t num_reqs, int64_t total_tokens,
                           const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                           const void* mixed_qkv, int64_t mixed_row_stride, const void* a_raw,
                           int64_t a_row_stride, const void* b_raw, int64_t b_row_stride,
                           gdn_dtype act_dtype, const void* conv_weight, const float* A_log,
                           const float* dt_bias, void* conv_state_pool, void* ssm_state_pool,
                           gdn_dtype state_dtype, int32_t num_slots, int32_t num_cols,
                           const int32_t* state_idx_dev, const int32_t* num_accepted_dev,
                           const int32_t* state_idx_host, const int32_t* num_accepted_host,
                           float scale, void* out, void* stream);

/*
 * gdn_kda_recurrent -- KDA, the gated delta rule with one log-decay per key
 * channel, token by token over varlen sequences against the slot-indexed
 * state pool ([P1] KdaHeadTokenStep, KdaGatedDeltaRuleKernel).  Per token t
 * of a sequence, value head h, key head kh = h / (Hv/Hk), [Dv, Dk] state S:
 *   S[:, d] <- exp(g[t,h,d]) S[:, d]   (each state column decays on its own)
 *   u = S k;  delta = beta[t,h] (v - u);  S <- S + delta k^T;  o = S (scale q)
 * With A_log non-NULL, g holds the gate's input and the log-decay is
 *   -exp(A_log[h]) * softplus(g[t,h,d] + dt_bias[h,d])   (dt_bias NULL = 0)
 * as [P1] KdaChunkPrefillKernel computes it.  q and k are used as given unless
 * use_qk_l2norm is set.  Sequence s starts from its slot's state (zero when
 * has_initial_state[s] is 0) and its final state is written back, rounded to
 * state_dtype; an empty sequence writes back its initial state.
 *
 * Arguments:
 *   dims                  as the other entry points (conv_kernel unused).
 *   num_seqs, total_tokens, cu_seqlens_host/_dev: N >= 0 sequences, T tokens; cu[0] = 0,
 *                         non-decreasing (empty sequences allowed), cu[N] = T.
 *   q, k                  device [T, Hk, Dk] in qkv_dtype (GDN_F32 or GDN_BF16).
 *   v                     device [T, Hv, Dv] in qkv_dtype.
 *   g                     device f32 [T, Hv, Dk].
 *   A_log                 device f32 [Hv] or NULL (g is then the log-decay itself).
 *   dt_bias               device f32 [Hv, Dk] or NULL; only with A_log.
 *   beta                  device f32 [T, Hv].
 *   ssm_state_pool        device [num_slots, Hv, Dv, Dk] in state_dtype, in place.
 *   slot_idx_host/_dev    int32 [N] (both NULL: slot s); -1 is refused.
 *   has_initial_state_dev device uint8 [N] or NULL (= all 1).
 *   scale                 query scale.
 *   use_qk_l2norm         1: L2-normalise q and k per (token, key head), eps 1e-6.
 *   out                   device [T, Hv, Dv] in qkv_dtype.
 * q, k, v, g, dt_bias, out and the pool must be 16-byte aligned.
 */
gdn_status gdn_kda_recurrent(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                             const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* q,
                             const void* k, const void* v, gdn_dtype qkv_dtype, const float* g,
                             const float* A_log, const float* dt_bias, const float* beta, void* ssm_state_pool,
                             gdn_dtype state_dtype, int32_t num_slots, const int32_t* slot_idx_host,
                             const int32_t* slot_idx_dev, const uint8_t* has_initial_state_dev, float scale,
                             int32_t use_qk_l2norm, void* out, void* stream);

/*
 * gdn_kda_prefill_varlen -- gdn_kda_recurrent's result computed in chunks of
 * 64 tokens (the WY / UT form with one decay per key channel), equal to it up
 * to rounding order ([P1] KdaChunkPrefillKernel, which defines the chunked
 * forward as the recurrence's output).  Head dims other than Dk = Dv in
 * {32, 64, 128} run the token-by-token kernel of gdn_kda_recurrent.
 *
 * Arguments: those of gdn_kda_recurrent, plus
 *   chunk_size            0 (= 64) or 64.
 *   workspace             device scratch of at least gdn_kda_prefill_workspace_size() bytes,
 *                         256-byte aligned; its contents need not be initialised.
 */
gdn_status gdn_kda_prefill_varlen(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                  const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* q,
                                  const void* k, const void* v, gdn_dtype qkv_dtype, const float* g,
                                  const float* A_log, const float* dt_bias, const float* beta, void* ssm_state_pool,
                                  gdn_dtype state_dtype, int32_t num_slots, const int32_t* slot_idx_host,
                                  const int32_t* slot_idx_dev, const uint8_t* has_initial_state_dev, float scale,
                                  int32_t use_qk_l2norm, int32_t chunk_size, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Workspace bytes gdn_kda_prefill_varlen needs for N sequences of T tokens
 * in total with q/k/v of qkv_dtype (0 when no workspace is used, or for
 * invalid arguments). */
size_t gdn_kda_prefill_workspace_size(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                      int32_t chunk_size, gdn_dtype qkv_dtype);

/*
 * gdn_mamba2_state_update -- one Mamba2 / SSD step per row against the
 * slot-indexed state pool [num_slots, H, P, N] ([P1] Mamba2StateUpdateKernel).
 * Not the delta rule: for row b, head h, group g = h / (H/G):
 *   dt = processed step (gdn_ssm_dt);  S <- exp(A[h] dt) S + dt x B^T
 *   y[p] = sum_n S[p][n] C[n] + D x[p];  y *= silu(z[p]) when z is given
 * S read at the pool dtype, computed in f32, stored back rounded.  A row whose
 * slot is -1 gets a zero output and touches nothing.
 *
 * Arguments:
 *   sdims                 H, P (1..1024), G, N in {16, 32, 64, 128, 256}.
 *   batch                 B >= 0 rows.
 *   x, z                  device [B, H, P] in act_dtype (z may be NULL).
 *   dt                    device [B, H] in act_dtype, the raw step.
 *   A                     device f32 [H], every entry < 0 (A = -exp(A_log)).
 *   B, C                  device [B, G, N] in act_dtype.
 *   D, D_per_head_dim     device f32 [H] (0) or [H, P] (1), or NULL.
 *   dtp                   step processing (dt_bias device f32 [H] or NULL); dt_min >= 0.
 *   act_dtype             GDN_F32 or GDN_BF16.
 *   state_pool            device [num_slots, H, P, N] in state_dtype, in place.
 *   slot_idx_dev/_host    int32 [B] as gdn_decode.
 *   out                   device [B, H, P] in act_dtype.
 * x, B, C, z, out and the pool must be 16-byte aligned.
 */
gdn_status gdn_mamba2_state_update(const gdn_ssm_dims* sdims, int32_t batch, const void* x, const void* dt,
                                   const float* A, const void* B, const void* C, const float* D,
                                   int32_t D_per_head_dim, const void* z, const gdn_ssm_dt* dtp,
                                   gdn_dtype act_dtype, void* state_pool, gdn_dtype state_dtype,
                                   int32_t num_slots, const int32_t* slot_idx_dev, const int32_t* slot_idx_host,
                                   void* out, void* stream);

/*
 * gdn_mamba2_chunk_scan -- Mamba2 / SSD over varlen sequences (the same
 * recurrence as gdn_mamba2_state_update, token by token), computed in chunks
 * of 64 tokens in the dual form ([P1] Mamba2ChunkScanKernel, whose five
 * stages compute it).  Sequence s starts from its slot's state (zero when
 * has_initial_state[s] is 0) and its final state is written back, rounded
 * once to the pool dtype; the states passed between chunks stay f32 (the
 * pages round them to the pool dtype as well).
 *
 * Arguments: those of gdn_mamba2_state_update over T tokens, plus
 *   num_seqs, total_tokens, cu_seqlens_host/_dev: as gdn_prepare (no empty sequence).
 *   sdims                 P in {32, 64, 128}, N in {32, 64, 128}.
 *   slot_idx_host/_dev    int32 [N] (both NULL: slot s); -1 is refused.
 *   has_initial_state_dev device uint8 [N] or NULL (= all 1).
 *   workspace             device scratch of at least gdn_mamba2_workspace_size() bytes,
 *                         256-byte aligned.
 */
gdn_status gdn_mamba2_chunk_scan(const gdn_ssm_dims* sdims, int32_t num_seqs, int64_t total_tokens,
                                 const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* x,
                                 const void* dt, const float* A, const void* B, const void* C, const float* D,
                                 int32_t D_per_head_dim, const void* z, const gdn_ssm_dt* dtp,
                                 gdn_dtype act_dtype, void* state_pool, gdn_dtype state_dtype, int32_t num_slots,
                                 const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                                 const uint8_t* has_initial_state_dev, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Workspace bytes gdn_mamba2_chunk_scan needs (0 for invalid arguments). */
size_t gdn_mamba2_workspace_size(const gdn_ssm_dims* sdims, int32_t num_seqs, int64_t total_tokens);

/*
 * gdn_gated_rmsnorm -- the layer's output epilogue, for the output of
 * gdn_prefill_varlen (or of gdn_decode): for every token t and value head h,
 * over the Dv values of the head,
 *   out[t,h,:] = x[t,h,:] / sqrt(mean_j x[t,h,j]^2 + eps) * weight[:] * act(z[t,h,:])
 * with act = silu, or the logistic function when sigmoid_gate is set: the
 * norm is taken before the gate, one group per head.  [P1]
 * RmsNormGatedKernel; [P3] gated_rms_norm_f32.
 *
 * Arguments:
 *   num_tokens            T >= 0 (T = 0 is a no-op).
 *   num_heads, head_dim   Hv > 0; Dv in {16, 32, 64, 128, 256}.
 *   x                     device [T, Hv, Dv] in io_dtype.
 *   z, z_row_stride       device gate in io_dtype: token t, head h, element j at
 *                         z[t * z_row_stride + h * Dv + j]; z_row_stride >= Hv * Dv.
 *   weight                device [Dv] in io_dtype.
 *   eps                   finite, >= 0.
 *   sigmoid_gate          0: silu gate; 1: logistic gate.
 *   out                   device [T, Hv, Dv] in io_dtype; may be x itself (in place), must not
 *                         otherwise overlap x or z.
 *   io_dtype              GDN_F32 or GDN_BF16.
 * x, z, weight and out must be 16-byte aligned and z_row_stride a whole number of 16-byte words.
 */
gdn_status gdn_gated_rmsnorm(int32_t num_tokens, int32_t num_heads, int32_t head_dim, const void* x,
                             const void* z, int64_t z_row_stride, const void* weight, float eps,
                             int32_t sigmoid_gate, void* out, gdn_dtype io_dtype, void* stream);

/*
 * gdn_prefill_varlen -- the gated delta rule over whole sequences, computed
 * in chunks of chunk_size tokens with the WY / UT-transform form, equal to
 * the token-by-token recurrence of gdn_decode up to rounding order ([P1]
 * GdnPrefillKernel; [P3] recurrent_gated_delta_rule_varlen_f32).  Sequence s
 * starts from its slot's state (or from zero when has_initial_state[s] is
 * 0) and its final state is written back to the same slot.
 *
 * Arguments:
 *   num_seqs, total_tokens, cu_seqlens_host/_dev: as gdn_prepare.
 *   q, k                  device [T, Hk, Dk] in qkv_dtype (GDN_F32 or GDN_BF16).
 *   v                     device [T, Hv, Dv] in qkv_dtype.
 *   g, beta               device f32 [T, Hv] (log decay and write strength).
 *   ssm_state_pool        device [num_slots, Hv, Dv, Dk] in state_dtype, in place.
 *   slot_idx_host/_dev    int32 [N] (both NULL: slot s); -1 is refused.
 *   has_initial_state_dev device uint8 [N] or NULL (= all 1).
 *   scale                 query scale.
 *   use_qk_l2norm         non-zero: L2-normalise q and k here (eps 1e-6), for callers whose
 *                         prepare step did not.
 *   chunk_size            0 (= 64) or 64.
 *   out                   device [T, Hv, Dv] in qkv_dtype.
 *   workspace             device scratch of at least gdn_prefill_workspace_size() bytes,
 *                         256-byte aligned; its contents need not be initialised.
 */
gdn_status gdn_prefill_varlen(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                              const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                              const void* q, const void* k, const void* v, gdn_dtype qkv_dtype,
                              const float* g, const float* beta, void* ssm_state_pool,
                              gdn_dtype state_dtype, int32_t num_slots,
                              const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                              const uint8_t* has_initial_state_dev, float scale,
                              int32_t use_qk_l2norm, int32_t chunk_size, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes gdn_prefill_varlen needs for at most num_seqs sequences and
 * total_tokens tokens (0 if the arguments are invalid). */
size_t gdn_prefill_workspace_size(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                  int32_t chunk_size);

/* Bytes of device memory the library holds, on every device it runs on, for
 * gdn_prefill_varlen_noalloc: a static array, resident until the process ends. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * gdn_prefill_varlen_noalloc -- gdn_prefill_varlen for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation): it takes no workspace and allocates
 * nothing.  Its scratch is a static device array of GDN_NOALLOC_SCRATCH_BYTES
 * per device (its address is looked up once per device, on the first call
 * made with that device current).  When the batch needs more scratch than
 * that, the value heads run in groups that fit, one group after another on
 * the stream; each head is computed exactly as gdn_prefill_varlen computes
 * it, so the results are the same.
 *
 * Arguments: those of gdn_prefill_varlen without workspace / workspace_bytes.
 * Errors: those of gdn_prefill_varlen; GDN_ERR_WORKSPACE when a single value
 *   head's scratch, gdn_prefill_workspace_size() with Hv = 1, exceeds
 *   GDN_NOALLOC_SCRATCH_BYTES (about 74 k tokens with Dk = Dv = 128).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (the prefill reads nothing of it that it has not written in
 * the same call): calls that overlap on one device, on different streams or
 * from different threads, race and must be ordered by the caller.
 */
gdn_status gdn_prefill_varlen_noalloc(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                      const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                                      const void* q, const void* k, const void* v, gdn_dtype qkv_dtype,
                                      const float* g, const float* beta, void* ssm_state_pool,
                                      gdn_dtype state_dtype, int32_t num_slots,
                                      const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                                      const uint8_t* has_initial_state_dev, float scale,
                                      int32_t use_qk_l2norm, int32_t chunk_size, void* out, void* stream);

/* Static English name of a status code. */
const char* gdn_status_string(gdn_status status);

/* Message of the last failing call on this thread ("" if none). */
const char* gdn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
