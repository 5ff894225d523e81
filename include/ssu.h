/*
 * ssu.h -- C ABI of libssu: the Mamba-style selective state update (SSU) over a
 * paged recurrent-state pool, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (page titles and the passage on each page):
 *   [SSU]  TensorRT-Edge-LLM, "Selective State Update" page:
 *          mamba_ssm::invokeSelectiveStateUpdate (decode, "Computes" paragraph
 *          and shape list), invokeSelectiveStateUpdatePrefill (prefill loop,
 *          replay stash), struct MambaReplayLayerInfo (replay reconstruct),
 *          invokeMambaReplayReconstructBatched (acceptedNodeIds, maxAcceptLen),
 *          invokeSelectiveStateUpdateDDTree (tree verify),
 *          struct MambaStateLayerInfo, invokeMambaStateClear (slot clear,
 *          slot -1 = all, every layer in one launch).
 *   [PAD]  FlashInfer, "flashinfer.gdn_fused_decode_step" page, parameters
 *          ssm_state (paged pool, padded row stride) and state_indices
 *          (negative index = padding row; index >= rows is a caller bug).
 *   [RSM]  TensorRT-Edge-LLM, "Recurrent State Manager" page: constructor
 *          (specs, slotCount, name, stream), spec, specs, clear, clearSlot,
 *          capture, restore, copySlotFrom, bytesPerSlot, stateBytesPerSlot,
 *          findState.
 *   [DNP]  Smile, "Class DeltaNetStatePool" page: activateStep, scatterActive
 *          (pack a cohort's home rows into working slots [0, B) and back).
 *   [GDN]  FlashInfer, "flashinfer.gdn_fused_decode_step" page: the fused
 *          gated-delta-rule decode step over paged conv / ssm pools.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, dense
 *     (C-contiguous) in the layout stated below, except that pool rows of
 *     `state` may be padded (state_row_stride). state, B, C and replay_B are
 *     read with 16-byte vector loads and must be 16-byte aligned; every other
 *     pointer must be aligned to its element size.
 *   - Every compute call is asynchronous on `stream` (0 = the null stream). It
 *     allocates nothing, never synchronises and never reads device data on the
 *     host, so it may be recorded under hipGraph stream capture.
 *   - Host-side argument checks only. A failed check returns SSU_EINVAL or
 *     SSU_ENOTSUP, launches nothing and writes nothing; ssu_last_error() then
 *     describes it. Errors never propagate as C++ exceptions.
 *   - Values inside device arrays are never validated: a negative state index
 *     is a padding row [PAD]; an index >= pool rows, or the same live index
 *     twice in one call, is undefined behaviour (a caller bug, as [PAD] states
 *     for out-of-range indices).
 *   - Floating-point arithmetic is fp32 whatever the storage dtype. fp16 and
 *     bf16 stores round to nearest even.
 */
#ifndef SSU_H
#define SSU_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ssu_status;
#define SSU_OK 0      /* success                                            */
#define SSU_EINVAL 1  /* invalid argument (null pointer, bad shape, range)   */
#define SSU_ENOTSUP 2 /* valid but unsupported (dtype, dstate)               */
#define SSU_EHIP 3    /* a HIP runtime call or kernel launch failed          */
#define SSU_ENOMEM 4  /* device allocation failed                            */

/* Storage dtypes (ssu_dims fields and ssu_state_spec.dtype). */
#define SSU_F32 0
#define SSU_F16 1
#define SSU_BF16 2
#define SSU_U8 3 /* raw bytes: pool specs only */

/* Geometry and dtypes of one call [SSU shape lists].
 *   nheads % ngroups == 0; head h reads group h / (nheads / ngroups).
 *   dstate in {16, 32, 64, 128, 256}; 1 <= dim <= 4096.
 *   state_dtype: SSU_F32, SSU_F16 or SSU_BF16 ([SSU] "half or float"; bf16 extra).
 *   io_dtype (x, z, out) and bc_dtype (B, C): SSU_F32, SSU_F16 or SSU_BF16.
 *   A, dt, dt_bias, D and the replay stash are always fp32.
 *   state_row_stride: elements between consecutive pool rows; 0 means dense
 *   (nheads*dim*dstate). A larger stride is allowed [PAD ssm_state]; stride
 *   times the element size must be a multiple of 16 bytes. */
typedef struct ssu_dims {
    int32_t batch;      /* rows of x / indices (decode, prefill); stash rows (replay) */
    int32_t nheads;
    int32_t dim;        /* head dimension */
    int32_t dstate;
    int32_t ngroups;
    int32_t pool_rows;  /* leading extent of `state`; with no state_indices, batch <= pool_rows */
    int64_t state_row_stride;
    int32_t state_dtype;
    int32_t io_dtype;
    int32_t bc_dtype;
    int32_t reserved;   /* must be 0 */
} ssu_dims;

/* ssu_decode -- one token (seq_len == 1) [SSU invokeSelectiveStateUpdate]:
 *   dt'       = dt[b,h] + dt_bias[h];  dt' = softplus(dt') if dt_softplus
 *   state[r,h,d,n] = state[r,h,d,n] * exp(A[h]*dt') + B[b,g,n] * dt' * x[b,h,d]
 *   out[b,h,d]     = sum_n state[r,h,d,n]*C[b,g,n] + D[h]*x[b,h,d], then
 *                    * silu(z[b,h,d]) if z is given
 * with r = state_indices[b] (or b when state_indices is NULL).
 * Layouts: x, z, out [batch, nheads, dim] (io_dtype); A, dt_bias, D [nheads];
 * dt [batch, nheads]; B, C [batch, ngroups, dstate] (bc_dtype);
 * state [pool_rows, nheads, dim, dstate] (state_dtype), updated in place.
 * Padding [PAD]: r < 0 -> state not read or written, out[b] = +0.0.
 * Optional (NULL allowed): dt_bias, D, z, state_indices. */
ssu_status ssu_decode(const ssu_dims *dims, const void *x, const float *A, const void *B,
                      const void *C, const float *dt, const float *dt_bias, const float *D,
                      const void *z, void *state, void *out, int32_t dt_softplus,
                      const int32_t *state_indices, hipStream_t stream);

/* ssu_prefill -- seq_len tokens in one launch [SSU invokeSelectiveStateUpdatePrefill].
 * Layouts: x, z, out [batch, seq_len, nheads, dim]; dt [batch, seq_len, nheads];
 * B, C [batch, seq_len, ngroups, dstate]; other tensors as ssu_decode.
 * context_lengths [batch] (NULL = all seq_len): row b runs tokens
 * t < L_b = clamp(context_lengths[b], 0, seq_len) through the decode step in
 * order and writes out[b,t] = +0.0 for t >= L_b; the state is left after L_b
 * tokens (untouched when L_b == 0).
 * Replay stash (all four or none) [SSU]: when given, the committed state is
 * read-only and, for t < L_b, the kernel stores
 *   replay_dA [batch, seq_len, nheads]          = A[h] * dt'   (log-decay)
 *   replay_dt [batch, seq_len, nheads]          = dt'
 *   replay_u  [batch, seq_len, nheads, dim]     = x  (unscaled, fp32)
 *   replay_B  [batch, seq_len, ngroups, dstate] = B  (fp32)
 * and zeros for t >= L_b; outputs are produced as without the stash.
 * Padding rows: out[b,:] = +0.0, state and stash rows untouched.
 * Numerics: fp32 state arithmetic either way. With x/z/out and B/C both bf16 or
 * both fp16, dstate a multiple of 32, dim a multiple of 8 and x, z, out and
 * replay_u 16-byte aligned, the tokens are evaluated 32 at a time in closed form
 * on the matrix cores; otherwise one at a time. Both agree with the token-by-token
 * recurrence to fp32 rounding, not bitwise; dt' and the stash are bit-identical. */
ssu_status ssu_prefill(const ssu_dims *dims, int32_t seq_len, const void *x, const float *A,
                       const void *B, const void *C, const float *dt, const float *dt_bias,
                       const float *D, const void *z, void *state, void *out,
                       int32_t dt_softplus, const int32_t *context_lengths,
                       const int32_t *state_indices, float *replay_dA, float *replay_u,
                       float *replay_B, float *replay_dt, hipStream_t stream);

/* ssu_replay -- commit accepted draft tokens [SSU MambaReplayLayerInfo,
 * invokeMambaReplayReconstructBatched]: for b < active_batch with
 * r = state_indices[b] >= 0, apply k tokens in place, in order:
 *   state[r,h,d,n] = state[r,h,d,n]*exp(replay_dA[b,p,h])
 *                    + replay_B[b,p,g,n]*replay_dt[b,p,h]*replay_u[b,p,h,d]
 * where token t reads stash position p = t and k = min(accepted_lengths[b], seq_len)
 * when accepted_node_ids is NULL; otherwise p = accepted_node_ids[b, t]
 * ([dims->batch, max_accept_len] int32, the accepted path of a tree verify,
 * root first), k = min(accepted_lengths[b], max_accept_len), and the row stops
 * before the first p outside [0, seq_len).
 * Stash layouts as ssu_prefill with dims->batch rows (the allocation);
 * accepted_lengths and state_indices [dims->batch] int32. Entries at
 * b >= active_batch are never read; rows with k == 0 are left untouched.
 * Requires 0 <= active_batch <= dims->batch, and max_accept_len >= 1 when
 * accepted_node_ids is given (ignored otherwise). state_indices may be NULL (r = b). */
ssu_status ssu_replay(const ssu_dims *dims, int32_t seq_len, void *state,
                      const float *replay_dA, const float *replay_u, const float *replay_B,
                      const float *replay_dt, const int32_t *accepted_lengths,
                      const int32_t *state_indices, int32_t active_batch,
                      const int32_t *accepted_node_ids, int32_t max_accept_len,
                      hipStream_t stream);

/* Most nodes one draft tree may hold (the verify budget of the tree kernel) [SSU]. */
#define SSU_MAX_TREE_NODES 128

/* ssu_tree_verify -- tree speculative verify [SSU invokeSelectiveStateUpdateDDTree].
 * Every batch row b carries a draft tree of num_nodes nodes
 * (0 <= num_nodes <= SSU_MAX_TREE_NODES) in topological order: the parent of
 * node m is parent_ids[b,m] < m, or negative when m hangs directly under the
 * committed state. The path of m is m, its parent, the parent's parent, ...,
 * taking at most depths[b,m] hops (any number when depths is NULL) and ending
 * at a parent id that is negative or not smaller than the node it belongs to.
 * The decode step of ssu_decode runs along the path, root first, starting
 * from pool row r = state_indices[b] (or b), and out[b,m] is the output of the
 * step of node m itself. The pool is only read: the committed state never
 * changes.
 * Layouts: x, z, out [batch, num_nodes, nheads, dim] (io_dtype);
 * dt [batch, num_nodes, nheads]; B, C [batch, num_nodes, ngroups, dstate]
 * (bc_dtype); parent_ids, depths [batch, num_nodes] int32; A, dt_bias, D
 * [nheads]; state [pool_rows, nheads, dim, dstate] (state_dtype).
 * Replay stash (all four or none): as ssu_prefill with the node axis in place
 * of the token axis, holding every node's own A[h]*dt', dt', x and B; commit an
 * accepted path with ssu_replay and accepted_node_ids.
 * z is optional (NULL: no gate; the page's form of this kernel has none), as
 * are dt_bias, D, depths and state_indices.
 * Padding rows (r < 0): out[b] = +0.0, stash rows untouched.
 * workspace: caller-owned device scratch of at least
 * ssu_tree_workspace_bytes(dims, num_nodes) bytes, 16-byte aligned (it
 * carries the B . C dots of every node pair, shared by all heads, from the
 * first of the two launches to the second); contents on entry ignored, on
 * return unspecified; calls sharing a workspace must be ordered (one stream). */
ssu_status ssu_tree_verify(const ssu_dims *dims, int32_t num_nodes, const void *x,
                           const float *A, const void *B, const void *C, const float *dt,
                           const float *dt_bias, const float *D, const void *z,
                           const void *state, void *out, int32_t dt_softplus,
                           const int32_t *state_indices, const int32_t *parent_ids,
                           const int32_t *depths, float *replay_dA, float *replay_u,
                           float *replay_B, float *replay_dt, void *workspace,
                           int64_t workspace_bytes, hipStream_t stream);

/* Bytes of the library-owned scratch of ssu_tree_verify_noalloc (per GPU). */
#define SSU_TREE_SCRATCH_BYTES 4194304

/* ssu_tree_verify_noalloc -- ssu_tree_verify for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same operation, arguments and kernels, except
 * that the B . C dots go to a device array the library holds for the life of
 * the process, SSU_TREE_SCRATCH_BYTES bytes on each GPU it runs on, instead of
 * a caller workspace. The caller still passes every input and output.
 * Limit: ssu_tree_workspace_bytes(dims, num_nodes) <= SSU_TREE_SCRATCH_BYTES
 * (e.g. batch 64 with one group and 128-node trees), else SSU_EINVAL before
 * any HIP call. The call allocates nothing: its first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress) once.
 * Every call on one GPU shares that GPU's array and leaves it holding its own
 * dots: calls that overlap on one GPU (other streams, or host threads whose
 * calls are not ordered) race on it and give undefined results; order them on
 * one stream. Calls through ssu_tree_verify never touch the array. */
ssu_status ssu_tree_verify_noalloc(const ssu_dims *dims, int32_t num_nodes, const void *x,
                                   const float *A, const void *B, const void *C, const float *dt,
                                   const float *dt_bias, const float *D, const void *z,
                                   const void *state, void *out, int32_t dt_softplus,
                                   const int32_t *state_indices, const int32_t *parent_ids,
                                   const int32_t *depths, float *replay_dA, float *replay_u,
                                   float *replay_B, float *replay_dt, hipStream_t stream);

/* Bytes of workspace ssu_tree_verify needs: 4 * batch * ngroups * num_nodes^2;
 * -1 if dims is NULL or num_nodes is outside [0, SSU_MAX_TREE_NODES] or
 * batch / ngroups is out of range. No HIP call. */
int64_t ssu_tree_workspace_bytes(const ssu_dims *dims, int32_t num_nodes);

/* One layer's buffers for ssu_replay_layers [SSU MambaReplayLayerInfo:
 * stateDst, replayDa, replayU, replayB, replayDt]. Layouts and alignment as
 * for ssu_replay; every layer shares the geometry in ssu_dims. */
typedef struct ssu_replay_layer {
    void *state;             /* [pool_rows, nheads, dim, dstate] state_dtype, in place */
    const float *replay_dA;  /* [dims->batch, seq_len, nheads] */
    const float *replay_u;   /* [dims->batch, seq_len, nheads, dim] */
    const float *replay_B;   /* [dims->batch, seq_len, ngroups, dstate] */
    const float *replay_dt;  /* [dims->batch, seq_len, nheads] */
} ssu_replay_layer;

/* ssu_replay_layers -- ssu_replay for num_layers layers in one launch
 * [SSU invokeMambaReplayReconstructBatched]. `layers` is a DEVICE array of
 * num_layers entries (the caller uploads it once and keeps it while calls that
 * use it are in flight); accepted_lengths, state_indices, accepted_node_ids
 * and active_batch are shared by every layer, exactly as in ssu_replay. The
 * pointers inside `layers` are not validated on the host: each must be
 * non-null and aligned as ssu_replay requires (undefined behaviour otherwise).
 * num_layers >= 0 (0: nothing to do). */
ssu_status ssu_replay_layers(const ssu_dims *dims, int32_t seq_len, const ssu_replay_layer *layers,
                             int32_t num_layers, const int32_t *accepted_lengths,
                             const int32_t *state_indices, int32_t active_batch,
                             const int32_t *accepted_node_ids, int32_t max_accept_len,
                             hipStream_t stream);

/* One layer's persistent states for ssu_state_clear_layers [SSU
 * MambaStateLayerInfo: recurrentState, convState]. Either may be NULL (that
 * buffer is skipped). */
typedef struct ssu_state_layer {
    void *recurrent_state; /* resident_rows rows of recurrent_row_bytes bytes */
    void *conv_state;      /* resident_rows rows of conv_row_bytes bytes */
} ssu_state_layer;

/* ssu_state_clear_layers -- zero resident row `slot` of both states of every
 * layer, or every row when slot == -1, in one launch [SSU
 * invokeMambaStateClear]. `layers` is a DEVICE array of num_layers entries.
 * Row bytes may be any non-negative count (0: that state is skipped); no
 * alignment is required. SSU_EINVAL unless num_layers >= 0, resident_rows >= 0,
 * -1 <= slot < resident_rows (slot -1 allowed with resident_rows == 0) and the
 * row byte counts are >= 0. */
ssu_status ssu_state_clear_layers(const ssu_state_layer *layers, int32_t num_layers,
                                  int32_t resident_rows, int32_t slot,
                                  int64_t recurrent_row_bytes, int64_t conv_row_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fused gated-delta-rule decode step [GDN]: one token per batch entry.
 * ---------------------------------------------------------------------- */
typedef struct ssu_gdn_dims {
    int32_t batch;
    int32_t hidden;           /* rows of w_ba */
    int32_t num_q_heads;      /* Hq: q and k heads */
    int32_t num_v_heads;      /* HV: value heads, HV/Hq in {1, 2, 4, 8} (else SSU_ENOTSUP) */
    int32_t head_dim;         /* D = K = V, in {32, 64, 128, 256} */
    int32_t conv_width;       /* W, 1..8 */
    int32_t pool_rows;        /* P: leading extent of both pools */
    int32_t use_qk_l2norm;
    int64_t ssm_row_stride;   /* elements between pool rows of ssm_state; 0 = HV*D*D */
    int64_t conv_slot_stride; /* conv_state element strides of its logical */
    int64_t conv_chan_stride; /* [P, qkv_dim, W-1] view: DS-dense pools are    */
    int64_t conv_tap_stride;  /* (qkv_dim*(W-1), W-1, 1), SD pools (.., 1, qkv_dim) */
} ssu_gdn_dims;

/* ssu_gdn_decode -- [GDN] with these readings of the steps the page names:
 *   ba = hidden_states[b] @ w_ba; beta = sigmoid(ba[:, h]);
 *   alpha = exp(-exp(A_log[h]) * softplus(ba[:, HV+h] + dt_bias[h]));
 *   conv: window = [conv_state[s, c, 0..W-2], mixed_qkv[b, c]] (oldest first),
 *         y_c = silu(sum_j window[j] conv_weight[c, j] + conv_bias[c]);
 *         conv_state[s, c, :] = window[1..];
 *   q | k | v = y channels [Hq D | Hq D | HV D]; value head h reads q/k head
 *   h / (HV/Hq); q, k /= sqrt(sum x^2 + 1e-6) when use_qk_l2norm; q *= scale
 *   (scale <= 0 or NaN selects 1/sqrt(D), as the page treats None and 0.0);
 *   S = ssm_state[s, h] ([D(v), D(k)], V-major, K-last): S *= alpha;
 *   S[v][:] += beta * (v[v] - S[v][:].k) k;  out[b, 0, h, v] = S[v][:].q.
 * s = state_indices[b]; a negative index is a padding entry: no pool access,
 * out[b] = +0.0. Indices >= P are undefined (the page: a caller bug).
 * Dtypes as the page: hidden_states [B, hidden], w_ba [hidden, 2 HV],
 * mixed_qkv [B, qkv_dim], conv_weight [qkv_dim, W], conv_bias [qkv_dim],
 * conv_state, dt_bias [HV] and out [B, 1, HV, D] bf16; A_log [HV] and
 * ssm_state [P, HV, D, D] fp32; qkv_dim = (2 Hq + HV) D. All device pointers;
 * ssm_state 16-byte aligned with a row stride that keeps rows 16-byte
 * aligned; w_ba 4-byte aligned; every other pointer aligned to its element
 * (SSU_EINVAL otherwise). Both pools are updated in place. HV <= 256.
 * workspace: caller-owned device scratch of at least ssu_gdn_workspace_bytes
 * (dims) bytes, 16-byte aligned (it carries the normalised q/k, v and the
 * b/a projection partial sums from the first of the two launches to the
 * second); its contents on
 * entry are ignored and on return unspecified. Calls that share a workspace
 * must be ordered (one stream). */
ssu_status ssu_gdn_decode(const ssu_gdn_dims *dims, const void *hidden_states, const void *w_ba,
                          const void *mixed_qkv, const void *conv_weight, const void *conv_bias,
                          void *conv_state, const float *A_log, const void *dt_bias, float scale,
                          float *ssm_state, const int32_t *state_indices, void *out,
                          void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace ssu_gdn_decode needs for these dims:
 * 4 * B * (2 Hq D + HV D + 2 HV ceil(hidden / 256)); -1 if dims is NULL or
 * has a non-positive hidden, head count or head_dim, or a negative batch.
 * No HIP call. */
int64_t ssu_gdn_workspace_bytes(const ssu_gdn_dims *dims);

/* ------------------------------------------------------------------------
 * Row movement between a resident pool and contiguous working rows. A row is
 * row_bytes bytes (the trailing dimensions of one pool row, any dtype); rows
 * of a buffer are `stride` bytes apart (0 = row_bytes, >= row_bytes
 * otherwise). Any alignment; 16-byte aligned rows and strides copy fastest.
 * Index arrays are device int32 arrays; values are not validated on the host.
 * ---------------------------------------------------------------------- */

/* ssu_state_gather -- active[b] = resident[state_indices[b]] for b < batch
 * [SSU invokeMambaStateGather]. A negative index is a padding entry [PAD]: its
 * active row is written as zeros. An index >= resident_rows is undefined. */
ssu_status ssu_state_gather(const void *resident, int32_t resident_rows, int64_t resident_stride,
                            void *active, int64_t active_stride, const int32_t *state_indices,
                            int32_t batch, int64_t row_bytes, hipStream_t stream);

/* ssu_state_scatter -- resident[state_indices[b]] = active[b] for b < batch with
 * a non-negative index [SSU invokeMambaStateScatter]; padding entries write
 * nothing. Duplicate live indices are undefined. */
ssu_status ssu_state_scatter(const void *active, int64_t active_stride, void *resident,
                             int32_t resident_rows, int64_t resident_stride,
                             const int32_t *state_indices, int32_t batch, int64_t row_bytes,
                             hipStream_t stream);

/* ssu_state_pack -- pack a cohort's home rows into the working slots [0, batch)
 * of the same pool [DNP activateStep]: afterwards slot b holds what row
 * homes[b] held before the call, for every b. Every source row is read before
 * any slot is written (a sequential home-to-slot copy would corrupt the cohort
 * when homes are not in ascending order), and the rows listed in
 * `bystanders` (live rows of other requests whose home lies in [0, batch);
 * each < batch, none a home of the cohort) are saved first so that
 * ssu_state_unpack can put them back. Slots whose home is the slot itself are
 * not copied. workspace: device buffer of (batch + n_bystanders) * row_bytes
 * bytes, kept by the caller until the matching ssu_state_unpack. homes must be
 * distinct and in [0, pool_rows); values are not validated. Two launches. */
ssu_status ssu_state_pack(void *pool, int32_t pool_rows, int64_t row_stride, int64_t row_bytes,
                          const int32_t *homes, int32_t batch, const int32_t *bystanders,
                          int32_t n_bystanders, void *workspace, hipStream_t stream);

/* ssu_state_unpack -- write the working slots [0, batch) back to the homes and
 * restore the bystander rows saved by ssu_state_pack [DNP scatterActive]; the
 * same arguments as the pack. Every slot is read before any home is written.
 * Two launches. */
ssu_status ssu_state_unpack(void *pool, int32_t pool_rows, int64_t row_stride, int64_t row_bytes,
                            const int32_t *homes, int32_t batch, const int32_t *bystanders,
                            int32_t n_bystanders, void *workspace, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Recurrent-state pool [RSM]: one zeroed, contiguous slab per state spec,
 * shaped [slot_count] + spec.shape, so slot s of state i starts at byte
 * s * stateBytesPerSlot(i) of slab i. Spec order is fixed: capture and
 * restore match buffers to states by position.
 * ---------------------------------------------------------------------- */
typedef struct ssu_pool ssu_pool; /* opaque; not copyable, freed once */

typedef struct ssu_state_spec {
    int32_t kind;     /* caller-defined state kind (e.g. 0 recurrent, 1 conv) */
    int32_t layer;    /* absolute layer index, >= 0 */
    int32_t rank;     /* entries of shape in use, 1..4 */
    int32_t dtype;    /* SSU_F32, SSU_F16, SSU_BF16 or SSU_U8 */
    int64_t shape[4]; /* per-slot shape; every used entry > 0 */
} ssu_state_spec;

/* Bytes one slot occupies across `specs` (static: no pool needed) [RSM bytesPerSlot].
 * Fails with SSU_EINVAL on an invalid spec list (see ssu_pool_alloc). */
ssu_status ssu_pool_bytes_per_slot(const ssu_state_spec *specs, int32_t n_specs, size_t *out);

/* Bytes of a caller slab that holds slot_count slots of every spec for
 * ssu_pool_alloc: the states' slabs in spec order, each starting at a
 * 256-byte boundary (sizing against a byte budget before any allocation, as
 * [RSM bytesPerSlot] does for one slot). No HIP call. */
ssu_status ssu_pool_slab_bytes(const ssu_state_spec *specs, int32_t n_specs, int32_t slot_count,
                               size_t *out);

/* Create a pool of slot_count zeroed slots of every spec on the current
 * device; the zeroing runs on `stream` [RSM constructor: specs, slotCount,
 * name, stream].
 *   name: NULL or a string copied into the pool, the prefix of its states in
 *         diagnostics ([RSM] "prefix for the slab tensor names");
 *   base: NULL -> the pool allocates one slab per spec (hipMalloc) and frees
 *         them in ssu_pool_free. Non-NULL -> a caller-owned device buffer of
 *         base_bytes >= ssu_pool_slab_bytes(specs, n_specs, slot_count)
 *         bytes, 256-byte aligned: the states are laid out in it as that call
 *         describes, the pool allocates nothing and ssu_pool_free leaves the
 *         buffer alone (the caller keeps it alive while the pool is used).
 * SSU_EINVAL if a spec has non-positive volume, a negative layer, a bad rank
 * or dtype, or repeats a {kind, layer} pair, or if the caller slab is
 * misaligned or too small (nothing is written then). slot_count == 0 or
 * n_specs == 0 gives a valid pool that uses no memory. The pool keeps its own
 * copy of the specs. Free with ssu_pool_free. */
ssu_status ssu_pool_alloc(const ssu_state_spec *specs, int32_t n_specs, int32_t slot_count,
                          const char *name, void *base, size_t base_bytes, hipStream_t stream,
                          ssu_pool **out);
/* Release the pool. Slabs the pool allocated are freed after synchronising
 * the device; a caller slab is left untouched (no HIP call). NULL is a no-op. */
ssu_status ssu_pool_free(ssu_pool *pool);
/* Geometry queries [RSM slotCount, numStates, state, stateBytesPerSlot, findState]. */
ssu_status ssu_pool_info(const ssu_pool *pool, int32_t *num_states, int32_t *slot_count);
ssu_status ssu_pool_state_ptr(const ssu_pool *pool, int32_t state_idx, void **dev_ptr);
ssu_status ssu_pool_state_bytes_per_slot(const ssu_pool *pool, int32_t state_idx, size_t *out);
/* The spec state state_idx was created from [RSM spec]. */
ssu_status ssu_pool_spec(const ssu_pool *pool, int32_t state_idx, ssu_state_spec *out);
/* Every spec in pool order [RSM specs]: the first min(capacity, numStates)
 * are written to out (NULL allowed when capacity is 0); *n_specs = numStates. */
ssu_status ssu_pool_specs(const ssu_pool *pool, ssu_state_spec *out, int32_t capacity,
                          int32_t *n_specs);
/* The pool's name ("" when created without one); the string is owned by the
 * pool and lives until ssu_pool_free. */
ssu_status ssu_pool_name(const ssu_pool *pool, const char **name);
/* *owns = 1 if the pool allocated its slabs, 0 if they lie in a caller slab. */
ssu_status ssu_pool_owns_memory(const ssu_pool *pool, int32_t *owns);
/* *state_idx = index of the state with this {kind, layer}, or -1 if none. */
ssu_status ssu_pool_find_state(const ssu_pool *pool, int32_t kind, int32_t layer,
                               int32_t *state_idx);
/* Zero every slot of every state, in one launch [RSM clear]. */
ssu_status ssu_pool_clear(ssu_pool *pool, hipStream_t stream);
/* Zero one slot of every state in one launch, leaving other slots untouched;
 * slot == -1 zeroes every slot [RSM clearSlot; SSU invokeMambaStateClear].
 * SSU_EINVAL unless -1 <= slot < slot_count. */
ssu_status ssu_pool_clear_slot(ssu_pool *pool, int32_t slot, hipStream_t stream);
/* Copy slot `slot` of state i into dst[i] (a caller-owned device buffer of
 * exactly dst_bytes[i] == stateBytesPerSlot(i) bytes), for every state, in one
 * launch [RSM capture]. n must equal the number of states. */
ssu_status ssu_pool_capture(const ssu_pool *pool, int32_t slot, void *const *dst,
                            const size_t *dst_bytes, int32_t n, hipStream_t stream);
/* Write a checkpoint back into one slot [RSM restore]: states 0..n_saved-1
 * from src[i] (src_bytes[i] must equal stateBytesPerSlot(i)); states beyond
 * n_saved are zeroed. Every entry is validated before anything is written. */
ssu_status ssu_pool_restore(ssu_pool *pool, int32_t slot, const void *const *src,
                            const size_t *src_bytes, int32_t n_saved, hipStream_t stream);
/* Copy slot src_slot of every state of `source` into slot dst_slot of `pool`;
 * both pools must hold identical specs in the same order [RSM copySlotFrom]. */
ssu_status ssu_pool_copy_slot_from(ssu_pool *pool, const ssu_pool *source, int32_t dst_slot,
                                   int32_t src_slot, hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *ssu_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int32_t ssu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSU_H */
