/*
 * ssu_oracle.c -- plain fp64 CPU oracle for the selective state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (all arithmetic in fp64, one element at a time, in the
 * order the definitions are written; built with -ffp-contract=off):
 *
 *  decode  -- TensorRT-Edge-LLM "Selective State Update" page,
 *             mamba_ssm::invokeSelectiveStateUpdate ("Computes" paragraph and
 *             the shape list under it):
 *               dt'       = dt + dt_bias, then softplus(dt') when dt_softplus
 *               new_state = state * exp(A * dt') + B * dt' * x
 *               out       = sum_n new_state[n] * C[n] + D * x
 *               out      *= silu(z)            (only when z is given)
 *             x [batch,nheads,dim], A [nheads], B/C [batch,ngroups,dstate],
 *             dt [batch,nheads], dt_bias/D [nheads], state [rows,nheads,dim,dstate].
 *  padding -- FlashInfer flashinfer.gdn_fused_decode_step page, parameter
 *             state_indices ("Padding / inactive rows"): a negative row index
 *             means the entry owns no pool row; its state is neither read nor
 *             written and its output row is written as zero.
 *  prefill -- same page, invokeSelectiveStateUpdatePrefill: all seq_len tokens
 *             of x [batch,seq_len,nheads,dim] in order, with contextLengths;
 *             with the replay stash given the committed state is left
 *             read-only and dA, x, B and dt' are stashed per token.
 *  replay  -- same page, struct MambaReplayLayerInfo: re-run the recurrence
 *             over the first acceptedLengths[b] stashed tokens, in place, for
 *             b < activeBatchSize; accepted == 0 leaves the row untouched.
 *             With acceptedNodeIds (invokeMambaReplayReconstructBatched) token
 *             t of row b is the stash entry of node acceptedNodeIds[b, t].
 *  tree    -- same page, invokeSelectiveStateUpdateDDTree: for every node of
 *             a draft tree, walk treeParentIds from the node to the root,
 *             replay the decode step along that path (root first) from the
 *             committed state, which stays read-only, and emit the node's
 *             output; stash the node's own dA, x, B and dt'.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): the bias is added before softplus; head h reads group
 * h / (nheads/ngroups); the stash holds dA = A*dt' (a log-decay) and replay
 * applies exp(dA); tokens t >= clamp(contextLengths[b], 0, seq_len) produce
 * zero outputs and zero stash entries and do not touch the state; replay runs
 * min(acceptedLengths[b], seq_len) tokens and skips negative row indices.
 * Tree readings: a node's parent id is that of an earlier node (smaller id) or
 * negative for a node whose predecessor is the committed state; treeDepths[n]
 * bounds the number of parent hops of the walk (NULL: no bound); a parent id
 * that is not smaller than the current node ends the walk there.  Replay with
 * node ids runs min(acceptedLengths[b], maxAcceptLen) tokens and stops at the
 * first id outside [0, seq_len).
 *
 * Parity pins: tests/test_oracle_pins.py checks this file against hand-derived
 * closed forms, invariants, the unrolled-sum form of the recurrence and an
 * independent pure-Python implementation (oracle/ref_tiny.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Node budget of one draft tree (the page's shared speculative verify budget). */
#define ORACLE_MAX_NODES 128

static double softplus(double v)
{
    /* log(1 + e^v), written so that neither branch overflows */
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

static double silu(double v)
{
    return v / (1.0 + exp(-v));
}

/* One token of one (batch row, head): updates st[dim*dstate] in place and
 * writes y[dim].  bvec/cvec point at the head's group row of B and C. */
static void head_step(int dim, int dstate, double *st, const double *xrow,
                      const double *bvec, const double *cvec, double dtp,
                      double decay, double dskip, int has_d, const double *zrow,
                      double *y)
{
    for (int d = 0; d < dim; ++d) {
        double *srow = st + (int64_t)d * dstate;
        double acc = 0.0;
        for (int n = 0; n < dstate; ++n) {
            srow[n] = srow[n] * decay + bvec[n] * dtp * xrow[d];
            acc += srow[n] * cvec[n];
        }
        double out = acc;
        if (has_d)
            out += dskip * xrow[d];
        if (zrow)
            out *= silu(zrow[d]);
        y[d] = out;
    }
}

static double processed_dt(double dt, const double *dt_bias, int h, int dt_softplus)
{
    double v = dt + (dt_bias ? dt_bias[h] : 0.0);
    return dt_softplus ? softplus(v) : v;
}

void oracle_ssu_decode(int32_t batch, int32_t nheads, int32_t dim, int32_t dstate,
                       int32_t ngroups, int64_t row_stride, const double *x,
                       const double *A, const double *B, const double *C,
                       const double *dt, const double *dt_bias, const double *D,
                       const double *z, double *state, double *out,
                       int32_t dt_softplus, const int32_t *state_indices)
{
    const int hpg = nheads / ngroups;
    const int64_t tile = (int64_t)dim * dstate;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < nheads; ++h) {
            const int64_t s = state_indices ? state_indices[b] : b;
            double *y = out + ((int64_t)b * nheads + h) * dim;
            if (s < 0) {
                for (int d = 0; d < dim; ++d)
                    y[d] = 0.0;
                continue;
            }
            const int g = h / hpg;
            const double dtp = processed_dt(dt[(int64_t)b * nheads + h], dt_bias, h, dt_softplus);
            const double decay = exp(A[h] * dtp);
            const int64_t xoff = ((int64_t)b * nheads + h) * dim;
            head_step(dim, dstate, state + s * row_stride + h * tile, x + xoff,
                      B + ((int64_t)b * ngroups + g) * dstate,
                      C + ((int64_t)b * ngroups + g) * dstate, dtp, decay,
                      D ? D[h] : 0.0, D != 0, z ? z + xoff : 0, y);
        }
    }
}

void oracle_ssu_prefill(int32_t batch, int32_t seq_len, int32_t nheads, int32_t dim,
                        int32_t dstate, int32_t ngroups, int64_t row_stride,
                        const double *x, const double *A, const double *B,
                        const double *C, const double *dt, const double *dt_bias,
                        const double *D, const double *z, double *state, double *out,
                        int32_t dt_softplus, const int32_t *context_lengths,
                        const int32_t *state_indices, double *st_dA, double *st_u,
                        double *st_B, double *st_dt, double *scratch)
{
    /* scratch: batch*nheads*dim*dstate doubles, used only in stash mode so the
     * committed state is never written. */
    const int hpg = nheads / ngroups;
    const int64_t tile = (int64_t)dim * dstate;
    const int stash = st_dA != 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < nheads; ++h) {
            const int64_t s = state_indices ? state_indices[b] : b;
            int L = seq_len;
            if (context_lengths) {
                L = context_lengths[b];
                if (L < 0) L = 0;
                if (L > seq_len) L = seq_len;
            }
            const int g = h / hpg;
            if (s < 0) {
                for (int t = 0; t < seq_len; ++t)
                    for (int d = 0; d < dim; ++d)
                        out[(((int64_t)b * seq_len + t) * nheads + h) * dim + d] = 0.0;
                continue;
            }
            double *st = state + s * row_stride + h * tile;
            if (stash) {
                double *priv = scratch + ((int64_t)b * nheads + h) * tile;
                memcpy(priv, st, sizeof(double) * tile);
                st = priv;
            }
            for (int t = 0; t < seq_len; ++t) {
                const int64_t bth = ((int64_t)b * seq_len + t) * nheads + h;
                const int64_t btg = ((int64_t)b * seq_len + t) * ngroups + g;
                double *y = out + bth * dim;
                if (t >= L) {
                    for (int d = 0; d < dim; ++d)
                        y[d] = 0.0;
                    if (stash) {
                        st_dA[bth] = 0.0;
                        st_dt[bth] = 0.0;
                        for (int d = 0; d < dim; ++d)
                            st_u[bth * dim + d] = 0.0;
                        if (h % hpg == 0)
                            for (int n = 0; n < dstate; ++n)
                                st_B[btg * dstate + n] = 0.0;
                    }
                    continue;
                }
                const double dtp = processed_dt(dt[bth], dt_bias, h, dt_softplus);
                const double decay = exp(A[h] * dtp);
                head_step(dim, dstate, st, x + bth * dim, B + btg * dstate,
                          C + btg * dstate, dtp, decay, D ? D[h] : 0.0, D != 0,
                          z ? z + bth * dim : 0, y);
                if (stash) {
                    st_dA[bth] = A[h] * dtp;
                    st_dt[bth] = dtp;
                    for (int d = 0; d < dim; ++d)
                        st_u[bth * dim + d] = x[bth * dim + d];
                    if (h % hpg == 0)
                        for (int n = 0; n < dstate; ++n)
                            st_B[btg * dstate + n] = B[btg * dstate + n];
                }
            }
        }
    }
}

void oracle_ssu_replay(int32_t active_batch, int32_t seq_len, int32_t nheads,
                       int32_t dim, int32_t dstate, int32_t ngroups,
                       int64_t row_stride, double *state, const double *st_dA,
                       const double *st_u, const double *st_B, const double *st_dt,
                       const int32_t *accepted_lengths, const int32_t *state_indices,
                       const int32_t *node_ids, int32_t max_accept_len)
{
    const int hpg = nheads / ngroups;
    const int64_t tile = (int64_t)dim * dstate;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int b = 0; b < active_batch; ++b) {
        for (int h = 0; h < nheads; ++h) {
            const int64_t s = state_indices ? state_indices[b] : b;
            const int limit = node_ids ? max_accept_len : seq_len;
            int k = accepted_lengths[b];
            if (k > limit) k = limit;
            if (s < 0 || k <= 0)
                continue;
            const int g = h / hpg;
            double *st = state + s * row_stride + h * tile;
            for (int t = 0; t < k; ++t) {
                /* stash position of the t-th accepted token */
                int pos = t;
                if (node_ids) {
                    pos = node_ids[(int64_t)b * max_accept_len + t];
                    if (pos < 0 || pos >= seq_len)
                        break;
                }
                const int64_t bth = ((int64_t)b * seq_len + pos) * nheads + h;
                const int64_t btg = ((int64_t)b * seq_len + pos) * ngroups + g;
                const double decay = exp(st_dA[bth]);
                for (int d = 0; d < dim; ++d)
                    for (int n = 0; n < dstate; ++n)
                        st[(int64_t)d * dstate + n] =
                            st[(int64_t)d * dstate + n] * decay +
                            st_B[btg * dstate + n] * st_dt[bth] * st_u[bth * dim + d];
            }
        }
    }
}

/* Root-to-node path of node n of one tree: path[0] is the node reached last by
 * the walk up treeParentIds, path[len-1] = n.  The walk takes at most
 * depths[n] hops (any number when depths is NULL) and stops at a parent id that
 * is negative or not smaller than the current node.  Returns len (<= n + 1). */
static int tree_path(const int32_t *parents, const int32_t *depths, int n, int *path)
{
    int up[ORACLE_MAX_NODES];
    int len = 0;
    int j = n;
    const int cap = depths ? depths[n] : n;
    up[len++] = j;
    while (len - 1 < cap) {
        const int p = parents[j];
        if (p < 0 || p >= j)
            break;
        j = p;
        up[len++] = j;
    }
    for (int i = 0; i < len; ++i)
        path[i] = up[len - 1 - i];
    return len;
}

void oracle_ssu_tree(int32_t batch, int32_t num_nodes, int32_t nheads, int32_t dim,
                     int32_t dstate, int32_t ngroups, int64_t row_stride,
                     const double *x, const double *A, const double *B, const double *C,
                     const double *dt, const double *dt_bias, const double *D,
                     const double *z, const double *state, double *out,
                     int32_t dt_softplus, const int32_t *state_indices,
                     const int32_t *parent_ids, const int32_t *depths, double *st_dA,
                     double *st_u, double *st_B, double *st_dt, double *scratch)
{
    /* scratch: batch*nheads*(dim*dstate + dim) doubles: a private copy of the
     * head's committed state per walk, and the outputs of the path's inner
     * nodes (discarded). num_nodes <= ORACLE_MAX_NODES. */
    const int hpg = nheads / ngroups;
    const int64_t tile = (int64_t)dim * dstate;
    const int stash = st_dA != 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < nheads; ++h) {
            const int64_t s = state_indices ? state_indices[b] : b;
            const int g = h / hpg;
            const int32_t *par = parent_ids + (int64_t)b * num_nodes;
            const int32_t *dep = depths ? depths + (int64_t)b * num_nodes : 0;
            if (s < 0) {
                for (int n = 0; n < num_nodes; ++n)
                    for (int d = 0; d < dim; ++d)
                        out[(((int64_t)b * num_nodes + n) * nheads + h) * dim + d] = 0.0;
                continue;
            }
            double *priv = scratch + ((int64_t)b * nheads + h) * (tile + dim);
            double *inner = priv + tile;
            const double *st0 = state + s * row_stride + h * tile;
            int path[ORACLE_MAX_NODES];
            for (int n = 0; n < num_nodes; ++n) {
                const int len = tree_path(par, dep, n, path);
                memcpy(priv, st0, sizeof(double) * tile);
                for (int i = 0; i < len; ++i) {
                    const int j = path[i];
                    const int64_t bjh = ((int64_t)b * num_nodes + j) * nheads + h;
                    const int64_t bjg = ((int64_t)b * num_nodes + j) * ngroups + g;
                    const double dtp = processed_dt(dt[bjh], dt_bias, h, dt_softplus);
                    head_step(dim, dstate, priv, x + bjh * dim, B + bjg * dstate,
                              C + bjg * dstate, dtp, exp(A[h] * dtp), D ? D[h] : 0.0, D != 0,
                              z ? z + bjh * dim : 0, i == len - 1 ? out + bjh * dim : inner);
                }
                if (stash) {
                    const int64_t bnh = ((int64_t)b * num_nodes + n) * nheads + h;
                    const int64_t bng = ((int64_t)b * num_nodes + n) * ngroups + g;
                    const double dtp = processed_dt(dt[bnh], dt_bias, h, dt_softplus);
                    st_dA[bnh] = A[h] * dtp;
                    st_dt[bnh] = dtp;
                    for (int d = 0; d < dim; ++d)
                        st_u[bnh * dim + d] = x[bnh * dim + d];
                    if (h % hpg == 0)
                        for (int k = 0; k < dstate; ++k)
                            st_B[bng * dstate + k] = B[bng * dstate + k];
                }
            }
        }
    }
}

/* Threads the OpenMP loops above use (reported beside the oracle's timing). */
int32_t oracle_num_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of the OpenMP loops above (for a single-thread timing
 * beside the parallel one); 0 or less keeps the current count. */
void oracle_set_num_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads((int)n);
#else
    (void)n;
#endif
}
