// C ABI of libssu: host-side argument checks, dispatch to the kernel
// launchers, and the recurrent-state pool. No entry point reads device memory
// on the host, synchronises, or allocates, except ssu_pool_alloc/ssu_pool_free.
#include <atomic>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "ssu.h"
#include "ssu_internal.h"

namespace {

thread_local std::string g_last_error;

ssu_status fail(ssu_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

ssu_status ok()
{
    g_last_error.clear();
    return SSU_OK;
}

ssu_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return ok();
    return fail(SSU_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t dtype_bytes(int32_t dt)
{
    switch (dt) {
    case SSU_F32: return 4;
    case SSU_F16: return 2;
    case SSU_BF16: return 2;
    case SSU_U8: return 1;
    default: return 0;
    }
}

bool compute_dtype(int32_t dt) { return dt == SSU_F32 || dt == SSU_F16 || dt == SSU_BF16; }

bool supported_dstate(int32_t n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }

// Shared geometry checks; fills the common part of the launch parameters.
ssu_status check_dims(const ssu_dims *d, const char *fn, bool need_pool_rows_for_batch,
                      bool have_indices, ssu::DecodeParams *out)
{
    if (!d)
        return fail(SSU_EINVAL, "%s: dims is NULL", fn);
    if (d->reserved != 0)
        return fail(SSU_EINVAL, "%s: dims.reserved must be 0", fn);
    if (d->batch < 0)
        return fail(SSU_EINVAL, "%s: batch %d < 0", fn, d->batch);
    if (d->nheads <= 0 || d->dim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
        return fail(SSU_EINVAL, "%s: nheads/dim/dstate/ngroups must be > 0 (got %d/%d/%d/%d)", fn,
                    d->nheads, d->dim, d->dstate, d->ngroups);
    if (d->nheads % d->ngroups != 0)
        return fail(SSU_EINVAL, "%s: nheads %d is not a multiple of ngroups %d", fn, d->nheads,
                    d->ngroups);
    if (d->pool_rows <= 0)
        return fail(SSU_EINVAL, "%s: pool_rows must be > 0 (got %d)", fn, d->pool_rows);
    if (d->dim > 4096)
        return fail(SSU_ENOTSUP, "%s: dim %d > 4096", fn, d->dim);
    if (!supported_dstate(d->dstate))
        return fail(SSU_ENOTSUP, "%s: dstate %d not in {16,32,64,128,256}", fn, d->dstate);
    if (!compute_dtype(d->state_dtype) || !compute_dtype(d->io_dtype) || !compute_dtype(d->bc_dtype))
        return fail(SSU_ENOTSUP, "%s: unsupported dtype (state %d, io %d, bc %d)", fn,
                    d->state_dtype, d->io_dtype, d->bc_dtype);
    const int64_t tile = (int64_t)d->nheads * d->dim * d->dstate;
    int64_t stride = d->state_row_stride;
    if (stride < 0)
        return fail(SSU_EINVAL, "%s: state_row_stride %lld < 0", fn, (long long)stride);
    if (stride == 0)
        stride = tile;
    if (stride < tile)
        return fail(SSU_EINVAL, "%s: state_row_stride %lld < nheads*dim*dstate %lld", fn,
                    (long long)stride, (long long)tile);
    if ((stride * (int64_t)dtype_bytes(d->state_dtype)) % 16 != 0)
        return fail(SSU_EINVAL, "%s: state row stride of %lld bytes is not a multiple of 16", fn,
                    (long long)(stride * (int64_t)dtype_bytes(d->state_dtype)));
    if (need_pool_rows_for_batch && !have_indices && d->batch > d->pool_rows)
        return fail(SSU_EINVAL, "%s: batch %d > pool_rows %d with no state_indices", fn, d->batch,
                    d->pool_rows);
    out->row_stride = stride;
    out->batch = d->batch;
    out->nheads = d->nheads;
    out->dim = d->dim;
    out->dstate = d->dstate;
    out->ngroups = d->ngroups;
    out->state_dtype = d->state_dtype;
    out->io_dtype = d->io_dtype;
    out->bc_dtype = d->bc_dtype;
    return SSU_OK;
}

size_t io_bytes(int32_t dt) { return dt == SSU_F32 ? 4 : 2; }

// Compute units of the current device, cached per device (a host-side attribute
// query; no device work, no synchronisation). 0 if the query fails.
int32_t current_cu_count()
{
    static std::atomic<int32_t> cache[64];  // zero-initialised; benign races between host threads
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < 64) {
        const int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < 64)
        cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Tensors read with 16-byte vector loads (state, B, C, replay_B) must be 16-byte
// aligned; every other tensor only needs the alignment of its element type.
#define SSU_REQUIRE_PTR(p, align, fn)                                                   \
    do {                                                                                \
        if (!(p))                                                                       \
            return fail(SSU_EINVAL, "%s: required pointer '%s' is NULL", fn, #p);       \
        if (((uintptr_t)(p) % (align)) != 0)                                            \
            return fail(SSU_EINVAL, "%s: pointer '%s' is not %d-byte aligned", fn, #p,  \
                        (int)(align));                                                  \
    } while (0)

#define SSU_OPTIONAL_PTR(p, align, fn)                                                  \
    do {                                                                                \
        if ((p) && ((uintptr_t)(p) % (align)) != 0)                                     \
            return fail(SSU_EINVAL, "%s: pointer '%s' is not %d-byte aligned", fn, #p,  \
                        (int)(align));                                                  \
    } while (0)

}  // namespace

extern "C" {

const char *ssu_last_error(void) { return g_last_error.c_str(); }

int32_t ssu_version(void) { return 10200; }

ssu_status ssu_decode(const ssu_dims *dims, const void *x, const float *A, const void *B,
                      const void *C, const float *dt, const float *dt_bias, const float *D,
                      const void *z, void *state, void *out, int32_t dt_softplus,
                      const int32_t *state_indices, hipStream_t stream)
{
    const char *fn = "ssu_decode";
    ssu::DecodeParams p = {};
    const ssu_status st = check_dims(dims, fn, true, state_indices != nullptr, &p);
    if (st != SSU_OK)
        return st;
    if (p.batch == 0)
        return ok();
    SSU_REQUIRE_PTR(x, io_bytes(dims->io_dtype), fn);
    SSU_REQUIRE_PTR(A, 4, fn);
    SSU_REQUIRE_PTR(B, 16, fn);
    SSU_REQUIRE_PTR(C, 16, fn);
    SSU_REQUIRE_PTR(dt, 4, fn);
    SSU_REQUIRE_PTR(state, 16, fn);
    SSU_REQUIRE_PTR(out, io_bytes(dims->io_dtype), fn);
    SSU_OPTIONAL_PTR(dt_bias, 4, fn);
    SSU_OPTIONAL_PTR(D, 4, fn);
    SSU_OPTIONAL_PTR(z, io_bytes(dims->io_dtype), fn);
    SSU_OPTIONAL_PTR(state_indices, 4, fn);
    p.x = x;
    p.A = A;
    p.B = B;
    p.C = C;
    p.dt = dt;
    p.dt_bias = dt_bias;
    p.D = D;
    p.z = z;
    p.state = state;
    p.out = out;
    p.idx = state_indices;
    p.dt_softplus = dt_softplus ? 1 : 0;
    return hip_status(ssu::launch_decode(p, stream), "ssu_decode launch");
}

ssu_status ssu_prefill(const ssu_dims *dims, int32_t seq_len, const void *x, const float *A,
                       const void *B, const void *C, const float *dt, const float *dt_bias,
                       const float *D, const void *z, void *state, void *out,
                       int32_t dt_softplus, const int32_t *context_lengths,
                       const int32_t *state_indices, float *replay_dA, float *replay_u,
                       float *replay_B, float *replay_dt, hipStream_t stream)
{
    const char *fn = "ssu_prefill";
    ssu::PrefillParams p = {};
    const ssu_status st = check_dims(dims, fn, true, state_indices != nullptr, &p.d);
    if (st != SSU_OK)
        return st;
    if (seq_len < 0)
        return fail(SSU_EINVAL, "%s: seq_len %d < 0", fn, seq_len);
    const int nstash = (replay_dA != nullptr) + (replay_u != nullptr) + (replay_B != nullptr) +
                       (replay_dt != nullptr);
    if (nstash != 0 && nstash != 4)
        return fail(SSU_EINVAL, "%s: replay stash must be all four buffers or none (%d given)",
                    fn, nstash);
    if (p.d.batch == 0 || seq_len == 0)
        return ok();
    if ((int64_t)p.d.batch * seq_len * p.d.nheads * p.d.dim > ((int64_t)1 << 40))
        return fail(SSU_ENOTSUP, "%s: problem too large", fn);
    SSU_REQUIRE_PTR(x, io_bytes(dims->io_dtype), fn);
    SSU_REQUIRE_PTR(A, 4, fn);
    SSU_REQUIRE_PTR(B, 16, fn);
    SSU_REQUIRE_PTR(C, 16, fn);
    SSU_REQUIRE_PTR(dt, 4, fn);
    SSU_REQUIRE_PTR(state, 16, fn);
    SSU_REQUIRE_PTR(out, io_bytes(dims->io_dtype), fn);
    SSU_OPTIONAL_PTR(dt_bias, 4, fn);
    SSU_OPTIONAL_PTR(D, 4, fn);
    SSU_OPTIONAL_PTR(z, io_bytes(dims->io_dtype), fn);
    SSU_OPTIONAL_PTR(context_lengths, 4, fn);
    SSU_OPTIONAL_PTR(state_indices, 4, fn);
    SSU_OPTIONAL_PTR(replay_dA, 4, fn);
    SSU_OPTIONAL_PTR(replay_u, 4, fn);
    SSU_OPTIONAL_PTR(replay_B, 16, fn);
    SSU_OPTIONAL_PTR(replay_dt, 4, fn);
    p.d.x = x;
    p.d.A = A;
    p.d.B = B;
    p.d.C = C;
    p.d.dt = dt;
    p.d.dt_bias = dt_bias;
    p.d.D = D;
    p.d.z = z;
    p.d.state = state;
    p.d.out = out;
    p.d.idx = state_indices;
    p.d.dt_softplus = dt_softplus ? 1 : 0;
    p.seq_len = seq_len;
    p.ctx = context_lengths;
    p.st_dA = replay_dA;
    p.st_u = replay_u;
    p.st_B = replay_B;
    p.st_dt = replay_dt;
    p.cu_count = current_cu_count();
    p.waves_per_wg = 0;
    return hip_status(ssu::launch_prefill(p, stream), "ssu_prefill launch");
}

ssu_status ssu_replay(const ssu_dims *dims, int32_t seq_len, void *state,
                      const float *replay_dA, const float *replay_u, const float *replay_B,
                      const float *replay_dt, const int32_t *accepted_lengths,
                      const int32_t *state_indices, int32_t active_batch,
                      const int32_t *accepted_node_ids, int32_t max_accept_len,
                      hipStream_t stream)
{
    const char *fn = "ssu_replay";
    ssu::DecodeParams d = {};
    const ssu_status st = check_dims(dims, fn, false, state_indices != nullptr, &d);
    if (st != SSU_OK)
        return st;
    if (seq_len < 0)
        return fail(SSU_EINVAL, "%s: seq_len %d < 0", fn, seq_len);
    if (active_batch < 0 || active_batch > d.batch)
        return fail(SSU_EINVAL, "%s: active_batch %d outside [0, batch %d]", fn, active_batch,
                    d.batch);
    if (!state_indices && active_batch > dims->pool_rows)
        return fail(SSU_EINVAL, "%s: active_batch %d > pool_rows %d with no state_indices", fn,
                    active_batch, dims->pool_rows);
    if (accepted_node_ids && max_accept_len < 1)
        return fail(SSU_EINVAL, "%s: max_accept_len %d < 1 with accepted_node_ids", fn,
                    max_accept_len);
    if (active_batch == 0 || seq_len == 0)
        return ok();
    SSU_REQUIRE_PTR(state, 16, fn);
    SSU_REQUIRE_PTR(replay_dA, 4, fn);
    SSU_REQUIRE_PTR(replay_u, 4, fn);
    SSU_REQUIRE_PTR(replay_B, 16, fn);
    SSU_REQUIRE_PTR(replay_dt, 4, fn);
    SSU_REQUIRE_PTR(accepted_lengths, 4, fn);
    SSU_OPTIONAL_PTR(state_indices, 4, fn);
    SSU_OPTIONAL_PTR(accepted_node_ids, 4, fn);
    ssu::ReplayParams p = {};
    p.state = state;
    p.dA = replay_dA;
    p.u = replay_u;
    p.B = replay_B;
    p.dt = replay_dt;
    p.accepted = accepted_lengths;
    p.idx = state_indices;
    p.row_stride = d.row_stride;
    p.active_batch = active_batch;
    p.seq_len = seq_len;
    p.nheads = d.nheads;
    p.dim = d.dim;
    p.dstate = d.dstate;
    p.ngroups = d.ngroups;
    p.state_dtype = d.state_dtype;
    p.node_ids = accepted_node_ids;
    p.max_accept_len = accepted_node_ids ? max_accept_len : 0;
    return hip_status(ssu::launch_replay(p, stream), "ssu_replay launch");
}

ssu_status ssu_replay_layers(const ssu_dims *dims, int32_t seq_len, const ssu_replay_layer *layers,
                             int32_t num_layers, const int32_t *accepted_lengths,
                             const int32_t *state_indices, int32_t active_batch,
                             const int32_t *accepted_node_ids, int32_t max_accept_len,
                             hipStream_t stream)
{
    const char *fn = "ssu_replay_layers";
    ssu::DecodeParams d = {};
    const ssu_status st = check_dims(dims, fn, false, state_indices != nullptr, &d);
    if (st != SSU_OK)
        return st;
    if (seq_len < 0)
        return fail(SSU_EINVAL, "%s: seq_len %d < 0", fn, seq_len);
    if (num_layers < 0 || num_layers > 65535)
        return fail(SSU_EINVAL, "%s: num_layers %d outside [0, 65535]", fn, num_layers);
    if (active_batch < 0 || active_batch > d.batch)
        return fail(SSU_EINVAL, "%s: active_batch %d outside [0, batch %d]", fn, active_batch,
                    d.batch);
    if (!state_indices && active_batch > dims->pool_rows)
        return fail(SSU_EINVAL, "%s: active_batch %d > pool_rows %d with no state_indices", fn,
                    active_batch, dims->pool_rows);
    if (accepted_node_ids && max_accept_len < 1)
        return fail(SSU_EINVAL, "%s: max_accept_len %d < 1 with accepted_node_ids", fn,
                    max_accept_len);
    if (num_layers == 0 || active_batch == 0 || seq_len == 0)
        return ok();
    SSU_REQUIRE_PTR(layers, alignof(ssu_replay_layer), fn);
    SSU_REQUIRE_PTR(accepted_lengths, 4, fn);
    SSU_OPTIONAL_PTR(state_indices, 4, fn);
    SSU_OPTIONAL_PTR(accepted_node_ids, 4, fn);
    ssu::ReplayParams p = {};
    p.layers = layers;
    p.num_layers = num_layers;
    p.accepted = accepted_lengths;
    p.idx = state_indices;
    p.row_stride = d.row_stride;
    p.active_batch = active_batch;
    p.seq_len = seq_len;
    p.nheads = d.nheads;
    p.dim = d.dim;
    p.dstate = d.dstate;
    p.ngroups = d.ngroups;
    p.state_dtype = d.state_dtype;
    p.node_ids = accepted_node_ids;
    p.max_accept_len = accepted_node_ids ? max_accept_len : 0;
    return hip_status(ssu::launch_replay(p, stream), "ssu_replay_layers launch");
}

ssu_status ssu_state_clear_layers(const ssu_state_layer *layers, int32_t num_layers,
                                  int32_t resident_rows, int32_t slot,
                                  int64_t recurrent_row_bytes, int64_t conv_row_bytes,
                                  hipStream_t stream)
{
    const char *fn = "ssu_state_clear_layers";
    if (num_layers < 0 || num_layers > 65535)
        return fail(SSU_EINVAL, "%s: num_layers %d outside [0, 65535]", fn, num_layers);
    if (resident_rows < 0)
        return fail(SSU_EINVAL, "%s: resident_rows %d < 0", fn, resident_rows);
    if (slot < -1 || (slot >= 0 && slot >= resident_rows))
        return fail(SSU_EINVAL, "%s: slot %d outside [-1, %d)", fn, slot, resident_rows);
    if (recurrent_row_bytes < 0 || conv_row_bytes < 0)
        return fail(SSU_EINVAL, "%s: row byte counts must be >= 0 (got %lld, %lld)", fn,
                    (long long)recurrent_row_bytes, (long long)conv_row_bytes);
    if (num_layers == 0 || resident_rows == 0)
        return ok();
    SSU_REQUIRE_PTR(layers, alignof(ssu_state_layer), fn);
    return hip_status(ssu::launch_clear_layers(layers, num_layers, resident_rows, slot,
                                               recurrent_row_bytes, conv_row_bytes, stream),
                      "ssu_state_clear_layers launch");
}

int64_t ssu_gdn_workspace_bytes(const ssu_gdn_dims *dims)
{
    if (!dims || dims->batch < 0 || dims->hidden <= 0 || dims->num_q_heads <= 0 ||
        dims->num_v_heads <= 0 || dims->head_dim <= 0)
        return -1;
    return 4 * ssu::gdn_workspace_floats(dims->batch, dims->hidden, dims->num_q_heads,
                                         dims->num_v_heads, dims->head_dim);
}

ssu_status ssu_gdn_decode(const ssu_gdn_dims *dims, const void *hidden_states, const void *w_ba,
                          const void *mixed_qkv, const void *conv_weight, const void *conv_bias,
                          void *conv_state, const float *A_log, const void *dt_bias, float scale,
                          float *ssm_state, const int32_t *state_indices, void *out,
                          void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    const char *fn = "ssu_gdn_decode";
    if (!dims)
        return fail(SSU_EINVAL, "%s: dims is NULL", fn);
    const ssu_gdn_dims &d = *dims;
    if (d.batch < 0 || d.hidden <= 0 || d.num_q_heads <= 0 || d.num_v_heads <= 0 ||
        d.pool_rows <= 0)
        return fail(SSU_EINVAL, "%s: batch >= 0, hidden/heads/pool_rows > 0 required", fn);
    if (d.num_v_heads % d.num_q_heads != 0)
        return fail(SSU_EINVAL, "%s: num_v_heads %d is not a multiple of num_q_heads %d", fn,
                    d.num_v_heads, d.num_q_heads);
    const int G = d.num_v_heads / d.num_q_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(SSU_ENOTSUP, "%s: num_v_heads / num_q_heads = %d not in {1, 2, 4, 8}", fn, G);
    if (d.num_v_heads > 256)
        return fail(SSU_ENOTSUP, "%s: num_v_heads %d > 256", fn, d.num_v_heads);
    if (d.head_dim != 32 && d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
        return fail(SSU_ENOTSUP, "%s: head_dim %d not in {32, 64, 128, 256}", fn, d.head_dim);
    if (d.conv_width < 1 || d.conv_width > 8)
        return fail(SSU_ENOTSUP, "%s: conv_width %d outside [1, 8]", fn, d.conv_width);
    const int64_t tile = (int64_t)d.num_v_heads * d.head_dim * d.head_dim;
    int64_t rs = d.ssm_row_stride ? d.ssm_row_stride : tile;
    if (rs < tile || (rs * 4) % 16 != 0)
        return fail(SSU_EINVAL, "%s: ssm_row_stride %lld must be >= HV*D*D and keep rows 16-byte aligned",
                    fn, (long long)d.ssm_row_stride);
    if (d.conv_slot_stride < 0 || d.conv_chan_stride < 0 || d.conv_tap_stride < 0)
        return fail(SSU_EINVAL, "%s: negative conv_state stride", fn);
    if (d.batch == 0)
        return ok();
    SSU_REQUIRE_PTR(hidden_states, 2, fn);
    SSU_REQUIRE_PTR(w_ba, 4, fn);
    SSU_REQUIRE_PTR(mixed_qkv, 2, fn);
    SSU_REQUIRE_PTR(conv_weight, 2, fn);
    SSU_REQUIRE_PTR(conv_bias, 2, fn);
    if (d.conv_width > 1)
        SSU_REQUIRE_PTR(conv_state, 2, fn);
    SSU_REQUIRE_PTR(A_log, 4, fn);
    SSU_REQUIRE_PTR(dt_bias, 2, fn);
    SSU_REQUIRE_PTR(ssm_state, 16, fn);
    SSU_REQUIRE_PTR(state_indices, 4, fn);
    SSU_REQUIRE_PTR(out, 2, fn);
    SSU_REQUIRE_PTR(workspace, 16, fn);
    const int64_t need = ssu_gdn_workspace_bytes(dims);
    if (workspace_bytes < need)
        return fail(SSU_EINVAL, "%s: workspace_bytes %lld < %lld required", fn,
                    (long long)workspace_bytes, (long long)need);
    ssu::GdnParams p = {};
    p.workspace = workspace;
    p.hs = hidden_states;
    p.w_ba = w_ba;
    p.qkv = mixed_qkv;
    p.conv_w = conv_weight;
    p.conv_b = conv_bias;
    p.conv_state = conv_state;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.scale = (scale > 0.0f) ? scale : 1.0f / sqrtf((float)d.head_dim);
    p.ssm = ssm_state;
    p.idx = state_indices;
    p.out = out;
    p.ssm_row_stride = rs;
    p.cs_slot = d.conv_slot_stride;
    p.cs_chan = d.conv_chan_stride;
    p.cs_tap = d.conv_tap_stride;
    p.batch = d.batch;
    p.hidden = d.hidden;
    p.hq = d.num_q_heads;
    p.hv = d.num_v_heads;
    p.dhead = d.head_dim;
    p.width = d.conv_width;
    p.use_l2 = d.use_qk_l2norm ? 1 : 0;
    return hip_status(ssu::launch_gdn(p, stream), "ssu_gdn_decode launch");
}

namespace {

ssu_status check_rows(const char *fn, int32_t rows, int64_t stride, int64_t row_bytes,
                      int32_t batch, int64_t *eff_stride)
{
    if (rows < 0)
        return fail(SSU_EINVAL, "%s: row count %d < 0", fn, rows);
    if (batch < 0 || batch > 65535)
        return fail(SSU_EINVAL, "%s: batch %d outside [0, 65535]", fn, batch);
    if (row_bytes < 0)
        return fail(SSU_EINVAL, "%s: row_bytes %lld < 0", fn, (long long)row_bytes);
    if (stride != 0 && stride < row_bytes)
        return fail(SSU_EINVAL, "%s: stride %lld < row_bytes %lld", fn, (long long)stride,
                    (long long)row_bytes);
    *eff_stride = stride ? stride : row_bytes;
    return SSU_OK;
}

}  // namespace

ssu_status ssu_state_gather(const void *resident, int32_t resident_rows, int64_t resident_stride,
                            void *active, int64_t active_stride, const int32_t *state_indices,
                            int32_t batch, int64_t row_bytes, hipStream_t stream)
{
    const char *fn = "ssu_state_gather";
    int64_t rs = 0, as = 0;
    ssu_status st = check_rows(fn, resident_rows, resident_stride, row_bytes, batch, &rs);
    if (st != SSU_OK)
        return st;
    st = check_rows(fn, batch, active_stride, row_bytes, batch, &as);
    if (st != SSU_OK)
        return st;
    if (batch == 0 || row_bytes == 0)
        return ok();
    SSU_REQUIRE_PTR(resident, 1, fn);
    SSU_REQUIRE_PTR(active, 1, fn);
    SSU_REQUIRE_PTR(state_indices, 4, fn);
    ssu::RowMove mv = {};
    mv.dst = active;
    mv.src = resident;
    mv.src_idx = state_indices;
    mv.dst_stride = as;
    mv.src_stride = rs;
    mv.rows = batch;
    return hip_status(ssu::launch_row_moves(&mv, 1, row_bytes, stream), "ssu_state_gather launch");
}

ssu_status ssu_state_scatter(const void *active, int64_t active_stride, void *resident,
                             int32_t resident_rows, int64_t resident_stride,
                             const int32_t *state_indices, int32_t batch, int64_t row_bytes,
                             hipStream_t stream)
{
    const char *fn = "ssu_state_scatter";
    int64_t rs = 0, as = 0;
    ssu_status st = check_rows(fn, resident_rows, resident_stride, row_bytes, batch, &rs);
    if (st != SSU_OK)
        return st;
    st = check_rows(fn, batch, active_stride, row_bytes, batch, &as);
    if (st != SSU_OK)
        return st;
    if (batch == 0 || row_bytes == 0)
        return ok();
    SSU_REQUIRE_PTR(active, 1, fn);
    SSU_REQUIRE_PTR(resident, 1, fn);
    SSU_REQUIRE_PTR(state_indices, 4, fn);
    ssu::RowMove mv = {};
    mv.dst = resident;
    mv.src = active;
    mv.dst_idx = state_indices;
    mv.dst_stride = rs;
    mv.src_stride = as;
    mv.rows = batch;
    return hip_status(ssu::launch_row_moves(&mv, 1, row_bytes, stream), "ssu_state_scatter launch");
}

namespace {

ssu_status pack_args(const char *fn, void *pool, int32_t pool_rows, int64_t row_stride,
                     int64_t row_bytes, const int32_t *homes, int32_t batch,
                     const int32_t *bystanders, int32_t n_bystanders, void *workspace,
                     int64_t *eff_stride)
{
    ssu_status st = check_rows(fn, pool_rows, row_stride, row_bytes, batch, eff_stride);
    if (st != SSU_OK)
        return st;
    if (batch > pool_rows)
        return fail(SSU_EINVAL, "%s: batch %d > pool_rows %d", fn, batch, pool_rows);
    if (n_bystanders < 0 || n_bystanders > batch)
        return fail(SSU_EINVAL, "%s: n_bystanders %d outside [0, batch %d]", fn, n_bystanders,
                    batch);
    if (batch == 0 || row_bytes == 0)
        return SSU_OK;
    SSU_REQUIRE_PTR(pool, 1, fn);
    SSU_REQUIRE_PTR(homes, 4, fn);
    SSU_REQUIRE_PTR(workspace, 1, fn);
    if (n_bystanders > 0)
        SSU_REQUIRE_PTR(bystanders, 4, fn);
    return SSU_OK;
}

}  // namespace

ssu_status ssu_state_pack(void *pool, int32_t pool_rows, int64_t row_stride, int64_t row_bytes,
                          const int32_t *homes, int32_t batch, const int32_t *bystanders,
                          int32_t n_bystanders, void *workspace, hipStream_t stream)
{
    const char *fn = "ssu_state_pack";
    int64_t rs = 0;
    const ssu_status st = pack_args(fn, pool, pool_rows, row_stride, row_bytes, homes, batch,
                                    bystanders, n_bystanders, workspace, &rs);
    if (st != SSU_OK)
        return st;
    if (batch == 0 || row_bytes == 0)
        return ok();
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    // 1. read every source: homes -> workspace rows [0, batch), bystanders ->
    //    workspace rows [batch, batch + n_bystanders)
    ssu::RowMove in[2] = {};
    in[0].dst = ws;
    in[0].src = pool;
    in[0].src_idx = homes;
    in[0].skip_same = homes;
    in[0].dst_stride = row_bytes;
    in[0].src_stride = rs;
    in[0].rows = batch;
    in[1].dst = ws + (int64_t)batch * row_bytes;
    in[1].src = pool;
    in[1].src_idx = bystanders;
    in[1].dst_stride = row_bytes;
    in[1].src_stride = rs;
    in[1].rows = n_bystanders;
    hipError_t e = ssu::launch_row_moves(in, n_bystanders > 0 ? 2 : 1, row_bytes, stream);
    if (e != hipSuccess)
        return hip_status(e, "ssu_state_pack launch");
    // 2. then write the slots
    ssu::RowMove out = {};
    out.dst = pool;
    out.src = ws;
    out.skip_same = homes;
    out.dst_stride = rs;
    out.src_stride = row_bytes;
    out.rows = batch;
    return hip_status(ssu::launch_row_moves(&out, 1, row_bytes, stream), "ssu_state_pack launch");
}

ssu_status ssu_state_unpack(void *pool, int32_t pool_rows, int64_t row_stride, int64_t row_bytes,
                            const int32_t *homes, int32_t batch, const int32_t *bystanders,
                            int32_t n_bystanders, void *workspace, hipStream_t stream)
{
    const char *fn = "ssu_state_unpack";
    int64_t rs = 0;
    const ssu_status st = pack_args(fn, pool, pool_rows, row_stride, row_bytes, homes, batch,
                                    bystanders, n_bystanders, workspace, &rs);
    if (st != SSU_OK)
        return st;
    if (batch == 0 || row_bytes == 0)
        return ok();
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    // 1. read every slot into the workspace (rows in place are left alone)
    ssu::RowMove in = {};
    in.dst = ws;
    in.src = pool;
    in.skip_same = homes;
    in.dst_stride = row_bytes;
    in.src_stride = rs;
    in.rows = batch;
    hipError_t e = ssu::launch_row_moves(&in, 1, row_bytes, stream);
    if (e != hipSuccess)
        return hip_status(e, "ssu_state_unpack launch");
    // 2. write the slots to their homes and the saved bystanders back (disjoint rows)
    ssu::RowMove out[2] = {};
    out[0].dst = pool;
    out[0].src = ws;
    out[0].dst_idx = homes;
    out[0].skip_same = homes;
    out[0].dst_stride = rs;
    out[0].src_stride = row_bytes;
    out[0].rows = batch;
    out[1].dst = pool;
    out[1].src = ws + (int64_t)batch * row_bytes;
    out[1].dst_idx = bystanders;
    out[1].dst_stride = rs;
    out[1].src_stride = row_bytes;
    out[1].rows = n_bystanders;
    return hip_status(ssu::launch_row_moves(out, n_bystanders > 0 ? 2 : 1, row_bytes, stream),
                      "ssu_state_unpack launch");
}

int64_t ssu_tree_workspace_bytes(const ssu_dims *dims, int32_t num_nodes)
{
    if (!dims || num_nodes < 0 || num_nodes > SSU_MAX_TREE_NODES || dims->batch < 0 ||
        dims->ngroups <= 0)
        return -1;
    return (int64_t)4 * dims->batch * dims->ngroups * num_nodes * num_nodes;
}

}  // extern "C"

namespace {

// ssu_tree_verify with a caller workspace, or (workspace == nullptr and
// own_scratch) the library's scratch.
ssu_status tree_verify(const char *fn, const ssu_dims *dims, int32_t num_nodes, const void *x,
                       const float *A, const void *B, const void *C, const float *dt,
                       const float *dt_bias, const float *D, const void *z, const void *state,
                       void *out, int32_t dt_softplus, const int32_t *state_indices,
                       const int32_t *parent_ids, const int32_t *depths, float *replay_dA,
                       float *replay_u, float *replay_B, float *replay_dt, void *workspace,
                       int64_t workspace_bytes, bool own_scratch, hipStream_t stream)
{
    ssu::TreeParams p = {};
    const ssu_status st = check_dims(dims, fn, true, state_indices != nullptr, &p.d);
    if (st != SSU_OK)
        return st;
    if (num_nodes < 0 || num_nodes > SSU_MAX_TREE_NODES)
        return fail(SSU_EINVAL, "%s: num_nodes %d outside [0, %d]", fn, num_nodes,
                    SSU_MAX_TREE_NODES);
    const int nstash = (replay_dA != nullptr) + (replay_u != nullptr) + (replay_B != nullptr) +
                       (replay_dt != nullptr);
    if (nstash != 0 && nstash != 4)
        return fail(SSU_EINVAL, "%s: replay stash must be all four buffers or none (%d given)",
                    fn, nstash);
    if (p.d.batch == 0 || num_nodes == 0)
        return ok();
    if ((int64_t)p.d.batch * num_nodes * p.d.nheads * p.d.dim > ((int64_t)1 << 40))
        return fail(SSU_ENOTSUP, "%s: problem too large", fn);
    SSU_REQUIRE_PTR(x, io_bytes(dims->io_dtype), fn);
    SSU_REQUIRE_PTR(A, 4, fn);
    SSU_REQUIRE_PTR(B, 16, fn);
    SSU_REQUIRE_PTR(C, 16, fn);
    SSU_REQUIRE_PTR(dt, 4, fn);
    SSU_REQUIRE_PTR(state, 16, fn);
    SSU_REQUIRE_PTR(out, io_bytes(dims->io_dtype), fn);
    SSU_REQUIRE_PTR(parent_ids, 4, fn);
    SSU_OPTIONAL_PTR(dt_bias, 4, fn);
    SSU_OPTIONAL_PTR(D, 4, fn);
    SSU_OPTIONAL_PTR(z, io_bytes(dims->io_dtype), fn);
    SSU_OPTIONAL_PTR(state_indices, 4, fn);
    SSU_OPTIONAL_PTR(depths, 4, fn);
    SSU_OPTIONAL_PTR(replay_dA, 4, fn);
    SSU_OPTIONAL_PTR(replay_u, 4, fn);
    SSU_OPTIONAL_PTR(replay_B, 16, fn);
    SSU_OPTIONAL_PTR(replay_dt, 4, fn);
    const int64_t need = ssu_tree_workspace_bytes(dims, num_nodes);
    if (own_scratch) {
        if (need > SSU_TREE_SCRATCH_BYTES)
            return fail(SSU_EINVAL,
                        "%s: batch * ngroups * num_nodes^2 * 4 = %lld bytes exceeds the library's "
                        "scratch of %d bytes (use ssu_tree_verify with a workspace)",
                        fn, (long long)need, SSU_TREE_SCRATCH_BYTES);
        const hipError_t e = ssu::tree_scratch(&workspace);
        if (e != hipSuccess)
            return hip_status(e, "ssu_tree_verify_noalloc scratch address");
    } else {
        SSU_REQUIRE_PTR(workspace, 16, fn);
        if (workspace_bytes < need)
            return fail(SSU_EINVAL, "%s: workspace_bytes %lld < %lld required", fn,
                        (long long)workspace_bytes, (long long)need);
    }
    p.gram = static_cast<float *>(workspace);
    p.d.x = x;
    p.d.A = A;
    p.d.B = B;
    p.d.C = C;
    p.d.dt = dt;
    p.d.dt_bias = dt_bias;
    p.d.D = D;
    p.d.z = z;
    p.d.state = const_cast<void *>(state);  // read only
    p.d.out = out;
    p.d.idx = state_indices;
    p.d.dt_softplus = dt_softplus ? 1 : 0;
    p.num_nodes = num_nodes;
    p.parents = parent_ids;
    p.depths = depths;
    p.st_dA = replay_dA;
    p.st_u = replay_u;
    p.st_B = replay_B;
    p.st_dt = replay_dt;
    return hip_status(ssu::launch_tree(p, stream), fn);
}

}  // namespace

extern "C" {

ssu_status ssu_tree_verify(const ssu_dims *dims, int32_t num_nodes, const void *x,
                           const float *A, const void *B, const void *C, const float *dt,
                           const float *dt_bias, const float *D, const void *z,
                           const void *state, void *out, int32_t dt_softplus,
                           const int32_t *state_indices, const int32_t *parent_ids,
                           const int32_t *depths, float *replay_dA, float *replay_u,
                           float *replay_B, float *replay_dt, void *workspace,
                           int64_t workspace_bytes, hipStream_t stream)
{
    return tree_verify("ssu_tree_verify", dims, num_nodes, x, A, B, C, dt, dt_bias, D, z, state,
                       out, dt_softplus, state_indices, parent_ids, depths, replay_dA, replay_u,
                       replay_B, replay_dt, workspace, workspace_bytes, false, stream);
}

ssu_status ssu_tree_verify_noalloc(const ssu_dims *dims, int32_t num_nodes, const void *x,
                                   const float *A, const void *B, const void *C, const float *dt,
                                   const float *dt_bias, const float *D, const void *z,
                                   const void *state, void *out, int32_t dt_softplus,
                                   const int32_t *state_indices, const int32_t *parent_ids,
                                   const int32_t *depths, float *replay_dA, float *replay_u,
                                   float *replay_B, float *replay_dt, hipStream_t stream)
{
    return tree_verify("ssu_tree_verify_noalloc", dims, num_nodes, x, A, B, C, dt, dt_bias, D, z,
                       state, out, dt_softplus, state_indices, parent_ids, depths, replay_dA,
                       replay_u, replay_B, replay_dt, nullptr, 0, true, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Recurrent-state pool
// ---------------------------------------------------------------------------
struct ssu_pool {
    std::vector<ssu_state_spec> specs;
    std::vector<size_t> bytes_per_slot;  // per state
    std::vector<void *> slabs;           // per state, slot_count * bytes_per_slot[i] bytes
    int32_t slot_count = 0;
    bool owns = true;                    // false: the slabs lie in a caller slab
    std::string name;                    // prefix of the state names in diagnostics
};

namespace {

constexpr size_t kSlabAlign = 256;  // every state's slab starts at this alignment

ssu_status check_specs(const ssu_state_spec *specs, int32_t n, const char *fn,
                       std::vector<size_t> *per_state)
{
    if (n < 0)
        return fail(SSU_EINVAL, "%s: n_specs %d < 0", fn, n);
    if (n > 0 && !specs)
        return fail(SSU_EINVAL, "%s: specs is NULL", fn);
    per_state->clear();
    for (int32_t i = 0; i < n; ++i) {
        const ssu_state_spec &s = specs[i];
        if (s.layer < 0)
            return fail(SSU_EINVAL, "%s: spec %d names negative layer %d", fn, i, s.layer);
        if (s.rank < 1 || s.rank > 4)
            return fail(SSU_EINVAL, "%s: spec %d has rank %d (1..4)", fn, i, s.rank);
        const size_t eb = dtype_bytes(s.dtype);
        if (eb == 0)
            return fail(SSU_EINVAL, "%s: spec %d has unknown dtype %d", fn, i, s.dtype);
        uint64_t vol = 1;
        for (int k = 0; k < s.rank; ++k) {
            if (s.shape[k] <= 0)
                return fail(SSU_EINVAL, "%s: spec %d has non-positive per-slot volume", fn, i);
            if (vol > (UINT64_MAX / 16) / (uint64_t)s.shape[k])
                return fail(SSU_EINVAL, "%s: spec %d volume overflows", fn, i);
            vol *= (uint64_t)s.shape[k];
        }
        for (int32_t j = 0; j < i; ++j)
            if (specs[j].kind == s.kind && specs[j].layer == s.layer)
                return fail(SSU_EINVAL, "%s: spec %d repeats {kind %d, layer %d} of spec %d", fn,
                            i, s.kind, s.layer, j);
        per_state->push_back((size_t)vol * eb);
    }
    return SSU_OK;
}

// Byte offset of every state's slab inside one slab holding all of them (each
// aligned to kSlabAlign), and the total; false if the sizes overflow.
bool slab_layout(const std::vector<size_t> &per, int32_t slot_count, std::vector<size_t> *offs,
                 size_t *total)
{
    size_t o = 0;
    offs->clear();
    for (size_t b : per) {
        if (slot_count > 0 && b > (SIZE_MAX / 4) / (size_t)slot_count)
            return false;
        offs->push_back(o);
        const size_t bytes = b * (size_t)slot_count;
        const size_t padded = (bytes + kSlabAlign - 1) / kSlabAlign * kSlabAlign;
        if (padded > SIZE_MAX / 4 - o)
            return false;
        o += padded;
    }
    *total = o;
    return true;
}

bool slot_ok(const ssu_pool *p, int32_t slot) { return slot >= 0 && slot < p->slot_count; }

// "pool 'name'" (or "pool") for diagnostics
std::string label(const ssu_pool *p)
{
    return p->name.empty() ? std::string("pool") : "pool '" + p->name + "'";
}

}  // namespace

extern "C" {

ssu_status ssu_pool_bytes_per_slot(const ssu_state_spec *specs, int32_t n_specs, size_t *out)
{
    const char *fn = "ssu_pool_bytes_per_slot";
    if (!out)
        return fail(SSU_EINVAL, "%s: out is NULL", fn);
    std::vector<size_t> per;
    const ssu_status st = check_specs(specs, n_specs, fn, &per);
    if (st != SSU_OK)
        return st;
    size_t total = 0;
    for (size_t b : per)
        total += b;
    *out = total;
    return ok();
}

ssu_status ssu_pool_slab_bytes(const ssu_state_spec *specs, int32_t n_specs, int32_t slot_count,
                               size_t *out)
{
    const char *fn = "ssu_pool_slab_bytes";
    if (!out)
        return fail(SSU_EINVAL, "%s: out is NULL", fn);
    if (slot_count < 0)
        return fail(SSU_EINVAL, "%s: slot_count %d < 0", fn, slot_count);
    std::vector<size_t> per, offs;
    const ssu_status st = check_specs(specs, n_specs, fn, &per);
    if (st != SSU_OK)
        return st;
    size_t total = 0;
    if (!slab_layout(per, slot_count, &offs, &total))
        return fail(SSU_EINVAL, "%s: slab size overflows", fn);
    *out = total;
    return ok();
}

ssu_status ssu_pool_alloc(const ssu_state_spec *specs, int32_t n_specs, int32_t slot_count,
                          const char *name, void *base, size_t base_bytes, hipStream_t stream,
                          ssu_pool **out)
{
    const char *fn = "ssu_pool_alloc";
    if (!out)
        return fail(SSU_EINVAL, "%s: out is NULL", fn);
    *out = nullptr;
    const std::string nm = name ? name : "";
    const std::string lb = nm.empty() ? std::string("pool") : "pool '" + nm + "'";
    if (slot_count < 0)
        return fail(SSU_EINVAL, "%s (%s): slot_count %d < 0", fn, lb.c_str(), slot_count);
    std::vector<size_t> per, offs;
    ssu_status st = check_specs(specs, n_specs, fn, &per);
    if (st != SSU_OK)
        return st;
    size_t need = 0;
    if (!slab_layout(per, slot_count, &offs, &need))
        return fail(SSU_EINVAL, "%s (%s): slab size overflows", fn, lb.c_str());
    if (base) {
        if ((reinterpret_cast<uintptr_t>(base) & (kSlabAlign - 1)) != 0)
            return fail(SSU_EINVAL, "%s (%s): caller slab is not %zu-byte aligned", fn, lb.c_str(),
                        kSlabAlign);
        if (base_bytes < need)
            return fail(SSU_EINVAL, "%s (%s): caller slab holds %zu bytes, the states need %zu", fn,
                        lb.c_str(), base_bytes, need);
    }
    ssu_pool *p = new (std::nothrow) ssu_pool();
    if (!p)
        return fail(SSU_ENOMEM, "%s (%s): host allocation failed", fn, lb.c_str());
    p->specs.assign(specs, specs + n_specs);
    p->bytes_per_slot = per;
    p->slot_count = slot_count;
    p->slabs.assign(n_specs, nullptr);
    p->owns = base == nullptr;
    p->name = nm;
    if (slot_count > 0) {
        std::vector<ssu::Segment> segs;
        for (int32_t i = 0; i < n_specs; ++i) {
            const size_t bytes = per[i] * (size_t)slot_count;
            if (base) {
                p->slabs[i] = static_cast<uint8_t *>(base) + offs[i];
            } else {
                const hipError_t e = hipMalloc(&p->slabs[i], bytes);
                if (e != hipSuccess) {
                    p->slabs[i] = nullptr;
                    ssu_pool_free(p);
                    return fail(e == hipErrorOutOfMemory ? SSU_ENOMEM : SSU_EHIP,
                                "%s (%s): hipMalloc of %zu bytes for state %d: %s", fn,
                                lb.c_str(), bytes, i, hipGetErrorString(e));
                }
            }
            segs.push_back({p->slabs[i], nullptr, (uint64_t)bytes});
        }
        const hipError_t e = ssu::launch_segments(segs.data(), (int)segs.size(), stream);
        if (e != hipSuccess) {
            ssu_pool_free(p);
            return fail(SSU_EHIP, "%s (%s): zero fill: %s", fn, lb.c_str(), hipGetErrorString(e));
        }
    }
    *out = p;
    return ok();
}

ssu_status ssu_pool_free(ssu_pool *pool)
{
    if (!pool)
        return ok();
    if (!pool->owns) {  // a caller slab: nothing to release or wait for
        delete pool;
        return ok();
    }
    bool any = false;
    for (void *s : pool->slabs)
        any = any || s;
    hipError_t first = hipSuccess;
    if (any)
        first = hipDeviceSynchronize();  // the slabs may still be in use by queued work
    for (void *s : pool->slabs) {
        if (s) {
            const hipError_t e = hipFree(s);
            if (first == hipSuccess)
                first = e;
        }
    }
    delete pool;
    return hip_status(first, "ssu_pool_free");
}

ssu_status ssu_pool_info(const ssu_pool *pool, int32_t *num_states, int32_t *slot_count)
{
    if (!pool)
        return fail(SSU_EINVAL, "ssu_pool_info: pool is NULL");
    if (num_states)
        *num_states = (int32_t)pool->specs.size();
    if (slot_count)
        *slot_count = pool->slot_count;
    return ok();
}

ssu_status ssu_pool_state_ptr(const ssu_pool *pool, int32_t state_idx, void **dev_ptr)
{
    if (!pool || !dev_ptr)
        return fail(SSU_EINVAL, "ssu_pool_state_ptr: NULL argument");
    if (state_idx < 0 || state_idx >= (int32_t)pool->specs.size())
        return fail(SSU_EINVAL, "ssu_pool_state_ptr: state %d outside [0, %zu)", state_idx,
                    pool->specs.size());
    *dev_ptr = pool->slabs[state_idx];
    return ok();
}

ssu_status ssu_pool_state_bytes_per_slot(const ssu_pool *pool, int32_t state_idx, size_t *out)
{
    if (!pool || !out)
        return fail(SSU_EINVAL, "ssu_pool_state_bytes_per_slot: NULL argument");
    if (state_idx < 0 || state_idx >= (int32_t)pool->specs.size())
        return fail(SSU_EINVAL, "ssu_pool_state_bytes_per_slot: state %d outside [0, %zu)",
                    state_idx, pool->specs.size());
    *out = pool->bytes_per_slot[state_idx];
    return ok();
}

ssu_status ssu_pool_spec(const ssu_pool *pool, int32_t state_idx, ssu_state_spec *out)
{
    if (!pool || !out)
        return fail(SSU_EINVAL, "ssu_pool_spec: NULL argument");
    if (state_idx < 0 || state_idx >= (int32_t)pool->specs.size())
        return fail(SSU_EINVAL, "ssu_pool_spec (%s): state %d outside [0, %zu)",
                    label(pool).c_str(), state_idx, pool->specs.size());
    *out = pool->specs[state_idx];
    return ok();
}

ssu_status ssu_pool_specs(const ssu_pool *pool, ssu_state_spec *out, int32_t capacity,
                          int32_t *n_specs)
{
    if (!pool || !n_specs)
        return fail(SSU_EINVAL, "ssu_pool_specs: NULL argument");
    if (capacity < 0 || (capacity > 0 && !out))
        return fail(SSU_EINVAL, "ssu_pool_specs (%s): capacity %d with %s buffer",
                    label(pool).c_str(), capacity, out ? "a" : "no");
    const int32_t n = (int32_t)pool->specs.size();
    for (int32_t i = 0; i < n && i < capacity; ++i)
        out[i] = pool->specs[i];
    *n_specs = n;
    return ok();
}

ssu_status ssu_pool_name(const ssu_pool *pool, const char **name)
{
    if (!pool || !name)
        return fail(SSU_EINVAL, "ssu_pool_name: NULL argument");
    *name = pool->name.c_str();
    return ok();
}

ssu_status ssu_pool_owns_memory(const ssu_pool *pool, int32_t *owns)
{
    if (!pool || !owns)
        return fail(SSU_EINVAL, "ssu_pool_owns_memory: NULL argument");
    *owns = pool->owns ? 1 : 0;
    return ok();
}

ssu_status ssu_pool_find_state(const ssu_pool *pool, int32_t kind, int32_t layer,
                               int32_t *state_idx)
{
    if (!pool || !state_idx)
        return fail(SSU_EINVAL, "ssu_pool_find_state: NULL argument");
    *state_idx = -1;
    for (size_t i = 0; i < pool->specs.size(); ++i)
        if (pool->specs[i].kind == kind && pool->specs[i].layer == layer)
            *state_idx = (int32_t)i;
    return ok();
}

ssu_status ssu_pool_clear_slot(ssu_pool *pool, int32_t slot, hipStream_t stream)
{
    const char *fn = "ssu_pool_clear_slot";
    if (!pool)
        return fail(SSU_EINVAL, "%s: pool is NULL", fn);
    if (slot < -1 || slot >= pool->slot_count || (slot == -1 && pool->slot_count < 0))
        return fail(SSU_EINVAL, "%s (%s): slot %d outside [-1, %d)", fn,
                    label(pool).c_str(), slot, pool->slot_count);
    if (pool->slot_count == 0)
        return ok();
    std::vector<ssu::Segment> segs;
    for (size_t i = 0; i < pool->specs.size(); ++i) {
        uint8_t *base = static_cast<uint8_t *>(pool->slabs[i]);
        const size_t b = pool->bytes_per_slot[i];
        if (slot < 0)
            segs.push_back({base, nullptr, (uint64_t)(b * (size_t)pool->slot_count)});
        else
            segs.push_back({base + b * (size_t)slot, nullptr, (uint64_t)b});
    }
    return hip_status(ssu::launch_segments(segs.data(), (int)segs.size(), stream), fn);
}

ssu_status ssu_pool_clear(ssu_pool *pool, hipStream_t stream)
{
    if (!pool)
        return fail(SSU_EINVAL, "ssu_pool_clear: pool is NULL");
    return ssu_pool_clear_slot(pool, -1, stream);
}

ssu_status ssu_pool_capture(const ssu_pool *pool, int32_t slot, void *const *dst,
                            const size_t *dst_bytes, int32_t n, hipStream_t stream)
{
    const char *fn = "ssu_pool_capture";
    if (!pool)
        return fail(SSU_EINVAL, "%s: pool is NULL", fn);
    if (!slot_ok(pool, slot))
        return fail(SSU_EINVAL, "%s (%s): slot %d outside [0, %d)", fn,
                    label(pool).c_str(), slot, pool->slot_count);
    if (n != (int32_t)pool->specs.size())
        return fail(SSU_EINVAL, "%s (%s): %d buffers given for %zu states", fn,
                    label(pool).c_str(), n, pool->specs.size());
    if (n > 0 && (!dst || !dst_bytes))
        return fail(SSU_EINVAL, "%s: dst or dst_bytes is NULL", fn);
    for (int32_t i = 0; i < n; ++i) {
        if (!dst[i])
            return fail(SSU_EINVAL, "%s (%s): dst[%d] is NULL", fn, label(pool).c_str(), i);
        if (dst_bytes[i] != pool->bytes_per_slot[i])
            return fail(SSU_EINVAL, "%s (%s): dst_bytes[%d] = %zu, state holds %zu bytes per slot", fn,
                        label(pool).c_str(),
                        i, dst_bytes[i], pool->bytes_per_slot[i]);
    }
    std::vector<ssu::Segment> segs;
    for (int32_t i = 0; i < n; ++i) {
        const uint8_t *base = static_cast<const uint8_t *>(pool->slabs[i]);
        segs.push_back({dst[i], base + pool->bytes_per_slot[i] * (size_t)slot,
                        (uint64_t)pool->bytes_per_slot[i]});
    }
    return hip_status(ssu::launch_segments(segs.data(), (int)segs.size(), stream), fn);
}

ssu_status ssu_pool_restore(ssu_pool *pool, int32_t slot, const void *const *src,
                            const size_t *src_bytes, int32_t n_saved, hipStream_t stream)
{
    const char *fn = "ssu_pool_restore";
    if (!pool)
        return fail(SSU_EINVAL, "%s: pool is NULL", fn);
    if (!slot_ok(pool, slot))
        return fail(SSU_EINVAL, "%s (%s): slot %d outside [0, %d)", fn,
                    label(pool).c_str(), slot, pool->slot_count);
    if (n_saved < 0 || n_saved > (int32_t)pool->specs.size())
        return fail(SSU_EINVAL, "%s (%s): n_saved %d outside [0, %zu]", fn,
                    label(pool).c_str(), n_saved,
                    pool->specs.size());
    if (n_saved > 0 && (!src || !src_bytes))
        return fail(SSU_EINVAL, "%s: src or src_bytes is NULL", fn);
    for (int32_t i = 0; i < n_saved; ++i) {  // validate everything before any write
        if (!src[i])
            return fail(SSU_EINVAL, "%s (%s): src[%d] is NULL", fn, label(pool).c_str(), i);
        if (src_bytes[i] != pool->bytes_per_slot[i])
            return fail(SSU_EINVAL, "%s (%s): src_bytes[%d] = %zu, state holds %zu bytes per slot", fn,
                        label(pool).c_str(),
                        i, src_bytes[i], pool->bytes_per_slot[i]);
    }
    std::vector<ssu::Segment> segs;
    for (size_t i = 0; i < pool->specs.size(); ++i) {
        uint8_t *base = static_cast<uint8_t *>(pool->slabs[i]);
        segs.push_back({base + pool->bytes_per_slot[i] * (size_t)slot,
                        (int32_t)i < n_saved ? src[i] : nullptr,
                        (uint64_t)pool->bytes_per_slot[i]});
    }
    return hip_status(ssu::launch_segments(segs.data(), (int)segs.size(), stream), fn);
}

ssu_status ssu_pool_copy_slot_from(ssu_pool *pool, const ssu_pool *source, int32_t dst_slot,
                                   int32_t src_slot, hipStream_t stream)
{
    const char *fn = "ssu_pool_copy_slot_from";
    if (!pool || !source)
        return fail(SSU_EINVAL, "%s: pool is NULL", fn);
    if (pool->specs.size() != source->specs.size())
        return fail(SSU_EINVAL, "%s (%s): pools hold %zu and %zu states", fn,
                    label(pool).c_str(), pool->specs.size(),
                    source->specs.size());
    for (size_t i = 0; i < pool->specs.size(); ++i) {
        const ssu_state_spec &a = pool->specs[i], &b = source->specs[i];
        bool same = a.kind == b.kind && a.layer == b.layer && a.rank == b.rank &&
                    a.dtype == b.dtype;
        for (int k = 0; same && k < a.rank; ++k)
            same = a.shape[k] == b.shape[k];
        if (!same)
            return fail(SSU_EINVAL, "%s (%s): state %zu differs between the pools", fn,
                        label(pool).c_str(), i);
    }
    if (!slot_ok(pool, dst_slot))
        return fail(SSU_EINVAL, "%s (%s): destination slot %d outside [0, %d)", fn,
                    label(pool).c_str(), dst_slot,
                    pool->slot_count);
    if (!slot_ok(source, src_slot))
        return fail(SSU_EINVAL, "%s (%s): source slot %d outside [0, %d)", fn,
                    label(source).c_str(), src_slot,
                    source->slot_count);
    std::vector<ssu::Segment> segs;
    for (size_t i = 0; i < pool->specs.size(); ++i) {
        const size_t b = pool->bytes_per_slot[i];
        segs.push_back({static_cast<uint8_t *>(pool->slabs[i]) + b * (size_t)dst_slot,
                        static_cast<const uint8_t *>(source->slabs[i]) + b * (size_t)src_slot,
                        (uint64_t)b});
    }
    return hip_status(ssu::launch_segments(segs.data(), (int)segs.size(), stream), fn);
}

}  // extern "C"
