// Replay reconstruct: commit the accepted prefix of a speculative verify.
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page, struct
// MambaReplayLayerInfo): re-run the recurrence over the first
// acceptedLengths[b] stashed tokens, in place, for b < activeBatchSize:
//   state <- state * exp(dA_t) + B_t * dt_t * u_t
// A row whose accepted count is 0, or whose state index is negative, is left
// untouched; entries at b >= activeBatchSize are never read. With
// acceptedNodeIds (invokeMambaReplayReconstructBatched) token t of row b is the
// stash entry of node acceptedNodeIds[b, t]; the count is capped at
// maxAcceptLen and the row ends before the first id outside the stash.
// invokeMambaReplayReconstructBatched runs every layer in one launch: the layer
// is blockIdx.y and its buffers come from a device array of
// MambaReplayLayerInfo-like entries.
//
// Mapping on gfx950: the decode mapping (the (batch row, head) tile split over
// workgroups of about 8 KiB of state; lanes along dstate with 16-byte vectors;
// non-temporal state traffic). The k <= seq_len stashed tokens are applied
// while the tile sits in registers, so the state is read and written once
// whatever k is: the kernel is bound by HBM bandwidth. When seq_len <= MAXT
// the stash values of every token are loaded together with the state, before
// any of them is used (tokens past k re-read token k-1 and are not applied).
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

struct ReplayShape {
    int64_t row_stride;
    int32_t seq_len, nheads, dim, ngroups, heads_per_group, parts;
    int32_t max_accept;  // row length of the node-id array (IDS only)
};

// MAXT > 0: at most MAXT tokens per row, all stash loads hoisted; MAXT == 0:
// any count. IDS: stash positions come from the node-id array.
template <typename ST, int NS, int PASSES, int MAXT, bool IDS>
__global__ __launch_bounds__(256) void ssu_replay_kernel(
    ST *__restrict__ state, const float *__restrict__ sdA, const float *__restrict__ su,
    const float *__restrict__ sB, const float *__restrict__ sdt,
    const int32_t *__restrict__ accepted, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ node_ids, const ssu_replay_layer *__restrict__ layers,
    const ReplayShape sh)
{
    if (layers) {  // batched over layers: this workgroup's layer is blockIdx.y
        const ssu_replay_layer &ly = layers[blockIdx.y];
        state = table_ptr<ST>(ly.state);
        sdA = table_ptr<const float>(ly.replay_dA);
        su = table_ptr<const float>(ly.replay_u);
        sB = table_ptr<const float>(ly.replay_B);
        sdt = table_ptr<const float>(ly.replay_dt);
    }
    constexpr int VEC = SV<ST>::VEC;
    constexpr int LPR = NS / VEC;
    constexpr int RPW = 64 / LPR;
    constexpr int RPP = 4 * RPW;
    constexpr int ROWS = PASSES * RPP;

    const int tile = blockIdx.x / sh.parts;
    const int part = blockIdx.x - tile * sh.parts;
    const int b = tile / sh.nheads;
    const int h = tile - b * sh.nheads;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (LPR - 1);
    const int rsub = (threadIdx.x >> 6) * RPW + lane / LPR;
    const int r0 = part * ROWS;

    const int row = idx ? idx[b] : b;
    const int k = min(accepted[b], IDS ? sh.max_accept : sh.seq_len);
    if (row < 0 || k <= 0)
        return;
    const int g = h / sh.heads_per_group;
    const int H = sh.nheads, Dm = sh.dim;
    const int64_t bT = (int64_t)b * sh.seq_len;
    ST *tp = state + (int64_t)row * sh.row_stride + (int64_t)h * Dm * NS + sub * VEC;

    u32x4 raw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = min(r0 + p * RPP + rsub, Dm - 1);
        raw[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(tp + (int64_t)r * NS));
    }
    float s[PASSES][VEC];
    if constexpr (MAXT > 0) {
        // stash position of every token slot (slots past k repeat token k-1);
        // kk = the tokens actually applied
        int pos[MAXT];
        int kk = k;
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            const int tc = min(t, k - 1);
            int p = tc;
            if constexpr (IDS) {
                p = node_ids[(int64_t)b * sh.max_accept + tc];
                const bool inside = p >= 0 && p < sh.seq_len;
                kk = inside ? kk : min(kk, tc);
                p = inside ? p : 0;
            }
            pos[t] = p;
        }
        float ut[MAXT][PASSES], bt[MAXT][VEC], at[MAXT], dtt[MAXT];
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            const int64_t bth = (bT + pos[t]) * H + h;
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
                ut[t][p] = su[bth * Dm + min(r0 + p * RPP + rsub, Dm - 1)];
            ld_typed<float, VEC>(sB, ((bT + pos[t]) * sh.ngroups + g) * NS + sub * VEC, bt[t]);
            at[t] = sdA[bth];
            dtt[t] = sdt[bth];
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
            SV<ST>::unpack(raw[p], s[p]);
        if (kk <= 0)
            return;  // the first node id is outside the stash: nothing to commit
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            if (t < kk) {
                const float a = expf(at[t]);
#pragma unroll
                for (int p = 0; p < PASSES; ++p) {
                    const float dtx = dtt[t] * ut[t][p];
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        s[p][e] = fmaf(dtx, bt[t][e], s[p][e] * a);
                }
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
            SV<ST>::unpack(raw[p], s[p]);
        int t = 0;
        for (; t < k; ++t) {
            int ps = t;
            if constexpr (IDS) {
                ps = node_ids[(int64_t)b * sh.max_accept + t];
                if (ps < 0 || ps >= sh.seq_len)
                    break;
            }
            const int64_t bth = (bT + ps) * H + h;
            const float a = expf(sdA[bth]);
            const float dtv = sdt[bth];
            float bv[VEC];
            ld_typed<float, VEC>(sB, ((bT + ps) * sh.ngroups + g) * NS + sub * VEC, bv);
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const float dtx = dtv * su[bth * Dm + min(r0 + p * RPP + rsub, Dm - 1)];
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    s[p][e] = fmaf(dtx, bv[e], s[p][e] * a);
            }
        }
        if (t == 0)
            return;  // nothing committed
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP + rsub;
        if (r < Dm)
            __builtin_nontemporal_store(SV<ST>::pack(s[p]),
                                        reinterpret_cast<u32x4 *>(tp + (int64_t)r * NS));
    }
}

template <typename ST, int NS>
hipError_t launch_ns(const ReplayParams &p, hipStream_t stream)
{
    constexpr int VEC = SV<ST>::VEC;
    constexpr int RPP = 4 * (64 / (NS / VEC));
    const int passes = p.dim > RPP ? 2 : 1;
    ReplayShape sh;
    sh.row_stride = p.row_stride;
    sh.seq_len = p.seq_len;
    sh.nheads = p.nheads;
    sh.dim = p.dim;
    sh.ngroups = p.ngroups;
    sh.heads_per_group = p.nheads / p.ngroups;
    sh.parts = (p.dim + passes * RPP - 1) / (passes * RPP);
    sh.max_accept = p.max_accept_len;
    const int64_t blocks = (int64_t)p.active_batch * p.nheads * sh.parts;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    if (p.layers && (p.num_layers <= 0 || p.num_layers > 65535))
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks, p.layers ? (unsigned)p.num_layers : 1u);
    ST *st = static_cast<ST *>(p.state);
    (void)hipGetLastError();
#define SSU_LAUNCH_REPLAY(PS, MT, ID)                                                         \
    hipLaunchKernelGGL((ssu_replay_kernel<ST, NS, PS, MT, ID>), grid, dim3(256), 0, stream, st, \
                       p.dA, p.u, p.B, p.dt, p.accepted, p.idx, p.node_ids, p.layers, sh)
#define SSU_LAUNCH_REPLAY_T(PS)           \
    if (p.node_ids) {                     \
        if (p.max_accept_len <= 4)        \
            SSU_LAUNCH_REPLAY(PS, 4, true);  \
        else if (p.max_accept_len <= 8)   \
            SSU_LAUNCH_REPLAY(PS, 8, true);  \
        else                              \
            SSU_LAUNCH_REPLAY(PS, 0, true);  \
    } else if (p.seq_len <= 1)            \
        SSU_LAUNCH_REPLAY(PS, 1, false);  \
    else if (p.seq_len <= 2)              \
        SSU_LAUNCH_REPLAY(PS, 2, false);  \
    else if (p.seq_len <= 4)              \
        SSU_LAUNCH_REPLAY(PS, 4, false);  \
    else if (p.seq_len <= 8)              \
        SSU_LAUNCH_REPLAY(PS, 8, false);  \
    else                                  \
        SSU_LAUNCH_REPLAY(PS, 0, false);
    if (passes == 2) {
        SSU_LAUNCH_REPLAY_T(2)
    } else {
        SSU_LAUNCH_REPLAY_T(1)
    }
#undef SSU_LAUNCH_REPLAY_T
#undef SSU_LAUNCH_REPLAY
    return hipGetLastError();
}

template <typename ST>
hipError_t launch_st(const ReplayParams &p, hipStream_t stream)
{
    switch (p.dstate) {
    case 16: return launch_ns<ST, 16>(p, stream);
    case 32: return launch_ns<ST, 32>(p, stream);
    case 64: return launch_ns<ST, 64>(p, stream);
    case 128: return launch_ns<ST, 128>(p, stream);
    case 256: return launch_ns<ST, 256>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_replay(const ReplayParams &p, hipStream_t stream)
{
    if (p.active_batch == 0 || p.seq_len == 0)
        return hipSuccess;
    switch (p.state_dtype) {
    case kF32: return launch_st<float>(p, stream);
    case kF16: return launch_st<_Float16>(p, stream);
    case kBF16: return launch_st<bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
