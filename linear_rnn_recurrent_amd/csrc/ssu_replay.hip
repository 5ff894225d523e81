// Replay reconstruct: commit the accepted prefix of a speculative verify.
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page, struct
// MambaReplayLayerInfo): re-run the recurrence over the first
// acceptedLengths[b] stashed tokens, in place, for b < activeBatchSize:
//   state <- state * exp(dA_t) + B_t * dt_t * u_t
// A row whose accepted count is 0, or whose state index is negative, is left
// untouched; entries at b >= activeBatchSize are never read.
//
// Mapping on gfx950: the same tile mapping as decode (one 256-thread
// workgroup per (batch row, head); lanes along dstate with 16-byte vectors; all
// state loads of a tile in flight before the first FMA). The k <= seq_len
// stashed tokens are applied while the tile sits in registers, so the state is
// read and written once whatever k is: the kernel is bound by HBM bandwidth.
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

struct ReplayShape {
    int64_t row_stride;
    int32_t seq_len, nheads, dim, ngroups, heads_per_group;
};

template <typename ST, int NS, int PASSES>
__global__ __launch_bounds__(256) void ssu_replay_kernel(
    ST *__restrict__ state, const float *__restrict__ sdA, const float *__restrict__ su,
    const float *__restrict__ sB, const float *__restrict__ sdt,
    const int32_t *__restrict__ accepted, const int32_t *__restrict__ idx, const ReplayShape sh)
{
    constexpr int VEC = SV<ST>::VEC;
    constexpr int LPR = NS / VEC;
    constexpr int RPW = 64 / LPR;
    constexpr int RPP = 4 * RPW;

    const int tile = blockIdx.x;
    const int b = tile / sh.nheads;
    const int h = tile - b * sh.nheads;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (LPR - 1);
    const int rsub = (threadIdx.x >> 6) * RPW + lane / LPR;

    const int row = idx ? idx[b] : b;
    const int k = min(accepted[b], sh.seq_len);
    if (row < 0 || k <= 0)
        return;
    const int g = h / sh.heads_per_group;
    const int H = sh.nheads, Dm = sh.dim;
    const int64_t bT = (int64_t)b * sh.seq_len;
    ST *tp = state + (int64_t)row * sh.row_stride + (int64_t)h * Dm * NS + sub * VEC;

    for (int r0 = 0; r0 < Dm; r0 += PASSES * RPP) {
        float s[PASSES][VEC];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = r0 + p * RPP + rsub;
            const u32x4 w = r < Dm ? *reinterpret_cast<const u32x4 *>(tp + (int64_t)r * NS)
                                   : u32x4{0u, 0u, 0u, 0u};
            SV<ST>::unpack(w, s[p]);
        }
        for (int t = 0; t < k; ++t) {
            const int64_t bth = (bT + t) * H + h;
            const float a = expf(sdA[bth]);
            const float dtv = sdt[bth];
            float bv[VEC];
            ld_vec<VEC>(sB, ((bT + t) * sh.ngroups + g) * NS + sub * VEC, kF32, bv);
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int r = r0 + p * RPP + rsub;
                const float dtx = dtv * (r < Dm ? su[bth * Dm + r] : 0.0f);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    s[p][e] = fmaf(dtx, bv[e], s[p][e] * a);
            }
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = r0 + p * RPP + rsub;
            if (r < Dm)
                *reinterpret_cast<u32x4 *>(tp + (int64_t)r * NS) = SV<ST>::pack(s[p]);
        }
    }
}

template <typename ST, int NS>
hipError_t launch_ns(const ReplayParams &p, hipStream_t stream)
{
    constexpr int VEC = SV<ST>::VEC;
    constexpr int RPP = 4 * (64 / (NS / VEC));
    const int need = (p.dim + RPP - 1) / RPP;
    ReplayShape sh;
    sh.row_stride = p.row_stride;
    sh.seq_len = p.seq_len;
    sh.nheads = p.nheads;
    sh.dim = p.dim;
    sh.ngroups = p.ngroups;
    sh.heads_per_group = p.nheads / p.ngroups;
    const dim3 grid((unsigned)((int64_t)p.active_batch * p.nheads));
    ST *st = static_cast<ST *>(p.state);
    (void)hipGetLastError();
#define SSU_LAUNCH_REPLAY(PS)                                                                  \
    hipLaunchKernelGGL((ssu_replay_kernel<ST, NS, PS>), grid, dim3(256), 0, stream, st, p.dA, \
                       p.u, p.B, p.dt, p.accepted, p.idx, sh)
    if (need >= 8)
        SSU_LAUNCH_REPLAY(8);
    else if (need >= 4)
        SSU_LAUNCH_REPLAY(4);
    else if (need >= 2)
        SSU_LAUNCH_REPLAY(2);
    else
        SSU_LAUNCH_REPLAY(1);
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
