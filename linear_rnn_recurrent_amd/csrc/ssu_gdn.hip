// Fused gated-delta-rule decode step over paged conv / ssm pools.
//
// Operation (FlashInfer, "flashinfer.gdn_fused_decode_step" page): per batch
// entry, the b/a projection GEMV, the causal conv1d update, the q/k/v split and
// the gated delta-rule decode with qk-L2-norm; both pools updated in place;
// negative state_indices are padding entries (no pool access, zero output).
// The formulas (the page names the steps only) are those stated in ssu.h.
//
// Mapping on gfx950. One 256-thread workgroup per (batch entry, q/k head h)
// owns every channel that head's outputs depend on: the D q and D k channels
// of h and the D v channels of each of its G = HV/Hq value heads, so each
// conv-state channel is read and written by exactly one workgroup. The state
// of the G value heads (G x D x D fp32, 128 KiB at D = 128, G = 2) dominates
// the traffic and is streamed once: 16 lanes per state row (D/16 columns
// each, 16-byte non-temporal loads and stores), four rows per wave, 16 rows
// per workgroup pass. The first passes' loads are issued before anything
// else, so they are in flight while the workgroup does its setup (the b/a
// dot products for its G value heads, the conv update of its (2+G) D
// channels, the q/k norms); later passes are prefetched a group of passes
// ahead. Per row: decay, the prediction S.k, the delta update, the output S.q
// -- the two row dots summed over the 16 lanes with DPP.
#include "ssu_device.h"
#include "ssu_dpp.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

constexpr int kGdnNT = 256;
constexpr int kGdnMaxG = 8;  // value heads per q/k head held in LDS

struct GdnShape {
    int64_t ssm_row_stride, cs_slot, cs_chan, cs_tap;
    int32_t hidden, hq, hv, width, use_l2, G;
    float scale;
};

__device__ __forceinline__ float bf16v(const void *p, int64_t i)
{
    return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}

template <int EPL>
__device__ __forceinline__ void ld_row(const float *p, float (&x)[EPL])
{
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + e));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[e + j] = __uint_as_float(w[j]);
        }
    } else {
        static_assert(EPL == 2, "rows split into 2, 4, 8 or 16 columns per lane");
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        x[0] = __uint_as_float(w[0]);
        x[1] = __uint_as_float(w[1]);
    }
}

template <int EPL>
__device__ __forceinline__ void st_row(float *p, const float (&x)[EPL])
{
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
            __builtin_nontemporal_store(
                u32x4{__float_as_uint(x[e]), __float_as_uint(x[e + 1]), __float_as_uint(x[e + 2]),
                      __float_as_uint(x[e + 3])},
                reinterpret_cast<u32x4 *>(p + e));
    } else {
        __builtin_nontemporal_store(u32x2{__float_as_uint(x[0]), __float_as_uint(x[1])},
                                    reinterpret_cast<u32x2 *>(p));
    }
}

template <int D>
__global__ __launch_bounds__(kGdnNT) void ssu_gdn_kernel(
    const void *__restrict__ hidden_states, const void *__restrict__ w_ba,
    const void *__restrict__ mixed_qkv, const void *__restrict__ conv_w,
    const void *__restrict__ conv_b, uint16_t *__restrict__ conv_state,
    const float *__restrict__ A_log, const void *__restrict__ dt_bias, float *__restrict__ ssm,
    const int32_t *__restrict__ idx, uint16_t *__restrict__ out, const GdnShape sh)
{
    constexpr int NT = kGdnNT;
    constexpr int EPL = D / 16;                             // state columns per lane
    constexpr int PF = EPL >= 16 ? 2 : (EPL >= 8 ? 4 : 8);  // passes of loads in flight
    __shared__ float ych[(2 + kGdnMaxG) * D];   // conv outputs: q | k | v of G heads
    __shared__ float red[4][2 * kGdnMaxG];      // per-wave partial b/a dots
    __shared__ float gates[2 * kGdnMaxG];       // alpha | beta per value head
    __shared__ float qk_inv[2];                 // norms of q and k (inverse)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = sh.G;
    const int Hq = sh.hq, HV = sh.hv, W = sh.width;
    const int b = blockIdx.x / Hq;
    const int h = blockIdx.x - b * Hq;
    const int hv0 = h * G;
    const int s = idx[b];
    const int64_t out0 = ((int64_t)b * HV + hv0) * D;

    if (s < 0) {  // padding entry: no pool access, zero output
        for (int i = tid; i < G * D; i += NT)
            out[out0 + i] = 0;
        return;
    }

    // ---- the first passes of state loads, before any setup ----
    const int l16 = lane & 15;
    const int rsub = wave * 4 + (lane >> 4);  // row within a 16-row pass
    const int NP = G * D / 16;                // passes
    float *ssm_h = ssm + (int64_t)s * sh.ssm_row_stride + (int64_t)hv0 * D * D + l16 * EPL;
    auto row_ptr = [&](int p) { return ssm_h + (int64_t)(16 * p + rsub) * D; };
    float cur[PF][EPL];
#pragma unroll
    for (int k = 0; k < PF; ++k)
        ld_row<EPL>(row_ptr(min(k, NP - 1)), cur[k]);

    // ---- setup: b/a dots, conv update, q/k norms ----
    {
        const int HD = Hq * D;
        float acc[2 * kGdnMaxG];
#pragma unroll
        for (int g = 0; g < 2 * kGdnMaxG; ++g)
            acc[g] = 0.0f;
        for (int i = tid; i < sh.hidden; i += NT) {
            const float hx = bf16v(hidden_states, (int64_t)b * sh.hidden + i);
            const int64_t wrow = (int64_t)i * 2 * HV;
#pragma unroll
            for (int g = 0; g < kGdnMaxG; ++g) {
                if (g < G) {
                    acc[g] = fmaf(hx, bf16v(w_ba, wrow + hv0 + g), acc[g]);
                    acc[kGdnMaxG + g] = fmaf(hx, bf16v(w_ba, wrow + HV + hv0 + g), acc[kGdnMaxG + g]);
                }
            }
        }
        // channels owned: q of h, k of h, v of the G value heads
        for (int j = tid; j < (2 + G) * D; j += NT) {
            const int c = j < D ? h * D + j : (j < 2 * D ? HD + h * D + (j - D) : 2 * HD + hv0 * D + (j - 2 * D));
            uint16_t *cs = conv_state + (int64_t)s * sh.cs_slot + (int64_t)c * sh.cs_chan;
            float y = bf16v(conv_b, c);
            const int64_t cw = (int64_t)c * W;
            for (int t = 0; t < W - 1; ++t) {
                const uint16_t raw = cs[t * sh.cs_tap];
                y = fmaf(bf16_to_f32(raw), bf16v(conv_w, cw + t), y);
                if (t > 0)
                    cs[(t - 1) * sh.cs_tap] = raw;  // shift: tap t-1 <- tap t
            }
            const uint16_t xnew = static_cast<const uint16_t *>(mixed_qkv)[(int64_t)b * (2 * HD + HV * D) + c];
            y = fmaf(bf16_to_f32(xnew), bf16v(conv_w, cw + W - 1), y);
            if (W > 1)
                cs[(W - 2) * sh.cs_tap] = xnew;
            ych[j] = silu_f32(y);
        }
        // wave partials of the b/a dots
#pragma unroll
        for (int g = 0; g < 2 * kGdnMaxG; ++g) {
            float v = acc[g];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1)
                v += __shfl_xor(v, m, 64);
            if (lane == 0)
                red[wave][g] = v;
        }
    }
    __syncthreads();
    if (wave == 0) {
        if (lane < G) {
            const float bb = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
            const float aa = (red[0][kGdnMaxG + lane] + red[1][kGdnMaxG + lane]) +
                             (red[2][kGdnMaxG + lane] + red[3][kGdnMaxG + lane]);
            const int hh = hv0 + lane;
            const float sp = softplus_f32(aa + bf16v(dt_bias, hh));
            gates[lane] = expf(-expf(A_log[hh]) * sp);   // alpha
            gates[kGdnMaxG + lane] = 1.0f / (1.0f + expf(-bb));  // beta
        }
    } else if (wave <= 2) {  // wave 1: |q|, wave 2: |k|
        const float *x = ych + (wave - 1) * D;
        float ss = 0.0f;
        for (int i = lane; i < D; i += 64)
            ss = fmaf(x[i], x[i], ss);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1)
            ss += __shfl_xor(ss, m, 64);
        if (lane == 0)
            qk_inv[wave - 1] = sh.use_l2 ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
    }
    __syncthreads();

    // this lane's slices of q (normalised, scaled) and k (normalised)
    float qv[EPL], kv[EPL];
    {
        const float iq = qk_inv[0] * sh.scale, ik = qk_inv[1];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qv[e] = ych[l16 * EPL + e] * iq;
            kv[e] = ych[D + l16 * EPL + e] * ik;
        }
    }

    // ---- stream the state: PF passes at a time, the next group in flight ----
    for (int p0 = 0; p0 < NP; p0 += PF) {
        float nxt[PF][EPL];
        const bool more = p0 + PF < NP;
        if (more) {
#pragma unroll
            for (int k = 0; k < PF; ++k)
                ld_row<EPL>(row_ptr(min(p0 + PF + k, NP - 1)), nxt[k]);
        }
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int p = p0 + k;
            if (p < NP) {
                const int r = 16 * p + rsub;   // row over the G heads
                const int g = r / D;
                const int v = r - g * D;
                const float alpha = gates[g], beta = gates[kGdnMaxG + g];
                float pk = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    cur[k][e] *= alpha;
                    pk = fmaf(cur[k][e], kv[e], pk);
                }
                pk = row_group_sum<16>(pk);
                const float delta = beta * (ych[(2 + g) * D + v] - pk);
                float po = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    cur[k][e] = fmaf(delta, kv[e], cur[k][e]);
                    po = fmaf(cur[k][e], qv[e], po);
                }
                po = row_group_sum<16>(po);
                st_row<EPL>(row_ptr(p), cur[k]);
                if (l16 == 0)
                    out[out0 + r] = (uint16_t)f32_to_bf16(po);
            }
        }
        if (more) {
#pragma unroll
            for (int k = 0; k < PF; ++k)
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    cur[k][e] = nxt[k][e];
        }
    }
}

template <int D>
hipError_t launch_d(const GdnParams &p, hipStream_t stream)
{
    GdnShape sh;
    sh.ssm_row_stride = p.ssm_row_stride;
    sh.cs_slot = p.cs_slot;
    sh.cs_chan = p.cs_chan;
    sh.cs_tap = p.cs_tap;
    sh.hidden = p.hidden;
    sh.hq = p.hq;
    sh.hv = p.hv;
    sh.width = p.width;
    sh.use_l2 = p.use_l2;
    sh.G = p.hv / p.hq;
    sh.scale = p.scale;
    const int64_t blocks = (int64_t)p.batch * p.hq;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    (void)hipGetLastError();
    hipLaunchKernelGGL((ssu_gdn_kernel<D>), dim3((unsigned)blocks), dim3(kGdnNT), 0, stream,
                       p.hs, p.w_ba, p.qkv, p.conv_w, p.conv_b,
                       static_cast<uint16_t *>(p.conv_state), p.A_log, p.dt_bias, p.ssm, p.idx,
                       static_cast<uint16_t *>(p.out), sh);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn(const GdnParams &p, hipStream_t stream)
{
    if (p.batch == 0)
        return hipSuccess;
    switch (p.dhead) {
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 256: return launch_d<256>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
