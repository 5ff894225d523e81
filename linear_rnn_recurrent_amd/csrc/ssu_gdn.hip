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
// each, interleaved in 16-byte chunks so that every non-temporal vector load
// or store covers whole cache lines), four rows per wave, 16 rows
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

struct GdnShape {
    int64_t ssm_row_stride, cs_slot, cs_chan, cs_tap;
    int32_t hidden, hq, hv, width, use_l2, G;
    float scale;
};

// The G (a power of two) consecutive bf16 weights of one head group in one
// projection row, as one load of 2 G bytes.
template <int GM> struct BaChunk;
template <> struct BaChunk<1> { typedef uint16_t T; };
template <> struct BaChunk<2> { typedef uint32_t T; };
template <> struct BaChunk<4> { typedef u32x2 T; };
template <> struct BaChunk<8> { typedef u32x4 T; };

template <int GM, int G>
__device__ __forceinline__ float ba_col(const typename BaChunk<GM>::T &w)
{
    if constexpr (GM == 1) {
        return bf16_to_f32(w);
    } else if constexpr (GM == 2) {
        return G == 0 ? __uint_as_float(w << 16) : __uint_as_float(w & 0xFFFF0000u);
    } else {
        const uint32_t x = w[G / 2];
        return (G & 1) ? __uint_as_float(x & 0xFFFF0000u) : __uint_as_float(x << 16);
    }
}

// A state row of D = 16 EPL fp32 is spread over 16 lanes. Column layout: a
// lane's e-th float is column col_of(l16, e); for EPL >= 4 its k-th 16-byte
// vector holds columns 64 k + 4 l16 .. + 3, so the 16 lanes of a row cover
// 256 consecutive bytes with each vector load or store (whole cache lines);
// for EPL = 2 a lane holds columns 2 l16, 2 l16 + 1.
template <int EPL>
__device__ __forceinline__ int col_of(int l16, int e)
{
    return EPL >= 4 ? (e / 4) * 64 + l16 * 4 + (e % 4) : l16 * 2 + e;
}

// p: the row's first element plus the lane's base offset lane_off<EPL>(l16)
template <int EPL>
__device__ __forceinline__ int lane_off(int l16) { return EPL >= 4 ? l16 * 4 : l16 * 2; }

template <int EPL>
__device__ __forceinline__ void ld_row(const float *p, float (&x)[EPL])
{
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + e * 16));
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
                reinterpret_cast<u32x4 *>(p + e * 16));
    } else {
        __builtin_nontemporal_store(u32x2{__float_as_uint(x[0]), __float_as_uint(x[1])},
                                    reinterpret_cast<u32x2 *>(p));
    }
}

// Workgroups per CU the register budget is held to: four keep a B = 64,
// Hq = 16 launch (1024 workgroups) resident in one round; the wide-window and
// D = 64, G = 8 variants need more registers than that allows.
template <int D, int GM, int WM>
constexpr int gdn_min_blocks() { return (WM > 4 || (D == 64 && GM == 8)) ? 1 : 4; }

// D: head dim; GM: value heads per q/k head (G = GM, a power of two); WM: conv width bound (the runtime width W <= WM; WM = 1
// exactly when W = 1, so the other instantiations always have a tap to read).
template <int D, int GM, int WM>
__global__ __launch_bounds__(kGdnNT, (gdn_min_blocks<D, GM, WM>())) void ssu_gdn_kernel(
    const uint16_t *__restrict__ hs, const uint16_t *__restrict__ w_ba,
    const uint16_t *__restrict__ mixed_qkv, const uint16_t *__restrict__ conv_w,
    const uint16_t *__restrict__ conv_b, uint16_t *__restrict__ conv_state,
    const float *__restrict__ A_log, const uint16_t *__restrict__ dt_bias, float *__restrict__ ssm,
    const int32_t *__restrict__ idx, uint16_t *__restrict__ out, const GdnShape sh)
{
    constexpr int NT = kGdnNT;
    constexpr int EPL = D / 16;                             // state columns per lane
    constexpr int PF = EPL >= 16 ? 2 : (EPL >= 8 ? 4 : 8);  // passes of loads in flight
    constexpr int KV = GM <= 2 ? 16 : (GM == 4 ? 8 : 4);     // projection rows per lane per batch
    constexpr int CPT = ((2 + GM) * D + NT - 1) / NT;       // owned channels per thread (bound)
    constexpr int CB = CPT < 2 ? CPT : 2;                   // channels per load batch
    constexpr int NTAP = WM > 1 ? WM - 1 : 1;
    constexpr int NRED = 2 * GM + 2;                        // b, a dots; |q|^2, |k|^2
    __shared__ float ych[(2 + GM) * D];                     // conv outputs: q | k | v of G heads
    __shared__ float red[NT / 64][NRED];                    // per-wave partial sums

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int G = GM;
    const int Hq = sh.hq, HV = sh.hv, W = sh.width, hidden = sh.hidden;
    const int b = blockIdx.x / Hq;
    const int h = blockIdx.x - b * Hq;
    const int hv0 = h * G;
    const int nch = (2 + G) * D;
    const int HD = Hq * D;
    const int s = idx[b];
    const int64_t out0 = ((int64_t)b * HV + hv0) * D;

    if (s < 0) {  // padding entry (uniform over the workgroup): no pool access, zero output
        for (int i = tid; i < G * D; i += NT)
            out[out0 + i] = 0;
        return;
    }

    // ---- issue every setup load before any use: b/a rows, conv inputs ----
    const uint16_t *hsb = hs + (int64_t)b * hidden;
    const int64_t wrow = 2 * (int64_t)HV;
    // Lane pairs share a projection row (one cache line): the even lane reads
    // the G beta-gate weights of this head group, the odd lane the G decay
    // weights, each as one chunk.
    typedef typename BaChunk<GM>::T WT;
    const int part = tid & 1;
    const int rlane = tid >> 1;
    uint32_t hx[KV];
    WT wv[KV];
    auto load_ba = [&](int i0) {
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int ic = min(i0 + rlane + (NT / 2) * k, hidden - 1);
            hx[k] = hsb[ic];
            wv[k] = *reinterpret_cast<const WT *>(w_ba + ic * wrow + part * HV + hv0);
        }
    };
    float acc[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g)
        acc[g] = 0.0f;
    auto fma_ba = [&](int i0) {
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const float x = (i0 + rlane + (NT / 2) * k < hidden) ? bf16_to_f32(hx[k]) : 0.0f;
            acc[0] = fmaf(x, ba_col<GM, 0>(wv[k]), acc[0]);
            if constexpr (GM > 1)
                acc[1] = fmaf(x, ba_col<GM, 1>(wv[k]), acc[1]);
            if constexpr (GM > 2) {
                acc[2] = fmaf(x, ba_col<GM, 2>(wv[k]), acc[2]);
                acc[3] = fmaf(x, ba_col<GM, 3>(wv[k]), acc[3]);
            }
            if constexpr (GM > 4) {
                acc[4] = fmaf(x, ba_col<GM, 4>(wv[k]), acc[4]);
                acc[5] = fmaf(x, ba_col<GM, 5>(wv[k]), acc[5]);
                acc[6] = fmaf(x, ba_col<GM, 6>(wv[k]), acc[6]);
                acc[7] = fmaf(x, ba_col<GM, 7>(wv[k]), acc[7]);
            }
        }
    };
    auto chan = [&](int j) {
        return j < D ? h * D + j : (j < 2 * D ? HD + h * D + (j - D) : 2 * HD + hv0 * D + (j - 2 * D));
    };
    const int64_t qkv_dim = 2 * (int64_t)HD + (int64_t)HV * D;
    uint32_t cbias[CB], cx[CB], cwt[CB][WM], ctap[CB][NTAP];
    auto load_conv = [&](int j0) {
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            const int c = chan(min(j0 + tid + NT * k, nch - 1));
            cbias[k] = conv_b[c];
            cx[k] = mixed_qkv[b * qkv_dim + c];
#pragma unroll
            for (int t = 0; t < WM; ++t)
                cwt[k][t] = conv_w[(int64_t)c * W + min(t, W - 1)];
            if constexpr (WM > 1) {  // here W >= 2: every tap index is in the pool
                const uint16_t *cs = conv_state + (int64_t)s * sh.cs_slot + (int64_t)c * sh.cs_chan;
#pragma unroll
                for (int t = 0; t < NTAP; ++t)
                    ctap[k][t] = cs[min(t, W - 2) * sh.cs_tap];
            }
        }
    };
    float ssq = 0.0f, ssk = 0.0f;
    auto conv_step = [&](int j0) {
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            const int j = j0 + tid + NT * k;
            if (j < nch) {
                const int c = chan(j);
                float y = bf16_to_f32(cbias[k]);
                float wl = 0.0f;
#pragma unroll
                for (int t = 0; t < WM; ++t) {
                    if (WM > 1 && t < W - 1 && t < NTAP)
                        y = fmaf(bf16_to_f32(ctap[k][t < NTAP ? t : 0]), bf16_to_f32(cwt[k][t]), y);
                    if (t == W - 1)
                        wl = bf16_to_f32(cwt[k][t]);
                }
                y = fmaf(bf16_to_f32(cx[k]), wl, y);
                // the pool keeps the last W-1 raw inputs: tap t <- tap t+1, newest last
                if constexpr (WM > 1) {
                    uint16_t *cs = conv_state + (int64_t)s * sh.cs_slot + (int64_t)c * sh.cs_chan;
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) {
                        if (t < W - 1) {
                            const uint32_t v = (t + 1 < NTAP && t + 1 < W - 1)
                                                   ? ctap[k][t + 1 < NTAP ? t + 1 : 0]
                                                   : cx[k];
                            cs[t * sh.cs_tap] = (uint16_t)v;
                        }
                    }
                }
                const float ys = silu_f32(y);
                ych[j] = ys;
                const float y2 = ys * ys;
                ssq += j < D ? y2 : 0.0f;
                ssk += (j >= D && j < 2 * D) ? y2 : 0.0f;
            }
        }
    };
    load_conv(0);  // pool taps first: they come from HBM, the projection from cache
    load_ba(0);

    // ---- then the first passes of state loads: in flight during the setup math ----
    const int l16 = lane & 15;
    const int rsub = wave * 4 + (lane >> 4);  // row within a 16-row pass
    const int NP = G * D / 16;                // passes
    float *ssm_h = ssm + (int64_t)s * sh.ssm_row_stride + (int64_t)hv0 * D * D + lane_off<EPL>(l16);
    auto row_ptr = [&](int p) { return ssm_h + (int64_t)(16 * p + rsub) * D; };
    float cur[PF][EPL];
    // vmcnt retires in order: the state loads go strictly after the setup
    // loads, so waiting for a setup value never waits for the state
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < PF; ++k)
        ld_row<EPL>(row_ptr(min(k, NP - 1)), cur[k]);
    __builtin_amdgcn_sched_barrier(0);

    fma_ba(0);
    for (int i0 = (NT / 2) * KV; i0 < hidden; i0 += (NT / 2) * KV) {
        load_ba(i0);
        fma_ba(i0);
    }
    conv_step(0);
    for (int j0 = NT * CB; j0 < nch; j0 += NT * CB) {
        load_conv(j0);
        conv_step(j0);
    }

    // ---- one exchange: per-wave partial sums; every wave finishes them itself ----
    {
        float red_w[NRED];
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            red_w[g] = wave_sum(part ? 0.0f : acc[g]);       // beta-gate input
            red_w[GM + g] = wave_sum(part ? acc[g] : 0.0f);  // decay input
        }
        red_w[2 * GM] = wave_sum(ssq);
        red_w[2 * GM + 1] = wave_sum(ssk);
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < NRED; ++i)
                red[wave][i] = red_w[i];
        }
    }
    __syncthreads();
    float alpha[GM], beta[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        const float bb = (red[0][g] + red[1][g]) + (red[2][g] + red[3][g]);
        const float aa = (red[0][GM + g] + red[1][GM + g]) + (red[2][GM + g] + red[3][GM + g]);
        const int hh = hv0 + g;
        const float sp = softplus_f32(aa + bf16_to_f32(dt_bias[hh]));
        alpha[g] = expf(-expf(A_log[hh]) * sp);
        beta[g] = 1.0f / (1.0f + expf(-bb));
    }
    float qv[EPL], kv[EPL];
    {
        const float sq = (red[0][2 * GM] + red[1][2 * GM]) + (red[2][2 * GM] + red[3][2 * GM]);
        const float sk =
            (red[0][2 * GM + 1] + red[1][2 * GM + 1]) + (red[2][2 * GM + 1] + red[3][2 * GM + 1]);
        const float iq = (sh.use_l2 ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) * sh.scale;
        const float ik = sh.use_l2 ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qv[e] = ych[col_of<EPL>(l16, e)] * iq;
            kv[e] = ych[D + col_of<EPL>(l16, e)] * ik;
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
                const int g = p / (D / 16);           // value head of this pass (uniform)
                const int v = 16 * (p - g * (D / 16)) + rsub;
                float al = alpha[0], be = beta[0];
#pragma unroll
                for (int gg = 1; gg < GM; ++gg) {
                    if (g == gg) {
                        al = alpha[gg];
                        be = beta[gg];
                    }
                }
                float pk = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    cur[k][e] *= al;
                    pk = fmaf(cur[k][e], kv[e], pk);
                }
                pk = row_group_sum<16>(pk);
                const float delta = be * (ych[(2 + g) * D + v] - pk);
                float po = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    cur[k][e] = fmaf(delta, kv[e], cur[k][e]);
                    po = fmaf(cur[k][e], qv[e], po);
                }
                po = row_group_sum<16>(po);
                st_row<EPL>(row_ptr(p), cur[k]);
                if (l16 == 0)
                    out[out0 + g * D + v] = (uint16_t)f32_to_bf16(po);
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

template <int D, int GM, int WM>
hipError_t launch_dgw(const GdnParams &p, const GdnShape &sh, hipStream_t stream)
{
    const int64_t blocks = (int64_t)p.batch * p.hq;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    (void)hipGetLastError();
    hipLaunchKernelGGL((ssu_gdn_kernel<D, GM, WM>), dim3((unsigned)blocks), dim3(kGdnNT), 0,
                       stream, static_cast<const uint16_t *>(p.hs),
                       static_cast<const uint16_t *>(p.w_ba), static_cast<const uint16_t *>(p.qkv),
                       static_cast<const uint16_t *>(p.conv_w),
                       static_cast<const uint16_t *>(p.conv_b),
                       static_cast<uint16_t *>(p.conv_state), p.A_log,
                       static_cast<const uint16_t *>(p.dt_bias), p.ssm, p.idx,
                       static_cast<uint16_t *>(p.out), sh);
    return hipGetLastError();
}

template <int D, int GM>
hipError_t launch_dg(const GdnParams &p, const GdnShape &sh, hipStream_t stream)
{
    if (p.width == 1)
        return launch_dgw<D, GM, 1>(p, sh, stream);
    return p.width <= 4 ? launch_dgw<D, GM, 4>(p, sh, stream) : launch_dgw<D, GM, 8>(p, sh, stream);
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
    switch (sh.G) {
    case 1: return launch_dg<D, 1>(p, sh, stream);
    case 2: return launch_dg<D, 2>(p, sh, stream);
    case 4: return launch_dg<D, 4>(p, sh, stream);
    case 8: return launch_dg<D, 8>(p, sh, stream);
    default: return hipErrorInvalidValue;
    }
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
