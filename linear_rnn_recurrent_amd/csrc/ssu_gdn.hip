// Fused gated-delta-rule decode step over paged conv / ssm pools.
//
// Operation (FlashInfer, "flashinfer.gdn_fused_decode_step" page): per batch
// entry, the b/a projection GEMV, the causal conv1d update, the q/k/v split and
// the gated delta-rule decode with qk-L2-norm; both pools updated in place;
// negative state_indices are padding entries (no pool access, zero output).
// The formulas (the page names the steps only) are those stated in ssu.h.
//
// Mapping on gfx950: two launches on the caller's stream.
//
// 1. gdn_prep: everything but the state. Workgroup (b, h) of the first B*Hq
//    owns every conv channel that q/k head h's outputs depend on (its D q and
//    D k channels and the D v channels of its G = HV/Hq value heads), so each
//    conv-state channel is read, shifted and written by exactly one thread;
//    it also takes the q/k L2 norms and writes q*scale/|q|, k/|k| and v to the
//    workspace (at width 4 on a dense channel-major pool a thread takes two
//    adjacent channels as 32-bit words). The remaining workgroups, one per (b, chunk of 256 hidden
//    rows), compute partial sums of the b/a projection (hidden x 2HV) over
//    their rows, reading the weight in whole rows (it is [hidden, 2HV]
//    row-major: a per-head column slice would touch a cache line per row for
//    a few useful bytes), one round of loads per thread.
// 2. gdn_stream: the state, all but a few percent of the bytes. Every wave is
//    independent (no barrier, no LDS): it owns a few rows of one value head's
//    D x D fp32 state, 16 lanes per row (8 below D = 128; at D = 128 its 16 KiB
//    of state per workgroup measured faster than 32 or 8) with the columns
//    interleaved in 16-byte chunks so that every non-temporal vector load or
//    store covers whole cache lines; it issues its state loads first, then
//    reads its q/k slices, v values and the b/a partial sums from the
//    workspace (cache hits), forms its head's gates, and per row applies decay,
//    prediction, delta update and output (row dots summed over the row's lanes
//    with DPP).
// Splitting the step in two lets the state stream run as many small,
// barrier-free waves that the dispatcher overlaps freely; in one launch each
// workgroup had to finish its latency-bound setup before streaming, and the
// workgroups sharing a CU spent much of the launch out of phase.
#include "ssu_device.h"
#include "ssu_dpp.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

constexpr int kGdnNT = 256;
constexpr int kProjRows = 256;  // hidden rows per projection workgroup

struct GdnPrepShape {
    int64_t cs_slot, cs_chan, cs_tap;
    int32_t batch, hidden, hq, hv, width, use_l2, proj_vec, nck;
    float scale;
};

// Workspace layout (fp32): qk [B][Hq][2][D] (q*scale/|q|, k/|k|), v [B][HV][D],
// part [B][NCK][2HV] (b/a projection partial sums per chunk of 256 rows).
__host__ __device__ inline int64_t ws_v_off(int64_t B, int64_t hq, int64_t d) { return B * hq * 2 * d; }
__host__ __device__ inline int64_t ws_p_off(int64_t B, int64_t hq, int64_t hv, int64_t d)
{
    return ws_v_off(B, hq, d) + B * hv * d;
}

// ---------------------------------------------------------------------------
// gdn_prep, b/a projection role: workgroup (b, chunk ck of 256 hidden rows),
// all 2HV columns. Thread t owns column chunk cc = t % NCH (CWC columns, one
// 16- or 4-byte load per row) and row phase rp = t / NCH; the partial sums are
// combined over the row phases through LDS and written per chunk.
// ---------------------------------------------------------------------------
// CWC bf16 weights of one row as raw words (loaded), then as floats
template <int CWC>
__device__ __forceinline__ void proj_load(const uint16_t *p, uint32_t (&v)[CWC / 2])
{
    if constexpr (CWC == 8) {
        const u32x4 q = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = q[j];
    } else {
        v[0] = *reinterpret_cast<const uint32_t *>(p);
    }
}

template <int CWC>
__device__ __forceinline__ void proj_cvt(const uint32_t (&v)[CWC / 2], float (&w)[CWC])
{
#pragma unroll
    for (int j = 0; j < CWC / 2; ++j) {
        w[2 * j] = __uint_as_float(v[j] << 16);
        w[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
    }
}

template <int CWC>
__device__ void gdn_projection(int b, int ck, const uint16_t *__restrict__ hs,
                               const uint16_t *__restrict__ w_ba, float *__restrict__ part_out,
                               const GdnPrepShape &sh, float *lds)
{
    constexpr int NT = kGdnNT;
    constexpr int U = 8;             // rows in flight per thread
    const int tid = threadIdx.x;
    const int NC = 2 * sh.hv;
    const int NCH = NC / CWC;        // column chunks (<= NT)
    const int RPH = NT / NCH;        // row phases
    const int cc = tid % NCH, rp = tid / NCH;
    const bool active = rp < RPH;
    const int r0 = ck * kProjRows;
    const int cn = min(kProjRows, sh.hidden - r0);
    float *hid = lds;                // this chunk's hidden values
    float *part = lds + kProjRows;   // [RPH][NC] partial sums
    const uint16_t *wb = w_ba + (int64_t)r0 * NC + cc * CWC;
    // the first U weight rows are loaded before the hidden values are staged
    // (they do not depend on them), so both loads are in flight together
    uint32_t wr[U][CWC / 2];
    auto load_rows = [&](int ra) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            proj_load<CWC>(wb + (int64_t)min(ra + u * RPH, cn - 1) * NC, wr[u]);
    };
    const uint16_t hval = hs[(int64_t)b * sh.hidden + r0 + min(tid, cn - 1)];
    load_rows(rp);  // rows clamped: in bounds for every thread
    if (tid < cn)
        hid[tid] = bf16_to_f32(hval);
    float acc[CWC];
#pragma unroll
    for (int j = 0; j < CWC; ++j)
        acc[j] = 0.0f;
    __syncthreads();
    if (active) {
        for (int ra = rp; ra < cn; ra += U * RPH) {
            if (ra != rp)
                load_rows(ra);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = ra + u * RPH;
                const float x = r < cn ? hid[r] : 0.0f;
                float w[CWC];
                proj_cvt<CWC>(wr[u], w);
#pragma unroll
                for (int j = 0; j < CWC; ++j)
                    acc[j] = fmaf(x, w[j], acc[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < CWC; ++j)
            part[rp * NC + cc * CWC + j] = acc[j];
    }
    __syncthreads();
    for (int t = tid; t < NC; t += NT) {
        float v = 0.0f;
        for (int r = 0; r < RPH; ++r)
            v += part[r * NC + t];
        part_out[((int64_t)b * sh.nck + ck) * NC + t] = v;
    }
}

// ---------------------------------------------------------------------------
// gdn_prep, conv role: workgroup (b, h). D: head dim; GM: G (a power of two);
// WM: conv width bound (W <= WM; WM = 1 exactly when W = 1, so the other
// instantiations always have a tap to read).
// ---------------------------------------------------------------------------
template <int D, int GM, int WM>
__device__ void gdn_conv(int b, int h, const uint16_t *__restrict__ mixed_qkv,
                         const uint16_t *__restrict__ conv_w, const uint16_t *__restrict__ conv_b,
                         uint16_t *__restrict__ conv_state, int s, float *__restrict__ ws,
                         const GdnPrepShape &sh, float *lds)
{
    constexpr int NT = kGdnNT;
    constexpr int G = GM;
    constexpr int NCH = (2 + G) * D;          // owned channels
    constexpr int CPT = (NCH + NT - 1) / NT;  // channels per thread
    constexpr int NTAP = WM > 1 ? WM - 1 : 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int Hq = sh.hq, HV = sh.hv, W = sh.width;
    const int hv0 = h * G;
    const int HD = Hq * D;
    const int64_t qkv_dim = 2 * (int64_t)HD + (int64_t)HV * D;
    auto chan = [&](int j) {
        return j < D ? h * D + j : (j < 2 * D ? HD + h * D + (j - D) : 2 * HD + hv0 * D + (j - 2 * D));
    };
    // every load first (pool taps from HBM, the rest from cache), then the math
    uint32_t cbias[CPT], cx[CPT], cwt[CPT][WM], ctap[CPT][NTAP];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int c = chan(min(tid + NT * k, NCH - 1));
        if constexpr (WM > 1) {  // here W >= 2: every tap index is in the pool
            const uint16_t *cs = conv_state + (int64_t)s * sh.cs_slot + (int64_t)c * sh.cs_chan;
#pragma unroll
            for (int t = 0; t < NTAP; ++t)
                ctap[k][t] = cs[min(t, W - 2) * sh.cs_tap];
        }
        cbias[k] = conv_b[c];
        cx[k] = mixed_qkv[b * qkv_dim + c];
#pragma unroll
        for (int t = 0; t < WM; ++t)
            cwt[k][t] = conv_w[(int64_t)c * W + min(t, W - 1)];
    }
    float y[CPT];
    float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int j = tid + NT * k;
        float acc = bf16_to_f32(cbias[k]);
        float wl = 0.0f;
#pragma unroll
        for (int t = 0; t < WM; ++t) {
            if (WM > 1 && t < W - 1 && t < NTAP)
                acc = fmaf(bf16_to_f32(ctap[k][t < NTAP ? t : 0]), bf16_to_f32(cwt[k][t]), acc);
            if (t == W - 1)
                wl = bf16_to_f32(cwt[k][t]);
        }
        acc = fmaf(bf16_to_f32(cx[k]), wl, acc);
        y[k] = silu_f32(acc);
        if (j < NCH) {
            // the pool keeps the last W-1 raw inputs: tap t <- tap t+1, newest last
            if constexpr (WM > 1) {
                uint16_t *cs = conv_state + (int64_t)s * sh.cs_slot + (int64_t)chan(j) * sh.cs_chan;
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
            const float y2 = y[k] * y[k];
            ssq += j < D ? y2 : 0.0f;
            ssk += (j >= D && j < 2 * D) ? y2 : 0.0f;
        }
    }
    const float wq = wave_sum(ssq), wk = wave_sum(ssk);
    if (lane == 0) {
        lds[2 * wave] = wq;
        lds[2 * wave + 1] = wk;
    }
    __syncthreads();
    const float sq = (lds[0] + lds[2]) + (lds[4] + lds[6]);
    const float sk = (lds[1] + lds[3]) + (lds[5] + lds[7]);
    const float iq = (sh.use_l2 ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) * sh.scale;
    const float ik = sh.use_l2 ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
    float *qk = ws + ((int64_t)b * Hq + h) * 2 * D;
    float *vv = ws + ws_v_off(sh.batch, Hq, D) + ((int64_t)b * HV + hv0) * D;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int j = tid + NT * k;
        if (j < D)
            qk[j] = y[k] * iq;
        else if (j < 2 * D)
            qk[j] = y[k] * ik;
        else if (j < NCH)
            vv[j - 2 * D] = y[k];
    }
}

// The conv role for width 4 on a dense channel-major pool ([slot][channel][3
// taps], 16-bit words 4-byte aligned): thread t takes channel pairs (2 jp,
// 2 jp + 1), jp = t + NT k. A pair's three taps each are six consecutive
// 16-bit values (three 32-bit words), its weights eight (four words), its bias
// and input two (one word each), so a thread moves its pair in six vector
// accesses where the per-channel path takes 24 16-bit ones. Same arithmetic,
// in the same order, as gdn_conv.
template <int D, int GM>
__device__ void gdn_conv_pairs(int b, int h, const uint16_t *__restrict__ mixed_qkv,
                               const uint16_t *__restrict__ conv_w, const uint16_t *__restrict__ conv_b,
                               uint16_t *__restrict__ conv_state, int s, float *__restrict__ ws,
                               const GdnPrepShape &sh, float *lds)
{
    constexpr int NT = kGdnNT;
    constexpr int G = GM;
    constexpr int NPR = (2 + G) * D / 2;      // owned channel pairs (D is even)
    constexpr int PPT = (NPR + NT - 1) / NT;  // pairs per thread
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int Hq = sh.hq, HV = sh.hv;
    const int hv0 = h * G;
    const int HD = Hq * D;
    const int64_t qkv_dim = 2 * (int64_t)HD + (int64_t)HV * D;
    // owned channel j (even) -> pool channel; a pair never straddles the q, k, v runs
    auto chan = [&](int j) {
        return j < D ? h * D + j : (j < 2 * D ? HD + h * D + (j - D) : 2 * HD + hv0 * D + (j - 2 * D));
    };
    uint32_t tw[PPT][3], ww[PPT][4], bw[PPT], xw[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int c = chan(2 * min(tid + NT * k, NPR - 1));
        const uint32_t *cs = reinterpret_cast<const uint32_t *>(conv_state + (int64_t)s * sh.cs_slot + (int64_t)c * 3);
        const uint32_t *cw = reinterpret_cast<const uint32_t *>(conv_w + (int64_t)c * 4);
#pragma unroll
        for (int i = 0; i < 3; ++i)
            tw[k][i] = cs[i];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ww[k][i] = cw[i];
        bw[k] = *reinterpret_cast<const uint32_t *>(conv_b + c);
        xw[k] = *reinterpret_cast<const uint32_t *>(mixed_qkv + b * qkv_dim + c);
    }
    auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
    auto hi = [](uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); };
    float y[PPT][2];
    float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int j = 2 * (tid + NT * k);
        // taps: (c0 t0, c0 t1), (c0 t2, c1 t0), (c1 t1, c1 t2); weights
        // (c0 w0, c0 w1), (c0 w2, c0 w3), (c1 w0, c1 w1), (c1 w2, c1 w3)
        float a0 = lo(bw[k]);
        a0 = fmaf(lo(tw[k][0]), lo(ww[k][0]), a0);
        a0 = fmaf(hi(tw[k][0]), hi(ww[k][0]), a0);
        a0 = fmaf(lo(tw[k][1]), lo(ww[k][1]), a0);
        a0 = fmaf(lo(xw[k]), hi(ww[k][1]), a0);
        float a1 = hi(bw[k]);
        a1 = fmaf(hi(tw[k][1]), lo(ww[k][2]), a1);
        a1 = fmaf(lo(tw[k][2]), hi(ww[k][2]), a1);
        a1 = fmaf(hi(tw[k][2]), lo(ww[k][3]), a1);
        a1 = fmaf(hi(xw[k]), hi(ww[k][3]), a1);
        y[k][0] = silu_f32(a0);
        y[k][1] = silu_f32(a1);
        if (j < 2 * NPR) {
            // the pool keeps the last 3 raw inputs, newest last: (c0 t1, c0 t2),
            // (c0 x, c1 t1), (c1 t2, c1 x)
            uint32_t *cs = reinterpret_cast<uint32_t *>(conv_state + (int64_t)s * sh.cs_slot + (int64_t)chan(j) * 3);
            cs[0] = __builtin_amdgcn_perm(tw[k][1], tw[k][0], 0x05040302u);
            cs[1] = __builtin_amdgcn_perm(tw[k][2], xw[k], 0x05040100u);
            cs[2] = __builtin_amdgcn_perm(xw[k], tw[k][2], 0x07060302u);
            const float y2 = y[k][0] * y[k][0] + y[k][1] * y[k][1];
            ssq += j < D ? y2 : 0.0f;
            ssk += (j >= D && j < 2 * D) ? y2 : 0.0f;
        }
    }
    const float wq = wave_sum(ssq), wk = wave_sum(ssk);
    if (lane == 0) {
        lds[2 * wave] = wq;
        lds[2 * wave + 1] = wk;
    }
    __syncthreads();
    const float sq = (lds[0] + lds[2]) + (lds[4] + lds[6]);
    const float sk = (lds[1] + lds[3]) + (lds[5] + lds[7]);
    const float iq = (sh.use_l2 ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) * sh.scale;
    const float ik = sh.use_l2 ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
    float *qk = ws + ((int64_t)b * Hq + h) * 2 * D;
    float *vv = ws + ws_v_off(sh.batch, Hq, D) + ((int64_t)b * HV + hv0) * D;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int j = 2 * (tid + NT * k);
        if (j < D) {
            qk[j] = y[k][0] * iq;
            qk[j + 1] = y[k][1] * iq;
        } else if (j < 2 * D) {
            qk[j] = y[k][0] * ik;
            qk[j + 1] = y[k][1] * ik;
        } else if (j < 2 * NPR) {
            vv[j - 2 * D] = y[k][0];
            vv[j - 2 * D + 1] = y[k][1];
        }
    }
}

template <int D, int GM, int WM, bool PAIRS>
__global__ __launch_bounds__(kGdnNT) void gdn_prep_kernel(
    const uint16_t *__restrict__ hs, const uint16_t *__restrict__ w_ba,
    const uint16_t *__restrict__ mixed_qkv, const uint16_t *__restrict__ conv_w,
    const uint16_t *__restrict__ conv_b, uint16_t *__restrict__ conv_state,
    const int32_t *__restrict__ idx, float *__restrict__ ws, const GdnPrepShape sh)
{
    __shared__ float lds[kProjRows + kGdnNT * 8];
    const int B = sh.batch;
    const int nconv = B * sh.hq;
    if ((int)blockIdx.x >= nconv) {  // projection role (uniform over the workgroup)
        const int j = blockIdx.x - nconv;
        const int b = j / sh.nck, ck = j - b * sh.nck;
        if (idx[b] < 0)
            return;
        float *part = ws + ws_p_off(B, sh.hq, sh.hv, D);
        if (sh.proj_vec)
            gdn_projection<8>(b, ck, hs, w_ba, part, sh, lds);
        else
            gdn_projection<2>(b, ck, hs, w_ba, part, sh, lds);
        return;
    }
    const int b = blockIdx.x / sh.hq;
    const int h = blockIdx.x - b * sh.hq;
    const int s = idx[b];
    if (s < 0)  // padding entry: no pool access; the stream writes its zero output
        return;
    if constexpr (PAIRS)
        gdn_conv_pairs<D, GM>(b, h, mixed_qkv, conv_w, conv_b, conv_state, s, ws, sh, lds);
    else
        gdn_conv<D, GM, WM>(b, h, mixed_qkv, conv_w, conv_b, conv_state, s, ws, sh, lds);
}

// ---------------------------------------------------------------------------
// gdn_stream
// ---------------------------------------------------------------------------
// A state row (D fp32) is spread over LPR lanes (16 at D >= 128, else 8), EPL = D /
// LPR floats each, as NV = EPL / 4 16-byte vectors: lane l's vector v holds
// columns 4 LPR v + 4 l .. + 3, so each vector access of a row's LPR lanes
// covers 16 LPR >= 128 consecutive bytes (whole cache lines). One wave
// instruction serves RPI = 64 / LPR rows; a wave runs PW such passes.
template <int D>
struct StreamCfg {
    static constexpr int LPR = D >= 128 ? 16 : 8;
    static constexpr int EPL = D / LPR;
    static constexpr int NV = EPL / 4;
    static constexpr int RPI = 64 / LPR;
    static constexpr int PW = D == 32 ? 1 : 2;
    static constexpr int RPW = RPI * PW;   // rows per wave
    static constexpr int RPB = 4 * RPW;    // rows per workgroup
    static constexpr int NPH = D / RPB;    // workgroups per value head
    static_assert(NV >= 1 && NPH >= 1 && NPH * RPB == D, "stream tiling");
};

// p: the row's first element + 4 l
template <int NV, int LPR>
__device__ __forceinline__ void ld_row(const float *p, float (&x)[4 * NV])
{
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + v * 4 * LPR));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[4 * v + j] = __uint_as_float(w[j]);
    }
}

template <int NV, int LPR>
__device__ __forceinline__ void st_row(float *p, const float (&x)[4 * NV])
{
#pragma unroll
    for (int v = 0; v < NV; ++v)
        __builtin_nontemporal_store(
            u32x4{__float_as_uint(x[4 * v]), __float_as_uint(x[4 * v + 1]),
                  __float_as_uint(x[4 * v + 2]), __float_as_uint(x[4 * v + 3])},
            reinterpret_cast<u32x4 *>(p + v * 4 * LPR));
}

// the same column layout for a (cached) D-vector in the workspace
template <int NV, int LPR>
__device__ __forceinline__ void ld_vec(const float *p, float (&x)[4 * NV])
{
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const float4 w = *reinterpret_cast<const float4 *>(p + v * 4 * LPR);
        x[4 * v] = w.x;
        x[4 * v + 1] = w.y;
        x[4 * v + 2] = w.z;
        x[4 * v + 3] = w.w;
    }
}

// exp via the hardware exp2 (relative error a few 1e-7 over the gates' range)
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// bf16 bits of f, round to nearest even, NaN kept quiet; selects, no branch
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : r;
}

struct GdnStreamShape {
    int64_t ssm_row_stride;
    int32_t batch, hq, hv, nck;
};

// Per row, with x the state row before the step, a = alpha, k / q the
// normalised key / scaled query: pk = x.k and po = x.q (both reduced over the
// row's lanes together), delta = beta (v - a pk), out = a po + delta (k.q),
// x' = a x + delta k -- the same values as decaying the row, predicting,
// updating and then reading the output, with the two reductions independent.
template <int D>
__global__ __launch_bounds__(kGdnNT) void gdn_stream_kernel(
    float *__restrict__ ssm, const int32_t *__restrict__ idx, const float *__restrict__ ws,
    const float *__restrict__ A_log, const uint16_t *__restrict__ dt_bias,
    uint16_t *__restrict__ out, const GdnStreamShape sh)
{
    using C = StreamCfg<D>;
    constexpr int LPR = C::LPR, EPL = C::EPL, NV = C::NV, PW = C::PW, RPI = C::RPI;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l = lane & (LPR - 1);
    const int HV = sh.hv;
    const int bh = blockIdx.x / C::NPH;  // b * HV + hv
    const int part = blockIdx.x - bh * C::NPH;
    const int b = bh / HV, hv = bh - b * HV;
    const int h = hv / (HV / sh.hq);     // q/k head of this value head
    const int row0 = part * C::RPB + wave * C::RPW + lane / LPR;  // rows row0 + RPI p
    const int s = idx[b];
    uint16_t *ob = out + (int64_t)bh * D;
    if (s < 0) {  // padding entry: zero output
        if (l == 0) {
#pragma unroll
            for (int p = 0; p < PW; ++p)
                ob[row0 + RPI * p] = 0;
        }
        return;
    }
    float *st = ssm + (int64_t)s * sh.ssm_row_stride + (int64_t)hv * D * D + 4 * l;
    float x[PW][EPL];
#pragma unroll
    for (int p = 0; p < PW; ++p)
        ld_row<NV, LPR>(st + (int64_t)(row0 + RPI * p) * D, x[p]);
    const float *qk = ws + ((int64_t)b * sh.hq + h) * 2 * D + 4 * l;
    float qv[EPL], kv[EPL];
    ld_vec<NV, LPR>(qk, qv);
    ld_vec<NV, LPR>(qk + D, kv);
    const float *vvp = ws + ws_v_off(sh.batch, sh.hq, D) + (int64_t)bh * D + row0;
    float vrow[PW];
#pragma unroll
    for (int p = 0; p < PW; ++p)
        vrow[p] = vvp[RPI * p];
    // gates: b/a sums of this value head over the projection chunks
    const float *pp = ws + ws_p_off(sh.batch, sh.hq, HV, D) + (int64_t)b * sh.nck * 2 * HV + hv;
    float pb = 0.0f, pa = 0.0f;
    for (int j = lane; j < sh.nck; j += 64) {
        pb += pp[(int64_t)j * 2 * HV];
        pa += pp[(int64_t)j * 2 * HV + HV];
    }
    pb = wave_sum(pb);
    pa = wave_sum(pa);
    const float t = pa + bf16_to_f32(dt_bias[hv]);
    const float sp = t > 20.0f ? t : __builtin_amdgcn_logf(1.0f + fast_exp(t)) * 0.6931471805599453f;
    const float alpha = fast_exp(-fast_exp(A_log[hv]) * sp);
    const float beta = __builtin_amdgcn_rcpf(1.0f + fast_exp(-pb));
    float kq = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        kq = fmaf(kv[e], qv[e], kq);
    kq = row_group_sum<LPR>(kq);
#pragma unroll
    for (int p = 0; p < PW; ++p) {
        float pk = 0.0f, po = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            pk = fmaf(x[p][e], kv[e], pk);
            po = fmaf(x[p][e], qv[e], po);
        }
        pk = row_group_sum<LPR>(pk);
        po = row_group_sum<LPR>(po);
        const float delta = beta * (vrow[p] - alpha * pk);
        const float o = fmaf(alpha, po, delta * kq);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            x[p][e] = fmaf(delta, kv[e], alpha * x[p][e]);
        st_row<NV, LPR>(st + (int64_t)(row0 + RPI * p) * D, x[p]);
        const uint32_t o16 = bf16_bits(o);
        if (l == 0)
            ob[row0 + RPI * p] = (uint16_t)o16;
    }
}

template <int D, int GM, int WM, bool PAIRS = false>
hipError_t launch_prep(const GdnParams &p, const GdnPrepShape &sh, hipStream_t stream)
{
    const int64_t blocks = (int64_t)p.batch * p.hq + (int64_t)p.batch * sh.nck;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_prep_kernel<D, GM, WM, PAIRS>), dim3((unsigned)blocks), dim3(kGdnNT), 0,
                       stream, static_cast<const uint16_t *>(p.hs),
                       static_cast<const uint16_t *>(p.w_ba), static_cast<const uint16_t *>(p.qkv),
                       static_cast<const uint16_t *>(p.conv_w),
                       static_cast<const uint16_t *>(p.conv_b),
                       static_cast<uint16_t *>(p.conv_state), p.idx,
                       static_cast<float *>(p.workspace), sh);
    return hipGetLastError();
}

template <int D, int GM>
hipError_t launch_prep_g(const GdnParams &p, const GdnPrepShape &sh, hipStream_t stream)
{
    if (p.width == 1)
        return launch_prep<D, GM, 1>(p, sh, stream);
    auto al4 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 3) == 0; };
    if (p.width == 4 && p.cs_tap == 1 && p.cs_chan == 3 && p.cs_slot % 2 == 0 && al4(p.conv_state) &&
        al4(p.conv_w) && al4(p.conv_b) && al4(p.qkv))
        return launch_prep<D, GM, 4, true>(p, sh, stream);
    return p.width <= 4 ? launch_prep<D, GM, 4>(p, sh, stream) : launch_prep<D, GM, 8>(p, sh, stream);
}

template <int D>
hipError_t launch_d(const GdnParams &p, hipStream_t stream)
{
    GdnPrepShape sh;
    sh.cs_slot = p.cs_slot;
    sh.cs_chan = p.cs_chan;
    sh.cs_tap = p.cs_tap;
    sh.batch = p.batch;
    sh.hidden = p.hidden;
    sh.hq = p.hq;
    sh.hv = p.hv;
    sh.width = p.width;
    sh.use_l2 = p.use_l2;
    sh.proj_vec = (p.hv % 4 == 0 && (reinterpret_cast<uintptr_t>(p.w_ba) & 15) == 0) ? 1 : 0;
    sh.scale = p.scale;
    sh.nck = (p.hidden + kProjRows - 1) / kProjRows;
    (void)hipGetLastError();
    hipError_t e;
    switch (p.hv / p.hq) {
    case 1: e = launch_prep_g<D, 1>(p, sh, stream); break;
    case 2: e = launch_prep_g<D, 2>(p, sh, stream); break;
    case 4: e = launch_prep_g<D, 4>(p, sh, stream); break;
    case 8: e = launch_prep_g<D, 8>(p, sh, stream); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    GdnStreamShape ss;
    ss.ssm_row_stride = p.ssm_row_stride;
    ss.batch = p.batch;
    ss.hq = p.hq;
    ss.hv = p.hv;
    ss.nck = sh.nck;
    const int64_t blocks = (int64_t)p.batch * p.hv * StreamCfg<D>::NPH;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_stream_kernel<D>), dim3((unsigned)blocks), dim3(kGdnNT), 0, stream,
                       p.ssm, p.idx, static_cast<const float *>(p.workspace), p.A_log,
                       static_cast<const uint16_t *>(p.dt_bias), static_cast<uint16_t *>(p.out), ss);
    return hipGetLastError();
}

}  // namespace

int64_t gdn_workspace_floats(int64_t batch, int64_t hidden, int64_t hq, int64_t hv, int64_t d)
{
    const int64_t nck = (hidden + kProjRows - 1) / kProjRows;
    return ws_p_off(batch, hq, hv, d) + batch * nck * 2 * hv;
}

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
