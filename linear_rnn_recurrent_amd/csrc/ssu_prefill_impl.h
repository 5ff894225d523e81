// Prefill selective state update: all seq_len tokens of every batch row in one
// launch, with contextLengths and the optional replay stash. Kernel template,
// instantiated once per state dtype by ssu_prefill_{f32,f16,bf16}.hip.
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page,
// invokeSelectiveStateUpdatePrefill): the decode step of
// invokeSelectiveStateUpdate applied to tokens t < L_b in order, where
// L_b = clamp(contextLengths[b], 0, seq_len); outputs beyond L_b are zero.
// With the replay stash the committed state is read-only and A*dt', dt', x and
// B are stashed per token in fp32 (zeros beyond L_b).
//
// Mapping on gfx950. The recurrence is sequential in t and every token does 3
// VALU operations per state element against a few hundred bytes of I/O per
// (token, head), so the loop is bound by the fp32 VALU, not by HBM. The state
// lives in registers for the whole sequence:
//   * a 256-thread workgroup owns one (batch row, head, block of 64 rows of
//     dim). dstate is cut into 16 slices of NS/16 columns: wave w, quarter q
//     (16 lanes) owns slice 4w+q, and lane rr of the quarter owns rows
//     rr, rr+16, rr+32, rr+48, so every B/C value read serves four rows;
//   * tokens go in chunks of TC. B and C (as fp32), x, dt' and exp(A dt') of a
//     chunk sit in LDS; the global loads of chunk c+1 are issued before the
//     token loop of chunk c (register prefetch) and written to the other LDS
//     buffer after it, so their latency hides behind a chunk of arithmetic;
//   * per token a lane reads its slice of B and C and its four x values with
//     16-byte LDS broadcasts and updates 4 x NS/16 state elements;
//   * the lane keeps S~ = S / P_t, P_t the running product of the decays, so a
//     token costs two FMAs per element instead of a multiply and two FMAs
//     (S~ += (dt'/P_t) x B; partial output = sum S~ C, scaled by P_t once per
//     output); S = P S~ is restored before the final store. Every term keeps the
//     relative rounding of the direct form. Before a product would leave
//     [1e-30, 1e30] the state is renormalised (S~ <- S~ * P_prev, P restarts),
//     which the staging marks per token in a bitmask read with scalar ops;
//   * the four slices of a wave are summed in registers with the gfx950
//     cross-lane swaps (v_permlane32_swap, v_permlane16_swap); the wave's
//     partial output per (token, row) goes to LDS, and after the chunk the
//     workgroup adds the four wave partials in a fixed order, applies D*x and
//     the gate, and stores the outputs (deterministic, no atomics);
//   * workgroups are ordered longest sequence first (the rank of each
//     contextLengths entry is computed on the device: no host read).
#pragma once

#include "ssu_device.h"
#include "ssu_internal.h"
#include "ssu_rowblock.h"

namespace ssu {
namespace {

struct PrefillShape {
    int64_t row_stride;
    int32_t batch, seq_len, nheads, dim, ngroups, heads_per_group, nrb;
    int32_t dt_softplus, sort_by_length, pass;
};

constexpr int kPrefillTC = 8;  // tokens per staged chunk

// Per-token operands of one lane: (dt', decay), its four x values and its
// slice of B and C, all read from LDS (16-byte broadcast reads).
template <int NSL>
struct Operands {
    float2 va;
    float4 xv;
    float b[NSL], c[NSL];
};

template <int NSL>
__device__ __forceinline__ void fetch_ops(Operands<NSL> &o, const float2 &va, const float *xp,
                                          const float *bp, const float *cp)
{
    o.va = va;
    o.xv = *reinterpret_cast<const float4 *>(xp);
    if constexpr (NSL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NSL; j += 4) {
            const float4 b4 = *reinterpret_cast<const float4 *>(bp + j);
            const float4 c4 = *reinterpret_cast<const float4 *>(cp + j);
            o.b[j] = b4.x; o.b[j + 1] = b4.y; o.b[j + 2] = b4.z; o.b[j + 3] = b4.w;
            o.c[j] = c4.x; o.c[j + 1] = c4.y; o.c[j + 2] = c4.z; o.c[j + 3] = c4.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NSL; ++j) {
            o.b[j] = bp[j];
            o.c[j] = cp[j];
        }
    }
}

// Renormalisation before a token: S~ <- (S~ * f.x) * f.y (see the staging).
template <int NSL>
__device__ __forceinline__ void apply_renorm(float (&S)[4][NSL], const float2 f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NSL; ++j)
            S[i][j] = (S[i][j] * f.x) * f.y;
}

// One token for a lane's 4 rows x NSL columns in the rescaled form: the lane
// holds S~ = S / P_t (P_t: the running product of decays since the last
// renormalisation) and o.va = (dt'/P_t, P_t). The update is one FMA per
// element, S~ += (dt'/P_t) x B, and so is the partial output sum of S~ C (the
// factor P_t is applied once per output in the epilogue). token_fma returns
// the lane's partials of its rows rr + 16 i, which quarter_reduce sums over the
// four quarters of the wave.
template <int NSL>
__device__ __forceinline__ float4 token_fma(float (&S)[4][NSL], const Operands<NSL> &o)
{
    const float qx[4] = {o.va.x * o.xv.x, o.va.x * o.xv.y, o.va.x * o.xv.z, o.va.x * o.xv.w};
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[i][j] = fmaf(qx[i], o.b[j], S[i][j]);
            p[i] = fmaf(S[i][j], o.c[j], p[i]);
        }
    }
    return make_float4(p[0], p[1], p[2], p[3]);
}

template <typename ST, typename IOT, typename BCT, int NS, int NW>
__global__ __launch_bounds__(64 * NW) void ssu_prefill_kernel(
    const void *__restrict__ x, const float *__restrict__ A, const void *__restrict__ Bm,
    const void *__restrict__ Cm, const float *__restrict__ dt, const float *__restrict__ dt_bias,
    const float *__restrict__ Dv, const void *__restrict__ z, ST *__restrict__ state,
    void *__restrict__ out, const int32_t *__restrict__ ctx, const int32_t *__restrict__ idx,
    float *__restrict__ st_dA, float *__restrict__ st_u, float *__restrict__ st_B,
    float *__restrict__ st_dt, const PrefillShape sh)
{
    constexpr int TC = kPrefillTC;
    constexpr int NT = 64 * NW;                   // threads
    constexpr int NSL = NS / (4 * NW);            // dstate columns per lane
    constexpr int BCN = TC * NS;                  // B (or C) elements per chunk
    constexpr int XT_PER = (TC * 64 + NT - 1) / NT; // x elements staged per thread
    static_assert(NSL >= 1 && NS % (4 * NW) == 0, "dstate must split into 4*NW slices");
    static_assert(TC % 2 == 0, "the token loop runs in pairs");

    __shared__ __attribute__((aligned(16))) float Bs[2][TC][NS];
    __shared__ __attribute__((aligned(16))) float Cs[2][TC][NS];
    __shared__ __attribute__((aligned(16))) float xs[2][TC][64];
    __shared__ float2 pp[2][TC];     // (dt'/P_t, P_t) per token
    __shared__ float2 renorm[2][TC]; // factors applied to S~ before a token (bit set in rmask)
    __shared__ uint32_t rmask[2];    // tokens preceded by a renormalisation
    __shared__ float ybuf[TC][NW][64];  // per (token, wave, row) partial sums
    __shared__ int sorted_b;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4;
    const int rr = lane & 15;
    const int sl = wave * 4 + q;
    const int n0 = sl * NSL;
    const int T = sh.seq_len, H = sh.nheads, Dm = sh.dim, G = sh.ngroups;
    // Work item u = blockIdx.x, or with length sorting a snake over passes of
    // sh.pass workgroups (one per CU): even passes take the longest remaining
    // rows first, odd passes the shortest, so the items that end up sharing a
    // CU mix long and short sequences.
    int u = blockIdx.x;
    if (sh.sort_by_length && sh.pass > 0) {
        const int pass = u / sh.pass, pos = u - pass * sh.pass;
        const int base = pass * sh.pass;
        const int width = min(sh.pass, (int)gridDim.x - base);
        u = base + ((pass & 1) ? width - 1 - pos : pos);
    }
    const int per_b = H * sh.nrb;
    const int qb = u / per_b;
    const int rem = u - qb * per_b;
    const int h = rem % H;
    const int rb = rem / H;

    int b = qb;
    if (sh.sort_by_length) {
        // b = the batch row whose length has rank qb (descending, ties by index)
        if (tid == 0)
            sorted_b = qb;
        __syncthreads();
        for (int c = tid; c < sh.batch; c += NT) {
            const int lc = clamp_len(ctx[c], T);
            int rank = 0;
            for (int c2 = 0; c2 < sh.batch; ++c2) {
                const int l2 = clamp_len(ctx[c2], T);
                rank += (l2 > lc) || (l2 == lc && c2 < c);
            }
            if (rank == qb)
                sorted_b = c;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(sorted_b);
    }

    const int srow = idx ? idx[b] : b;
    const int L = ctx ? clamp_len(ctx[b], T) : T;
    const int64_t bT = (int64_t)b * T;
    const int rbase = rb * 64;

    if (srow < 0) {  // padding row: outputs zero, state and stash untouched
        for (int i = tid; i < T * 64; i += NT) {
            const int r = rbase + (i & 63);
            if (r < Dm)
                st_elem<IOT>(out, ((bT + (i >> 6)) * H + h) * Dm + r, 0.0f);
        }
        return;
    }

    const bool stash = st_dA != nullptr;
    const int g = h / sh.heads_per_group;
    const float Ah = A[h];
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    const float dskip = Dv ? Dv[h] : 0.0f;
    const bool writes_B = stash && rb == 0 && (h % sh.heads_per_group) == 0;

    // ---- the state slice: rows rbase + rr + 16 i, columns n0 .. n0+NSL-1 ----
    float S[4][NSL];
    ST *sbase = state + (int64_t)srow * sh.row_stride + (int64_t)h * Dm * NS + n0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rc = min(rbase + rr + 16 * i, Dm - 1);
#pragma unroll
        for (int j = 0; j < NSL; ++j)
            S[i][j] = ld_elem<ST>(sbase, (int64_t)rc * NS + j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool rv = rbase + rr + 16 * i < Dm;  // rows past dim hold zeros
#pragma unroll
        for (int j = 0; j < NSL; ++j)
            S[i][j] = rv ? S[i][j] : 0.0f;
    }
    // Consume the state here: otherwise the token loop, not knowing whether these
    // loads are still in flight, waits on every outstanding load, including the
    // next chunk's prefetch. Emits no instruction beyond that one wait.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NSL; ++j)
            asm volatile("" ::"v"(S[i][j]));

    // ---- chunk staging: global -> registers (prefetch) -> LDS ----
    // Every prefetch load is unconditional (indices past the chunk or past dim
    // are clamped to valid ones and masked when written to LDS) and keeps raw
    // bits, so nothing waits on it until the chunk is written to LDS after the
    // token loop.
    constexpr int BCV = (BCN / 4 + NT - 1) / NT;  // 4-element B/C vectors per thread
    float pcarry = 1.0f;  // wave 0: S = pcarry * S~ after the last staged chunk
    typename Raw4<BCT>::type rB[BCV], rC[BCV];
    uint32_t rX[XT_PER], rDt;
    auto load_chunk = [&](int t0, int nt) {
#pragma unroll
        for (int k = 0; k < BCV; ++k) {
            const int e = min((tid + NT * k) * 4, nt * NS - 4);
            const int64_t o = ((bT + t0 + e / NS) * G + g) * NS + (e % NS);
            rB[k] = ld_raw4<BCT>(Bm, o);
            rC[k] = ld_raw4<BCT>(Cm, o);
        }
#pragma unroll
        for (int k = 0; k < XT_PER; ++k) {
            const int e = tid + NT * k;
            const int tt = min(e >> 6, nt - 1);
            const int r = min(rbase + (e & 63), Dm - 1);
            rX[k] = ld_raw1<IOT>(x, ((bT + t0 + tt) * H + h) * Dm + r);
        }
        rDt = ld_raw1<float>(dt, (bT + t0 + min(tid & (TC - 1), nt - 1)) * H + h);
    };
    auto store_chunk = [&](int buf, int t0, int nt) {
#pragma unroll
        for (int k = 0; k < BCV; ++k) {
            const int e = (tid + NT * k) * 4;
            if (e < BCN) {
                float vb[4], vc[4];
                cvt_raw4<BCT>(rB[k], vb);
                cvt_raw4<BCT>(rC[k], vc);
                *reinterpret_cast<float4 *>(&Bs[buf][e / NS][e % NS]) =
                    make_float4(vb[0], vb[1], vb[2], vb[3]);
                *reinterpret_cast<float4 *>(&Cs[buf][e / NS][e % NS]) =
                    make_float4(vc[0], vc[1], vc[2], vc[3]);
                if (writes_B && e < nt * NS) {
                    const int64_t o = ((bT + t0 + e / NS) * G + g) * NS + (e % NS);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        st_B[o + j] = vb[j];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < XT_PER; ++k) {
            const int e = tid + NT * k;
            if (e < TC * 64) {
                const int r = rbase + (e & 63);
                const bool valid = e < nt * 64 && r < Dm;
                const float xv = valid ? cvt_raw1<IOT>(rX[k]) : 0.0f;
                xs[buf][e >> 6][xpos(e & 63)] = xv;
                if (stash && valid)
                    st_u[((bT + t0 + (e >> 6)) * H + h) * Dm + r] = xv;
            }
        }
        if (wave == 0) {
            // lanes < TC: one token each; slots past the chunk are neutral tokens
            // (dt' = 0, decay = 1). P_t = pcarry * (prefix product of the decays);
            // common case: every P_t within [1e-30, 1e30], no renormalisation.
            float v = __uint_as_float(rDt) + bias;
            if (sh.dt_softplus)
                v = softplus_f32(v);
            const bool live = lane < nt;
            const float dtp = live ? v : 0.0f;
            const float a = live ? expf(Ah * v) : 1.0f;
            float pre = a;
#pragma unroll
            for (int d = 1; d < TC; d <<= 1) {
                const float o = __shfl_up(pre, d, 64);
                if ((lane & (TC - 1)) >= d)
                    pre *= o;
            }
            float P = pcarry * pre;
            float m1 = 1.0f, m2 = 1.0f;
            uint32_t mask = 0;
            if (__ballot(lane < TC && !(P >= 1e-30f && P <= 1e30f)) != 0) {
                if (__ballot(lane < TC && !(pre >= 1e-30f && pre <= 1e30f)) == 0) {
                    // renormalise once, before the chunk's first token
                    mask = 1;
                    if (lane == 0)
                        m1 = pcarry;
                    P = pre;
                } else {
                    // rare: extreme decays inside the chunk; walk the tokens in order
                    float pr = pcarry;
                    for (int t = 0; t < TC; ++t) {
                        const float at = __shfl(a, t, 64);
                        const float cand = pr * at;
                        float pt = cand, f1 = 1.0f, f2 = 1.0f;
                        if (!(cand >= 1e-30f && cand <= 1e30f)) {
                            mask |= 1u << t;
                            f1 = pr;               // S~ * P_prev = true state
                            if (at >= 1e-30f && at <= 1e30f) {
                                pt = at;
                            } else {
                                f2 = at;           // decay applied directly
                                pt = 1.0f;
                            }
                        }
                        if (lane == t) {
                            P = pt;
                            m1 = f1;
                            m2 = f2;
                        }
                        pr = pt;
                    }
                }
            }
            if (lane < TC) {
                pp[buf][lane] = make_float2(dtp / P, P);
                renorm[buf][lane] = make_float2(m1, m2);
                if (stash && rb == 0 && live) {
                    st_dA[(bT + t0 + lane) * H + h] = Ah * v;
                    st_dt[(bT + t0 + lane) * H + h] = v;
                }
            }
            if (lane == 0)
                rmask[buf] = mask;
            pcarry = __shfl(P, TC - 1, 64);  // neutral slots keep P of the last token
        }
    };

    const int nchunks = (L + TC - 1) / TC;
    if (nchunks > 0) {
        load_chunk(0, min(TC, L));
        store_chunk(0, 0, min(TC, L));
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const int t0 = c * TC;
        const int nt = min(TC, L - t0);
        if (c + 1 < nchunks)
            load_chunk(t0 + TC, min(TC, L - t0 - TC));
        // gate inputs of this chunk's outputs (raw bits, clamped indices; without
        // z the x values are re-read and never used), consumed after the token loop
        const void *zsrc = z ? z : x;
        uint32_t zq[XT_PER];
#pragma unroll
        for (int k = 0; k < XT_PER; ++k) {
            const int e = tid + NT * k;
            const int tt = min(e >> 6, nt - 1);
            const int r = min(rbase + (e & 63), Dm - 1);
            zq[k] = ld_raw1<IOT>(zsrc, ((bT + t0 + tt) * H + h) * Dm + r);
        }

        // ---- the recurrence over the chunk, state in registers ----
        // Unrolled by two with ping-pong operand sets: the LDS reads of token
        // tt+1 are in flight while token tt is computed. The body has no
        // condition: with an odd token count the last pair ends with the
        // neutral slot nt (dt' = 0, decay = 1 and x = 0 leave the state
        // unchanged; its partial sums are never read).
        Operands<NSL> opa, opb;
        const uint32_t mask = __builtin_amdgcn_readfirstlane(rmask[buf]);
        fetch_ops<NSL>(opa, pp[buf][0], &xs[buf][0][rr * 4], &Bs[buf][0][n0], &Cs[buf][0][n0]);
        for (int tt = 0; tt < nt; tt += 2) {
            const int t1 = tt + 1;
            fetch_ops<NSL>(opb, pp[buf][t1], &xs[buf][t1][rr * 4], &Bs[buf][t1][n0], &Cs[buf][t1][n0]);
            if (mask & (1u << tt))
                apply_renorm<NSL>(S, renorm[buf][tt]);
            ybuf[tt][wave][lane] = quarter_reduce(token_fma<NSL>(S, opa));
            const int t2 = min(tt + 2, TC - 1);
            fetch_ops<NSL>(opa, pp[buf][t2], &xs[buf][t2][rr * 4], &Bs[buf][t2][n0], &Cs[buf][t2][n0]);
            if (mask & (1u << t1))
                apply_renorm<NSL>(S, renorm[buf][t1]);
            ybuf[t1][wave][lane] = quarter_reduce(token_fma<NSL>(S, opb));
        }
        __syncthreads();

        // ---- combine the 4 wave partials, skip term and gate; store outputs ----
#pragma unroll
        for (int k = 0; k < XT_PER; ++k) {
            const int e = tid + NT * k;
            const int r = rbase + (e & 63);
            if (e < nt * 64 && r < Dm) {
                const int tt = e >> 6;
                float y = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; w += 2)
                    y += ybuf[tt][w][e & 63] + ybuf[tt][w + 1][e & 63];
                y *= pp[buf][tt].y;
                y += dskip * xs[buf][tt][xpos(e & 63)];
                if (z)
                    y *= silu_f32(cvt_raw1<IOT>(zq[k]));
                st_elem<IOT>(out, ((bT + t0 + tt) * H + h) * Dm + r, y);
            }
        }
        if (c + 1 < nchunks)
            store_chunk(buf ^ 1, t0 + TC, min(TC, L - t0 - TC));
        __syncthreads();
    }

    // ---- tokens beyond the context: zero outputs and zero stash ----
    for (int i = tid; i < (T - L) * 64; i += NT) {
        const int r = rbase + (i & 63);
        if (r < Dm) {
            const int64_t o = ((bT + L + (i >> 6)) * H + h) * Dm + r;
            st_elem<IOT>(out, o, 0.0f);
            if (stash)
                st_u[o] = 0.0f;
        }
    }
    if (stash && rb == 0) {
        for (int t = L + tid; t < T; t += NT) {
            st_dA[(bT + t) * H + h] = 0.0f;
            st_dt[(bT + t) * H + h] = 0.0f;
        }
    }
    if (writes_B) {
        for (int i = tid; i < (T - L) * NS; i += NT)
            st_B[((bT + L + i / NS) * G + g) * NS + (i % NS)] = 0.0f;
    }

    if (!stash && L > 0) {
        // S = P_last * S~ (P of the last real token of the last chunk)
        const float plast = pp[((L + TC - 1) / TC - 1) & 1][(L - 1) % TC].y;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NSL; ++j)
                S[i][j] *= plast;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + rr + 16 * i;
            if (r < Dm) {
#pragma unroll
                for (int j = 0; j < NSL; ++j)
                    st_elem<ST>(sbase, (int64_t)r * NS + j, S[i][j]);
            }
        }
    }
}

}  // namespace
}  // namespace ssu

// the matrix-core prefill (bf16 or fp16 operands), dispatched to from launch_prefill_bc
#include "ssu_prefill_mm.h"

namespace ssu {
namespace {

inline PrefillShape prefill_shape(const PrefillParams &p)
{
    const DecodeParams &d = p.d;
    PrefillShape sh;
    sh.row_stride = d.row_stride;
    sh.batch = d.batch;
    sh.seq_len = p.seq_len;
    sh.nheads = d.nheads;
    sh.dim = d.dim;
    sh.ngroups = d.ngroups;
    sh.heads_per_group = d.nheads / d.ngroups;
    sh.nrb = (d.dim + 63) / 64;
    sh.dt_softplus = d.dt_softplus;
    sh.sort_by_length = (p.ctx != nullptr && d.batch <= 256) ? 1 : 0;
    sh.pass = p.cu_count;
    return sh;
}

template <typename ST, typename IOT, typename BCT, int NS, int NW>
hipError_t launch_prefill_cfg(const PrefillParams &p, hipStream_t stream)
{
    const DecodeParams &d = p.d;
    const PrefillShape sh = prefill_shape(p);
    const int64_t blocks = (int64_t)d.batch * d.nheads * sh.nrb;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    (void)hipGetLastError();
    hipLaunchKernelGGL((ssu_prefill_kernel<ST, IOT, BCT, NS, NW>), dim3((unsigned)blocks),
                       dim3(64 * NW), 0, stream, d.x, d.A, d.B, d.C, d.dt, d.dt_bias, d.D, d.z,
                       static_cast<ST *>(d.state), d.out, p.ctx, d.idx, p.st_dA, p.st_u, p.st_B,
                       p.st_dt, sh);
    return hipGetLastError();
}

template <typename ST, typename IOT, typename BCT>
hipError_t launch_prefill_bc(const PrefillParams &p, hipStream_t stream)
{
    if constexpr (__is_same(IOT, BCT) && (__is_same(IOT, bf16_t) || __is_same(IOT, _Float16))) {
        if (prefill_mm_fits(p)) {
            const PrefillShape sh = prefill_shape(p);
            switch (p.d.dstate) {
            case 32: return launch_prefill_mm<ST, IOT, BCT, 32>(p, sh, stream);
            case 64: return launch_prefill_mm<ST, IOT, BCT, 64>(p, sh, stream);
            case 128: return launch_prefill_mm<ST, IOT, BCT, 128>(p, sh, stream);
            case 256: return launch_prefill_mm<ST, IOT, BCT, 256>(p, sh, stream);
            default: break;
            }
        }
    }
    // Eight waves per workgroup when every CU gets at most one workgroup: a lone
    // wave issues well below its SIMD's VALU rate, so two per SIMD finish the
    // sequence sooner. With more workgroups the larger footprint would keep
    // some of them from being resident, so four waves are used.
    const bool wide = p.waves_per_wg == 8 ||
                      (p.waves_per_wg == 0 && p.cu_count > 0 &&
                       (int64_t)p.d.batch * p.d.nheads * ((p.d.dim + 63) / 64) <= p.cu_count);
    switch (p.d.dstate) {
    case 16: return launch_prefill_cfg<ST, IOT, BCT, 16, 4>(p, stream);
    case 32: return wide ? launch_prefill_cfg<ST, IOT, BCT, 32, 8>(p, stream)
                         : launch_prefill_cfg<ST, IOT, BCT, 32, 4>(p, stream);
    case 64: return wide ? launch_prefill_cfg<ST, IOT, BCT, 64, 8>(p, stream)
                         : launch_prefill_cfg<ST, IOT, BCT, 64, 4>(p, stream);
    case 128: return wide ? launch_prefill_cfg<ST, IOT, BCT, 128, 8>(p, stream)
                          : launch_prefill_cfg<ST, IOT, BCT, 128, 4>(p, stream);
    case 256: return wide ? launch_prefill_cfg<ST, IOT, BCT, 256, 8>(p, stream)
                          : launch_prefill_cfg<ST, IOT, BCT, 256, 4>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST, typename IOT>
hipError_t launch_prefill_io(const PrefillParams &p, hipStream_t stream)
{
    switch (p.d.bc_dtype) {
    case kF32: return launch_prefill_bc<ST, IOT, float>(p, stream);
    case kF16: return launch_prefill_bc<ST, IOT, _Float16>(p, stream);
    case kBF16: return launch_prefill_bc<ST, IOT, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST>
hipError_t launch_prefill_state(const PrefillParams &p, hipStream_t stream)
{
    switch (p.d.io_dtype) {
    case kF32: return launch_prefill_io<ST, float>(p, stream);
    case kF16: return launch_prefill_io<ST, _Float16>(p, stream);
    case kBF16: return launch_prefill_io<ST, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace ssu
