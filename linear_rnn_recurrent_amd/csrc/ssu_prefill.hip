// Prefill selective state update: all seq_len tokens of every batch row in one
// launch, with contextLengths and the optional replay stash.
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page,
// invokeSelectiveStateUpdatePrefill): the decode step of
// invokeSelectiveStateUpdate applied to tokens t < L_b in order, where
// L_b = clamp(contextLengths[b], 0, seq_len); outputs beyond L_b are zero.
// With the replay stash the committed state is read-only and A*dt', dt', x and
// B are stashed per token in fp32 (zeros beyond L_b).
//
// Mapping on gfx950. The recurrence is sequential in t, and every token does
// 3 VALU operations per state element against a few hundred bytes of I/O per
// (token, head), so the loop is bound by the fp32 VALU, not by HBM. The state
// therefore lives in registers for the whole sequence:
//   * a workgroup owns one (batch row, head, block of 64 rows of dim); lane =
//     row of dim, wave w = a slice of NSL dstate columns (NW waves cover dstate);
//   * per token the wave needs B and C only for its own slice and the same for
//     all 64 lanes: they are wave-uniform loads that land in scalar registers,
//     so each update is v_mul + v_fma with a scalar operand and the output dot
//     product is one v_fma per element, with no cross-lane traffic;
//   * dt' and exp(A dt') are computed once per token for a chunk of TC tokens
//     (one lane per token) and x is staged as fp32, both in LDS, double buffered;
//   * each wave writes its partial output sum per (token, row) to LDS; after the
//     chunk the workgroup adds the NW partials in a fixed order, applies D*x and
//     the gate, and stores the outputs (deterministic, no atomics);
//   * workgroups are ordered longest sequence first (rank of contextLengths
//     computed on the device, so no host read is needed).
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

struct PrefillShape {
    int64_t row_stride;
    int32_t batch, seq_len, nheads, dim, ngroups, heads_per_group, nrb;
    int32_t io_dtype, bc_dtype, dt_softplus, sort_by_length;
};

constexpr int kTC = 16;  // tokens per staged chunk

template <typename ST, typename BT, int NSL, int NW>
__global__ __launch_bounds__(64 * NW) void ssu_prefill_kernel(
    const void *__restrict__ x, const float *__restrict__ A, const void *__restrict__ Bm,
    const void *__restrict__ Cm, const float *__restrict__ dt, const float *__restrict__ dt_bias,
    const float *__restrict__ Dv, const void *__restrict__ z, ST *__restrict__ state,
    void *__restrict__ out, const int32_t *__restrict__ ctx, const int32_t *__restrict__ idx,
    float *__restrict__ st_dA, float *__restrict__ st_u, float *__restrict__ st_B,
    float *__restrict__ st_dt, const PrefillShape sh)
{
    constexpr int NS = NSL * NW;
    constexpr int NT = 64 * NW;
    constexpr int VEC = SV<ST>::VEC;
    static_assert(NSL % VEC == 0, "slice must hold whole 16-byte vectors");

    __shared__ float xs[2][kTC][64];
    __shared__ float pdt[2][kTC];
    __shared__ float pda[2][kTC];
    __shared__ float ybuf[kTC][NW][64];
    __shared__ int sorted_b;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = sh.seq_len, H = sh.nheads, Dm = sh.dim, G = sh.ngroups;
    const int per_b = H * sh.nrb;
    const int q = blockIdx.x / per_b;
    const int rem = blockIdx.x - q * per_b;
    const int h = rem % H;
    const int rb = rem / H;

    int b = q;
    if (sh.sort_by_length) {
        // b = the batch row whose length has rank q (descending, ties by index)
        if (tid == 0)
            sorted_b = q;
        __syncthreads();
        for (int c = tid; c < sh.batch; c += NT) {
            const int lc = clamp_len(ctx[c], T);
            int rank = 0;
            for (int c2 = 0; c2 < sh.batch; ++c2) {
                const int l2 = clamp_len(ctx[c2], T);
                rank += (l2 > lc) || (l2 == lc && c2 < c);
            }
            if (rank == q)
                sorted_b = c;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(sorted_b);
    }

    const int row = rb * 64 + lane;
    const bool rv = row < Dm;
    const int srow = idx ? idx[b] : b;
    const int L = ctx ? clamp_len(ctx[b], T) : T;
    const int64_t bT = (int64_t)b * T;
    const int io = sh.io_dtype;

    if (srow < 0) {  // padding row: outputs zero, state and stash untouched
        for (int i = tid; i < T * 64; i += NT) {
            const int r = rb * 64 + (i & 63);
            if (r < Dm)
                st_io(out, ((bT + (i >> 6)) * H + h) * Dm + r, 0.0f, io);
        }
        return;
    }

    const bool stash = st_dA != nullptr;
    const int g = h / sh.heads_per_group;
    const int nlo = wave * NSL;
    const float Ah = A[h];
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    const float dskip = Dv ? Dv[h] : 0.0f;
    const bool writes_B = stash && rb == 0 && (h % sh.heads_per_group) == 0;

    float S[NSL];
    ST *sp = state + (int64_t)srow * sh.row_stride + ((int64_t)h * Dm + (rv ? row : 0)) * NS + nlo;
#pragma unroll
    for (int k = 0; k < NSL / VEC; ++k) {
        const u32x4 w = rv ? reinterpret_cast<const u32x4 *>(sp)[k] : u32x4{0u, 0u, 0u, 0u};
        float e[VEC];
        SV<ST>::unpack(w, e);
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            S[k * VEC + j] = e[j];
    }

    for (int t0 = 0; t0 < L; t0 += kTC) {
        const int nt = min(kTC, L - t0);
        const int buf = (t0 / kTC) & 1;
        // ---- stage the chunk: dt', decay, x (and the stash) ----
        if (wave == 0 && lane < nt) {
            const int64_t bth = (bT + t0 + lane) * H + h;
            float v = dt[bth] + bias;
            if (sh.dt_softplus)
                v = softplus_f32(v);
            pdt[buf][lane] = v;
            pda[buf][lane] = expf(Ah * v);
            if (stash && rb == 0) {
                st_dA[bth] = Ah * v;
                st_dt[bth] = v;
            }
        }
        for (int i = tid; i < nt * 64; i += NT) {
            const int tt = i >> 6, r = i & 63, row2 = rb * 64 + r;
            float xv = 0.0f;
            if (row2 < Dm) {
                const int64_t xo = ((bT + t0 + tt) * H + h) * Dm + row2;
                xv = ld_io(x, xo, io);
                if (stash)
                    st_u[xo] = xv;
            }
            xs[buf][tt][r] = xv;
        }
        if (writes_B) {
            for (int i = tid; i < nt * NS; i += NT) {
                const int64_t o = ((bT + t0 + i / NS) * G + g) * NS + (i % NS);
                st_B[o] = ld_io(Bm, o, sh.bc_dtype);
            }
        }
        __syncthreads();
        // ---- the recurrence over the chunk, state in registers ----
        for (int tt = 0; tt < nt; ++tt) {
            const float v = pdt[buf][tt];
            const float a = pda[buf][tt];
            const float dtx = v * xs[buf][tt][lane];
            const int64_t bo = ((bT + t0 + tt) * G + g) * NS + nlo;
            float bj[NSL], cj[NSL];
            ld_bc<BT, NSL>(Bm, bo, bj);
            ld_bc<BT, NSL>(Cm, bo, cj);
            float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
#pragma unroll
            for (int j = 0; j < NSL; j += 4) {
                S[j] = fmaf(dtx, bj[j], S[j] * a);
                p0 = fmaf(S[j], cj[j], p0);
                S[j + 1] = fmaf(dtx, bj[j + 1], S[j + 1] * a);
                p1 = fmaf(S[j + 1], cj[j + 1], p1);
                S[j + 2] = fmaf(dtx, bj[j + 2], S[j + 2] * a);
                p2 = fmaf(S[j + 2], cj[j + 2], p2);
                S[j + 3] = fmaf(dtx, bj[j + 3], S[j + 3] * a);
                p3 = fmaf(S[j + 3], cj[j + 3], p3);
            }
            ybuf[tt][wave][lane] = (p0 + p1) + (p2 + p3);
        }
        __syncthreads();
        // ---- combine the dstate slices, skip term and gate; store outputs ----
        for (int i = tid; i < nt * 64; i += NT) {
            const int tt = i >> 6, r = i & 63, row2 = rb * 64 + r;
            if (row2 < Dm) {
                float y = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    y += ybuf[tt][w][r];
                const int64_t xo = ((bT + t0 + tt) * H + h) * Dm + row2;
                y += dskip * xs[buf][tt][r];
                if (z)
                    y *= silu_f32(ld_io(z, xo, io));
                st_io(out, xo, y, io);
            }
        }
    }

    // ---- tokens beyond the context: zero outputs and zero stash ----
    for (int i = tid; i < (T - L) * 64; i += NT) {
        const int r = rb * 64 + (i & 63);
        if (r < Dm) {
            const int64_t xo = ((bT + L + (i >> 6)) * H + h) * Dm + r;
            st_io(out, xo, 0.0f, io);
            if (stash)
                st_u[xo] = 0.0f;
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

    if (!stash && L > 0 && rv) {
#pragma unroll
        for (int k = 0; k < NSL / VEC; ++k) {
            float e[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                e[j] = S[k * VEC + j];
            reinterpret_cast<u32x4 *>(sp)[k] = SV<ST>::pack(e);
        }
    }
}

template <typename ST, typename BT, int NSL, int NW>
hipError_t launch_cfg(const PrefillParams &p, hipStream_t stream)
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
    sh.io_dtype = d.io_dtype;
    sh.bc_dtype = d.bc_dtype;
    sh.dt_softplus = d.dt_softplus;
    sh.sort_by_length = (p.ctx != nullptr && d.batch <= 256) ? 1 : 0;
    const dim3 grid((unsigned)((int64_t)d.batch * d.nheads * sh.nrb));
    (void)hipGetLastError();
    hipLaunchKernelGGL((ssu_prefill_kernel<ST, BT, NSL, NW>), grid, dim3(64 * NW), 0, stream, d.x,
                       d.A, d.B, d.C, d.dt, d.dt_bias, d.D, d.z, static_cast<ST *>(d.state),
                       d.out, p.ctx, d.idx, p.st_dA, p.st_u, p.st_B, p.st_dt, sh);
    return hipGetLastError();
}

template <typename ST, typename BT>
hipError_t launch_bt(const PrefillParams &p, hipStream_t stream)
{
    switch (p.d.dstate) {
    case 16: return launch_cfg<ST, BT, 16, 1>(p, stream);
    case 32: return launch_cfg<ST, BT, 16, 2>(p, stream);
    case 64: return launch_cfg<ST, BT, 16, 4>(p, stream);
    case 128: return launch_cfg<ST, BT, 32, 4>(p, stream);
    case 256: return launch_cfg<ST, BT, 32, 8>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST>
hipError_t launch_st(const PrefillParams &p, hipStream_t stream)
{
    switch (p.d.bc_dtype) {
    case kF32: return launch_bt<ST, float>(p, stream);
    case kF16: return launch_bt<ST, _Float16>(p, stream);
    case kBF16: return launch_bt<ST, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream)
{
    if (p.d.batch == 0 || p.seq_len == 0)
        return hipSuccess;
    switch (p.d.state_dtype) {
    case kF32: return launch_st<float>(p, stream);
    case kF16: return launch_st<_Float16>(p, stream);
    case kBF16: return launch_st<bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
