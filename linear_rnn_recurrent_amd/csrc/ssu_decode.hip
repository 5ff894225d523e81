// Decode selective state update (one token per batch row).
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page,
// mamba_ssm::invokeSelectiveStateUpdate, "Computes" paragraph):
//   state <- state * exp(A*dt') + B * dt' * x;  out = sum_n state*C + D*x;  out *= silu(z)
// with dt' = softplus(dt + dt_bias) and padding rows (negative index) skipped
// with a zero output (FlashInfer gdn_fused_decode_step page, state_indices).
//
// Mapping on gfx950: one 256-thread workgroup (4 waves) per (batch row, head)
// tile of dim x dstate state elements, contiguous in HBM. Lanes run along
// dstate with one 16-byte vector each (4 fp32 or 8 fp16/bf16), so every wave
// load or store covers 1 KiB of consecutive bytes. A wave covers 64/LPR rows
// per pass, where LPR = dstate/VEC lanes share a row; PASSES passes of the
// four waves are issued back to back so that a lane has PASSES independent
// 16-byte loads in flight before the first FMA. The per-row reduction over
// dstate is a butterfly across the LPR lanes of the row. The op is bound by
// HBM bandwidth (each state element is read and written once, 3 VALU ops),
// so no matrix cores are involved.
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

struct DecodeShape {
    int64_t row_stride;
    int32_t nheads, dim, ngroups, heads_per_group;
    int32_t io_dtype, bc_dtype, dt_softplus;
};

template <typename ST, int NS, int PASSES>
__global__ __launch_bounds__(256) void ssu_decode_kernel(
    const void *__restrict__ x, const float *__restrict__ A, const void *__restrict__ Bm,
    const void *__restrict__ Cm, const float *__restrict__ dt, const float *__restrict__ dt_bias,
    const float *__restrict__ Dv, const void *__restrict__ z, ST *__restrict__ state,
    void *__restrict__ out, const int32_t *__restrict__ idx, const DecodeShape sh)
{
    constexpr int VEC = SV<ST>::VEC;
    constexpr int LPR = NS / VEC;  // lanes per state row
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "dstate/VEC must divide 64");
    constexpr int RPW = 64 / LPR;  // rows per wave per pass
    constexpr int RPP = 4 * RPW;   // rows per workgroup pass

    const int tile = blockIdx.x;
    const int b = tile / sh.nheads;
    const int h = tile - b * sh.nheads;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (LPR - 1);
    const int rsub = (threadIdx.x >> 6) * RPW + lane / LPR;
    const int64_t bh = (int64_t)b * sh.nheads + h;
    const int64_t obase = bh * sh.dim;

    const int row = idx ? idx[b] : b;
    if (row < 0) {  // padding row: no state access, zero output
        for (int d = threadIdx.x; d < sh.dim; d += 256)
            st_io(out, obase + d, 0.0f, sh.io_dtype);
        return;
    }

    float v = dt[bh] + (dt_bias ? dt_bias[h] : 0.0f);
    if (sh.dt_softplus)
        v = softplus_f32(v);
    const float decay = expf(A[h] * v);
    const float dskip = Dv ? Dv[h] : 0.0f;
    const int g = h / sh.heads_per_group;

    float bv[VEC], cv[VEC];
    const int64_t bcoff = ((int64_t)b * sh.ngroups + g) * NS + sub * VEC;
    ld_vec<VEC>(Bm, bcoff, sh.bc_dtype, bv);
    ld_vec<VEC>(Cm, bcoff, sh.bc_dtype, cv);

    ST *tp = state + (int64_t)row * sh.row_stride + (int64_t)h * sh.dim * NS + sub * VEC;

    for (int r0 = 0; r0 < sh.dim; r0 += PASSES * RPP) {
        u32x4 raw[PASSES];
        float xr[PASSES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = r0 + p * RPP + rsub;
            if (r < sh.dim) {
                raw[p] = *reinterpret_cast<const u32x4 *>(tp + (int64_t)r * NS);
                xr[p] = ld_io(x, obase + r, sh.io_dtype);
            } else {
                raw[p] = u32x4{0u, 0u, 0u, 0u};
                xr[p] = 0.0f;
            }
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = r0 + p * RPP + rsub;
            float s[VEC];
            SV<ST>::unpack(raw[p], s);
            const float dtx = v * xr[p];
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s[e] = fmaf(dtx, bv[e], s[e] * decay);
                part = fmaf(s[e], cv[e], part);
            }
            if (r < sh.dim)
                *reinterpret_cast<u32x4 *>(tp + (int64_t)r * NS) = SV<ST>::pack(s);
            part = group_sum<LPR>(part);
            if (sub == 0 && r < sh.dim) {
                float y = part + dskip * xr[p];
                if (z)
                    y *= silu_f32(ld_io(z, obase + r, sh.io_dtype));
                st_io(out, obase + r, y, sh.io_dtype);
            }
        }
    }
}

template <typename ST, int NS>
hipError_t launch_ns(const DecodeParams &p, hipStream_t stream)
{
    constexpr int VEC = SV<ST>::VEC;
    constexpr int RPP = 4 * (64 / (NS / VEC));
    const int need = (p.dim + RPP - 1) / RPP;
    DecodeShape sh;
    sh.row_stride = p.row_stride;
    sh.nheads = p.nheads;
    sh.dim = p.dim;
    sh.ngroups = p.ngroups;
    sh.heads_per_group = p.nheads / p.ngroups;
    sh.io_dtype = p.io_dtype;
    sh.bc_dtype = p.bc_dtype;
    sh.dt_softplus = p.dt_softplus;
    const dim3 grid((unsigned)((int64_t)p.batch * p.nheads));
    const dim3 block(256);
    ST *st = static_cast<ST *>(p.state);
    (void)hipGetLastError();  // report only this launch's status
#define SSU_LAUNCH_DECODE(PS)                                                                   \
    hipLaunchKernelGGL((ssu_decode_kernel<ST, NS, PS>), grid, block, 0, stream, p.x, p.A, p.B, \
                       p.C, p.dt, p.dt_bias, p.D, p.z, st, p.out, p.idx, sh)
    if (need >= 8)
        SSU_LAUNCH_DECODE(8);
    else if (need >= 4)
        SSU_LAUNCH_DECODE(4);
    else if (need >= 2)
        SSU_LAUNCH_DECODE(2);
    else
        SSU_LAUNCH_DECODE(1);
#undef SSU_LAUNCH_DECODE
    return hipGetLastError();
}

template <typename ST>
hipError_t launch_st(const DecodeParams &p, hipStream_t stream)
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

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream)
{
    if (p.batch == 0)
        return hipSuccess;
    switch (p.state_dtype) {
    case kF32: return launch_st<float>(p, stream);
    case kF16: return launch_st<_Float16>(p, stream);
    case kBF16: return launch_st<bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
