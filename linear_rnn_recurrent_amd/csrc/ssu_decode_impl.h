// Decode selective state update (one token per batch row): kernel template.
// Instantiated once per state dtype by ssu_decode_{f32,f16,bf16}.hip.
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page,
// mamba_ssm::invokeSelectiveStateUpdate, "Computes" paragraph):
//   state <- state * exp(A*dt') + B * dt' * x;  out = sum_n state*C + D*x;  out *= silu(z)
// with dt' = softplus(dt + dt_bias) and padding rows (negative index) skipped
// with a zero output (FlashInfer gdn_fused_decode_step page, state_indices).
//
// Mapping on gfx950: the (batch row, head) tile of dim x dstate state
// elements is contiguous in HBM and is split over ceil(dim / ROWS) workgroups
// of 256 threads (4 waves), each owning ROWS consecutive rows, about 8 KiB of
// state. Lanes run along dstate with one 16-byte vector each (4 fp32 or 8
// fp16/bf16), so every wave load or store covers 1 KiB of consecutive bytes; a
// lane issues its PASSES loads before the first FMA. State loads and stores
// carry the non-temporal hint: every byte is touched exactly once per launch,
// and keeping it out of the caches measured faster than the default policy.
// Rows past dim are loaded from the last valid row (so every load is issued
// unconditionally) and never stored. The per-row reduction over dstate is a
// butterfly across the LPR lanes of the row. The op is bound by HBM bandwidth
// (each state element is read and written once, 3 VALU ops), so no matrix
// cores are involved.
#pragma once

#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

struct DecodeShape {
    int64_t row_stride;
    int32_t nheads, dim, ngroups, heads_per_group, parts;
    int32_t dt_softplus;
};

// ST: state storage type; IOT: x/z/out storage type; BCT: B/C storage type.
template <typename ST, typename IOT, typename BCT, int NS, int PASSES>
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
    constexpr int ROWS = PASSES * RPP;

    const int tile = blockIdx.x / sh.parts;
    const int part = blockIdx.x - tile * sh.parts;
    const int b = tile / sh.nheads;
    const int h = tile - b * sh.nheads;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (LPR - 1);
    const int rsub = (threadIdx.x >> 6) * RPW + lane / LPR;
    const int64_t bh = (int64_t)b * sh.nheads + h;
    const int64_t obase = bh * sh.dim;
    const int r0 = part * ROWS;

    const int row = idx ? idx[b] : b;
    if (row < 0) {  // padding row: no state access, zero output
        for (int d = r0 + (int)threadIdx.x; d < min(sh.dim, r0 + ROWS); d += 256)
            st_elem<IOT>(out, obase + d, 0.0f);
        return;
    }

    // Every load is issued before the first use of any loaded value, state
    // first, so that a lane has all of them in flight together.
    ST *tp = state + (int64_t)row * sh.row_stride + (int64_t)h * sh.dim * NS + sub * VEC;
    u32x4 raw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = min(r0 + p * RPP + rsub, sh.dim - 1);
        raw[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(tp + (int64_t)r * NS));
    }
    // Without z the gate operand is read from x (a cached re-read, never used),
    // which keeps this load phase free of branches.
    const void *zsrc = z ? z : x;
    float xr[PASSES], zr[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int64_t o = obase + min(r0 + p * RPP + rsub, sh.dim - 1);
        xr[p] = ld_elem<IOT>(x, o);
        zr[p] = ld_elem<IOT>(zsrc, o);
    }
    const int g = h / sh.heads_per_group;
    float bv[VEC], cv[VEC];
    const int64_t bcoff = ((int64_t)b * sh.ngroups + g) * NS + sub * VEC;
    ld_typed<BCT, VEC>(Bm, bcoff, bv);
    ld_typed<BCT, VEC>(Cm, bcoff, cv);

    float v = dt[bh] + (dt_bias ? dt_bias[h] : 0.0f);
    if (sh.dt_softplus)
        v = softplus_f32(v);
    const float decay = expf(A[h] * v);
    const float dskip = Dv ? Dv[h] : 0.0f;

    // All arithmetic before the first store: on gfx9 stores share the vector
    // memory counter with loads, so a load consumed after a store would have
    // to wait for that store as well.
    float s[PASSES][VEC], part_sum[PASSES], skip[PASSES], gate[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        skip[p] = dskip * xr[p];
        gate[p] = z ? silu_f32(zr[p]) : 1.0f;
        SV<ST>::unpack(raw[p], s[p]);
        const float dtx = v * xr[p];
        part_sum[p] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            s[p][e] = fmaf(dtx, bv[e], s[p][e] * decay);
            part_sum[p] = fmaf(s[p][e], cv[e], part_sum[p]);
        }
    }
    // Pin the values derived from loads above the stores (the optimiser would
    // otherwise sink the dot products below them). Emits no instruction.
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        asm volatile("" ::"v"(part_sum[p]), "v"(skip[p]), "v"(gate[p]));
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP + rsub;
        if (r < sh.dim)
            __builtin_nontemporal_store(SV<ST>::pack(s[p]),
                                        reinterpret_cast<u32x4 *>(tp + (int64_t)r * NS));
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = r0 + p * RPP + rsub;
        const float sum = group_sum<LPR>(part_sum[p]);
        if (sub == 0 && r < sh.dim)
            st_elem<IOT>(out, obase + r, (sum + skip[p]) * gate[p]);
    }
}

template <typename ST, typename IOT, typename BCT, int NS>
hipError_t launch_decode_cfg(const DecodeParams &p, hipStream_t stream)
{
    constexpr int VEC = SV<ST>::VEC;
    constexpr int RPP = 4 * (64 / (NS / VEC));
    const int passes = p.dim > RPP ? 2 : 1;  // ~8 KiB of state per workgroup
    DecodeShape sh;
    sh.row_stride = p.row_stride;
    sh.nheads = p.nheads;
    sh.dim = p.dim;
    sh.ngroups = p.ngroups;
    sh.heads_per_group = p.nheads / p.ngroups;
    sh.parts = (p.dim + passes * RPP - 1) / (passes * RPP);
    sh.dt_softplus = p.dt_softplus;
    const int64_t blocks = (int64_t)p.batch * p.nheads * sh.parts;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const dim3 block(256);
    ST *st = static_cast<ST *>(p.state);
    (void)hipGetLastError();  // report only this launch's status
    if (passes == 2)
        hipLaunchKernelGGL((ssu_decode_kernel<ST, IOT, BCT, NS, 2>), grid, block, 0, stream, p.x,
                           p.A, p.B, p.C, p.dt, p.dt_bias, p.D, p.z, st, p.out, p.idx, sh);
    else
        hipLaunchKernelGGL((ssu_decode_kernel<ST, IOT, BCT, NS, 1>), grid, block, 0, stream, p.x,
                           p.A, p.B, p.C, p.dt, p.dt_bias, p.D, p.z, st, p.out, p.idx, sh);
    return hipGetLastError();
}

template <typename ST, typename IOT, typename BCT>
hipError_t launch_decode_bc(const DecodeParams &p, hipStream_t stream)
{
    switch (p.dstate) {
    case 16: return launch_decode_cfg<ST, IOT, BCT, 16>(p, stream);
    case 32: return launch_decode_cfg<ST, IOT, BCT, 32>(p, stream);
    case 64: return launch_decode_cfg<ST, IOT, BCT, 64>(p, stream);
    case 128: return launch_decode_cfg<ST, IOT, BCT, 128>(p, stream);
    case 256: return launch_decode_cfg<ST, IOT, BCT, 256>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST, typename IOT>
hipError_t launch_decode_io(const DecodeParams &p, hipStream_t stream)
{
    switch (p.bc_dtype) {
    case kF32: return launch_decode_bc<ST, IOT, float>(p, stream);
    case kF16: return launch_decode_bc<ST, IOT, _Float16>(p, stream);
    case kBF16: return launch_decode_bc<ST, IOT, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST>
hipError_t launch_decode_state(const DecodeParams &p, hipStream_t stream)
{
    switch (p.io_dtype) {
    case kF32: return launch_decode_io<ST, float>(p, stream);
    case kF16: return launch_decode_io<ST, _Float16>(p, stream);
    case kBF16: return launch_decode_io<ST, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace ssu
