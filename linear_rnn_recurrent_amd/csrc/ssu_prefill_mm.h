// Prefill on the matrix cores: the same operation as ssu_prefill_kernel
// (TensorRT-Edge-LLM, "Selective State Update" page,
// invokeSelectiveStateUpdatePrefill: the decode step applied to tokens
// t < L_b in order, outputs beyond L_b zero, optional replay stash with the
// committed state read-only), evaluated a chunk of 32 tokens at a time in
// closed form. Used for bf16 x/z/out with bf16 B/C (both exact as bf16
// matrix-core operands) and dstate a multiple of 32.
//
// Within a chunk that starts from state S0 (a_k = A dt'_k, Lc[t] = sum of a_k
// over k <= t, both within the chunk):
//   y_t   = e^{Lc[t]} (S0 C_t) + sum_{j<=t} e^{Lc[t]-Lc[j]} dt'_j (B_j . C_t) x_j + D x_t
//   S_end = e^{Lc[last]} S0 + sum_j e^{Lc[last]-Lc[j]} dt'_j x_j B_j^T
// which is the token-by-token recurrence regrouped (the tree verify's closed
// form on a chain, plus the state the chain ends in). Four products per chunk
// and wave (16 rows of dim), all v_mfma_f32_16x16x32_bf16:
//   Y^T  = C . S^T            (inter-chunk term; S as bf16 hi + lo)
//   G^T  = B . C^T            (the B_j . C_t dots, lower triangle)
//   Y^T += Q . X^T            (Q[t][j] = e^{Lc[t]-Lc[j]} dt'_j G[t][j]; Q as
//                              bf16 hi + lo; D x_t added in fp32 after it)
//   S^T  = e^{Lc[last]} S^T + B^T . X'^T   (X'[r][j] = w_j x_j[r], w_j the
//                              suffix weight; X' as three bf16 terms, so the
//                              carried fp32 state keeps fp32 accuracy)
// The state never leaves registers: each lane holds S[r][16 nt + 4 qg + v],
// the accumulator layout of the last product, and the inter-chunk product
// takes it as its B operand directly by ordering the dstate index of the
// contraction as that layout does (the C operand follows the same order).
// Likewise the token index of Q . X^T is ordered as the G^T accumulator
// holds it, so Q is formed in registers.
#pragma once

#include <atomic>
#include "ssu_device.h"
#include "ssu_dpp.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

typedef float pm_f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 pm_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pm_bf16x2 __attribute__((ext_vector_type(2)));
typedef float pm_f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPmTT = 32;   // tokens per chunk (two 16-token MFMA tiles)
constexpr int kPmNT = 256;  // threads: four waves of 16 rows
constexpr int kPmSeg = 16;  // chunks whose decay tables are formed together

// LDS layout (bytes) of one workgroup
struct PmLds {
    int cs, bs, bt, xt, zs, ys, lc, rd, sf, tot, sb, total;
};
__host__ __device__ constexpr int pm_row_pitch(int NS) { return NS * 2 + 16; }   // C, B rows
__host__ __device__ constexpr int pm_t_pitch() { return kPmTT * 2 + 8; }          // B^T, x^T rows
__host__ __device__ constexpr int pm_y_pitch() { return 64 * 4 + 16; }            // fp32 outputs
__host__ __device__ constexpr int pm_z_pitch() { return 64 * 2 + 16; }            // z rows
__host__ __device__ inline PmLds pm_lds(int NS)
{
    PmLds L;
    int o = 0;
    auto take = [&o](int bytes) { const int r = o; o += (bytes + 15) & ~15; return r; };
    L.cs = take(kPmTT * pm_row_pitch(NS));   // C of the chunk [t][n]
    L.bs = take(kPmTT * pm_row_pitch(NS));   // B of the chunk [j][n]
    L.bt = take(NS * pm_t_pitch());          // B^T [n][j]
    L.xt = take(64 * pm_t_pitch());          // x^T [row][j]
    L.zs = take(kPmTT * pm_z_pitch());       // z [t][row]
    L.ys = take(kPmTT * pm_y_pitch());       // outputs before the gate [t][row], fp32
    // decay tables of kPmSeg chunks, [chunk][token]
    L.lc = take(kPmSeg * kPmTT * 4);         // Lc[t] log2(e) (base-2 exponent)
    L.rd = take(kPmSeg * kPmTT * 4);         // 2^((Lc[j0]-Lc[j]) log2(e)) dt'_j, j0 = j's quad start
    L.sf = take(kPmSeg * kPmTT * 4);         // w_j = e^{Lc[last]-Lc[j]} dt'_j
    L.tot = take(kPmSeg * 4);                // e^{Lc[last]}
    L.sb = take(16);                         // the batch row of this workgroup
    L.total = o;
    return L;
}

// An 8-element operand from two runs of 4 bf16 in LDS: at p and at p + 32
// bytes (16 elements on)
__device__ __forceinline__ pm_bf16x8 pm_op(const unsigned char *p)
{
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(p + 32);
    return __builtin_bit_cast(pm_bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// fp32 values as `terms` bf16 parts (round to nearest, the remainder split again)
template <int TERMS>
__device__ __forceinline__ void pm_split(const float (&f)[8], pm_bf16x8 (&o)[TERMS])
{
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        r[e] = f[e];
#pragma unroll
    for (int u = 0; u < TERMS; ++u) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const pm_bf16x2 p = __builtin_convertvector((pm_f32x2){r[e], r[e + 1]}, pm_bf16x2);
            o[u][e] = p[0];
            o[u][e + 1] = p[1];
            if (u + 1 < TERMS) {
                r[e] -= (float)p[0];
                r[e + 1] -= (float)p[1];
            }
        }
    }
}

template <typename ST, int NS>
__global__ __launch_bounds__(kPmNT) __attribute__((amdgpu_waves_per_eu(NS <= 128 ? 3 : 1))) void ssu_prefill_mm_kernel(
    const void *__restrict__ x, const float *__restrict__ A, const void *__restrict__ Bm,
    const void *__restrict__ Cm, const float *__restrict__ dt, const float *__restrict__ dt_bias,
    const float *__restrict__ Dv, const void *__restrict__ z, ST *__restrict__ state,
    void *__restrict__ out, const int32_t *__restrict__ ctx, const int32_t *__restrict__ idx,
    float *__restrict__ st_dA, float *__restrict__ st_u, float *__restrict__ st_B,
    float *__restrict__ st_dt, const PrefillShape sh)
{
    constexpr int TT = kPmTT;
    constexpr int NT = kPmNT;
    constexpr int KN = NS / 32;          // k-steps over dstate
    constexpr int NT16 = NS / 16;        // dstate tiles of the state
    constexpr int PC = pm_row_pitch(NS), PT = pm_t_pitch(), PY = pm_y_pitch(), PZ = pm_z_pitch();
    constexpr int NCB = NS / 8;                      // 16-byte column blocks of a B (C) row
    constexpr int NVP = (16 * NCB + NT - 1) / NT;    // token pairs x column blocks per thread
    static_assert(NS % 32 == 0, "dstate in whole 32-column steps");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const PmLds L = pm_lds(NS);
    unsigned char *Cs = lds + L.cs, *Bs = lds + L.bs, *Bt = lds + L.bt, *Xt = lds + L.xt;
    unsigned char *Zs = lds + L.zs;
    float *Ys = reinterpret_cast<float *>(lds + L.ys);
    float *const lcs_all = reinterpret_cast<float *>(lds + L.lc);
    float *const rds_all = reinterpret_cast<float *>(lds + L.rd);
    float *const sfs_all = reinterpret_cast<float *>(lds + L.sf);
    float *const tot_all = reinterpret_cast<float *>(lds + L.tot);
    int *sorted_b = reinterpret_cast<int *>(lds + L.sb);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = lane >> 4, ln = lane & 15;
    const int T = sh.seq_len, H = sh.nheads, Dm = sh.dim, G = sh.ngroups;

    // work item: as ssu_prefill_kernel (longest rows first, snake over passes)
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
        if (tid == 0)
            *sorted_b = qb;
        __syncthreads();
        for (int c = tid; c < sh.batch; c += NT) {
            const int lc = clamp_len(ctx[c], T);
            int rank = 0;
            for (int c2 = 0; c2 < sh.batch; ++c2) {
                const int l2 = clamp_len(ctx[c2], T);
                rank += (l2 > lc) || (l2 == lc && c2 < c);
            }
            if (rank == qb)
                *sorted_b = c;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(*sorted_b);
    }

    const int srow = idx ? idx[b] : b;
    const int Lb = ctx ? clamp_len(ctx[b], T) : T;
    const int64_t bT = (int64_t)b * T;
    const int rbase = rb * 64;
    const int NSTR = H * Dm;  // elements between tokens of x, z, out, st_u

    if (srow < 0) {  // padding row: outputs zero, state and stash untouched
        for (int i = tid; i < T * 64; i += NT) {
            const int r = rbase + (i & 63);
            if (r < Dm)
                st_elem<bf16_t>(out, ((bT + (i >> 6)) * H + h) * Dm + r, 0.0f);
        }
        return;
    }

    const bool stash = st_dA != nullptr;
    const int g = h / sh.heads_per_group;
    const float Ah = A[h];
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    const float dskip = Dv ? Dv[h] : 0.0f;
    const bool writes_B = stash && rb == 0 && (h % sh.heads_per_group) == 0;
    // per-row bases (elements); offsets from them are 32-bit
    const unsigned char *xrow = static_cast<const unsigned char *>(x) + (bT * H + h) * Dm * 2;
    const unsigned char *zrow = z ? static_cast<const unsigned char *>(z) + (bT * H + h) * Dm * 2 : nullptr;
    unsigned char *orow = static_cast<unsigned char *>(out) + (bT * H + h) * Dm * 2;
    const unsigned char *brow = static_cast<const unsigned char *>(Bm) + (bT * G + g) * NS * 2;
    const unsigned char *crow = static_cast<const unsigned char *>(Cm) + (bT * G + g) * NS * 2;
    const float *dtrow = dt + bT * H + h;
    // stash bases of this (batch row, head / group): token t at t H (dA, dt),
    // t NSTR (x, from the block's first row), t G NS (B)
    float *sArow = stash ? st_dA + bT * H + h : nullptr;
    float *sDrow = stash ? st_dt + bT * H + h : nullptr;
    float *sUrow = stash ? st_u + (bT * H + h) * Dm + rbase : nullptr;
    float *sBrow = writes_B ? st_B + (bT * G + g) * NS : nullptr;

    // ---- the state: lane (ln, qg) of wave w holds S[r][16 nt + 4 qg + v] ----
    const int rl = 16 * wave + ln;  // row within the block
    const int r = rbase + rl;
    const bool rv = r < Dm;
    ST *srowp = state + (int64_t)srow * sh.row_stride + (int64_t)h * Dm * NS + (int64_t)min(r, Dm - 1) * NS;
    pm_f32x4 S[NT16];

    // ---- chunk staging: global -> registers (prefetch) -> LDS ----
    // B and C: item v = (token pair p = v % 16, column block cb = v / 16), two
    // 16-byte loads (tokens 2p, 2p+1); B^T takes the pair as one 32-bit word
    // per column. x: threads < 128 take (token pair tid % 16, rows
    // 8 (tid / 16) ..+7) and x^T the pair as one word per row. z (and the
    // outputs): token tid / 8, rows 8 (tid % 8) ..+7.
    u32x4 rB[NVP][2], rC[NVP][2], rX[2], rZ;
    const int xtok = tid >> 3, xr8 = 8 * (tid & 7);  // z / output mapping
    const bool xrv = rbase + xr8 < Dm;               // Dm is a multiple of 8
    const int xp = tid & 15, xb8 = 8 * ((tid >> 4) & 7);  // x mapping (threads < 128)
    const bool xbv = rbase + xb8 < Dm;
    auto load_chunk = [&](int t0, int nv) {
#pragma unroll
        for (int k = 0; k < NVP; ++k) {
            const int v = min(tid + NT * k, 16 * NCB - 1);
            const int p = v & 15, col = 8 * (v >> 4);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tok = min(2 * p + q, nv - 1);
                const uint32_t o = (uint32_t)((((t0 + tok) * G) * NS + col) * 2);
                rB[k][q] = *reinterpret_cast<const u32x4 *>(brow + o);
                rC[k][q] = *reinterpret_cast<const u32x4 *>(crow + o);
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tok = min(2 * xp + q, nv - 1);
            rX[q] = *reinterpret_cast<const u32x4 *>(
                xrow + (uint32_t)(((t0 + tok) * NSTR + min(rbase + xb8, Dm - 8)) * 2));
        }
        // (without z the same words of x: a load on every path, never waited for
        // out of turn)
        rZ = *reinterpret_cast<const u32x4 *>(
            (zrow ? zrow : xrow) + (uint32_t)(((t0 + min(xtok, nv - 1)) * NSTR + min(rbase + xr8, Dm - 8)) * 2));
    };
    // 16-bit element i of a 16-byte register group; the elements i of two
    // groups as one word (one v_perm_b32: bytes of the low or high halves)
    auto h16 = [](const u32x4 &w, int i) { return (w[i >> 1] >> (16 * (i & 1))) & 0xffffu; };
    auto pair16 = [](const u32x4 &w0, const u32x4 &w1, int i) {
        // selector bytes 0-3 pick from w0's word, 4-7 from w1's (perm takes (hi, lo))
        return __builtin_amdgcn_perm(w1[i >> 1], w0[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
    };
    auto store_chunk = [&](int t0, int nv) {
#pragma unroll
        for (int k = 0; k < NVP; ++k) {
            const int v = tid + NT * k;
            if (v < 16 * NCB) {
                const int p = v & 15, col = 8 * (v >> 4);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    *reinterpret_cast<u32x4 *>(Bs + (2 * p + q) * PC + col * 2) = rB[k][q];
                    *reinterpret_cast<u32x4 *>(Cs + (2 * p + q) * PC + col * 2) = rC[k][q];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint32_t *>(Bt + (col + i) * PT + 4 * p) = pair16(rB[k][0], rB[k][1], i);
                if (writes_B) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        if (2 * p + q < nv) {
                            float *sb = sBrow + (uint32_t)((t0 + 2 * p + q) * G * NS + col);
#pragma unroll
                            for (int i = 0; i < 8; i += 4)
                                *reinterpret_cast<float4 *>(sb + i) =
                                    make_float4(bf16_to_f32(h16(rB[k][q], i)), bf16_to_f32(h16(rB[k][q], i + 1)),
                                                bf16_to_f32(h16(rB[k][q], i + 2)), bf16_to_f32(h16(rB[k][q], i + 3)));
                        }
                    }
                }
            }
        }
        if (tid < 128) {
            u32x4 w[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bool live = 2 * xp + q < nv && xbv;
                w[q] = live ? rX[q] : u32x4{0u, 0u, 0u, 0u};
                if (stash && live) {
                    float *su = sUrow + (uint32_t)((t0 + 2 * xp + q) * NSTR + xb8);
#pragma unroll
                    for (int i = 0; i < 8; i += 4)
                        *reinterpret_cast<float4 *>(su + i) =
                            make_float4(bf16_to_f32(h16(w[q], i)), bf16_to_f32(h16(w[q], i + 1)),
                                        bf16_to_f32(h16(w[q], i + 2)), bf16_to_f32(h16(w[q], i + 3)));
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint32_t *>(Xt + (xb8 + i) * PT + 4 * xp) = pair16(w[0], w[1], i);
        }
        *reinterpret_cast<u32x4 *>(Zs + xtok * PZ + xr8 * 2) = rZ;
    };

    // ---- decay tables of chunks c0 .. c0 + kPmSeg - 1, all four waves: wave w
    // takes chunk pairs w, w + 4 (lanes 0-31 the first chunk, 32-63 the
    // second), one token per lane (a = 0, dt' = 0 past the context); Lc by an
    // inclusive prefix scan, the suffix sums by a second scan (not as
    // differences of prefix sums: no cancellation) ----
    auto fill_tables = [&](int c0) {
        constexpr int NPASS = kPmSeg / 8;
        float rdt[NPASS];
#pragma unroll
        for (int k = 0; k < NPASS; ++k) {
            const int t = (c0 + 2 * (wave + 4 * k)) * TT + lane;
            rdt[k] = dtrow[(uint32_t)(min(t, Lb - 1) * H)];
        }
#pragma unroll
        for (int k = 0; k < NPASS; ++k) {
            const int cl = 2 * (wave + 4 * k) + (lane >> 5);  // chunk within the tables
            const int t = (c0 + 2 * (wave + 4 * k)) * TT + lane;
            float v = rdt[k] + bias;
            if (sh.dt_softplus)  // as every other kernel computes it: the same dt' bits
                v = softplus_f32(v);
            const bool live = t < Lb;
            const float dtp = live ? v : 0.0f;
            const float a = live ? Ah * v : 0.0f;
            // inclusive prefix and suffix sums within each 32-lane half (two
            // rows of 16: row sums by DPP, then the other row's total added)
            float pre = row_prefix_sum16(a), suf = row_suffix_sum16(a);
            const float p15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pre), 15));
            const float p47 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pre), 47));
            const float s16 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, suf), 16));
            const float s48 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, suf), 48));
            const int row = lane >> 4;
            if (row == 1)
                pre += p15;
            else if (row == 3)
                pre += p47;
            if (row == 0)
                suf += s16;
            else if (row == 2)
                suf += s48;
            // suf includes a_j itself: the weight of x_j in the chunk's end state
            // takes the decays after j only
            const float l2 = pre * 1.4426950408889634f;
            const float l2q = dpp_f32<0x00>(l2);  // quad_perm [0,0,0,0]: the quad's first token
            const int o = cl * TT + (lane & 31);
            lcs_all[o] = l2;
            rds_all[o] = __builtin_amdgcn_exp2f(l2q - l2) * dtp;
            sfs_all[o] = expf(suf - a) * dtp;
            if (stash && rb == 0 && live) {
                sArow[(uint32_t)(t * H)] = a;
                sDrow[(uint32_t)(t * H)] = v;
            }
            if ((lane & 31) == 31)  // the chunk's total decay
                tot_all[cl] = expf(pre);
        }
    };

    // Every load is consumed on every path: the state and the first chunk
    // before the loop, each prefetch by the same iteration's store_chunk (the
    // last iteration loads its own chunk again and stores nothing live). No
    // load is then outstanding at the loop head on any path, and the chunk's
    // matrix products do not wait for the prefetch.
    const int nchunks = (Lb + TT - 1) / TT;
    if (nchunks > 0) {
#pragma unroll
        for (int nt = 0; nt < NT16; ++nt) {
            float f[4];  // four consecutive dstate entries (the row pointer is clamped)
            cvt_raw4<ST>(ld_raw4<ST>(srowp, 16 * nt + 4 * qg), f);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                S[nt][v] = rv ? f[v] : 0.0f;
        }
        load_chunk(0, min(TT, Lb));
        fill_tables(0);
        store_chunk(0, min(TT, Lb));
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * TT;
        const int nv = min(TT, Lb - t0);
        const int tn = min(t0 + TT, (nchunks - 1) * TT);  // the next chunk, or this one again
        const int cs = c % kPmSeg;
        if (cs == 0 && c > 0) {  // the next kPmSeg chunks' tables (their readers are past the barrier)
            fill_tables(c);
            __syncthreads();
        }
        load_chunk(tn, min(TT, Lb - tn));
        // the prefetch stays here, a whole chunk of work ahead of its use (the
        // scheduler would otherwise sink it towards store_chunk to save registers)
        __builtin_amdgcn_sched_barrier(0);
        const float *lcs = lcs_all + cs * TT, *rds = rds_all + cs * TT;
        const float *sfs = sfs_all + cs * TT;

        // ---- Y^T = C . S^T and G^T = B . C^T over dstate ----
        pm_f32x4 ay[2] = {pm_f32x4{0.0f, 0.0f, 0.0f, 0.0f}, pm_f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        pm_f32x4 ag[3] = {pm_f32x4{0.0f, 0.0f, 0.0f, 0.0f}, pm_f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                          pm_f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
            // dstate order of step kk for lane group qg: 32kk+4qg+e (e<4), 32kk+16+4qg+e-4
            pm_bf16x8 cop[2], bop[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                cop[t] = pm_op(Cs + (16 * t + ln) * PC + (32 * kk + 4 * qg) * 2);
                bop[t] = pm_op(Bs + (16 * t + ln) * PC + (32 * kk + 4 * qg) * 2);
            }
            float sv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sv[e] = S[2 * kk][e];
                sv[4 + e] = S[2 * kk + 1][e];
            }
            pm_bf16x8 sp[2];
            pm_split<2>(sv, sp);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int uu = 0; uu < 2; ++uu)
                    ay[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cop[t], sp[uu], ay[t], 0, 0, 0);
            ag[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop[0], cop[0], ag[0], 0, 0, 0);
            ag[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop[0], cop[1], ag[1], 0, 0, 0);
            ag[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop[1], cop[1], ag[2], 0, 0, 0);
        }

        // inter-chunk term decays to token t: lanes hold tokens 16t + 4qg + v
        // (the outputs are bf16: the hardware exp2 is accurate enough here; the
        // state's own weights use expf)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const float4 l4 = *reinterpret_cast<const float4 *>(lcs + 16 * t + 4 * qg);
            ay[t][0] *= __builtin_amdgcn_exp2f(l4.x);
            ay[t][1] *= __builtin_amdgcn_exp2f(l4.y);
            ay[t][2] *= __builtin_amdgcn_exp2f(l4.z);
            ay[t][3] *= __builtin_amdgcn_exp2f(l4.w);
        }

        // ---- Q in registers: lane (t = 16tt + ln, qg) element e holds source
        // j = 4qg + e (e < 4) or 16 + 4qg + e - 4, as the G^T accumulators do ----
        const float4 lj0 = *reinterpret_cast<const float4 *>(lcs + 4 * qg);
        const float4 lj1 = *reinterpret_cast<const float4 *>(lcs + 16 + 4 * qg);
        const float4 rd0 = *reinterpret_cast<const float4 *>(rds + 4 * qg);
        const float4 rd1 = *reinterpret_cast<const float4 *>(rds + 16 + 4 * qg);
        // 2^(Lc[t]-Lc[j]) dt'_j as 2^(Lc[t]-Lc[j0]) (2^(Lc[j0]-Lc[j]) dt'_j): one exp2 per quad
        const float rd[8] = {rd0.x, rd0.y, rd0.z, rd0.w, rd1.x, rd1.y, rd1.z, rd1.w};
        // x^T operand in the same source order: lane (row rl, qg)
        const pm_bf16x8 xop = pm_op(Xt + rl * PT + (4 * qg) * 2);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int tq = 16 * t + ln;  // this lane's token as a Q row
            const float lt = lcs[tq];
            const float eq0 = __builtin_amdgcn_exp2f(lt - lj0.x);
            const float eq1 = t == 1 ? __builtin_amdgcn_exp2f(lt - lj1.x) : 0.0f;
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = e < 4 ? 4 * qg + e : 12 + 4 * qg + e;
                float q = 0.0f;
                if (t == 1 || e < 4) {  // sources 16.. lie past every token of tile 0
                    const float gv = e < 4 ? ag[t][e] : ag[2][e - 4];
                    // (rows t past the chunk's end are formed too but never stored;
                    // their sources past the end have dt' = 0)
                    if (j <= tq)
                        q = (e < 4 ? eq0 : eq1) * rd[e] * gv;
                }
                qv[e] = q;
            }
            pm_bf16x8 qp[2];
            pm_split<2>(qv, qp);
#pragma unroll
            for (int uu = 0; uu < 2; ++uu)
                ay[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[uu], xop, ay[t], 0, 0, 0);
        }
        // D x_t in fp32: the x^T operand holds x of tokens 4qg + v (elements
        // 0-3) and 16 + 4qg + v (4-7) of row rl, the tokens of ay[0][v], ay[1][v]
        float xf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            xf[e] = (float)xop[e];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            ay[0][v] = fmaf(dskip, xf[v], ay[0][v]);
            ay[1][v] = fmaf(dskip, xf[4 + v], ay[1][v]);
        }

        // outputs before the gate: Ys[t][row]
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                Ys[(16 * t + 4 * qg + v) * (PY / 4) + rl] = ay[t][v];

        // ---- S^T = e^{Lc[last]} S^T + B^T . X'^T ----
        {
            const float4 w0 = *reinterpret_cast<const float4 *>(sfs + 4 * qg);
            const float4 w1 = *reinterpret_cast<const float4 *>(sfs + 16 + 4 * qg);
            const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            float xw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xw[e] = wj[e] * xf[e];
            pm_bf16x8 xp[3];
            pm_split<3>(xw, xp);
            const float ws = tot_all[cs];
#pragma unroll
            for (int nt = 0; nt < NT16; ++nt) {
                const pm_bf16x8 bt = pm_op(Bt + (16 * nt + ln) * PT + (4 * qg) * 2);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    S[nt][v] *= ws;
#pragma unroll
                for (int uu = 0; uu < 3; ++uu)
                    S[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt, xp[uu], S[nt], 0, 0, 0);
            }
        }
        __syncthreads();

        // ---- gate and store the chunk's outputs: 8 rows of one token per thread ----
        if (xtok < nv && xrv) {
            const float4 y0 = *reinterpret_cast<const float4 *>(Ys + xtok * (PY / 4) + xr8);
            const float4 y1 = *reinterpret_cast<const float4 *>(Ys + xtok * (PY / 4) + xr8 + 4);
            float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            if (zrow) {
                const u32x4 zw = *reinterpret_cast<const u32x4 *>(Zs + xtok * PZ + xr8 * 2);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float zi = bf16_to_f32((zw[i >> 1] >> (16 * (i & 1))) & 0xffffu);
                    y[i] *= zi * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * zi));
                }
            }
            u32x4 ow;  // round to nearest even, two values per conversion
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ow[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((pm_f32x2){y[2 * i], y[2 * i + 1]}, pm_bf16x2));
            *reinterpret_cast<u32x4 *>(orow + (uint32_t)(((t0 + xtok) * NSTR + rbase + xr8) * 2)) = ow;
        }
        store_chunk(t0 + TT, min(TT, Lb - t0 - TT));  // nothing live past the last chunk
        __syncthreads();
    }

    // ---- tokens beyond the context: zero outputs and zero stash ----
    for (int i = tid; i < (T - Lb) * 64; i += NT) {
        const int rr = rbase + (i & 63);
        if (rr < Dm) {
            const int64_t o = ((bT + Lb + (i >> 6)) * H + h) * Dm + rr;
            st_elem<bf16_t>(out, o, 0.0f);
            if (stash)
                st_u[o] = 0.0f;
        }
    }
    if (stash && rb == 0) {
        for (int t = Lb + tid; t < T; t += NT) {
            st_dA[(bT + t) * H + h] = 0.0f;
            st_dt[(bT + t) * H + h] = 0.0f;
        }
    }
    if (writes_B) {
        for (int i = tid; i < (T - Lb) * NS; i += NT)
            st_B[((bT + Lb + i / NS) * G + g) * NS + (i % NS)] = 0.0f;
    }

    // ---- the final state (without the stash the pool row is updated) ----
    if (!stash && Lb > 0 && rv) {
        ST *sp = state + (int64_t)srow * sh.row_stride + (int64_t)h * Dm * NS + (int64_t)r * NS;
#pragma unroll
        for (int nt = 0; nt < NT16; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                st_elem<ST>(sp, 16 * nt + 4 * qg + v, S[nt][v]);
    }
}

template <typename ST, int NS>
hipError_t launch_prefill_mm(const PrefillParams &p, const PrefillShape &sh, hipStream_t stream)
{
    const DecodeParams &d = p.d;
    const int64_t blocks = (int64_t)d.batch * d.nheads * sh.nrb;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const int lds = pm_lds(NS).total;
    auto kern = ssu_prefill_mm_kernel<ST, NS>;
    if (lds > 64 * 1024) {
        // above 64 KiB of dynamic LDS the kernel must be allowed it, once per device
        static std::atomic<int> allowed[64];  // zero-initialised; benign races between host threads
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess)
                return e;
            if (dev >= 0 && dev < 64)
                allowed[dev].store(1, std::memory_order_relaxed);
        }
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kPmNT), (unsigned)lds, stream, d.x, d.A,
                       d.B, d.C, d.dt, d.dt_bias, d.D, d.z, static_cast<ST *>(d.state), d.out, p.ctx,
                       d.idx, p.st_dA, p.st_u, p.st_B, p.st_dt, sh);
    return hipGetLastError();
}

// The matrix-core prefill takes bf16 x/z/out and B/C (exact operands), dstate a
// multiple of 32, dim a multiple of 8 and 16-byte aligned x, z, out and x
// stash (whole 8-row vectors); everything else runs on ssu_prefill_kernel.
inline bool prefill_mm_fits(const PrefillParams &p)
{
    const DecodeParams &d = p.d;
    auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    return d.io_dtype == kBF16 && d.bc_dtype == kBF16 && d.dstate % 32 == 0 && d.dim % 8 == 0 &&
           al16(d.x) && al16(d.out) && (d.z == nullptr || al16(d.z)) &&
           (p.st_u == nullptr || al16(p.st_u)) && p.waves_per_wg == 0;
}

}  // namespace
}  // namespace ssu
