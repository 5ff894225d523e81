// Prefill on the matrix cores: the same operation as ssu_prefill_kernel
// (TensorRT-Edge-LLM, "Selective State Update" page,
// invokeSelectiveStateUpdatePrefill: the decode step applied to tokens
// t < L_b in order, outputs beyond L_b zero, optional replay stash with the
// committed state read-only), evaluated a chunk of 32 tokens at a time in
// closed form. Used for x/z/out and B/C both bf16 or both fp16 (exact as
// 16-bit matrix-core operands) and dstate a multiple of 32.
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
// With fp16 operands B . C^T runs on v_mfma_f32_16x16x32_f16 as it is, and
// C . S^T and B^T . X'^T with S and X' scaled per row, by the power of two that
// puts the largest magnitude in [2^14, 2^15), then cut into two fp16 parts, the
// scale undone on the fp32 result; Q . X^T (32 sources) runs on
// v_mfma_f32_16x16x4_f32 with Q as formed and x exact in fp32.
// The state never leaves registers: each lane holds S[r][16 nt + 4 qg + v],
// the accumulator layout of the last product, and the inter-chunk product
// takes it as its B operand directly by ordering the dstate index of the
// contraction as that layout does (the C operand follows the same order).
// Likewise the token index of Q . X^T is ordered as the G^T accumulator
// holds it, so Q is formed in registers.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>
#include "ssu_device.h"
#include "ssu_dpp.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

typedef float pm_f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 pm_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pm_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 pm_f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 pm_f16x2 __attribute__((ext_vector_type(2)));
typedef float pm_f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPmTT = 32;   // tokens per chunk (two 16-token MFMA tiles)
constexpr int kPmNT = 256;  // threads: four waves of 16 rows
constexpr int kPmSeg = 16;  // chunks whose decay tables are formed together

// LDS layout (bytes) of one workgroup
struct PmLds {
    int cs, bs, xs, zs, ys, lc, rd, sf, tot, big, sb, total;
};
// C, B rows: a pitch of 32 bytes past whole 64-byte runs puts consecutive rows
// 8 banks apart (of the 32 4-byte LDS banks), so the four rows a transposed
// read takes per 16 lanes (32 bytes each) cover all 32 banks; row r permutes
// the four 8-byte slots of every 32-byte block by XOR with 8 ((r / 4) % 4)
// (pm_swz), so that the 16 rows a row-major operand read touches at once (8
// bytes each, one column) fall in 16 different bank pairs as well. A 16-byte
// row store stays one 16-byte store, its halves swapped for odd r / 4.
__host__ __device__ constexpr int pm_row_pitch(int NS) { return NS * 2 + 32; }
__device__ __forceinline__ int pm_swz(int row) { return ((row >> 2) & 3) * 8; }
__host__ __device__ constexpr int pm_y_pitch() { return 64 * 4 + 16; }            // fp32 outputs
__host__ __device__ constexpr int pm_z_pitch() { return 64 * 2 + 16; }            // z rows
__host__ __device__ constexpr int pm_x_pitch() { return 64 * 2 + 32; }            // x rows (8 banks apart)
__host__ __device__ inline PmLds pm_lds(int NS)
{
    PmLds L;
    int o = 0;
    auto take = [&o](int bytes) { const int r = o; o += (bytes + 15) & ~15; return r; };
    L.cs = take(kPmTT * pm_row_pitch(NS));   // C of the chunk [t][n]
    L.bs = take(kPmTT * pm_row_pitch(NS));   // B of the chunk [j][n]
    L.xs = take(kPmTT * pm_x_pitch());       // x [j][row]
    L.zs = take(kPmTT * pm_z_pitch());       // z [t][row]
    L.ys = take(kPmTT * pm_y_pitch());       // outputs before the gate [t][row], fp32
    // decay tables of kPmSeg chunks, [chunk][token]
    L.lc = take(kPmSeg * kPmTT * 4);         // Lc[t] log2(e) (base-2 exponent)
    L.rd = take(kPmSeg * kPmTT * 4);         // 2^((Lc[j0]-Lc[j]) log2(e)) dt'_j, j0 = j's quad start
                                             // (dt'_j alone in a chunk marked in `big`)
    L.sf = take(kPmSeg * kPmTT * 4);         // w_j = e^{Lc[last]-Lc[j]} dt'_j
    L.tot = take(kPmSeg * 4);                // e^{Lc[last]}
    L.big = take(kPmSeg * 4);                // 1: a quad of the chunk spans more than 2^64 of decay
    L.sb = take(16);                         // the batch row of this workgroup
    L.total = o;
    return L;
}

// An 8-element operand from two runs of 4 bf16 in LDS: at p and at p + 32
// bytes (16 elements on)
__device__ __forceinline__ u32x4 pm_op(const unsigned char *p)
{
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(p + 32);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

typedef short pm_i16x4 __attribute__((ext_vector_type(4)));

// Eight 16-bit values of one column of a row-major [token][column] LDS tile,
// for tokens 4 qg + e and 16 + 4 qg + e (e < 4), as the MFMA operand order
// used here: ds_read_b64_tr_b16 gives lane i of each 16-lane group element
// i % 4 of the 8 bytes that lane 4 e + i / 4 addressed, for e = 0 .. 3, so
// lane s of the group addresses token row 4 qg + s / 4, columns c0 + 4 (s % 4)
// .. + 3, and lane i ends up with column c0 + i of four consecutive tokens.
// p: the lane's address in token row 4 qg + s / 4; p + hi_off: the same
// columns in token row 16 + 4 qg + s / 4
__device__ __forceinline__ u32x4 pm_op_tr(const unsigned char *p, int hi_off)
{
    typedef __attribute__((address_space(3))) pm_i16x4 *lds_v4p;
    const pm_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)p);
    const pm_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(p + hi_off));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// D += A B on the matrix cores for 16-bit operands of type T (bf16_t or
// _Float16), eight per lane given as their bits
template <typename T>
__device__ __forceinline__ pm_f32x4 pm_mfma(const u32x4 &a, const u32x4 &b, const pm_f32x4 &c)
{
    if constexpr (__is_same(T, _Float16))
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(pm_f16x8, a),
                                                      __builtin_bit_cast(pm_f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pm_bf16x8, a),
                                                       __builtin_bit_cast(pm_bf16x8, b), c, 0, 0, 0);
}

// a 16-bit value of type T (its bits) as fp32, and eight of them
template <typename T>
__device__ __forceinline__ float pm_to_f32(uint32_t h)
{
    if constexpr (__is_same(T, _Float16))
        return f16_to_f32(h);
    else
        return bf16_to_f32(h);
}
template <typename T>
__device__ __forceinline__ void pm_to_f32x8(const u32x4 &w, float (&f)[8])
{
    if constexpr (__is_same(T, _Float16)) {
        const pm_f16x8 v = __builtin_bit_cast(pm_f16x8, w);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = (float)v[e];
    } else {
        const pm_bf16x8 v = __builtin_bit_cast(pm_bf16x8, w);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = (float)v[e];
    }
}

// two fp32 values rounded to nearest-even in type T, packed into one word
template <typename T>
__device__ __forceinline__ uint32_t pm_pack2(float a, float b)
{
    if constexpr (__is_same(T, _Float16))
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((pm_f32x2){a, b}, pm_f16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((pm_f32x2){a, b}, pm_bf16x2));
}

// The largest of m over the four lanes ln + 16 q of a wave (the lanes that
// hold one row's values in the accumulator and operand layouts used here)
__device__ __forceinline__ float pm_row_max(float m)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The power of two 2^k that puts a row's largest magnitude m in [2^14, 2^15)
// (k clamped to the normal range; m = 0 gives 2^15), and its inverse
__device__ __forceinline__ void pm_row_scale(float m, float &sc, float &inv)
{
    const int k = min(max(15 - __builtin_amdgcn_frexp_expf(m), -113), 126);
    sc = __builtin_amdgcn_ldexpf(1.0f, k);
    inv = __builtin_amdgcn_ldexpf(1.0f, -k);
}

// sc f (|sc f| < 2^15) as two fp16 parts: the nearest fp16, then the nearest
// fp16 to the remainder (exact in fp32); relative error 2^-22, or 2^-25 absolute
// where the remainder falls below fp16's normal range
__device__ __forceinline__ void pm_split_f16(const float (&f)[8], float sc, u32x4 (&o)[2])
{
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const float a = f[e] * sc, b = f[e + 1] * sc;
        const pm_f16x2 p = __builtin_convertvector((pm_f32x2){a, b}, pm_f16x2);
        const pm_f16x2 q = __builtin_convertvector((pm_f32x2){a - (float)p[0], b - (float)p[1]}, pm_f16x2);
        o[0][e >> 1] = __builtin_bit_cast(uint32_t, p);
        o[1][e >> 1] = __builtin_bit_cast(uint32_t, q);
    }
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

// IOT: x/z/out type, BCT: B/C type (bf16_t or _Float16)
template <typename ST, typename IOT, typename BCT, int NS>
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
    constexpr int PC = pm_row_pitch(NS), PY = pm_y_pitch(), PZ = pm_z_pitch(), PX = pm_x_pitch();
    constexpr int NCB = NS / 8;                      // 16-byte column blocks of a B (C) row
    constexpr int NVP = (16 * NCB + NT - 1) / NT;    // token pairs x column blocks per thread
    static_assert(NS % 32 == 0, "dstate in whole 32-column steps");
    constexpr bool BCH = __is_same(BCT, _Float16);  // fp16 B/C: scaled fp16 parts of S and X'
    constexpr bool IOH = __is_same(IOT, _Float16);  // fp16 x: Q . X^T on the fp32 matrix cores

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const PmLds L = pm_lds(NS);
    unsigned char *Cs = lds + L.cs, *Bs = lds + L.bs, *Xs = lds + L.xs;
    unsigned char *Zs = lds + L.zs;
    float *Ys = reinterpret_cast<float *>(lds + L.ys);
    float *const lcs_all = reinterpret_cast<float *>(lds + L.lc);
    float *const rds_all = reinterpret_cast<float *>(lds + L.rd);
    float *const sfs_all = reinterpret_cast<float *>(lds + L.sf);
    float *const tot_all = reinterpret_cast<float *>(lds + L.tot);
    int *const big_all = reinterpret_cast<int *>(lds + L.big);
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
    // 16-byte loads (tokens 2p, 2p+1). x, z (and the outputs): token tid / 8,
    // rows 8 (tid % 8) ..+7. Every tile is stored row-major ([token][column]);
    // the operands that need it transposed read it with ds_read_b64_tr_b16.
    u32x4 rB[NVP][2], rC[NVP][2], rX, rZ;
    const int xtok = tid >> 3, xr8 = 8 * (tid & 7);  // x / z / output mapping
    const bool xrv = rbase + xr8 < Dm;               // Dm is a multiple of 8
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
        const uint32_t ox = (uint32_t)(((t0 + min(xtok, nv - 1)) * NSTR + min(rbase + xr8, Dm - 8)) * 2);
        rX = *reinterpret_cast<const u32x4 *>(xrow + ox);
        // (without z the same words of x: a load on every path, never waited for
        // out of turn)
        rZ = *reinterpret_cast<const u32x4 *>((zrow ? zrow : xrow) + ox);
    };
    // 16-bit element i of a 16-byte register group; the elements i of two
    // groups as one word (one v_perm_b32: bytes of the low or high halves)
    auto h16 = [](const u32x4 &w, int i) { return (w[i >> 1] >> (16 * (i & 1))) & 0xffffu; };
    // the same element as fp32 bits, for the stash (bf16: the bits shifted up)
    auto c32 = [&](const u32x4 &w, int i) { return __float_as_uint(pm_to_f32<BCT>(h16(w, i))); };
    auto x32 = [&](const u32x4 &w, int i) { return __float_as_uint(pm_to_f32<IOT>(h16(w, i))); };
    auto store_chunk = [&](int t0, int nv) {
#pragma unroll
        for (int k = 0; k < NVP; ++k) {
            const int v = tid + NT * k;
            if (v < 16 * NCB) {
                const int p = v & 15, col = 8 * (v >> 4);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int row = 2 * p + q;
                    const u32x4 b = rB[k][q], c = rC[k][q];
                    const int sz = pm_swz(row);
                    const bool sw = (sz & 8) != 0;  // the block's 8-byte halves swapped
                    const int o = row * PC + ((col * 2) ^ (sz & 16));
                    *reinterpret_cast<u32x4 *>(Bs + o) = sw ? u32x4{b[2], b[3], b[0], b[1]} : b;
                    *reinterpret_cast<u32x4 *>(Cs + o) = sw ? u32x4{c[2], c[3], c[0], c[1]} : c;
                }
            }
        }
        // x past the context or beyond dim as zeros (their loads were clamped)
        *reinterpret_cast<u32x4 *>(Xs + xtok * PX + xr8 * 2) = xtok < nv && xrv ? rX : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(Zs + xtok * PZ + xr8 * 2) = rZ;
    };
    // The stash stores of the staged chunk (B and x as fp32), issued after every
    // prefetched register has been read: loads and stores share one in-order
    // memory counter, so a store issued before the last use of a prefetched
    // register would be waited for there (a write round trip per chunk); here
    // the next such wait is a chunk later.
    auto stash_chunk = [&](int t0, int nv) {
        __builtin_amdgcn_sched_barrier(0);
        if (writes_B) {
#pragma unroll
            for (int k = 0; k < NVP; ++k) {
                const int v = tid + NT * k;
                const int p = v & 15, col = 8 * (v >> 4);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (v < 16 * NCB && 2 * p + q < nv) {
                        float *sb = sBrow + (uint32_t)((t0 + 2 * p + q) * G * NS + col);
#pragma unroll
                        for (int i = 0; i < 8; i += 4)
                            __builtin_nontemporal_store(u32x4{c32(rB[k][q], i), c32(rB[k][q], i + 1),
                                                              c32(rB[k][q], i + 2), c32(rB[k][q], i + 3)},
                                                        reinterpret_cast<u32x4 *>(sb + i));
                    }
                }
            }
        }
        if (stash && xtok < nv && xrv) {
            float *su = sUrow + (uint32_t)((t0 + xtok) * NSTR + xr8);
#pragma unroll
            for (int i = 0; i < 8; i += 4)
                __builtin_nontemporal_store(u32x4{x32(rX, i), x32(rX, i + 1), x32(rX, i + 2), x32(rX, i + 3)},
                                            reinterpret_cast<u32x4 *>(su + i));
        }
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
            // suf includes a_j itself; the weight of x_j in the chunk's end state
            // takes the decays after j only: the next token's suffix sum (taken
            // as it is, not as suf - a_j, which loses the small sum after an
            // extreme decay to cancellation)
            float after = __shfl_down(suf, 1, 64);
            if ((lane & 31) == 31)
                after = 0.0f;
            const float l2 = pre * 1.4426950408889634f;
            const float l2q = dpp_f32<0x00>(l2);  // quad_perm [0,0,0,0]: the quad's first token
            // Q's per-quad factoring 2^(Lc[t]-Lc[j0]) * 2^(Lc[j0]-Lc[j]) overflows
            // (inf * 0) once a quad's decays span more than ~2^127; chunks with a
            // span above 2^64 form every Q entry from its own exponent instead
            const uint64_t wide = __ballot(!(fabsf(l2q - l2) <= 64.0f));
            const bool big = ((lane & 32) ? (wide >> 32) : (wide & 0xffffffffull)) != 0;
            const int o = cl * TT + (lane & 31);
            lcs_all[o] = l2;
            rds_all[o] = big ? dtp : __builtin_amdgcn_exp2f(l2q - l2) * dtp;
            sfs_all[o] = expf(after) * dtp;
            if ((lane & 31) == 0)
                big_all[cl] = big ? 1 : 0;
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
        stash_chunk(0, min(TT, Lb));
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
        // fp16 B/C: S enters C . S^T scaled per row (this lane's row rl)
        float ssc = 1.0f, sinv = 1.0f;
        if constexpr (BCH) {
            float m = 0.0f;
#pragma unroll
            for (int nt = 0; nt < NT16; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    m = fmaxf(m, fabsf(S[nt][v]));
            pm_row_scale(pm_row_max(m), ssc, sinv);
        }
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
            // dstate order of step kk for lane group qg: 32kk+4qg+e (e<4), 32kk+16+4qg+e-4
            u32x4 cop[2], bop[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int o = (16 * t + ln) * PC + (((32 * kk + 4 * qg) * 2) ^ pm_swz(ln));
                cop[t] = pm_op(Cs + o);
                bop[t] = pm_op(Bs + o);
            }
            float sv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sv[e] = S[2 * kk][e];
                sv[4 + e] = S[2 * kk + 1][e];
            }
            u32x4 sp[2];
            if constexpr (BCH) {
                pm_split_f16(sv, ssc, sp);
            } else {
                pm_bf16x8 sb[2];
                pm_split<2>(sv, sb);
                sp[0] = __builtin_bit_cast(u32x4, sb[0]);
                sp[1] = __builtin_bit_cast(u32x4, sb[1]);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int uu = 0; uu < 2; ++uu)
                    ay[t] = pm_mfma<BCT>(cop[t], sp[uu], ay[t]);
            ag[0] = pm_mfma<BCT>(bop[0], cop[0], ag[0]);
            ag[1] = pm_mfma<BCT>(bop[0], cop[1], ag[1]);
            ag[2] = pm_mfma<BCT>(bop[1], cop[1], ag[2]);
        }

        // inter-chunk term decays to token t: lanes hold tokens 16t + 4qg + v
        // (the outputs are 16-bit: the hardware exp2 is accurate enough here; the
        // state's own weights use expf); with fp16 B/C the row scale is undone
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const float4 l4 = *reinterpret_cast<const float4 *>(lcs + 16 * t + 4 * qg);
            ay[t][0] *= __builtin_amdgcn_exp2f(l4.x) * sinv;
            ay[t][1] *= __builtin_amdgcn_exp2f(l4.y) * sinv;
            ay[t][2] *= __builtin_amdgcn_exp2f(l4.z) * sinv;
            ay[t][3] *= __builtin_amdgcn_exp2f(l4.w) * sinv;
        }

        // ---- Q in registers: lane (t = 16tt + ln, qg) element e holds source
        // j = 4qg + e (e < 4) or 16 + 4qg + e - 4, as the G^T accumulators do ----
        const float4 lj0 = *reinterpret_cast<const float4 *>(lcs + 4 * qg);
        const float4 lj1 = *reinterpret_cast<const float4 *>(lcs + 16 + 4 * qg);
        const float4 rd0 = *reinterpret_cast<const float4 *>(rds + 4 * qg);
        const float4 rd1 = *reinterpret_cast<const float4 *>(rds + 16 + 4 * qg);
        // 2^(Lc[t]-Lc[j]) dt'_j as 2^(Lc[t]-Lc[j0]) (2^(Lc[j0]-Lc[j]) dt'_j): one exp2 per quad
        const float rd[8] = {rd0.x, rd0.y, rd0.z, rd0.w, rd1.x, rd1.y, rd1.z, rd1.w};
        const float lj[8] = {lj0.x, lj0.y, lj0.z, lj0.w, lj1.x, lj1.y, lj1.z, lj1.w};
        // x^T operand in the same source order, lane (row rl, qg), read
        // transposed from the row-major x tile: this lane addresses token row
        // 4 qg + ln / 4 at rows 16 wave + 4 (ln % 4) ..+3
        const u32x4 xop = pm_op_tr(Xs + (4 * qg + (ln >> 2)) * PX + 32 * wave + 8 * (ln & 3), 16 * PX);
        float xf[8];  // the same x in fp32 (fp16 x: before the Q tiles, which use it)
        if constexpr (IOH)
            pm_to_f32x8<IOT>(xop, xf);
        // Q of token tile t: per quad, or (chunks with extreme decays) per entry
        auto q_tile = [&](auto per_entry, int t) {
            const int tq = 16 * t + ln;  // this lane's token as a Q row
            const float lt = lcs[tq];
            const float eq0 = per_entry ? 0.0f : __builtin_amdgcn_exp2f(lt - lj0.x);
            const float eq1 = (per_entry || t == 0) ? 0.0f : __builtin_amdgcn_exp2f(lt - lj1.x);
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = e < 4 ? 4 * qg + e : 12 + 4 * qg + e;
                float q = 0.0f;
                if (t == 1 || e < 4) {  // sources 16.. lie past every token of tile 0
                    const float gv = e < 4 ? ag[t][e] : ag[2][e - 4];
                    // (rows t past the chunk's end are formed too but never stored;
                    // their sources past the end have dt' = 0)
                    if (j <= tq) {
                        const float f = per_entry ? __builtin_amdgcn_exp2f(lt - lj[e]) : (e < 4 ? eq0 : eq1);
                        q = f * rd[e] * gv;
                    }
                }
                qv[e] = q;
            }
            if constexpr (IOH) {
                // fp16 x: on the fp32 matrix cores, Q as formed and x exact in
                // fp32, one 4-source step per element (lane group qg holds
                // source 4qg + e, resp. 16 + 4qg + e - 4, in both operands);
                // sources 16.. are past every token of tile 0
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t == 1 || e < 4)
                        ay[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[e], xf[e], ay[t], 0, 0, 0);
            } else {
                pm_bf16x8 qp[2];
                pm_split<2>(qv, qp);
#pragma unroll
                for (int uu = 0; uu < 2; ++uu)
                    ay[t] = pm_mfma<bf16_t>(__builtin_bit_cast(u32x4, qp[uu]), xop, ay[t]);
            }
        };
        if (__builtin_amdgcn_readfirstlane(big_all[cs]) != 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                q_tile(std::true_type{}, t);
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                q_tile(std::false_type{}, t);
        }
        // D x_t in fp32: the x^T operand holds x of tokens 4qg + v (elements
        // 0-3) and 16 + 4qg + v (4-7) of row rl, the tokens of ay[0][v], ay[1][v]
        if constexpr (!IOH)
            pm_to_f32x8<IOT>(xop, xf);
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
            const float ws = tot_all[cs];
            // B^T operand reads straight from the row-major B tile: this lane
            // addresses token row 4 qg + ln / 4 at columns 16 nt + 4 (ln % 4)
            // (the row's slot permutation is the same for row + 16)
            const int trow = 4 * qg + (ln >> 2);
            const unsigned char *btr = Bs + trow * PC + ((8 * (ln & 3)) ^ pm_swz(trow));
            if constexpr (BCH) {
                // X' scaled per row into two fp16 parts; the product, unscaled,
                // is added to the decayed state
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    m = fmaxf(m, fabsf(xw[e]));
                float xsc, xinv;
                pm_row_scale(pm_row_max(m), xsc, xinv);
                u32x4 xh[2];
                pm_split_f16(xw, xsc, xh);
#pragma unroll
                for (int nt = 0; nt < NT16; ++nt) {
                    const u32x4 bt = pm_op_tr(btr + 32 * nt, 16 * PC);
                    pm_f32x4 pr = pm_mfma<_Float16>(bt, xh[0], pm_f32x4{0.0f, 0.0f, 0.0f, 0.0f});
                    pr = pm_mfma<_Float16>(bt, xh[1], pr);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        S[nt][v] = fmaf(pr[v], xinv, S[nt][v] * ws);
                }
            } else {
                pm_bf16x8 xp[3];
                pm_split<3>(xw, xp);
#pragma unroll
                for (int nt = 0; nt < NT16; ++nt) {
                    const u32x4 bt = pm_op_tr(btr + 32 * nt, 16 * PC);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        S[nt][v] *= ws;
#pragma unroll
                    for (int uu = 0; uu < 3; ++uu)
                        S[nt] = pm_mfma<bf16_t>(bt, __builtin_bit_cast(u32x4, xp[uu]), S[nt]);
                }
            }
        }
        __syncthreads();

        // ---- gate the chunk's outputs: 8 rows of one token per thread (stored
        // below, once the next chunk is staged) ----
        const bool olive = xtok < nv && xrv;
        u32x4 ow = u32x4{0u, 0u, 0u, 0u};
        if (olive) {
            const float4 y0 = *reinterpret_cast<const float4 *>(Ys + xtok * (PY / 4) + xr8);
            const float4 y1 = *reinterpret_cast<const float4 *>(Ys + xtok * (PY / 4) + xr8 + 4);
            float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            if (zrow) {
                const u32x4 zw = *reinterpret_cast<const u32x4 *>(Zs + xtok * PZ + xr8 * 2);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float zi = pm_to_f32<IOT>((zw[i >> 1] >> (16 * (i & 1))) & 0xffffu);
                    y[i] *= zi * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * zi));
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)  // round to nearest even, two values per conversion
                ow[i] = pm_pack2<IOT>(y[2 * i], y[2 * i + 1]);
        }
        // the next chunk into LDS (z over this chunk's z: read above, in the same
        // thread), then every global store of this iteration: loads and stores
        // share one in-order memory counter, so a store issued before the last
        // use of a prefetched register would be waited for there
        store_chunk(t0 + TT, min(TT, Lb - t0 - TT));  // nothing live past the last chunk
        __builtin_amdgcn_sched_barrier(0);
        if (olive)
            *reinterpret_cast<u32x4 *>(orow + (uint32_t)(((t0 + xtok) * NSTR + rbase + xr8) * 2)) = ow;
        stash_chunk(t0 + TT, min(TT, Lb - t0 - TT));
        __syncthreads();
    }

    // ---- tokens beyond the context: zero outputs and zero stash (+0.0 is all
    // zero bits in every type), in 16-byte
    // stores (dim is a multiple of 8 and out, the x stash 16-byte aligned) ----
    {
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
        for (int i = tid; i < (T - Lb) * 8; i += NT) {  // 8 16-bit outputs per store
            const int rr = rbase + 8 * (i & 7);
            if (rr < Dm)
                *reinterpret_cast<u32x4 *>(orow + (uint32_t)(((Lb + (i >> 3)) * NSTR + rr) * 2)) = zero;
        }
        if (stash) {
            for (int i = tid; i < (T - Lb) * 16; i += NT) {  // 4 fp32 stash values per store
                const int rr = 4 * (i & 15);
                if (rbase + rr < Dm)
                    __builtin_nontemporal_store(zero, reinterpret_cast<u32x4 *>(sUrow + (uint32_t)((Lb + (i >> 4)) * NSTR + rr)));
            }
        }
    }
    if (stash && rb == 0) {
        for (int t = Lb + tid; t < T; t += NT) {
            st_dA[(bT + t) * H + h] = 0.0f;
            st_dt[(bT + t) * H + h] = 0.0f;
        }
    }
    if (writes_B) {  // B rows are 16-byte aligned (dstate a multiple of 32)
        for (int i = tid; i < (T - Lb) * (NS / 4); i += NT)
            __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                        reinterpret_cast<u32x4 *>(sBrow + (uint32_t)((Lb + i / (NS / 4)) * G * NS + 4 * (i % (NS / 4)))));
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

template <typename ST, typename IOT, typename BCT, int NS>
hipError_t launch_prefill_mm(const PrefillParams &p, const PrefillShape &sh, hipStream_t stream)
{
    const DecodeParams &d = p.d;
    const int64_t blocks = (int64_t)d.batch * d.nheads * sh.nrb;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const int lds = pm_lds(NS).total;
    auto kern = ssu_prefill_mm_kernel<ST, IOT, BCT, NS>;
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

// The matrix-core prefill takes x/z/out and B/C both bf16 or both fp16 (exact
// operands), dstate a multiple of 32, dim a multiple of 8 and 16-byte aligned x, z, out and x
// stash (whole 8-row vectors); everything else runs on ssu_prefill_kernel.
// Offsets within one batch row's tokens are formed in 32 bits: a row's x, z,
// out, B and C (and the fp32 x and B stash) must span under 2^31 bytes, with a
// factor of two to spare.
inline bool prefill_mm_fits(const PrefillParams &p)
{
    const DecodeParams &d = p.d;
    auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    const int64_t per_token = std::max((int64_t)d.nheads * d.dim, (int64_t)d.ngroups * d.dstate);
    const bool offsets_fit = (int64_t)p.seq_len * per_token * 4 < ((int64_t)1 << 31);
    const bool types = (d.io_dtype == kBF16 || d.io_dtype == kF16) && d.bc_dtype == d.io_dtype;
    return offsets_fit && types && d.dstate % 32 == 0 && d.dim % 8 == 0 &&
           al16(d.x) && al16(d.out) && (d.z == nullptr || al16(d.z)) &&
           (p.st_u == nullptr || al16(p.st_u)) && p.waves_per_wg == 0;
}

}  // namespace
}  // namespace ssu
