// Tree speculative verify: the output of every node of a draft tree, each
// computed along its own ancestor path from the read-only committed state.
// Kernel template, instantiated once per state dtype by ssu_tree_{f32,f16,bf16}.hip.
//
// Operation (TensorRT-Edge-LLM, "Selective State Update" page,
// invokeSelectiveStateUpdateDDTree): for node m, walk the parent ids from m
// to the root, run the decode step of invokeSelectiveStateUpdate along that
// path root first, starting from the committed state, and emit the output of
// m's own step; stash m's A*dt', dt', x and B for the commit of the accepted
// path.
//
// Form used here. Along a path c_k -> ... -> c_1 -> c_0 = m (root first) the
// recurrence is affine in the state, so the state after m's step is
//   S_m = w_S S0 + sum_i w_i dt'_{c_i} x_{c_i} B_{c_i}^T,
//   w_i = prod of exp(A dt') over c_0 .. c_{i-1},  w_S = prod over c_0 .. c_k,
// and m's output row is
//   y_m = w_S (S0 C_m) + sum_i [w_i dt'_{c_i} (B_{c_i} . C_m)] x_{c_i} + D x_m.
// This costs one dstate-long dot per (row, node) for S0 C_m, plus one
// dstate-long dot per (node, path entry) shared by all rows, instead of a
// full state update per path entry and row. The weights are running products
// of the per-node decays from m upwards, the same products the step-by-step
// recurrence forms.
//
// The dots B_{c_i} . C_m depend on the batch row and group only, so a first
// launch (ssu_tree_gram_kernel) forms G[b,g][m][j] = B_j . C_m for every
// j <= m (ancestors precede their node) once, for all heads, into a caller
// workspace, and copies B to the stash. The main launch then writes, per node
// and head, the dense coefficient matrix Q[m][j] = w_j dt'_j G[m][j] (zero off
// the path), and the path sum becomes a second matrix product Q . X.
//
// Mapping on gfx950 (one (batch row, head, block of 64 rows of dim) per
// 256-thread workgroup):
//   1. prologue: every global load is issued first: the state slice (straight
//      into MFMA operand registers), x of every node (16-byte vectors, kept in
//      LDS in their storage dtype), dt / parent / depth per node and C of the
//      first chunk. Per node a record {exp(A dt'), dt', parent, hop bound}
//      goes to LDS; one lane per node walks the parent ids and writes the
//      node's path (ancestor ids, node first) into a fixed slot of a
//      triangular table; each lane then keeps the x values it feeds to the
//      path product in registers;
//   2. nodes go in chunks of 16 (the N side of one MFMA tile). S0 . C_m is a
//      dense contraction [64 rows x dstate] x [dstate x nodes] on the matrix
//      cores in fp32 (v_mfma_f32_16x16x4_f32): wave w owns rows 16w .. 16w+15,
//      lane group g = lane/16 the dstate slice [g dstate/4, (g+1) dstate/4),
//      C of the chunk (LDS) is the B operand;
//   3. the 16 lanes of each chunk node take one path entry each: its decay,
//      dt' and G value (prefetched from the workspace a chunk ahead), the
//      weights as a running product across the lanes (DPP prefix product),
//      giving Q[m][j] (written into a zeroed LDS matrix, transposed) and the
//      weight w_S of S0 for the node;
//   4. after one barrier the accumulators are scaled by w_S per node and the
//      path terms are added on the matrix cores: acc += X . Q^T over the
//      source nodes j < the chunk's end (ancestors only), with X from the
//      registers of step 1; then D x, gate, store.
#pragma once

#include <atomic>
#include "ssu_device.h"
#include "ssu_dpp.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

struct TreeShape {
    int64_t row_stride;
    int32_t num_nodes, nheads, dim, ngroups, heads_per_group, nrb;
    int32_t dt_softplus;
};

constexpr int kXcds = 8;     // accelerator dies, each with its own L2
constexpr int kTreeTC = 16;   // nodes per chunk (the N side of one 16x16 MFMA tile)
constexpr int kTreeNT = 256;  // threads: four waves of 16 rows each

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// With bf16 C (exact as a bf16 MFMA operand) S0 . C runs on the bf16 matrix
// cores: S0 = hi + mid + lo, each a bf16 (round to nearest, the remainder
// split again), so each product is that of fp32 S0 to within ~2^-24 of S0 and
// the sums stay fp32; three v_mfma_f32_16x16x32_bf16 (16 cycles each) replace
// eight v_mfma_f32_16x16x4_f32 (32 cycles each) per 32 dstate columns. When
// the outputs are 16-bit, hi + mid suffice for an fp32 state (~2^-17 of S0,
// 2^6 below an fp16 output's own rounding). A 16-bit state needs fewer terms
// (bf16: hi only; fp16: hi + mid, exact).
// With bf16 x (exact as an operand) the path product X . Q^T also runs on the
// bf16 matrix cores, Q split into hi + lo bf16 terms (relative error ~2^-16
// per coefficient, far below the bf16 rounding of the outputs).
template <typename IOT>
struct TreePathSplit {
    static constexpr bool on = __is_same(IOT, bf16_t);
};

template <typename ST, typename IOT, typename BCT, int NS>
struct TreeSplit {
    static constexpr bool on = __is_same(BCT, bf16_t) && NS % 32 == 0;
    static constexpr int terms =
        __is_same(ST, bf16_t) ? 1 : (sizeof(ST) == 4 && sizeof(IOT) == 4 ? 3 : 2);
    static constexpr int T = NS / 32;  // 16x16x32 steps over dstate
};

// Waves per SIMD the register budget is cut for (5: 96 VGPRs, 4: 128): the
// most at which the operand registers (state slice, x of the path product,
// C and Q reads) fit without spilling; dstate 256 is left to the compiler.
template <typename IOT, typename BCT, int NS>
constexpr int tree_waves()
{
    if (NS <= 16 || (TreePathSplit<IOT>::on && NS <= (__is_same(BCT, bf16_t) ? 128 : 64)))
        return 5;
    return NS <= 128 ? 4 : 1;
}

// Byte offsets of the LDS arrays for a tree of M nodes (host and device).
struct TreeLds {
    int xs, cs, rec, pc, path, len, qt, cws, total;
};

__host__ __device__ inline int tree_lds_take(int &o, int bytes)
{
    const int r = o;
    o += (bytes + 15) & ~15;
    return r;
}

// Row pitches (bytes) in LDS: one 16-byte pad per row spreads the rows that
// the lanes of one instruction read together over the banks (C rows of
// dstate elements; x rows of the block's 64 rows of dim).
__host__ __device__ constexpr int tree_row_bytes(int NS, int bc_bytes) { return NS * bc_bytes + 16; }
// (16-bit x: an 8-byte pad, which already puts the four lane groups of the
// path-operand reads, 8 nodes apart, on disjoint banks)
__host__ __device__ constexpr int tree_x_pitch(int io_bytes) { return 64 * io_bytes + (io_bytes == 2 ? 8 : 16); }
// source-node rows of the coefficient matrix: every chunk's range, padded
__host__ __device__ constexpr int tree_q_rows(int M) { return (M + 15) & ~15; }
// row pitch (elements) of Q in its split-bf16 form [term][node][source]: whole
// 32-source MFMA steps plus a 16-byte pad against bank conflicts
__host__ __device__ constexpr int tree_q_pitch(int M) { return ((M + 31) & ~31) + 8; }

__host__ __device__ inline TreeLds tree_lds(int M, int NS, int io_bytes, int bc_bytes)
{
    TreeLds L;
    int o = 0;
    const int rb = tree_row_bytes(NS, bc_bytes);
    // x [M][64 rows] is staged here until every lane holds its share of it
    // in registers; the same bytes then hold the chunk coefficients Q, double
    // buffered: fp32 Q^T [source][chunk node] or the split-bf16 [2 terms]
    // [chunk node][source pitch] (the larger of the two)
    const int xs_bytes = ((M + 31) & ~31) * tree_x_pitch(io_bytes);  // whole 32-node steps
    const int q_bytes = 2 * kTreeTC * tree_q_pitch(M) * 4;
    L.xs = L.qt = tree_lds_take(o, xs_bytes > q_bytes ? xs_bytes : q_bytes);
    L.cs = tree_lds_take(o, kTreeTC * rb);                // C of the current chunk [TC][NS]
    L.rec = tree_lds_take(o, M * 8);                      // {exp(A dt'), dt'} per node
    L.pc = tree_lds_take(o, M * 4);                       // {parent, hop bound} per node
    L.path = tree_lds_take(o, M * (M + 1) / 2);           // path of node m at m(m+1)/2
    L.len = tree_lds_take(o, M);                          // path lengths (<= 128)
    L.cws = tree_lds_take(o, kTreeTC * 4);                // weights of S0 of the chunk's nodes
    L.total = o;
    return L;
}

// Triangular table slot of node m's path (m(m+1)/2, 32-bit).
__device__ __forceinline__ uint32_t tri(int m) { return ((uint32_t)m * (uint32_t)(m + 1)) >> 1; }

// fp32 at a 32-bit byte offset from a base (the offset zero-extends, so the
// access takes a scalar base and one vector offset register).
__device__ __forceinline__ float ld_f32_at(const float *base, uint32_t byte_off)
{
    return *reinterpret_cast<const float *>(reinterpret_cast<const unsigned char *>(base) + byte_off);
}

// n consecutive storage-dtype elements (16-bit or fp32) as fp32, from LDS or
// global memory; n * element size is a multiple of 8 bytes and the address is
// aligned to it.
template <typename T, int N>
__device__ __forceinline__ void ld_row_f32(const unsigned char *p, float (&f)[N])
{
    if constexpr (sizeof(T) == 4) {
        static_assert(N % 4 == 0, "fp32 rows go in 16-byte pieces");
#pragma unroll
        for (int k = 0; k < N; k += 4) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(p + 4 * k);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[k + e] = __uint_as_float(w[e]);
        }
    } else if constexpr (N % 8 == 0) {
#pragma unroll
        for (int k = 0; k < N; k += 8) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(p + 2 * k);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[k + 2 * e] = cvt_raw1<T>(w[e] & 0xffffu);
                f[k + 2 * e + 1] = cvt_raw1<T>(w[e] >> 16);
            }
        }
    } else {
        static_assert(N == 4, "16-bit rows go in 8- or 16-byte pieces");
        const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            f[2 * e] = cvt_raw1<T>(w[e] & 0xffffu);
            f[2 * e + 1] = cvt_raw1<T>(w[e] >> 16);
        }
    }
}

// G[b,g][m][j] = B_j . C_m (fp32) for j <= m, on the matrix cores: the
// 16 x 16 tiles (node block mb, source block jb <= mb) of every (b, g), one
// tile per wave, four per workgroup. With 16-bit B and C the tile is
// v_mfma_f32_16x16x32_{bf16,f16} over dstate (the products are exact, the
// sums fp32), else v_mfma_f32_16x16x4_f32. The lane holding G[m][j..j+3]
// writes it as one vector; entries above the diagonal of a diagonal tile are
// written too (the verify kernel never reads them). Padded batch rows are
// skipped.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename BCT, int NS>
__global__ __launch_bounds__(kTreeNT) void ssu_tree_gram_kernel(
    const void *__restrict__ Bm, const void *__restrict__ Cm, const int32_t *__restrict__ idx,
    float *__restrict__ gram, int32_t M, int32_t G)
{
    constexpr int BB = (int)sizeof(BCT);
    constexpr bool MF16 = BB == 2 && NS % 32 == 0;  // 16x16x32 on 16-bit operands
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qg = lane >> 4, ln = lane & 15;
    const int nmb = (M + 15) / 16;
    const int ntile = nmb * (nmb + 1) / 2;
    const int nq = (ntile + 3) / 4;  // workgroups per (b, g)
    // (the workgroups of one (b, g) on one XCD, as in the verify kernel)
    int wg = blockIdx.x;
    if (gridDim.x % kXcds == 0)
        wg = (wg % kXcds) * (gridDim.x / kXcds) + wg / kXcds;
    const int bg = wg / nq;
    const int q = wg - bg * nq;
    const int b = bg / G, g = bg - b * G;
    if (idx && idx[b] < 0)
        return;
    // the rows of (b, g): node n at n G NS elements
    const unsigned char *brow = static_cast<const unsigned char *>(Bm) + ((int64_t)b * M * G + g) * NS * BB;
    const unsigned char *crow = static_cast<const unsigned char *>(Cm) + ((int64_t)b * M * G + g) * NS * BB;
    const uint32_t nstride = (uint32_t)G * NS * BB;
    const int k = 4 * q + wave;  // tile k = mb (mb + 1) / 2 + jb
    if (k < ntile) {
        int mb = 0;
        while ((mb + 1) * (mb + 2) / 2 <= k)
            ++mb;
        const int jb = k - mb * (mb + 1) / 2;
        const uint32_t jn = min(16 * jb + ln, M - 1), mn = min(16 * mb + ln, M - 1);
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (MF16) {
            // A: B_{16 jb + ln}[32 t + 8 qg ..], B: C_{16 mb + ln}[32 t + 8 qg ..]
            u32x4 av[NS / 32], bv[NS / 32];
#pragma unroll
            for (int t = 0; t < NS / 32; ++t) {
                av[t] = *reinterpret_cast<const u32x4 *>(brow + jn * nstride + (32 * t + 8 * qg) * BB);
                bv[t] = *reinterpret_cast<const u32x4 *>(crow + mn * nstride + (32 * t + 8 * qg) * BB);
            }
#pragma unroll
            for (int t = 0; t < NS / 32; ++t) {
                if constexpr (__is_same(BCT, bf16_t))
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[t]),
                                                                  __builtin_bit_cast(bf16x8, bv[t]), acc, 0, 0, 0);
                else
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[t]),
                                                                 __builtin_bit_cast(f16x8, bv[t]), acc, 0, 0, 0);
            }
        } else {
            // lane group qg sums the dstate slice [qg NS/4, (qg+1) NS/4)
            constexpr int KS = NS / 4;
            float ca[KS], bw[KS];
            ld_row_f32<BCT, KS>(crow + mn * nstride + qg * KS * BB, ca);
            ld_row_f32<BCT, KS>(brow + jn * nstride + qg * KS * BB, bw);
#pragma unroll
            for (int s = 0; s < KS; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bw[s], ca[s], acc, 0, 0, 0);
        }
        // acc[v] = B_{16 jb + 4 qg + v} . C_{16 mb + ln}
        const int m = 16 * mb + ln, j0 = 16 * jb + 4 * qg;
        if (m < M) {
            float *gp = gram + ((int64_t)bg * M + m) * M + j0;
            if (M % 4 == 0 && j0 < M && (reinterpret_cast<uintptr_t>(gram) & 15) == 0) {
                *reinterpret_cast<float4 *>(gp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (j0 + v < M)
                        gp[v] = acc[v];
            }
        }
    }
}

template <typename ST, typename IOT, typename BCT, int NS>
__global__ __launch_bounds__(kTreeNT) __attribute__((amdgpu_waves_per_eu(tree_waves<IOT, BCT, NS>()))) void ssu_tree_kernel(
    const void *__restrict__ x, const float *__restrict__ A, const void *__restrict__ Cm,
    const float *__restrict__ dt, const float *__restrict__ dt_bias, const float *__restrict__ Dv,
    const void *__restrict__ z, const ST *__restrict__ state, void *__restrict__ out,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ depths, const float *__restrict__ gram, const void *__restrict__ Bm,
    float *__restrict__ st_dA, float *__restrict__ st_u, float *__restrict__ st_B, float *__restrict__ st_dt,
    const TreeShape sh)
{
    constexpr int NT = kTreeNT;
    constexpr int TC = kTreeTC;
    constexpr int MX = SSU_MAX_TREE_NODES;
    constexpr int KS = NS / 4;                        // dstate columns per lane group
    constexpr int XB = (int)sizeof(IOT), BB = (int)sizeof(BCT);
    constexpr int RB = tree_row_bytes(NS, BB);        // LDS row pitch of C
    constexpr int XP = tree_x_pitch(XB);              // LDS row pitch of x
    constexpr int CV = (TC * NS * BB / 16 + NT - 1) / NT;  // 16-byte C vectors per thread
    constexpr int XV = 16 / XB;                       // x elements per 16-byte vector
    constexpr int BVE = 16 / BB;                      // C elements per 16-byte vector
    constexpr int XVEC = (MX * 64 / XV + NT - 1) / NT;  // x vectors per thread
    constexpr int NPT = (MX + NT - 1) / NT;           // node records per thread
    static_assert(KS % 4 == 0 && (KS * BB) % 8 == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int M = sh.num_nodes;
    const TreeLds L = tree_lds(M, NS, XB, BB);
    const int RM = tree_q_rows(M);
    unsigned char *xs = lds + L.xs;
    unsigned char *cs = lds + L.cs;
    float2 *rec = reinterpret_cast<float2 *>(lds + L.rec);  // {exp(A dt'), dt'}
    int *n_pc = reinterpret_cast<int *>(lds + L.pc);         // parent (low 16 bits), hop bound
    uint8_t *n_path = lds + L.path;                          // triangular path table
    uint8_t *n_len = lds + L.len;
    float *qt = reinterpret_cast<float *>(lds + L.qt);       // 2 x [RM][TC] (fp32 form)
    constexpr bool PX = TreePathSplit<IOT>::on;
    const int QP = tree_q_pitch(M);
    uint16_t *qs = reinterpret_cast<uint16_t *>(lds + L.qt);  // 2 x [2][TC][QP] (split form)
    float *c_wS = reinterpret_cast<float *>(lds + L.cws);    // [TC]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = lane >> 4;     // lane group: dstate slice / source node (MFMA A/B), row quad (D)
    const int ln = lane & 15;     // MFMA A row / B and D column (node of the chunk)
    const int H = sh.nheads, Dm = sh.dim, G = sh.ngroups;
    const int per_b = H * sh.nrb;
    // workgroup i runs on XCD i % 8: the workgroups of one batch row (which
    // share its C, B and G) are given consecutive slots of one XCD, so that
    // its L2 serves them (identity when the grid is not a multiple of 8)
    int wg = blockIdx.x;
    if (gridDim.x % kXcds == 0)
        wg = (wg % kXcds) * (gridDim.x / kXcds) + wg / kXcds;
    const int b = wg / per_b;
    const int rem = wg - b * per_b;
    const int h = rem % H;
    const int rb = rem / H;
    const int64_t bM = (int64_t)b * M;
    const int rbase = rb * 64;

    const int srow = idx ? idx[b] : b;
    if (srow < 0) {  // padding row: outputs zero, stash untouched
        for (int i = tid; i < M * 64; i += NT) {
            const int r = rbase + (i & 63);
            if (r < Dm)
                st_elem<IOT>(out, ((bM + (i >> 6)) * H + h) * Dm + r, 0.0f);
        }
        return;
    }

    const bool stash = st_dA != nullptr;
    const int g = h / sh.heads_per_group;
    const float *gbg = gram + ((int64_t)b * G + g) * M * M;  // G[m][j] of this (b, g)
    // out and z of this (batch row, head): node m, row r at m H Dm + r
    void *obase = static_cast<unsigned char *>(out) + (bM * H + h) * Dm * XB;
    const void *zbase = z ? static_cast<const unsigned char *>(z) + (bM * H + h) * Dm * XB : nullptr;
    const bool ovec = Dm % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & (4 * XB - 1)) == 0;
    // per-(batch row, head) bases; the offsets from them below are 32-bit
    const int NSTR = H * Dm;                                  // elements between nodes
    const float *dtb = dt + bM * H + h;                       // dt of node m at m H
    const unsigned char *xbase = static_cast<const unsigned char *>(x) + (bM * H + h) * Dm * XB;
    float *ubase = stash ? st_u + (bM * H + h) * Dm : nullptr;
    const float Ah = A[h];
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    const float dskip = Dv ? Dv[h] : 0.0f;

    // ---- 1. prologue: every global load first ----
    // MFMA A operand, fp32 form: lane (ln, qg) of wave w holds
    // S0[row 16 w + ln][qg KS + s]; split-bf16 form: S0[row][32 t + 8 qg + e]
    // as `terms` bf16 parts per element
    using SP = TreeSplit<ST, IOT, BCT, NS>;
    const int arow = rbase + 16 * wave + ln;
    float sa[SP::on ? 1 : KS];
    bf16x8 sb[SP::on ? SP::terms * SP::T : 1];
    {
        const ST *sp = state + (int64_t)srow * sh.row_stride + (int64_t)h * Dm * NS +
                       (int64_t)min(arow, Dm - 1) * NS;
        if constexpr (SP::on) {
#pragma unroll
            for (int t = 0; t < SP::T; ++t) {
                float r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    r[e] = ld_elem<ST>(sp, 32 * t + 8 * qg + e);
                // two elements per conversion (v_cvt_pk_bf16_f32, round to nearest)
#pragma unroll
                for (int u = 0; u < SP::terms; ++u) {
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const bf16x2 p = __builtin_convertvector((f32x2){r[e], r[e + 1]}, bf16x2);
                        sb[u * SP::T + t][e] = p[0];
                        sb[u * SP::T + t][e + 1] = p[1];
                        if (u + 1 < SP::terms) {
                            r[e] -= (float)p[0];
                            r[e + 1] -= (float)p[1];
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < KS; ++s)
                sa[s] = ld_elem<ST>(sp, qg * KS + s);
        }
    }
    // per node: dt, parent id, hop bound
    float ndt[NPT];
    int npar[NPT], ncap[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const uint32_t m = min(tid + NT * k, M - 1);
        ndt[k] = dtb[m * H];
        npar[k] = parents[bM + m];
        ncap[k] = depths ? depths[bM + m] : m;
    }
    // C of chunk c: 16-byte vectors of the storage dtype (nodes past M clamp to M-1)
    u32x4 rc[CV];
    const unsigned char *cbase = static_cast<const unsigned char *>(Cm) + (bM * G + g) * NS * BB;
    auto load_c = [&](int t0) {
#pragma unroll
        for (int k = 0; k < CV; ++k) {
            const int v = tid + NT * k;               // vector v: node v / (NS/BVE)
            const int m = min(t0 + v / (NS / BVE), M - 1);
            rc[k] = *reinterpret_cast<const u32x4 *>(
                cbase + (uint32_t)(m * (G * NS * BB) + 16 * (v % (NS / BVE))));
        }
    };
    auto store_c = [&]() {
#pragma unroll
        for (int k = 0; k < CV; ++k) {
            const int v = tid + NT * k;
            if (v < TC * NS / BVE)
                *reinterpret_cast<u32x4 *>(cs + (v / (NS / BVE)) * RB + (v % (NS / BVE)) * 16) =
                    rc[k];
        }
    };
    load_c(0);
    // x of every node, rows of the block, as 16-byte vectors when dim allows
    // (vector v: node v / (64/XV), rows XV*(v % (64/XV)) ..); rows past dim are 0
    const bool xvec = Dm % XV == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                      (!stash || (reinterpret_cast<uintptr_t>(st_u) & 15) == 0);
    if (xvec) {
        constexpr int VPN = 64 / XV;  // vectors per node
        const int nvec = M * VPN;
        u32x4 xr[XVEC];
#pragma unroll
        for (int k = 0; k < XVEC; ++k) {
            const int v = min(tid + NT * k, nvec - 1);
            const int r = min(rbase + XV * (v % VPN), Dm - XV);
            xr[k] = *reinterpret_cast<const u32x4 *>(xbase + (uint32_t)(((v / VPN) * NSTR + r) * XB));
        }
#pragma unroll
        for (int k = 0; k < XVEC; ++k) {
            const int v = tid + NT * k;
            if (v < nvec) {
                const int m = v / VPN, rl = XV * (v % VPN);
                const bool valid = rbase + rl < Dm;
                u32x4 w = xr[k];
                if (!valid)
                    w = u32x4{0u, 0u, 0u, 0u};
                unsigned char *xw = xs + m * XP + rl * XB;  // 8-byte aligned at least
                if constexpr (XP % 16 == 0) {
                    *reinterpret_cast<u32x4 *>(xw) = w;
                } else {
                    reinterpret_cast<u32x2 *>(xw)[0] = u32x2{w[0], w[1]};
                    reinterpret_cast<u32x2 *>(xw)[1] = u32x2{w[2], w[3]};
                }
            }
        }
        // (the fp32 x stash of this path is written after the chunk loop)
    } else {
        for (int e = tid; e < M * 64; e += NT) {
            const int m = e >> 6, rl = e & 63, r = rbase + rl;
            uint32_t w = 0;
            if (r < Dm) {
                const int64_t o = ((bM + m) * H + h) * Dm + r;
                w = ld_raw1<IOT>(x, o);
                if (stash)
                    st_u[o] = cvt_raw1<IOT>(w);
            }
            if constexpr (XB == 4)
                *reinterpret_cast<uint32_t *>(xs + m * XP + rl * 4) = w;
            else
                *reinterpret_cast<uint16_t *>(xs + m * XP + rl * 2) = (uint16_t)w;
        }
    }
    // node records {decay exp(A dt'), dt'} and {parent id (-1 unless it
    // precedes the node), hop bound}
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int m = tid + NT * k;
        if (m < M) {
            float v = ndt[k] + bias;
            if (sh.dt_softplus)
                v = softplus_f32(v);
            const int p = npar[k];
            rec[m] = make_float2(expf(Ah * v), v);
            // a walk never takes more than m hops, and a bound below 0 acts as 0
            const int cap = max(0, min(ncap[k], m));
            n_pc[m] = (int)(uint16_t)(p >= 0 && p < m ? p : -1) | (cap << 16);
            if (stash && rb == 0) {
                const int64_t o = (bM + m) * H + h;
                st_dA[o] = Ah * v;
                st_dt[o] = v;
            }
        }
    }
    // B of every node to the fp32 stash: the workgroups of row block 0 of
    // the group's heads take equal shares of the nodes
    if (st_B && rb == 0) {
        const int hpg = sh.heads_per_group;
        const int R = (M + hpg - 1) / hpg, n0 = (h - g * hpg) * R, n1 = min(M, n0 + R);
        const unsigned char *brow = static_cast<const unsigned char *>(Bm) + (bM * G + g) * NS * BB;
        float *sbrow = st_B + (bM * G + g) * NS;
        for (int e = tid; e < (n1 - n0) * (NS / 4); e += NT) {
            const int n = n0 + e / (NS / 4), c4 = 4 * (e % (NS / 4));
            float f[4];
            ld_row_f32<BCT, 4>(brow + (uint32_t)((n * G * NS + c4) * BB), f);
            *reinterpret_cast<float4 *>(sbrow + (uint32_t)(n * G * NS + c4)) = make_float4(f[0], f[1], f[2], f[3]);
        }
    }
    // x rows of the nodes past M up to a whole 32-node step read as zeros
    for (int i = tid; i < (((M + 31) & ~31) - M) * XP / 8; i += NT)
        *reinterpret_cast<u32x2 *>(xs + M * XP + 8 * i) = u32x2{0u, 0u};
    store_c();
    __syncthreads();

    // ---- the path of every node (one lane per node), node first ----
    for (int m = tid; m < M; m += NT) {
        uint8_t *pp = n_path + tri(m);
        const int cap = n_pc[m] >> 16;
        int j = m, hops = 0;
        while (true) {
            pp[hops] = (uint8_t)j;
            const int p = (int16_t)n_pc[j];
            if (hops >= cap || p < 0)
                break;
            j = p;
            ++hops;
        }
        n_len[m] = hops + 1;
    }
    // this lane's MFMA A operand of the path product: x_{4s+qg}[row 16w+ln]
    // (fp32 form) or x_{32t+8qg+e}[row 16w+ln] (bf16 form)
    float xa[PX ? 1 : MX / 4];
    bf16x8 xb[PX ? MX / 32 : 1];
    {
        // this lane's row; the staging holds whole 32-node steps (zero past M)
        const unsigned char *xl = xs + (16 * wave + ln) * XB;
        if constexpr (PX) {
#pragma unroll
            for (int t = 0; t < MX / 32; ++t) {
                xb[t] = bf16x8{};
                if (32 * t < M) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xb[t][e] = __builtin_bit_cast(
                            __bf16, *reinterpret_cast<const uint16_t *>(xl + (32 * t + 8 * qg + e) * XP));
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < MX / 4; ++s) {
                float v = 0.0f;
                if (4 * s < M) {
                    const unsigned char *p = xl + (4 * s + qg) * XP;
                    if constexpr (XB == 4)
                        v = *reinterpret_cast<const float *>(p);
                    else
                        v = cvt_raw1<IOT>(*reinterpret_cast<const uint16_t *>(p));
                }
                xa[s] = v;
            }
        }
    }
    __syncthreads();  // x staging read by every lane; paths in place

    // G value of this lane's path entry (entry tid%16 of chunk node tid/16) of
    // the chunk starting at t0; entries past 16 are read in the loop below
    // (issued on every lane, at a clamped entry, so that no branch hides the
    // load from the wait counting: a wait for it then leaves the later
    // loads in flight; lanes past the path never use the value)
    auto load_g = [&](int t0) {
        const int m = min(t0 + (tid >> 4), M - 1), l = tid & 15;
        const int j = n_path[tri(m) + min(l, (int)n_len[m] - 1)];
        return ld_f32_at(gbg, (m * M + j) * 4u);
    };
    float gcur = load_g(0);
    // both coefficient buffers (over the x staging) start at zero; from then
    // on each chunk clears the entries that the chunk before it set
    {
        constexpr int QB = PX ? 2 * 2 * TC * 2 : 2 * TC * 4;  // bytes per unit of QP / RM
        const int n16 = (PX ? QP : RM) * QB / 16;
        u32x4 *q = reinterpret_cast<u32x4 *>(lds + L.qt);
        for (int i = tid; i < n16; i += NT)
            q[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    const int nchunks = (M + TC - 1) / TC;
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * TC;
        const int nt = min(TC, M - t0);
        const int mo = t0 + ln;                       // this lane's output node
        const int orow = rbase + 16 * wave + 4 * qg;  // and its first output row
        float *q = qt + (c & 1) * RM * TC;
        uint16_t *qc = qs + (c & 1) * 2 * TC * QP;

        // S0 . C: 16 rows x 16 nodes per wave on the matrix cores, four
        // independent accumulators so that the MFMAs issue back to back
        constexpr int NACC = SP::on ? 2 : 4;  // a 16-cycle bf16 MFMA needs two in flight
        f32x4 acc4[NACC];
#pragma unroll
        for (int a4 = 0; a4 < NACC; ++a4)
            acc4[a4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (SP::on) {
            // B operand: C_{node ln}[32 t + 8 qg .. + 7], one 16-byte LDS read
            const unsigned char *cb = cs + ln * RB + 16 * qg;
            bf16x8 cv[SP::T];
#pragma unroll
            for (int t = 0; t < SP::T; ++t)
                cv[t] = *reinterpret_cast<const bf16x8 *>(cb + 64 * t);
#pragma unroll
            for (int t = 0; t < SP::T; ++t)
#pragma unroll
                for (int u = 0; u < SP::terms; ++u)
                    acc4[(u + t) % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        sb[u * SP::T + t], cv[t], acc4[(u + t) % NACC], 0, 0, 0);
        } else {
            const unsigned char *cb = cs + ln * RB + qg * KS * BB;
#pragma unroll
            for (int s0 = 0; s0 < KS; s0 += 4) {
                float cv[4];
                ld_row_f32<BCT, 4>(cb + s0 * BB, cv);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc4[e % NACC] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(sa[s0 + e], cv[e], acc4[e % NACC], 0, 0, 0);
            }
        }

        // next chunk's C and G values, in flight during the coefficients
        // (unconditional: past the last chunk they read clamped nodes). G
        // goes first: the wait for C before it is stored to LDS then also
        // covers G, and the end-of-chunk hand-over of G waits for nothing
        const float gnext = load_g(t0 + TC);
        load_c(t0 + TC);

        // coefficients: the 16 lanes of chunk node tt take path entries
        // l, l+16, ..; w of entry i is the product of the decays of entries
        // 0 .. i-1 (a running product across the lanes, carried across blocks)
        {
            const int tt = tid >> 4, l = tid & 15;
            const int m = t0 + tt;
            const int len = tt < nt ? n_len[m] : 0;   // uniform over the node's 16 lanes
            const uint8_t *pp = n_path + (tt < nt ? tri(m) : 0u);
            float carry = 1.0f;
            for (int i0 = 0; i0 < len; i0 += 16) {
                const int i = i0 + l;
                const bool v = i < len;
                const int j = v ? pp[i] : m;
                const float2 r = rec[j];
                const float gv = i0 == 0 ? gcur : (v ? ld_f32_at(gbg, (m * M + j) * 4u) : 0.0f);
                const float incl = row_prefix_prod16(v ? r.x : 1.0f);
                const float excl = dpp_f32_fill<0x111>(1.0f, incl);  // row_shr:1
                if (v) {
                    // entry 0 is the node itself (the only j == m): D x_m joins
                    // the path sum
                    const float qv = carry * excl * r.y * gv + (j == m ? dskip : 0.0f);
                    if constexpr (PX) {
                        const __bf16 hi = (__bf16)qv;
                        qc[tt * QP + j] = __builtin_bit_cast(uint16_t, hi);
                        qc[(TC + tt) * QP + j] =
                            __builtin_bit_cast(uint16_t, (__bf16)(qv - (float)hi));
                    } else {
                        q[j * TC + tt] = qv;
                    }
                }
                carry *= __shfl(incl, (lane & ~15) | 15, 64);
            }
            if (l == 0 && tt < nt)
                c_wS[tt] = carry;
            // back to zero: the entries chunk c - 1 set in the other buffer
            // (every lane read them before the last barrier; chunk c + 1
            // writes there after the next one). Chunks before the last are full.
            if (c > 0) {
                const int mp = m - TC;
                const int lenp = n_len[mp];
                const uint8_t *ppp = n_path + tri(mp);
                for (int i = l; i < lenp; i += 16) {
                    const int j = ppp[i];
                    if constexpr (PX) {
                        uint16_t *qo = qs + ((c - 1) & 1) * 2 * TC * QP;
                        qo[tt * QP + j] = 0;
                        qo[(TC + tt) * QP + j] = 0;
                    } else {
                        qt[((c - 1) & 1) * RM * TC + j * TC + tt] = 0.0f;
                    }
                }
            }
        }
        __syncthreads();
        if (c + 1 < nchunks)
            store_c();  // every read of this chunk's C is done

        // outputs held in the accumulators: node mo, rows orow .. orow+3
        {
            // gate inputs of this lane's four outputs (raw bits; clamped indices)
            uint32_t zq[4] = {0u, 0u, 0u, 0u};
            if (z) {
                const int e = min(mo, M - 1) * (H * Dm);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    zq[v] = ld_raw1<IOT>(static_cast<const unsigned char *>(zbase) +
                                             (uint32_t)((e + min(orow + v, Dm - 1)) * XB), 0);
            }
            f32x4 acc = acc4[0] + acc4[1];
            if constexpr (NACC == 4)
                acc += acc4[2] + acc4[3];
            const float wS = c_wS[ln];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc[v] *= wS;
            // path terms: acc[row][node] += sum_j x_j[row] Q[node][j] over the
            // chunk's sources j < t0 + TC, in groups of four k-steps whose Q^T
            // reads are issued together (group indices are constants, so the
            // x operands stay in registers)
            if constexpr (PX) {
                // B operand: Q[node ln][32 t + 8 qg .. + 7], hi and lo terms
                const uint16_t *qr = qc + ln * QP + 8 * qg;
#pragma unroll
                for (int t = 0; t < MX / 32; ++t) {
                    if (32 * t < t0 + TC) {
                        const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(qr + 32 * t);
                        const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(qr + TC * QP + 32 * t);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[t], qh, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[t], ql, acc, 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int gq = 0; gq < MX / 16; ++gq) {
                    if (gq <= c) {
                        float qv[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            qv[u] = q[(16 * gq + 4 * u + qg) * TC + ln];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[4 * gq + u], qv[u], acc, 0, 0, 0);
                    }
                }
            }
            if (ln < nt) {
                float o[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    o[v] = acc[v];
                    if (z)
                        o[v] *= silu_f32(cvt_raw1<IOT>(zq[v]));
                }
                unsigned char *op = static_cast<unsigned char *>(obase) + (uint32_t)((mo * (H * Dm) + orow) * XB);
                if (ovec) {  // rows orow .. orow+3 are in range together
                    if (orow < Dm)
                        st_raw4<IOT>(op, 0, o);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (orow + v < Dm)
                            st_elem<IOT>(op, v, o[v]);
                }
            }
        }
        gcur = gnext;
        __syncthreads();
    }

    // ---- the fp32 x stash (16-byte x vectors): written last, from a second
    // read of x, with non-temporal stores. Every workgroup starts together and
    // streams its state and x in the prologue; stash stores there (twice the
    // bytes of x) lengthened that memory-bound phase, while here they overlap
    // other workgroups' chunk loops, which move little data ----
    if (stash && xvec) {
        constexpr int VPN = 64 / XV;  // vectors per node
        for (int v = tid; v < M * VPN; v += NT) {
            const int m = v / VPN, rl = XV * (v % VPN);
            if (rbase + rl < Dm) {
                const uint32_t o = (uint32_t)(m * NSTR + rbase + rl);
                const u32x4 w = *reinterpret_cast<const u32x4 *>(xbase + o * XB);
                float f[XV];
                if constexpr (XB == 4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        f[e] = __uint_as_float(w[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[2 * e] = cvt_raw1<IOT>(w[e] & 0xffffu);
                        f[2 * e + 1] = cvt_raw1<IOT>(w[e] >> 16);
                    }
                }
                float *dst = ubase + o;
#pragma unroll
                for (int e = 0; e < XV; e += 4)
                    __builtin_nontemporal_store(
                        u32x4{__float_as_uint(f[e]), __float_as_uint(f[e + 1]),
                              __float_as_uint(f[e + 2]), __float_as_uint(f[e + 3])},
                        reinterpret_cast<u32x4 *>(dst + e));
            }
        }
    }
}

template <typename ST, typename IOT, typename BCT, int NS>
hipError_t launch_tree_cfg(const TreeParams &p, hipStream_t stream)
{
    const DecodeParams &d = p.d;
    TreeShape sh;
    sh.row_stride = d.row_stride;
    sh.num_nodes = p.num_nodes;
    sh.nheads = d.nheads;
    sh.dim = d.dim;
    sh.ngroups = d.ngroups;
    sh.heads_per_group = d.nheads / d.ngroups;
    sh.nrb = (d.dim + 63) / 64;
    sh.dt_softplus = d.dt_softplus;
    const int64_t blocks = (int64_t)d.batch * d.nheads * sh.nrb;
    const int nmb = (p.num_nodes + 15) / 16;
    const int64_t gblocks = (int64_t)d.batch * d.ngroups * ((nmb * (nmb + 1) / 2 + 3) / 4);
    if (blocks > 0x7fffffff || gblocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    constexpr int XB = (int)sizeof(IOT), BB = (int)sizeof(BCT);
    const TreeLds L = tree_lds(p.num_nodes, NS, XB, BB);
    auto kern = ssu_tree_kernel<ST, IOT, BCT, NS>;
    if (L.total > 64 * 1024) {
        // Above 64 KiB of dynamic LDS the kernel must be allowed it first, once
        // per device: raise the limit to the largest tree this kernel can get,
        // so that later launches (under stream capture too) need no call.
        static std::atomic<int> allowed[64];  // zero-initialised; benign races between host threads
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        if (dev < 0 || dev >= 64 || allowed[dev].load(std::memory_order_relaxed) < L.total) {
            const int most = tree_lds(SSU_MAX_TREE_NODES, NS, XB, BB).total;
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, most);
            if (e != hipSuccess)
                return e;
            if (dev >= 0 && dev < 64)
                allowed[dev].store(most, std::memory_order_relaxed);
        }
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL((ssu_tree_gram_kernel<BCT, NS>), dim3((unsigned)gblocks), dim3(kTreeNT), 0,
                       stream, d.B, d.C, d.idx, p.gram, p.num_nodes, d.ngroups);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kTreeNT), (unsigned)L.total, stream,
                       d.x, d.A, d.C, d.dt, d.dt_bias, d.D, d.z,
                       static_cast<const ST *>(d.state), d.out, d.idx, p.parents, p.depths,
                       p.gram, d.B, p.st_dA, p.st_u, p.st_B, p.st_dt, sh);
    return hipGetLastError();
}

template <typename ST, typename IOT, typename BCT>
hipError_t launch_tree_bc(const TreeParams &p, hipStream_t stream)
{
    switch (p.d.dstate) {
    case 16: return launch_tree_cfg<ST, IOT, BCT, 16>(p, stream);
    case 32: return launch_tree_cfg<ST, IOT, BCT, 32>(p, stream);
    case 64: return launch_tree_cfg<ST, IOT, BCT, 64>(p, stream);
    case 128: return launch_tree_cfg<ST, IOT, BCT, 128>(p, stream);
    case 256: return launch_tree_cfg<ST, IOT, BCT, 256>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST, typename IOT>
hipError_t launch_tree_io(const TreeParams &p, hipStream_t stream)
{
    switch (p.d.bc_dtype) {
    case kF32: return launch_tree_bc<ST, IOT, float>(p, stream);
    case kF16: return launch_tree_bc<ST, IOT, _Float16>(p, stream);
    case kBF16: return launch_tree_bc<ST, IOT, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename ST>
hipError_t launch_tree_state(const TreeParams &p, hipStream_t stream)
{
    switch (p.d.io_dtype) {
    case kF32: return launch_tree_io<ST, float>(p, stream);
    case kF16: return launch_tree_io<ST, _Float16>(p, stream);
    case kBF16: return launch_tree_io<ST, bf16_t>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace ssu
