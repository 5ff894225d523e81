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
//   w_i = exp(sum of A dt' over c_0 .. c_{i-1}),  w_S = exp(sum over c_0 .. c_k),
// and m's output row is
//   y_m = w_S (S0 C_m) + sum_i [w_i dt'_{c_i} (B_{c_i} . C_m)] x_{c_i} + D x_m.
// This costs one dstate-long dot per (row, node) for S0 C_m, plus one
// dstate-long dot per (node, path entry) shared by all rows, instead of a
// full state update per path entry and row. The exponent sums are formed
// from m upwards, so each weight carries the rounding of its own few terms
// (a weight far up the path is small whatever its relative error).
//
// Mapping on gfx950 (256 threads, one (batch row, head, block of 64 rows of
// dim) per workgroup; the prefill's lane layout, state slice in registers):
//   1. per node (one lane each): dt', A dt', parent id into LDS;
//   2. per node: walk the parents once to count the path, a workgroup prefix
//      sum places every node's path entries, a second walk writes each
//      entry's ancestor id and weight w_i dt'_{c_i} (the path entries of all
//      nodes fit in M(M+1)/2 slots: a node's path has at most m+1 entries);
//   3. per path entry: B_{c_i} . C_m over dstate by 4..16 lanes from global
//      memory (B and C are shared by all heads of a group, so L2 serves
//      them), folded into the entry's coefficient;
//   4. C of TC nodes at a time is staged in LDS (register prefetch of the next
//      chunk); each lane forms its rows' partial S0 . C_m over its dstate
//      slice, the four quarters of a wave are summed with cross-lane swaps and
//      the four waves' partials meet in LDS;
//   5. per (node, row): w_S * (sum of wave partials) + sum over the node's path
//      entries of coefficient * x (x of every node of the row block sits in
//      LDS) + D x, gate, store.
#pragma once

#include "ssu_device.h"
#include "ssu_internal.h"
#include "ssu_rowblock.h"

namespace ssu {
namespace {

struct TreeShape {
    int64_t row_stride;
    int32_t num_nodes, nheads, dim, ngroups, heads_per_group, nrb;
    int32_t dt_softplus;
};

constexpr int kTreeTC = 8;  // nodes per staged chunk of C
constexpr int kTreeNW = 4;  // waves per workgroup

// Byte offsets of the LDS arrays for a tree of M nodes (host and device).
struct TreeLds {
    int xs, cs, ybuf, dtp, dA, wS, par, off, len, ew, ej, en, wsum, total;
};

__host__ __device__ inline int tree_lds_take(int &o, int bytes)
{
    const int r = o;
    o += (bytes + 15) & ~15;
    return r;
}

__host__ __device__ inline TreeLds tree_lds(int M, int NS)
{
    TreeLds L;
    int o = 0;
    const int E = M * (M + 1) / 2;
    L.xs = tree_lds_take(o, M * 64 * 4);                    // x of the row block [M][64]
    L.cs = tree_lds_take(o, 2 * kTreeTC * NS * 4);          // C chunks [2][TC][NS]
    L.ybuf = tree_lds_take(o, kTreeTC * kTreeNW * 64 * 4);  // wave partials [TC][NW][64]
    L.dtp = tree_lds_take(o, M * 4);                        // dt'
    L.dA = tree_lds_take(o, M * 4);                         // A dt'
    L.wS = tree_lds_take(o, M * 4);                         // weight of S0 per node
    L.par = tree_lds_take(o, M * 4);                        // parent id
    L.off = tree_lds_take(o, M * 4);                        // first path entry
    L.len = tree_lds_take(o, M * 4);                        // path entries
    L.ew = tree_lds_take(o, E * 4);                         // entry weight / coefficient
    L.ej = tree_lds_take(o, E);                             // entry: ancestor id
    L.en = tree_lds_take(o, E);                             // entry: node id
    L.wsum = tree_lds_take(o, kTreeNW * 4);                 // per-wave path counts
    L.total = o;
    return L;
}

template <int NSL>
__device__ __forceinline__ void fetch_c(float (&c)[NSL], const float *cp)
{
    if constexpr (NSL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NSL; j += 4) {
            const float4 c4 = *reinterpret_cast<const float4 *>(cp + j);
            c[j] = c4.x;
            c[j + 1] = c4.y;
            c[j + 2] = c4.z;
            c[j + 3] = c4.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NSL; ++j)
            c[j] = cp[j];
    }
}

// The lane's partial S0 . C over its slice, for its rows rr + 16 i.
template <int NSL>
__device__ __forceinline__ float4 rows_dot(const float (&S)[4][NSL], const float (&c)[NSL])
{
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < NSL; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p[i] = fmaf(S[i][j], c[j], p[i]);
    return make_float4(p[0], p[1], p[2], p[3]);
}

template <typename ST, typename IOT, typename BCT, int NS>
__global__ __launch_bounds__(64 * kTreeNW) void ssu_tree_kernel(
    const void *__restrict__ x, const float *__restrict__ A, const void *__restrict__ Bm,
    const void *__restrict__ Cm, const float *__restrict__ dt, const float *__restrict__ dt_bias,
    const float *__restrict__ Dv, const void *__restrict__ z, const ST *__restrict__ state,
    void *__restrict__ out, const int32_t *__restrict__ idx, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ depths, float *__restrict__ st_dA, float *__restrict__ st_u,
    float *__restrict__ st_B, float *__restrict__ st_dt, const TreeShape sh)
{
    constexpr int NW = kTreeNW;
    constexpr int NT = 64 * NW;
    constexpr int TC = kTreeTC;
    constexpr int NSL = NS / (4 * NW);             // dstate columns per lane
    constexpr int BCN = TC * NS;                   // C elements per chunk
    constexpr int BCV = (BCN / 4 + NT - 1) / NT;   // 4-element C vectors per thread
    constexpr int XT_PER = TC * 64 / NT;           // (node, row) outputs per thread per chunk
    constexpr int EPL = NS / 16 >= 4 ? NS / 16 : 4;  // B/C elements per lane in a path dot
    constexpr int LPE = NS / EPL;                  // lanes per path entry
    constexpr int EPP = NT / LPE;                  // path entries per pass
    static_assert(NSL >= 1 && NS % (4 * NW) == 0, "dstate must split into 16 slices");
    static_assert(TC % 2 == 0 && XT_PER * NT == TC * 64, "chunk shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int M = sh.num_nodes;
    const TreeLds L = tree_lds(M, NS);
    float *xs = reinterpret_cast<float *>(lds + L.xs);
    float(*Cs)[TC][NS] = reinterpret_cast<float(*)[TC][NS]>(lds + L.cs);
    float(*ybuf)[NW][64] = reinterpret_cast<float(*)[NW][64]>(lds + L.ybuf);
    float *n_dtp = reinterpret_cast<float *>(lds + L.dtp);
    float *n_dA = reinterpret_cast<float *>(lds + L.dA);
    float *n_wS = reinterpret_cast<float *>(lds + L.wS);
    int *n_par = reinterpret_cast<int *>(lds + L.par);
    int *n_off = reinterpret_cast<int *>(lds + L.off);
    int *n_len = reinterpret_cast<int *>(lds + L.len);
    float *e_w = reinterpret_cast<float *>(lds + L.ew);
    uint8_t *e_j = lds + L.ej;
    uint8_t *e_n = lds + L.en;
    int *wsum = reinterpret_cast<int *>(lds + L.wsum);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4;
    const int rr = lane & 15;
    const int n0 = (wave * 4 + q) * NSL;
    const int H = sh.nheads, Dm = sh.dim, G = sh.ngroups;
    const int per_b = H * sh.nrb;
    const int b = blockIdx.x / per_b;
    const int rem = blockIdx.x - b * per_b;
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
    const float Ah = A[h];
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    const float dskip = Dv ? Dv[h] : 0.0f;

    // ---- the committed state slice: rows rbase + rr + 16 i, columns n0 .. n0+NSL-1 ----
    float S[4][NSL];
    const ST *sbase = state + (int64_t)srow * sh.row_stride + (int64_t)h * Dm * NS + n0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rc = min(rbase + rr + 16 * i, Dm - 1);
#pragma unroll
        for (int j = 0; j < NSL; ++j)
            S[i][j] = ld_elem<ST>(sbase, (int64_t)rc * NS + j);
    }

    // ---- 1. per node: dt', A dt', parent; x of every node into LDS ----
    if (tid < M) {
        float v = dt[(bM + tid) * H + h] + bias;
        if (sh.dt_softplus)
            v = softplus_f32(v);
        n_dtp[tid] = v;
        n_dA[tid] = Ah * v;
        n_par[tid] = parents[bM + tid];
        if (stash && rb == 0) {
            st_dA[(bM + tid) * H + h] = Ah * v;
            st_dt[(bM + tid) * H + h] = v;
        }
    }
#pragma unroll 4
    for (int e = tid; e < M * 64; e += NT) {
        const int m = e >> 6;
        const int r = rbase + (e & 63);
        float v = 0.0f;
        if (r < Dm) {
            const int64_t o = ((bM + m) * H + h) * Dm + r;
            v = ld_elem<IOT>(x, o);
            if (stash)
                st_u[o] = v;
        }
        xs[m * 64 + xpos(e & 63)] = v;
    }
    if (stash && rb == 0 && (h % sh.heads_per_group) == 0) {
        for (int i = tid; i < M * NS; i += NT) {
            const int64_t o = ((bM + i / NS) * G + g) * NS + (i % NS);
            st_B[o] = ld_elem<BCT>(Bm, o);
        }
    }
    __syncthreads();

    // ---- 2. the path of every node: length, placement, entries ----
    int len = 0;
    if (tid < M) {
        const int cap = depths ? depths[bM + tid] : tid;
        int j = tid, hops = 0;
        while (hops < cap) {
            const int p = n_par[j];
            if (p < 0 || p >= j)
                break;
            j = p;
            ++hops;
        }
        len = hops + 1;
    }
    int incl = len;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += o;
    }
    if (lane == 63)
        wsum[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = wsum[w];
        base += w < wave ? c : 0;
        total += c;
    }
    if (tid < M) {
        const int e0 = base + incl - len;
        n_off[tid] = e0;
        n_len[tid] = len;
        int j = tid;
        float acc = 0.0f;  // sum of A dt' over the path nodes after j
        for (int k = 0; k < len; ++k) {
            e_j[e0 + k] = (uint8_t)j;
            e_n[e0 + k] = (uint8_t)tid;
            e_w[e0 + k] = expf(acc) * n_dtp[j];
            acc += n_dA[j];
            j = n_par[j];
        }
        n_wS[tid] = expf(acc);
    }
    __syncthreads();

    // ---- 3. coefficient of every path entry: weight * (B_ancestor . C_node) ----
    {
        const int grp = tid / LPE;
        const int l = tid - grp * LPE;
        for (int e0 = 0; e0 < total; e0 += 2 * EPP) {
            float bv[2][EPL], cv[2][EPL];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ec = min(e0 + u * EPP + grp, total - 1);
                const int j = e_j[ec], m = e_n[ec];
                ld_typed<BCT, EPL>(Bm, ((bM + j) * G + g) * NS + l * EPL, bv[u]);
                ld_typed<BCT, EPL>(Cm, ((bM + m) * G + g) * NS + l * EPL, cv[u]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float d = 0.0f;
#pragma unroll
                for (int k = 0; k < EPL; ++k)
                    d = fmaf(bv[u][k], cv[u][k], d);
                d = group_sum<LPE>(d);
                const int e = e0 + u * EPP + grp;
                if (l == 0 && e < total)
                    e_w[e] *= d;
            }
        }
    }

    // ---- 4./5. S0 . C per node in chunks of TC nodes, then the outputs ----
    typename Raw4<BCT>::type rC[BCV];
    auto load_chunk = [&](int t0, int nt) {
#pragma unroll
        for (int k = 0; k < BCV; ++k) {
            const int e = min((tid + NT * k) * 4, nt * NS - 4);
            rC[k] = ld_raw4<BCT>(Cm, ((bM + t0 + e / NS) * G + g) * NS + (e % NS));
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int k = 0; k < BCV; ++k) {
            const int e = (tid + NT * k) * 4;
            if (e < BCN) {
                float vc[4];
                cvt_raw4<BCT>(rC[k], vc);
                *reinterpret_cast<float4 *>(&Cs[buf][e / NS][e % NS]) =
                    make_float4(vc[0], vc[1], vc[2], vc[3]);
            }
        }
    };

    const int nchunks = (M + TC - 1) / TC;
    load_chunk(0, min(TC, M));
    store_chunk(0);
    __syncthreads();
    const void *zsrc = z ? z : x;
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const int t0 = c * TC;
        const int nt = min(TC, M - t0);
        if (c + 1 < nchunks)
            load_chunk(t0 + TC, min(TC, M - t0 - TC));
        uint32_t zq[XT_PER];
#pragma unroll
        for (int k = 0; k < XT_PER; ++k) {
            const int e = tid + NT * k;
            const int tt = min(e >> 6, nt - 1);
            const int r = min(rbase + (e & 63), Dm - 1);
            zq[k] = ld_raw1<IOT>(zsrc, ((bM + t0 + tt) * H + h) * Dm + r);
        }

        // Pairs of nodes with ping-pong operands; slots past nt hold clamped
        // copies of the chunk's last node and their partials are never read.
        float ca[NSL], cb[NSL];
        fetch_c<NSL>(ca, &Cs[buf][0][n0]);
        for (int tt = 0; tt < nt; tt += 2) {
            fetch_c<NSL>(cb, &Cs[buf][tt + 1][n0]);
            ybuf[tt][wave][lane] = quarter_reduce(rows_dot<NSL>(S, ca));
            fetch_c<NSL>(ca, &Cs[buf][min(tt + 2, TC - 1)][n0]);
            ybuf[tt + 1][wave][lane] = quarter_reduce(rows_dot<NSL>(S, cb));
        }
        __syncthreads();

#pragma unroll
        for (int k = 0; k < XT_PER; ++k) {
            const int e = tid + NT * k;
            const int tt = e >> 6;  // uniform across the wave
            const int rl = e & 63;
            const int r = rbase + rl;
            if (tt < nt && r < Dm) {
                const int m = t0 + tt;
                const int xp = xpos(rl);
                float y = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; w += 2)
                    y += ybuf[tt][w][rl] + ybuf[tt][w + 1][rl];
                y *= n_wS[m];
                const int off = n_off[m], nl = n_len[m];
                int k2 = 0;
                for (; k2 + 1 < nl; k2 += 2) {
                    const int j0 = e_j[off + k2], j1 = e_j[off + k2 + 1];
                    const float w0 = e_w[off + k2], w1 = e_w[off + k2 + 1];
                    const float x0 = xs[j0 * 64 + xp], x1 = xs[j1 * 64 + xp];
                    y = fmaf(w0, x0, y);
                    y = fmaf(w1, x1, y);
                }
                if (k2 < nl)
                    y = fmaf(e_w[off + k2], xs[e_j[off + k2] * 64 + xp], y);
                y += dskip * xs[m * 64 + xp];
                if (z)
                    y *= silu_f32(cvt_raw1<IOT>(zq[k]));
                st_elem<IOT>(out, ((bM + m) * H + h) * Dm + r, y);
            }
        }
        if (c + 1 < nchunks)
            store_chunk(buf ^ 1);
        __syncthreads();
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
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const TreeLds L = tree_lds(p.num_nodes, NS);
    auto kern = ssu_tree_kernel<ST, IOT, BCT, NS>;
    if (L.total > 64 * 1024) {
        // Above 64 KiB of dynamic LDS the kernel must be allowed it first, once
        // per device: raise the limit to the largest tree this kernel can get,
        // so that later launches (under stream capture too) need no call.
        static int allowed[64] = {0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        if (dev < 0 || dev >= 64 || allowed[dev] < L.total) {
            const int most = tree_lds(SSU_MAX_TREE_NODES, NS).total;
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, most);
            if (e != hipSuccess)
                return e;
            if (dev >= 0 && dev < 64)
                allowed[dev] = most;
        }
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kTreeNW), (unsigned)L.total,
                       stream, d.x, d.A, d.B, d.C, d.dt, d.dt_bias, d.D, d.z,
                       static_cast<const ST *>(d.state), d.out, d.idx, p.parents, p.depths,
                       p.st_dA, p.st_u, p.st_B, p.st_dt, sh);
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
