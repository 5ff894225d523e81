// Byte-range copy/zero kernel behind the pool operations (clear, clear of one
// slot across every state, capture, restore with zero fill, slot copy between
// pools). One launch serves up to kMaxSeg ranges, so clearing one slot of every
// state of a layer stack is a single launch, as TensorRT-Edge-LLM's
// invokeMambaStateClear does ("Selective State Update" page). A kernel rather
// than hipMemsetAsync/hipMemcpyAsync keeps the operations capturable in a HIP
// graph without memset nodes.
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {
namespace {

constexpr int kMaxSeg = 32;

struct SegBatch {
    Segment seg[kMaxSeg];
};

__global__ __launch_bounds__(256) void ssu_segments_kernel(const SegBatch sb)
{
    const Segment sg = sb.seg[blockIdx.y];
    uint8_t *d = static_cast<uint8_t *>(sg.dst);
    const uint8_t *s = static_cast<const uint8_t *>(sg.src);
    const uint64_t n = sg.bytes;
    const uint64_t first = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    const bool aligned = ((uintptr_t)d % 16 == 0) && (s == nullptr || (uintptr_t)s % 16 == 0);
    uint64_t done = 0;
    if (aligned) {
        const uint64_t n16 = n / 16;
        u32x4 *d4 = reinterpret_cast<u32x4 *>(d);
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(s);
        for (uint64_t i = first; i < n16; i += step)
            d4[i] = s4 ? s4[i] : u32x4{0u, 0u, 0u, 0u};
        done = n16 * 16;
    }
    for (uint64_t i = done + first; i < n; i += step)
        d[i] = s ? s[i] : (uint8_t)0;
}

// invokeMambaStateClear ("Selective State Update" page): zero row `slot` (or
// every row, slot -1) of the recurrent and conv state of every layer, whose
// pointers come from a device array of MambaStateLayerInfo-like entries. A
// one-dimensional grid of (layer, piece) workgroups, the recurrent pieces of a
// layer first and then its conv pieces, so that no workgroup is launched
// without bytes to clear. A layer's pieces interleave in 4 KiB blocks (piece p
// takes blocks p, p + np, ..), so the workgroups of a layer sweep its range
// together instead of each writing a separate stretch: fewer write fronts
// open in the memory at once. Any alignment: the bytes before the first
// 16-byte boundary and after the last one go to piece 0.
constexpr uint64_t kClearPiece = 16 * 1024;

__global__ __launch_bounds__(256) void ssu_clear_layers_kernel(const ssu_state_layer *layers,
                                                               int rows, int slot,
                                                               int64_t rec_row_bytes,
                                                               int64_t conv_row_bytes,
                                                               uint32_t nrec, uint32_t nconv)
{
    const uint32_t per = nrec + nconv;
    const uint32_t l = blockIdx.x / per;
    const uint32_t k = blockIdx.x - l * per;
    const bool conv = k >= nrec;
    const uint64_t piece = conv ? k - nrec : k;
    const void *raw = conv ? layers[l].conv_state : layers[l].recurrent_state;
    const uint64_t rb = (uint64_t)(conv ? conv_row_bytes : rec_row_bytes);
    if (raw == nullptr || rb == 0)
        return;
    uint8_t *base = table_ptr<uint8_t>(raw);
    uint8_t *d = base + (slot >= 0 ? (uint64_t)slot * rb : 0);
    const uint64_t n = slot >= 0 ? rb : (uint64_t)rows * rb;
    const uint64_t mis = (uint64_t)((16 - ((uintptr_t)d & 15)) & 15);
    const uint64_t head = mis < n ? mis : n;
    const uint64_t body = (n - head) / 16;  // 16-byte vectors
    constexpr uint64_t kVec = kClearPiece / 16;
    const int tid = threadIdx.x;
    if (piece == 0) {
        if ((uint64_t)tid < head)
            d[tid] = 0;
        const uint64_t tail = n - head - body * 16;
        if ((uint64_t)tid < tail)
            d[head + body * 16 + tid] = 0;
    }
    const uint64_t np = conv ? nconv : nrec;
    u32x4 *d4 = reinterpret_cast<u32x4 *>(d + head);
#pragma unroll
    for (int j = 0; j < (int)(kVec / 256); ++j) {
        const uint64_t i = ((uint64_t)j * np + piece) * 256 + tid;
        if (i < body)
            __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, &d4[i]);
    }
}

// Row moves between a pool and working rows (invokeMambaStateGather /
// invokeMambaStateScatter, "Selective State Update" page; the activateStep /
// scatterActive packing of the "Class DeltaNetStatePool" page): workgroup
// (x, y, z) moves piece x of row y of move set z. When both rows are 16-byte
// aligned the row's pieces interleave in 4 KiB blocks (piece x takes blocks
// x, x + np, ..), each lane issuing its four streaming 16-byte loads before
// its four stores, so the workgroups of a row sweep it together; otherwise
// piece x is the byte range [x * kRowPiece, (x+1) * kRowPiece), copied bytewise.
constexpr int64_t kRowPiece = 16 * 1024;

struct RowMoves {
    RowMove m[2];
    int64_t row_bytes;
};

__global__ __launch_bounds__(256) void ssu_row_moves_kernel(const RowMoves rm)
{
    const RowMove mv = rm.m[blockIdx.z];
    const int b = blockIdx.y;
    if (b >= mv.rows)
        return;
    if (mv.skip_same && mv.skip_same[b] == b)
        return;
    const int d = mv.dst_idx ? mv.dst_idx[b] : b;
    if (d < 0)
        return;
    const int s = mv.src ? (mv.src_idx ? mv.src_idx[b] : b) : -1;
    const uint64_t n = (uint64_t)rm.row_bytes;
    const uint64_t x = blockIdx.x, np = gridDim.x;
    const int tid = threadIdx.x;
    uint8_t *dp = static_cast<uint8_t *>(mv.dst) + (uint64_t)d * mv.dst_stride;
    const uint8_t *sp = s >= 0 ? static_cast<const uint8_t *>(mv.src) + (uint64_t)s * mv.src_stride : nullptr;
    const bool aligned = (((uintptr_t)dp | (sp ? (uintptr_t)sp : 0)) & 15) == 0;
    if (aligned) {
        constexpr int kIt = (int)(kRowPiece / 16 / 256);  // 16-byte vectors per lane
        const uint64_t nv = n / 16;
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dp);
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(sp);
        u32x4 v[kIt];
#pragma unroll
        for (int k = 0; k < kIt; ++k) {
            const uint64_t j = ((uint64_t)k * np + x) * 256 + tid;
            v[k] = (s4 && j < nv) ? __builtin_nontemporal_load(&s4[j]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kIt; ++k) {
            const uint64_t j = ((uint64_t)k * np + x) * 256 + tid;
            if (j < nv)
                __builtin_nontemporal_store(v[k], &d4[j]);
        }
        if (x == 0 && (uint64_t)tid < n - nv * 16)  // tail bytes
            dp[nv * 16 + tid] = sp ? sp[nv * 16 + tid] : (uint8_t)0;
        return;
    }
    const uint64_t lo = x * (uint64_t)kRowPiece;
    if (lo >= n)
        return;
    const uint64_t len = n - lo < (uint64_t)kRowPiece ? n - lo : (uint64_t)kRowPiece;
    for (uint64_t i = tid; i < len; i += blockDim.x)
        dp[lo + i] = sp ? sp[lo + i] : (uint8_t)0;
}

}  // namespace

hipError_t launch_row_moves(const RowMove *moves, int n, int64_t row_bytes, hipStream_t stream)
{
    if (n < 1 || n > 2)
        return hipErrorInvalidValue;
    RowMoves rm = {};
    int rows = 0;
    for (int i = 0; i < n; ++i) {
        rm.m[i] = moves[i];
        rows = moves[i].rows > rows ? moves[i].rows : rows;
    }
    rm.row_bytes = row_bytes;
    if (rows == 0 || row_bytes == 0)
        return hipSuccess;
    if (rows > 65535)
        return hipErrorInvalidConfiguration;
    const uint64_t chunks = ((uint64_t)row_bytes + kRowPiece - 1) / kRowPiece;
    if (chunks > 0x7fffffffull)
        return hipErrorInvalidConfiguration;
    (void)hipGetLastError();
    hipLaunchKernelGGL(ssu_row_moves_kernel, dim3((unsigned)chunks, (unsigned)rows, (unsigned)n),
                       dim3(256), 0, stream, rm);
    return hipGetLastError();
}

hipError_t launch_clear_layers(const ssu_state_layer *layers, int num_layers, int rows, int slot,
                               int64_t rec_row_bytes, int64_t conv_row_bytes, hipStream_t stream)
{
    if (num_layers == 0 || rows == 0)
        return hipSuccess;
    // pieces per layer of each kind (every layer has the same row sizes)
    auto pieces = [&](int64_t row_bytes) -> uint64_t {
        const uint64_t n = slot >= 0 ? (uint64_t)row_bytes : (uint64_t)rows * (uint64_t)row_bytes;
        return (n + kClearPiece - 1) / kClearPiece;
    };
    const uint64_t nrec = pieces(rec_row_bytes), nconv = pieces(conv_row_bytes);
    const uint64_t blocks = (uint64_t)num_layers * (nrec + nconv);
    if (blocks == 0)
        return hipSuccess;
    if (blocks > 0x7fffffffull)
        return hipErrorInvalidConfiguration;
    (void)hipGetLastError();
    hipLaunchKernelGGL(ssu_clear_layers_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, layers,
                       rows, slot, rec_row_bytes, conv_row_bytes, (uint32_t)nrec, (uint32_t)nconv);
    return hipGetLastError();
}

hipError_t launch_segments(const Segment *segs, int n, hipStream_t stream)
{
    (void)hipGetLastError();
    for (int base = 0; base < n; base += kMaxSeg) {
        const int m = n - base < kMaxSeg ? n - base : kMaxSeg;
        SegBatch sb = {};
        uint64_t maxb = 0;
        for (int i = 0; i < m; ++i) {
            sb.seg[i] = segs[base + i];
            maxb = sb.seg[i].bytes > maxb ? sb.seg[i].bytes : maxb;
        }
        if (maxb == 0)
            continue;
        uint64_t blocks = (maxb / 16 + 255) / 256;
        blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
        hipLaunchKernelGGL(ssu_segments_kernel, dim3((unsigned)blocks, (unsigned)m), dim3(256), 0,
                           stream, sb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace ssu
