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
// every row, slot -1) of the recurrent (blockIdx.z == 0) and conv (== 1) state
// of layer blockIdx.y, whose pointers come from a device array of
// MambaStateLayerInfo-like entries. Any alignment: bytes up to the first
// 16-byte boundary, then 16-byte stores, then the tail bytes.
__global__ __launch_bounds__(256) void ssu_clear_layers_kernel(const ssu_state_layer *layers,
                                                               int rows, int slot,
                                                               int64_t rec_row_bytes,
                                                               int64_t conv_row_bytes)
{
    const ssu_state_layer ly = layers[blockIdx.y];
    uint8_t *base = static_cast<uint8_t *>(blockIdx.z ? ly.conv_state : ly.recurrent_state);
    const uint64_t rb = (uint64_t)(blockIdx.z ? conv_row_bytes : rec_row_bytes);
    if (base == nullptr || rb == 0)
        return;
    uint8_t *d = base + (slot >= 0 ? (uint64_t)slot * rb : 0);
    const uint64_t n = slot >= 0 ? rb : (uint64_t)rows * rb;
    const uint64_t mis = (uint64_t)((16 - ((uintptr_t)d & 15)) & 15);
    const uint64_t head = mis < n ? mis : n;
    const uint64_t body = (n - head) / 16;
    const uint64_t first = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    if (first < head)
        d[first] = 0;
    // four 16-byte stores per thread per pass, a workgroup's lanes side by side
    u32x4 *d4 = reinterpret_cast<u32x4 *>(d + head);
    const uint64_t b0 = (uint64_t)blockIdx.x * blockDim.x * 4 + threadIdx.x;
    const uint64_t bstep = (uint64_t)gridDim.x * blockDim.x * 4;
    for (uint64_t i = b0; i < body; i += bstep) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i + (uint64_t)k * blockDim.x < body)
                __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, &d4[i + (uint64_t)k * blockDim.x]);
    }
    for (uint64_t i = head + body * 16 + first; i < n; i += step)
        d[i] = 0;
}

// Row moves between a pool and working rows (invokeMambaStateGather /
// invokeMambaStateScatter, "Selective State Update" page; the activateStep /
// scatterActive packing of the "Class DeltaNetStatePool" page): workgroup
// (x, y, z) moves bytes [x * kRowChunk, (x+1) * kRowChunk) of row y of move set
// z. Streaming 16-byte non-temporal loads and stores when both rows are
// 16-byte aligned, bytes otherwise.
constexpr int64_t kRowChunk = 64 * 1024;

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
    const uint64_t lo = (uint64_t)blockIdx.x * kRowChunk;
    const uint64_t n = (uint64_t)rm.row_bytes;
    if (lo >= n)
        return;
    const uint64_t len = n - lo < (uint64_t)kRowChunk ? n - lo : (uint64_t)kRowChunk;
    uint8_t *dp = static_cast<uint8_t *>(mv.dst) + (uint64_t)d * mv.dst_stride + lo;
    const uint8_t *sp =
        s >= 0 ? static_cast<const uint8_t *>(mv.src) + (uint64_t)s * mv.src_stride + lo : nullptr;
    const bool aligned = (((uintptr_t)dp | (sp ? (uintptr_t)sp : 0)) & 15) == 0;
    uint64_t done = 0;
    if (aligned) {
        const uint64_t nv = len / 16;
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dp);
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(sp);
        for (uint64_t i = threadIdx.x; i < nv; i += 4 * blockDim.x) {
            u32x4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t j = i + (uint64_t)k * blockDim.x;
                v[k] = (s4 && j < nv) ? __builtin_nontemporal_load(&s4[j]) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t j = i + (uint64_t)k * blockDim.x;
                if (j < nv)
                    __builtin_nontemporal_store(v[k], &d4[j]);
            }
        }
        done = nv * 16;
    }
    for (uint64_t i = done + threadIdx.x; i < len; i += blockDim.x)
        dp[i] = sp ? sp[i] : (uint8_t)0;
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
    const uint64_t chunks = ((uint64_t)row_bytes + kRowChunk - 1) / kRowChunk;
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
    if (num_layers > 65535)
        return hipErrorInvalidConfiguration;
    const uint64_t rb = (uint64_t)(rec_row_bytes > conv_row_bytes ? rec_row_bytes : conv_row_bytes);
    const uint64_t maxb = slot >= 0 ? rb : (uint64_t)rows * rb;
    if (maxb == 0)
        return hipSuccess;
    uint64_t blocks = (maxb / 16 + 1023) / 1024;  // 256 threads x 4 vectors each
    blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
    (void)hipGetLastError();
    hipLaunchKernelGGL(ssu_clear_layers_kernel, dim3((unsigned)blocks, (unsigned)num_layers, 2),
                       dim3(256), 0, stream, layers, rows, slot, rec_row_bytes, conv_row_bytes);
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
