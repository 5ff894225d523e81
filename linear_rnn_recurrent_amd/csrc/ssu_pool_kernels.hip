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

}  // namespace

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
