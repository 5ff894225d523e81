// Lane layout shared by the kernels that keep a (batch row, head) block of 64
// state rows in registers across a 256-thread workgroup (prefill, tree
// verify): dstate is cut into 16 slices, wave w quarter q (16 lanes) owns
// slice 4w+q, and lane rr of a quarter owns rows rr, rr+16, rr+32, rr+48.
#pragma once

#include <hip/hip_runtime.h>

namespace ssu {

// Position of row r (0..63) of a row block in the LDS x / partial-sum arrays:
// lane rr of a quarter reads its rows rr, rr+16, rr+32, rr+48 as one float4.
__device__ __forceinline__ int xpos(int r) { return (r & 15) * 4 + (r >> 4); }

// Sums a lane's four row partials (rows rr + 16 i) over the four quarters of
// the wave with two swap-and-add steps (32-lane halves, then 16-lane rows),
// leaving in lane rr + 16 q the wave's partial of row rr + 16 q.
__device__ __forceinline__ float quarter_reduce(const float4 p)
{
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p.x), __float_as_uint(p.z),
                                                      false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p.y), __float_as_uint(p.w),
                                                      false, false);
    const float u0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
    const float u1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
    const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(u0), __float_as_uint(u1),
                                                    false, false);
    return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

}  // namespace ssu
