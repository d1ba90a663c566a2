// q4_plan.hpp -- the K-segment schedule of the fixed reduction order
// (host and device).  See q4_device.hpp for the whole order.
#pragma once

#include <hip/hip_runtime.h>

namespace q4 {

struct Plan {
    int nb;  // blocks of 32 along K
    int G;   // quads of 4 blocks
    int S;   // segments (power of two, 1..16)
};

__host__ __device__ inline Plan make_plan(int K)
{
    Plan p;
    p.nb = K / 32;
    p.G = (p.nb + 3) / 4;
    int s = 1;
    while (s * 2 <= p.G && s < 16)
        s *= 2;
    p.S = s;
    return p;
}

__host__ __device__ inline int seg_first_block(const Plan &p, int j)
{
    return 4 * (int)(((long long)j * p.G) / p.S);
}

__host__ __device__ inline int seg_end_block(const Plan &p, int j)
{
    const int e = 4 * (int)(((long long)(j + 1) * p.G) / p.S);
    return e < p.nb ? e : p.nb;
}

}  // namespace q4
