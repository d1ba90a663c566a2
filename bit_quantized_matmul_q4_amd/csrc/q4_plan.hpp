// q4_plan.hpp -- the K-segment schedule of the fixed reduction order
// (host and device).  See q4_device.hpp for the whole order.
#pragma once

#include <hip/hip_runtime.h>

namespace q4 {

struct Plan {
    int nb;     // blocks of 32 along K
    int G;      // quads of 4 blocks
    int S;      // segments (power of two, 1..16)
    int log2S;  // log2(S)
};

__host__ __device__ inline Plan make_plan(int K)
{
    Plan p;
    p.nb = K / 32;
    p.G = (p.nb + 3) / 4;
    int s = 1, l = 0;
    while (s * 2 <= p.G && s < 16) {
        s *= 2;
        ++l;
    }
    p.S = s;
    p.log2S = l;
    return p;
}

// j * G < 2^31 for every valid K (G < 2^26, j <= 16).
__host__ __device__ inline int seg_first_block(const Plan &p, int j)
{
    return 4 * ((j * p.G) >> p.log2S);
}

__host__ __device__ inline int seg_end_block(const Plan &p, int j)
{
    const int e = 4 * (((j + 1) * p.G) >> p.log2S);
    return e < p.nb ? e : p.nb;
}

}  // namespace q4
