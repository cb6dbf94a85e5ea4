// Device side of the split-K partials a consumer kernel sums itself: the
// same order and arithmetic as the GEMM's own reduce pass (splits added in
// order, then alpha, then the residual).
#pragma once
#include "qlx_internal.h"

namespace qlx {

// Four consecutive elements at flat index i (a multiple of 4; mn too); the
// residual R at row-major index ri.
__device__ inline float4 part_sum4(const Partials& q, int64_t i, int64_t ri) {
    const float4* src = reinterpret_cast<const float4*>(q.p + i);
    const int64_t st = q.mn / 4;
    auto add = [](float4& a, const float4& b) {
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    };
    float4 v = src[0];
    int s = 1;
    for (; s + 4 <= q.splits; s += 4) {  // four loads in flight, added in split order
        const float4 w0 = src[s * st], w1 = src[(s + 1) * st], w2 = src[(s + 2) * st], w3 = src[(s + 3) * st];
        add(v, w0);
        add(v, w1);
        add(v, w2);
        add(v, w3);
    }
    for (; s < q.splits; ++s) add(v, src[s * st]);
    v.x *= q.alpha;
    v.y *= q.alpha;
    v.z *= q.alpha;
    v.w *= q.alpha;
    if (q.R) add(v, *reinterpret_cast<const float4*>(q.R + ri));
    return v;
}

}  // namespace qlx
