// AdamW on the LoRA factors: the optimizer update of the training step.
//
// The pages fix only the learning rate (2e-5, the training section of their
// example configuration, guillermodelpino.com article, "Qué es Soup") and name
// no optimizer; AdamW is the reading: decoupled weight decay (Loshchilov &
// Hutter, "Decoupled Weight Decay Regularization", Algorithm 2) with
// bias-corrected moments, the decay scaled by the learning rate as PyTorch's
// AdamW does:
//   theta <- theta * (1 - lr * wd)
//   m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g^2
//   theta <- theta - (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// fp32 throughout, elementwise, so the kernel is bound by HBM: 16 bytes read
// and 12 written per parameter.
#include "qlx_internal.h"

namespace qlx {

namespace {
struct AdamTable {
    AdamTensor t[kAdamMaxTensors];
    int64_t start[kAdamMaxTensors + 1];  // prefix sums of 4-element groups
    int n;
};

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, const AdamScalars& c) {
    p *= c.decay;
    m = c.b1 * m + c.one_m_b1 * g;
    v = c.b2 * v + c.one_m_b2 * (g * g);
    p -= c.step_size * (m / (sqrtf(v) * c.inv_bc2_sqrt + c.eps));
}

// Thread = 4 consecutive elements of one tensor (a float4 when the tensor's
// length is a multiple of 4; the launcher checks alignment).
__global__ __launch_bounds__(256) void k_adamw(const AdamTable tab, const AdamScalars c) {
    const int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (q >= tab.start[tab.n]) return;
    int i = 0;
    while (q >= tab.start[i + 1]) ++i;
    const AdamTensor& T = tab.t[i];
    const int64_t e0 = (q - tab.start[i]) * 4;
    if ((T.n & 3) == 0) {
        float4 p = *reinterpret_cast<const float4*>(T.p + e0);
        const float4 g = *reinterpret_cast<const float4*>(T.g + e0);
        float4 m = *reinterpret_cast<const float4*>(T.m + e0);
        float4 v = *reinterpret_cast<const float4*>(T.v + e0);
        adam_one(p.x, g.x, m.x, v.x, c);
        adam_one(p.y, g.y, m.y, v.y, c);
        adam_one(p.z, g.z, m.z, v.z, c);
        adam_one(p.w, g.w, m.w, v.w, c);
        *reinterpret_cast<float4*>(T.p + e0) = p;
        *reinterpret_cast<float4*>(T.m + e0) = m;
        *reinterpret_cast<float4*>(T.v + e0) = v;
        return;
    }
    for (int64_t e = e0; e < e0 + 4 && e < T.n; ++e) {
        float p = T.p[e], m = T.m[e], v = T.v[e];
        adam_one(p, T.g[e], m, v, c);
        T.p[e] = p;
        T.m[e] = m;
        T.v[e] = v;
    }
}
}  // namespace

void launch_adamw(const AdamTensor* ts, int n, const AdamScalars& c, hipStream_t s) {
    QLX_REQUIRE(n >= 0 && n <= kAdamMaxTensors, QLX_EINVAL, "adamw: too many tensors in one launch");
    AdamTable tab{};
    tab.n = n;
    tab.start[0] = 0;
    double bytes = 0;
    for (int i = 0; i < n; ++i) {
        const AdamTensor& T = ts[i];
        QLX_REQUIRE(T.n >= 0, QLX_EINVAL, "adamw: negative tensor size");
        if ((T.n & 3) == 0) {
            for (const void* ptr : {static_cast<const void*>(T.p), static_cast<const void*>(T.g),
                                    static_cast<const void*>(T.m), static_cast<const void*>(T.v)})
                QLX_REQUIRE((reinterpret_cast<uintptr_t>(ptr) & 15) == 0, QLX_EINVAL,
                            "adamw: tensors whose length is a multiple of 4 must be 16-byte aligned");
        }
        tab.t[i] = T;
        tab.start[i + 1] = tab.start[i] + (T.n + 3) / 4;
        bytes += 28.0 * T.n;
    }
    const int64_t groups = tab.start[n];
    if (groups == 0) return;
    ProfScope prof("adamw", 0.0, bytes, s);
    hipLaunchKernelGGL(k_adamw, dim3(unsigned((groups + 255) / 256)), dim3(256), 0, s, tab, c);
    check_launch("adamw");
}

}  // namespace qlx
