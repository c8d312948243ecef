// combine.hip -- weighted combine ("sum" stage of the fused MoE profiling plan,
// "Decode 吞吐专项实验分析报告", subsection "下一步 profiling 方向"):
//   y[t][n] = sum_{j ascending} w[t,j] * o[slot_pos[t*k+j]][n]
// in fp32, stored once in the activation dtype (round to nearest even).
// A gather (each output element summed by one thread in a fixed order), so
// the result is deterministic.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// one thread per 4 consecutive outputs of one token row
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o, const float *__restrict__ w,
                                                      const int32_t *__restrict__ slot_pos,
                                                      uint8_t *__restrict__ y, int T, int H, int k, int act_f32) {
    const int t = blockIdx.x;
    const int n4 = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
    if (t >= T || n4 >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto fma4 = [&](float wj, const float4 v) {
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    };
    // up to eight rows in flight, summed in j order; a slot left out of the grouping
    // (pos < 0, a bad expert id) adds nothing
    const int32_t *sp = slot_pos + (size_t)t * k;
    const float *wt = w + (size_t)t * k;
    int j = 0;
    for (; j + 8 <= k; j += 8) {
        int pos[8];
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) pos[u] = sp[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u)   // row 0 stands in for a left-out slot (not added)
            v[u] = *reinterpret_cast<const float4 *>(o + (size_t)max(pos[u], 0) * H + n4);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (pos[u] >= 0) fma4(wt[j + u], v[u]);
    }
    for (; j < k; ++j) {
        const int pos = sp[j];
        if (pos >= 0) fma4(wt[j], *reinterpret_cast<const float4 *>(o + (size_t)pos * H + n4));
    }
    if (act_f32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + (size_t)t * H + n4) = acc;
    } else {
        uint2 pk;
        pk.x = pack_bf16x2(acc.x, acc.y);
        pk.y = pack_bf16x2(acc.z, acc.w);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + (size_t)t * H + n4) = pk;
    }
}

hipError_t launch_combine(const moe_shape &s, const float *o, const float *w, const int32_t *slot_pos, void *y,
                          hipStream_t st) {
    const int H = s.hidden;
    dim3 grid(s.num_tokens, (H / 4 + 255) / 256);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, o, w, slot_pos, static_cast<uint8_t *>(y),
                       s.num_tokens, H, s.top_k, s.act_dtype == MOE_F32);
    return hipGetLastError();
}

}  // namespace moe
