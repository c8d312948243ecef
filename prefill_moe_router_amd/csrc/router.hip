// router.hip -- router gate and top-k softmax ("gate" and "topk" stages of the
// fused MoE profiling plan, "Decode 吞吐专项实验分析报告", subsection
// "下一步 profiling 方向").
//
//   s[t,e] = bias[e] + sum_h x[t,h] w_router[e,h]            (fp32 accumulate)
//   keep the k largest s[t,.] by (score desc, expert id asc), report them in
//   ascending id; weight = softmax over all E at the kept ids, divided by the
//   kept sum when renormalising.
#include <float.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int RT_TOK = 8;  // tokens per router wave tile

// One wave per (token tile of up to 8 tokens, expert).  The wave holds the
// expert's router row in registers (CPL 16-byte chunks per lane, K split over
// the 64 lanes, coalesced) and dots it with each token row.
template <class F, int CPL>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint8_t *__restrict__ x,
                                                            const uint8_t *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ logits, int T, int H,
                                                            int E, int experts_per_block) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t0 = blockIdx.x * RT_TOK;
    const int nt = min(RT_TOK, T - t0);
    const int e_begin = blockIdx.y * experts_per_block;
    const int e_end = min(E, e_begin + experts_per_block);
    const int nch = H / F::EPC;
    const size_t row_bytes = (size_t)nch * 16;
    for (int e = e_begin + wave; e < e_end; e += 4) {
        uint4 wq[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lane + WAVE * c;
            wq[c] = ch < nch ? *reinterpret_cast<const uint4 *>(wr + (size_t)e * row_bytes + (size_t)ch * 16)
                             : make_uint4(0, 0, 0, 0);
        }
        float acc[RT_TOK];
#pragma unroll
        for (int tt = 0; tt < RT_TOK; ++tt) {
            acc[tt] = 0.f;
            if (tt < nt) {
                const uint8_t *xr = x + (size_t)(t0 + tt) * row_bytes;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = lane + WAVE * c;
                    if (ch < nch) acc[tt] = chunk_dot<F>(wq[c], 0, xr + (size_t)ch * F::XB, acc[tt]);
                }
            }
        }
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int tt = 0; tt < RT_TOK; ++tt) {
            if (tt < nt) {
                const float v = wave_sum(acc[tt]);
                if (lane == 0) logits[(size_t)(t0 + tt) * E + e] = v + b;
            }
        }
    }
}

// One wave per token.  E <= 1024: each lane holds up to 16 scores (expert
// lane + 64*j).  k rounds of a wave arg-max under the total order (score desc,
// id asc) select the kept set; the kept ids are then ranked to ascending order.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, int T, int E, int k, int renorm) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float *s = logits + (size_t)t * E;
    float v[16];
    float m = -FLT_MAX;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = lane + WAVE * j;
        v[j] = e < E ? s[e] : -FLT_MAX;
        if (e < E) m = fmaxf(m, v[j]);
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) m = fmaxf(m, __shfl_xor(m, msk, WAVE));
    uint32_t taken = 0;
    int sel_e = 0x7fffffff;
    float sel_v = -FLT_MAX;
    for (int r = 0; r < k; ++r) {
        float bv = -FLT_MAX;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + WAVE * j;
            if (e < E && !((taken >> j) & 1u) && (v[j] > bv || be == 0x7fffffff)) {
                bv = v[j];
                be = e;
            }
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) {
            const float ov = __shfl_xor(bv, msk, WAVE);
            const int oe = __shfl_xor(be, msk, WAVE);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if (lane == r) {
            sel_e = be;
            sel_v = bv;
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
    }
    float p = 0.f;
    if (lane < k) p = __expf(sel_v - m);
    float denom;
    if (renorm) {
        denom = wave_sum(p);
    } else {
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + WAVE * j;
            if (e < E) z += __expf(v[j] - m);
        }
        denom = wave_sum(z);
    }
    int rank = 0;
    for (int r = 0; r < k; ++r) {
        const int oe = __shfl(sel_e, r, WAVE);
        rank += oe < sel_e ? 1 : 0;
    }
    if (lane < k) {
        ids[(size_t)t * k + rank] = sel_e;
        w[(size_t)t * k + rank] = p / denom;
    }
}

template <class F>
static hipError_t router_dispatch(const moe_shape &s, const void *x, const void *wr, const float *bias,
                                  float *logits, hipStream_t st) {
    const int T = s.num_tokens, H = s.hidden, E = s.num_experts;
    const int nch = H / F::EPC;
    const int tiles = (T + RT_TOK - 1) / RT_TOK;
    // few token tiles: spread the experts over many blocks (4 per block)
    const int epb = tiles >= 256 ? E : 4;
    dim3 grid(tiles, (E + epb - 1) / epb);
    const uint8_t *xb = static_cast<const uint8_t *>(x), *wb = static_cast<const uint8_t *>(wr);
    const int cpl = (nch + WAVE - 1) / WAVE;
#define MOE_RT(C) hipLaunchKernelGGL((router_logits_kernel<F, C>), grid, dim3(256), 0, st, xb, wb, bias, logits, T, H, E, epb)
    if (cpl <= 1) MOE_RT(1);
    else if (cpl <= 2) MOE_RT(2);
    else if (cpl <= 4) MOE_RT(4);
    else if (cpl <= 8) MOE_RT(8);
    else MOE_RT(16);
#undef MOE_RT
    return hipGetLastError();
}

hipError_t launch_router_logits(const moe_shape &s, const void *x, const void *wr, const float *bias,
                                float *logits, hipStream_t st) {
    if (s.act_dtype == MOE_F32) return router_dispatch<FmtF32>(s, x, wr, bias, logits, st);
    return router_dispatch<FmtBF16>(s, x, wr, bias, logits, st);
}

hipError_t launch_topk(const moe_shape &s, const float *logits, int32_t *ids, float *w, hipStream_t st) {
    const int T = s.num_tokens;
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, ids, w, T, s.num_experts,
                       s.top_k, s.renormalize ? 1 : 0);
    return hipGetLastError();
}

}  // namespace moe
