// decode_ffn.hip -- expert FFN for few tokens per expert ("expert kernel" and
// "activation" stages; the decode batches of at most 8 rows that the
// MMVQ ncols<=8 kernels of "第 9 章 prefill：最大的瓶颈" §9.5 serve).
//
// Bandwidth-bound: every weight byte of an active expert is read once.  One
// wave owns one weight row; the row's 16-byte chunks are spread over the 64
// lanes (coalesced), held in registers, and dotted with the rows of all
// tokens routed to that expert (8 at a time), then reduced across the wave.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int DT = 8;  // token rows per pass over a weight row held in registers

template <class F, int CPL>
__device__ __forceinline__ void load_row(const uint8_t *__restrict__ row, const uint8_t *__restrict__ srow,
                                         int nch, int lane, uint4 (&q)[CPL], uint32_t (&sc)[CPL]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + WAVE * c;
        q[c] = ch < nch ? *reinterpret_cast<const uint4 *>(row + (size_t)ch * 16) : make_uint4(0, 0, 0, 0);
        sc[c] = (F::SCALED && ch < nch) ? (uint32_t)srow[ch] : 0u;
    }
}

__device__ __forceinline__ void store_act(uint8_t *dst, size_t idx, float v, bool f32) {
    if (f32)
        reinterpret_cast<float *>(dst)[idx] = v;
    else
        reinterpret_cast<uint16_t *>(dst)[idx] = (uint16_t)f32_to_bf16_rne(v);
}

// h[p][i] = scale_p * silu(Wg[e,i,:].x_t) * (Wu[e,i,:].x_t) for every slot p
// grouped to expert e = active[1 + blockIdx.y]; one wave per row i.
template <class F, int CPL>
__global__ __launch_bounds__(256) void decode_gateup_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, const uint8_t *__restrict__ wu,
    const uint8_t *__restrict__ sg, const uint8_t *__restrict__ su, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted, const int32_t *__restrict__ active, const float *__restrict__ wts,
    uint8_t *__restrict__ h, int H, int I, int k, int act_f32) {
    const int a = blockIdx.y;
    if (a >= active[0]) return;
    const int e = active[1 + a];
    const int g0 = offsets[e], ne = offsets[e + 1] - g0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + wave;
    if (row >= I) return;
    const int nch = H / F::EPC;
    const size_t rsel = (size_t)e * I + row;
    uint4 gq[CPL], uq[CPL];
    uint32_t gs[CPL], us[CPL];
    load_row<F, CPL>(wg + rsel * nch * 16, F::SCALED ? sg + rsel * nch : nullptr, nch, lane, gq, gs);
    load_row<F, CPL>(wu + rsel * nch * 16, F::SCALED ? su + rsel * nch : nullptr, nch, lane, uq, us);
    const size_t xrow = (size_t)nch * F::XB;
    for (int tt0 = 0; tt0 < ne; tt0 += DT) {
        const int nt = min(DT, ne - tt0);
        float ag[DT], au[DT];
        int slot[DT];
#pragma unroll
        for (int tt = 0; tt < DT; ++tt) {
            ag[tt] = 0.f;
            au[tt] = 0.f;
            slot[tt] = tt < nt ? sorted[g0 + tt0 + tt] : 0;
            if (tt < nt) {
                const uint8_t *xr = x + (size_t)(slot[tt] / k) * xrow;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = lane + WAVE * c;
                    if (ch < nch) {
                        const uint8_t *xp = xr + (size_t)ch * F::XB;
                        ag[tt] = chunk_dot<F>(gq[c], gs[c], xp, ag[tt]);
                        au[tt] = chunk_dot<F>(uq[c], us[c], xp, au[tt]);
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < DT; ++tt) {
            if (tt < nt) {
                const float g = wave_sum(ag[tt]);
                const float u = wave_sum(au[tt]);
                if (lane == 0) {
                    const float sc = wts ? wts[slot[tt]] : 1.f;
                    store_act(h, (size_t)(g0 + tt0 + tt) * I + row, sc * swiglu(g, u), act_f32);
                }
            }
        }
    }
}

// o[p][n] = Wd[e,n,:].h[p,:] for every slot p grouped to expert e; one wave per row n.
template <class F, int CPL>
__global__ __launch_bounds__(256) void decode_down_kernel(const uint8_t *__restrict__ wd,
                                                          const uint8_t *__restrict__ sd,
                                                          const int32_t *__restrict__ offsets,
                                                          const int32_t *__restrict__ active,
                                                          const uint8_t *__restrict__ h, float *__restrict__ o,
                                                          int H, int I) {
    const int a = blockIdx.y;
    if (a >= active[0]) return;
    const int e = active[1 + a];
    const int g0 = offsets[e], ne = offsets[e + 1] - g0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + wave;
    if (n >= H) return;
    const int nch = I / F::EPC;
    const size_t rsel = (size_t)e * H + n;
    uint4 q[CPL];
    uint32_t sc[CPL];
    load_row<F, CPL>(wd + rsel * nch * 16, F::SCALED ? sd + rsel * nch : nullptr, nch, lane, q, sc);
    const size_t hrow = (size_t)nch * F::XB;
    for (int tt0 = 0; tt0 < ne; tt0 += DT) {
        const int nt = min(DT, ne - tt0);
        float acc[DT];
#pragma unroll
        for (int tt = 0; tt < DT; ++tt) {
            acc[tt] = 0.f;
            if (tt < nt) {
                const uint8_t *hr = h + (size_t)(g0 + tt0 + tt) * hrow;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = lane + WAVE * c;
                    if (ch < nch) acc[tt] = chunk_dot<F>(q[c], sc[c], hr + (size_t)ch * F::XB, acc[tt]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < DT; ++tt) {
            if (tt < nt) {
                const float v = wave_sum(acc[tt]);
                if (lane == 0) o[(size_t)(g0 + tt0 + tt) * H + n] = v;
            }
        }
    }
}

static int cpl_bucket(int nch) {
    const int c = (nch + WAVE - 1) / WAVE;
    return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 16;
}

template <class F>
static hipError_t gateup_dispatch(const moe_shape &s, const void *x, const moe_expert_weights &w,
                                  const int32_t *offsets, const int32_t *sorted, const int32_t *active,
                                  const float *wts, void *h, hipStream_t st) {
    const int H = s.hidden, I = s.intermediate;
    const int maxa = std::min(s.num_experts, s.num_tokens * s.top_k);
    dim3 grid((I + 3) / 4, maxa);
    const int cpl = cpl_bucket(H / F::EPC);
    auto xb = static_cast<const uint8_t *>(x);
    auto g = static_cast<const uint8_t *>(w.w_gate);
    auto u = static_cast<const uint8_t *>(w.w_up);
    auto hb = static_cast<uint8_t *>(h);
    const int f32 = s.act_dtype == MOE_F32;
#define MOE_GU(C)                                                                                            \
    hipLaunchKernelGGL((decode_gateup_kernel<F, C>), grid, dim3(256), 0, st, xb, g, u, w.s_gate, w.s_up, offsets, \
                       sorted, active, wts, hb, H, I, s.top_k, f32)
    switch (cpl) {
        case 1: MOE_GU(1); break;
        case 2: MOE_GU(2); break;
        case 4: MOE_GU(4); break;
        case 8: MOE_GU(8); break;
        default: MOE_GU(16); break;
    }
#undef MOE_GU
    return hipGetLastError();
}

template <class F>
static hipError_t down_dispatch(const moe_shape &s, const moe_expert_weights &w, const int32_t *offsets,
                                const int32_t *active, const void *h, float *o, hipStream_t st) {
    const int H = s.hidden, I = s.intermediate;
    const int maxa = std::min(s.num_experts, s.num_tokens * s.top_k);
    dim3 grid((H + 3) / 4, maxa);
    const int cpl = cpl_bucket(I / F::EPC);
    auto d = static_cast<const uint8_t *>(w.w_down);
    auto hb = static_cast<const uint8_t *>(h);
#define MOE_DN(C) \
    hipLaunchKernelGGL((decode_down_kernel<F, C>), grid, dim3(256), 0, st, d, w.s_down, offsets, active, hb, o, H, I)
    switch (cpl) {
        case 1: MOE_DN(1); break;
        case 2: MOE_DN(2); break;
        case 4: MOE_DN(4); break;
        case 8: MOE_DN(8); break;
        default: MOE_DN(16); break;
    }
#undef MOE_DN
    return hipGetLastError();
}

hipError_t launch_decode_gateup(const moe_shape &s, const void *x, const moe_expert_weights &w,
                                const int32_t *offsets, const int32_t *sorted, const int32_t *active,
                                const float *wts, void *h, hipStream_t st) {
    switch (s.weight_dtype) {
        case MOE_F32: return gateup_dispatch<FmtF32>(s, x, w, offsets, sorted, active, wts, h, st);
        case MOE_BF16: return gateup_dispatch<FmtBF16>(s, x, w, offsets, sorted, active, wts, h, st);
        default: return gateup_dispatch<FmtMX4>(s, x, w, offsets, sorted, active, wts, h, st);
    }
}

hipError_t launch_decode_down(const moe_shape &s, const moe_expert_weights &w, const int32_t *offsets,
                              const int32_t *active, const void *h, float *o, hipStream_t st) {
    switch (s.weight_dtype) {
        case MOE_F32: return down_dispatch<FmtF32>(s, w, offsets, active, h, o, st);
        case MOE_BF16: return down_dispatch<FmtBF16>(s, w, offsets, active, h, o, st);
        default: return down_dispatch<FmtMX4>(s, w, offsets, active, h, o, st);
    }
}

}  // namespace moe
