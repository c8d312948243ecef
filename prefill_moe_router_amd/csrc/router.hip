// router.hip -- router gate and top-k softmax ("gate" and "topk" stages of the
// fused MoE profiling plan, "Decode 吞吐专项实验分析报告", subsection
// "下一步 profiling 方向").
//
//   s[t,e] = bias[e] + sum_h x[t,h] w_router[e,h]            (fp32 accumulate)
//   keep the k largest s[t,.] by (score desc, expert id asc), report them in
//   ascending id; weight = softmax over all E at the kept ids, divided by the
//   kept sum when renormalising.
#include <float.h>

#include <hip/hip_ext.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int RT_TOK = 8;  // tokens per router wave tile

// One wave per (token tile of up to 8 tokens, expert).  The wave holds the
// expert's router row in registers (CPL 16-byte chunks per lane, K split over
// the 64 lanes, coalesced) and dots it with each token row.  Every token row of
// the tile is loaded before any product (rows past the end repeat the last
// token and are not written), and the eight sums are reduced together through
// DPP, so the tile costs about one memory round trip.
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
        float acc[RT_TOK];
        if constexpr (CPL <= 8) {
            // chunks past the row end (lanes beyond nch) read the last chunk with zero
            // weights, so no load or product sits behind a branch; tokens in batches of TB
            // so that a batch's activation chunks fit in registers
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + WAVE * c;
                const uint4 v =
                    *reinterpret_cast<const uint4 *>(wr + (size_t)e * row_bytes + (size_t)min(ch, nch - 1) * 16);
                wq[c] = ch < nch ? v : make_uint4(0, 0, 0, 0);
            }
            constexpr int TB = CPL >= 8 ? 2 : RT_TOK;
#pragma unroll
            for (int t8 = 0; t8 < RT_TOK; t8 += TB) {
#pragma unroll
                for (int tt = t8; tt < t8 + TB; ++tt) {
                    acc[tt] = 0.f;
                    const uint8_t *xr = x + (size_t)(t0 + min(tt, nt - 1)) * row_bytes;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int ch = min(lane + WAVE * c, nch - 1);
                        acc[tt] = chunk_dot<F>(wq[c], 0, xr + (size_t)ch * F::XB, acc[tt]);
                    }
                }
                if (TB < RT_TOK) __builtin_amdgcn_sched_barrier(0);   // keep the batches apart
            }
        } else {
            // very wide rows: guarded chunks, one token at a time (fits the register file)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + WAVE * c;
                wq[c] = ch < nch ? *reinterpret_cast<const uint4 *>(wr + (size_t)e * row_bytes + (size_t)ch * 16)
                                 : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int tt = 0; tt < RT_TOK; ++tt) {
                acc[tt] = 0.f;
                const uint8_t *xr = x + (size_t)(t0 + min(tt, nt - 1)) * row_bytes;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = lane + WAVE * c;
                    if (ch < nch) acc[tt] = chunk_dot<F>(wq[c], 0, xr + (size_t)ch * F::XB, acc[tt]);
                }
            }
        }
        wave_fsum_n(acc);
        const float b = bias ? bias[e] : 0.f;
        if (lane < nt) {
            float v = acc[0];
#pragma unroll
            for (int tt = 1; tt < RT_TOK; ++tt) v = lane == tt ? acc[tt] : v;
            logits[(size_t)(t0 + lane) * E + e] = v + b;
        }
    }
}

// One wave per token (E <= 1024): radix top-k selection of the token's logits row,
// ids ascending, softmax weights (renormalised over the kept set when asked).
template <int NJ>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, int T, int E, int k, int renorm) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    wave_topk<NJ>(logits + (size_t)t * E, E, k, renorm, nullptr, nullptr, ids + (size_t)t * k, w + (size_t)t * k);
}

// ---- router GEMM + top-k in one kernel (bf16 activations, MFMA) --------------------------
//
// A work-group takes kRouterRows (32) tokens and all E (a multiple of 32, <= 128)
// experts, so the top-k of each token is taken in the same work-group.  The k loop
// runs in 64-wide steps: each step's 32 token rows and E expert rows (128 bytes of
// each) are staged in an LDS ring by direct-to-LDS loads in which eight lanes read
// one whole 128-byte line (whole-line requests: reading half lines or less per
// request measured ~2.6x slower from L2 on gfx950).  Wave w computes the 32 x 16
// expert tiles w and w + 4 with v_mfma_f32_16x16x32_bf16, so every logit is one
// fp32 accumulation over k in a fixed order; bias is added once at the end.  Each
// wave then selects the top-k of eight tokens.
//
// With grouping outputs the kernel also produces the first half of the stable counting
// sort by expert: the number of the block's slots that chose each expert
// (counts[block][e]) and each slot's rank among the block's slots with the same expert
// (slot_rank[p]); the slots of a block are consecutive and each token chooses an expert
// at most once, so the rank is the number of earlier tokens of the block that chose it.
constexpr int RM_MAXNT = 8;   // expert tiles of 16

struct RouterTopkParams {
    const uint8_t *x, *wr;
    const float *bias;
    int32_t *ids;
    float *w;
    int32_t *slot_rank, *counts;   // both null without grouping outputs
    int T, H, E, K, renorm;
};

#ifndef MOE_RT_NSTAGE
#define MOE_RT_NSTAGE 4
#endif
constexpr int RT_NSTAGE = MOE_RT_NSTAGE;   // LDS ring depth (64-wide k steps)
#ifndef MOE_RT_WAVES
#define MOE_RT_WAVES 8
#endif
constexpr int RT_WAVES = MOE_RT_WAVES;    // 4 or 8: each computes NT / RT_WAVES expert tiles
constexpr int RT_ROUNDS_MAX_K = 12;       // arg-max rounds up to this k, radix walk above

// The 16-byte chunk c of staged row R sits at chunk slot c ^ rt_swz(R) of the row's 128
// bytes: the 16 rows read by one 16-lane group of an MFMA operand load then fall on
// distinct 16-byte bank groups (rows two apart share banks and differ in the key).
__device__ __forceinline__ int rt_swz(int row) { return (row >> 1) & 7; }

template <int NT>
__global__ __launch_bounds__(64 * RT_WAVES) void router_topk_mfma_kernel(RouterTopkParams p) {
    constexpr int E = 16 * NT;
    constexpr int ROWS = kRouterRows + E;          // staged rows per step: tokens, then experts
    constexpr int STAGE = ROWS * 128;
    constexpr int NLOAD = ROWS / 8;                // 1 KB direct loads per step (8 rows each)
    constexpr int UPW = NLOAD / 4;                 // per loading wave (waves 0-3; NT even: NLOAD % 4 == 0)
    constexpr int NJW = (NT + RT_WAVES - 1) / RT_WAVES;   // expert tiles per wave
    constexpr int TPW = kRouterRows / RT_WAVES;    // tokens per wave in the top-k
    static_assert(NT % 2 == 0 && NLOAD % 4 == 0, "E must be a multiple of 32");
    extern __shared__ __attribute__((aligned(16))) uint8_t rsm[];   // ring; then logits [32][E] fp32
    __shared__ int s_ids[kRouterRows * 32];
    __shared__ float s_w[kRouterRows * 32];
    __shared__ uint32_t s_trash[RT_WAVES * 64];
    __shared__ uint32_t s_mask[E];
    __shared__ float s_bias[E];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int H = p.H;
    if (threadIdx.x < E) {
        s_mask[threadIdx.x] = 0u;
        s_bias[threadIdx.x] = p.bias ? p.bias[threadIdx.x] : 0.f;
    }
    const int t0 = blockIdx.x * kRouterRows;
    const int rows = min(kRouterRows, p.T - t0);
    // this lane's source in each of the wave's loads: staged row R = 8j + lane/8 (padding
    // token rows of a ragged block read the last token), chunk slot lane%8
    const bool loader = wave < 4;
    const uint8_t *src[UPW];
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const int R = min(8 * (wave + 4 * u) + (lane >> 3), ROWS - 1);
        const int c = (lane & 7) ^ rt_swz(R);
        src[u] = (R < kRouterRows ? p.x + (size_t)(t0 + min(R, rows - 1)) * H * 2
                                  : p.wr + (size_t)(R - kRouterRows) * H * 2) + c * 16;
    }
    auto issue = [&](int step, int slot) __attribute__((always_inline)) {
        if (loader) {
#pragma unroll
            for (int u = 0; u < UPW; ++u)
                load_lds16(src[u] + (size_t)step * 128, rsm + slot * STAGE + (wave + 4 * u) * 1024);
        }
    };
    f32x4_t acc[2][NJW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int r16 = lane & 15, q = lane >> 4;
    auto compute = [&](int slot) __attribute__((always_inline)) {
        const uint8_t *st = rsm + slot * STAGE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 4 * s + q;
            bf16x8_t a[2], b[NJW];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int R = 16 * i + r16;
                a[i] = *reinterpret_cast<const bf16x8_t *>(st + R * 128 + ((c ^ rt_swz(R)) << 4));
            }
#pragma unroll
            for (int j = 0; j < NJW; ++j) {
                const int n = wave + RT_WAVES * j;
                const int R = kRouterRows + 16 * min(n, NT - 1) + r16;
                b[j] = *reinterpret_cast<const bf16x8_t *>(st + R * 128 + ((c ^ rt_swz(R)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJW; ++j)
                    if (wave + RT_WAVES * j < NT)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    const int nsteps = H / 64;   // >= RT_NSTAGE (H % 512 == 0)
#pragma unroll
    for (int s = 0; s < RT_NSTAGE - 1; ++s) issue(s, s);
    for (int t = 0; t < nsteps; ++t) {
        // this wave's loads of step t are done once at most the later issued steps' remain
        const int later = min(RT_NSTAGE - 2, nsteps - 1 - t);
        if (later >= RT_NSTAGE - 2) wait_vm<(RT_NSTAGE - 2) * UPW>();
        else if (later == 4) wait_vm<4 * UPW>();
        else if (later == 3) wait_vm<3 * UPW>();
        else if (later == 2) wait_vm<2 * UPW>();
        else if (later == 1) wait_vm<UPW>();
        else wait_vm<0>();
        barrier_nofence();   // everyone's loads of step t are in; step t-1's slot is free
        if (t + RT_NSTAGE - 1 < nsteps) issue(t + RT_NSTAGE - 1, (t + RT_NSTAGE - 1) % RT_NSTAGE);
        compute(t % RT_NSTAGE);
    }
    static_assert(RT_NSTAGE >= 3 && RT_NSTAGE <= 7 && (RT_NSTAGE - 2) * UPW < 64, "ring depth the waits cover");
    wait_lgkm0();
    barrier_nofence();   // all operand reads are done: the ring becomes the logits table
    float *lg = reinterpret_cast<float *>(rsm);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJW; ++j) {
            const int n = wave + RT_WAVES * j;
            if (n < NT) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    lg[(16 * i + 4 * q + g) * E + 16 * n + r16] = acc[i][j][g] + s_bias[16 * n + r16];
            }
        }
    __syncthreads();

    const int K = p.K, rr0 = wave * TPW;
    if (K <= RT_ROUNDS_MAX_K)
        wave_topk_multi<(E + 63) / 64, TPW, true>(lg + rr0 * E, E, K, p.renorm, rows - rr0, s_ids + rr0 * K,
                                                s_w + rr0 * K, s_mask, rr0, s_trash + wave * 64);
    else
        wave_topk_multi<(E + 63) / 64, TPW, false>(lg + rr0 * E, E, K, p.renorm, rows - rr0, s_ids + rr0 * K,
                                                 s_w + rr0 * K, s_mask, rr0, s_trash + wave * 64);
    __syncthreads();
    // the block's ids and weights are one contiguous run of rows * K slots
    const size_t g0 = (size_t)t0 * K;
    for (int i = threadIdx.x; i < rows * K; i += 64 * RT_WAVES) {
        p.ids[g0 + i] = s_ids[i];
        p.w[g0 + i] = s_w[i];
    }
    if (!p.counts) return;
    if (threadIdx.x < E) p.counts[(size_t)blockIdx.x * E + threadIdx.x] = __popc(s_mask[threadIdx.x]);
    for (int i = threadIdx.x; i < rows * K; i += 64 * RT_WAVES) {
        const int rr = i / K;
        p.slot_rank[g0 + i] = __popc(s_mask[s_ids[i]] & ((1u << rr) - 1u));
    }
}

bool router_topk_mfma_supported(const moe_shape &s) {
    return s.act_dtype == MOE_BF16 && s.num_experts % 32 == 0 && s.num_experts <= 16 * RM_MAXNT &&
           s.hidden % 512 == 0 && s.top_k <= 32;
}

int router_topk_blocks(const moe_shape &s) { return (s.num_tokens + kRouterRows - 1) / kRouterRows; }

template <int NT>
static hipError_t router_topk_go(const RouterTopkParams &prm, int blocks, hipStream_t st, hipEvent_t ev0,
                                 hipEvent_t ev1) {
    constexpr size_t lds = (size_t)RT_NSTAGE * (kRouterRows + 16 * NT) * 128;
    static bool attr_done = false;
    if (!attr_done) {
        const hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void *>(router_topk_mfma_kernel<NT>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (r != hipSuccess) return r;
        attr_done = true;
    }
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(router_topk_mfma_kernel<NT>, dim3(blocks), dim3(64 * RT_WAVES), lds, st, ev0, ev1, 0,
                              prm);
    else
        hipLaunchKernelGGL(router_topk_mfma_kernel<NT>, dim3(blocks), dim3(64 * RT_WAVES), lds, st, prm);
    return hipGetLastError();
}

hipError_t launch_router_topk_mfma(const moe_shape &s, const void *x, const void *wr, const float *bias,
                                   int32_t *ids, float *w, int32_t *slot_rank, int32_t *counts, hipStream_t st,
                                   hipEvent_t ev0, hipEvent_t ev1) {
    const RouterTopkParams prm{static_cast<const uint8_t *>(x), static_cast<const uint8_t *>(wr), bias, ids, w,
                               slot_rank, counts, s.num_tokens, s.hidden, s.num_experts, s.top_k,
                               s.renormalize ? 1 : 0};
    const int nb = router_topk_blocks(s);
    switch (s.num_experts / 32) {
        case 1: return router_topk_go<2>(prm, nb, st, ev0, ev1);
        case 2: return router_topk_go<4>(prm, nb, st, ev0, ev1);
        case 3: return router_topk_go<6>(prm, nb, st, ev0, ev1);
        default: return router_topk_go<8>(prm, nb, st, ev0, ev1);
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
    const int E = s.num_experts, k = s.top_k, rn = s.renormalize ? 1 : 0;
    const dim3 grid((T + 3) / 4), blk(256);
    if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, grid, blk, 0, st, logits, ids, w, T, E, k, rn);
    else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, grid, blk, 0, st, logits, ids, w, T, E, k, rn);
    else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, blk, 0, st, logits, ids, w, T, E, k, rn);
    else if (E <= 512) hipLaunchKernelGGL(topk_kernel<8>, grid, blk, 0, st, logits, ids, w, T, E, k, rn);
    else hipLaunchKernelGGL(topk_kernel<16>, grid, blk, 0, st, logits, ids, w, T, E, k, rn);
    return hipGetLastError();
}

}  // namespace moe
