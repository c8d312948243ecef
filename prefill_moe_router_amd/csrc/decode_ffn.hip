// decode_ffn.hip -- expert FFN when each expert sees few tokens: the decode
// batches beyond the fused single-launch kernel and the medium batches (tens to a
// few hundred tokens) below the point where the MFMA grouped GEMMs win ("expert
// kernel" and "activation" stages; the small-batch regime that the MMVQ ncols<=8
// kernels of "第 9 章 prefill：最大的瓶颈" §9.5 serve, without their 8-column cap).
//
// Bandwidth-bound: every weight byte of an active expert is read once, and the
// few tokens routed to the expert reuse it from registers.
//  * A work-group (4 waves) owns one active expert and four passes of weight rows;
//    the activation rows of the expert's tokens (x rows for gate/up, h' rows for
//    down) are staged in LDS once per work-group when they fit in 64 KB, and each
//    pass's weights are loaded while the previous pass computes.
//  * A lane group of LPR lanes owns one weight row: the row's 16-byte chunks are
//    spread over the group (coalesced), loaded once, and MXFP4 codes are decoded to
//    bf16 in registers once -- not once per token.
//  * Every token of the expert is then dotted with the row from LDS (v_dot2 on bf16
//    pairs, fp32 FMA for fp32 weights), summed over the lane group by DPP, and the
//    group's last lane stores the result.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int SNT = 256;                    // threads per work-group
constexpr int SWAVES = SNT / WAVE;
constexpr size_t STAGE_BYTES = 64 * 1024;   // LDS for staged activation rows

// 16-byte words per weight chunk once decoded: 4 for MXFP4 / NVFP4 (32 bf16), 2 for
// MXINT8 (16 bf16), else 1
template <class F>
constexpr int dec_words() { return F::EPC == 32 ? 4 : F::EPC == 16 ? 2 : 1; }

// sum over groups of LPR consecutive lanes; the total lands in the group's last lane
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if (LPR == 64) return dpp_sum64(v);
    if (LPR == 32) return dpp_sum32(v);
    return dpp_sum16(v);
}

// load chunk ch of a weight row (16 bytes, plus its scale code for MXFP4 / NVFP4) and
// decode it into W 16-byte words: bf16 pairs (bf16, MXFP4, NVFP4) or 4 fp32 (fp32).
// NVFP4 elements are E2M1 codes times their 16-element block's E4M3 scale, exact in bf16.
template <class F>
__device__ __forceinline__ void load_chunk(const uint8_t *row, const uint8_t *srow, int ch, bool ok,
                                           u32x4_t (&w)[dec_words<F>()]) {
    constexpr int W = dec_words<F>();
    if (!ok) {
#pragma unroll
        for (int u = 0; u < W; ++u) w[u] = u32x4_t{0u, 0u, 0u, 0u};
        return;
    }
    const u32x4_t q = *reinterpret_cast<const u32x4_t *>(row + (size_t)ch * 16);
    if constexpr (W == 4 && F::SB == 2) {
        // NVFP4: the power-of-two part of the block's E4M3 scale in the convert, then the
        // remaining factor (the products are exact in bf16)
        const uint32_t code = load_scale<F>(srow, ch);
        float p2[2], fm[2];
        e4m3_split(code & 0xffu, p2[0], fm[0]);
        e4m3_split(code >> 8, p2[1], fm[1]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float s = p2[u >> 1], f = fm[u >> 1];
            w[u][0] = bf16x2_mul_exact(fp4x2_to_bf16x2<0>(q[u], s), f);
            w[u][1] = bf16x2_mul_exact(fp4x2_to_bf16x2<1>(q[u], s), f);
            w[u][2] = bf16x2_mul_exact(fp4x2_to_bf16x2<2>(q[u], s), f);
            w[u][3] = bf16x2_mul_exact(fp4x2_to_bf16x2<3>(q[u], s), f);
        }
    } else if constexpr (W == 2) {
        // MXINT8: codes times the block's power of two (exact in bf16)
        const float s = mxint8_scale(load_scale<F>(srow, ch));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            w[u][0] = i8x2_to_bf16x2<0>(q[2 * u], s);
            w[u][1] = i8x2_to_bf16x2<1>(q[2 * u], s);
            w[u][2] = i8x2_to_bf16x2<0>(q[2 * u + 1], s);
            w[u][3] = i8x2_to_bf16x2<1>(q[2 * u + 1], s);
        }
    } else if constexpr (W == 4) {
        const float s = e8m0_to_f32(srow[ch]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            w[u][0] = fp4x2_to_bf16x2<0>(q[u], s);
            w[u][1] = fp4x2_to_bf16x2<1>(q[u], s);
            w[u][2] = fp4x2_to_bf16x2<2>(q[u], s);
            w[u][3] = fp4x2_to_bf16x2<3>(q[u], s);
        }
    } else {
        w[0] = q;
    }
}

// dot of one decoded chunk with the matching activation bytes at xp (LDS)
template <class F>
__device__ __forceinline__ float chunk_dot_dec(const u32x4_t (&w)[dec_words<F>()], const uint8_t *xp, float acc) {
    constexpr int W = dec_words<F>();
    if constexpr (F::EPC == 4) {
        const float4 xv = *reinterpret_cast<const float4 *>(xp);
        acc = fmaf(__uint_as_float(w[0][0]), xv.x, acc);
        acc = fmaf(__uint_as_float(w[0][1]), xv.y, acc);
        acc = fmaf(__uint_as_float(w[0][2]), xv.z, acc);
        acc = fmaf(__uint_as_float(w[0][3]), xv.w, acc);
    } else {
#pragma unroll
        for (int u = 0; u < W; ++u) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xp + 16 * u);
            acc = dot2_bf16(w[u][0], xv[0], acc);
            acc = dot2_bf16(w[u][1], xv[1], acc);
            acc = dot2_bf16(w[u][2], xv[2], acc);
            acc = dot2_bf16(w[u][3], xv[3], acc);
        }
    }
    return acc;
}

__device__ __forceinline__ void store_act(uint8_t *dst, size_t idx, float v, bool f32) {
    if (f32)
        reinterpret_cast<float *>(dst)[idx] = v;
    else
        reinterpret_cast<uint16_t *>(dst)[idx] = (uint16_t)f32_to_bf16_rne(v);
}

// weight rows per lane group so that the decoded rows stay near 64 registers
template <class F, int CPL, int NMAT>
constexpr int rows_per_group() {
    constexpr int regs = NMAT * CPL * dec_words<F>() * 4;
    constexpr int r = 64 / regs;
    return r < 1 ? 1 : (r > 4 ? 4 : r);
}

// Row passes per work-group: MXFP4 rows are a quarter of the bytes of the activation
// rows they meet, so a work-group covers four passes of rows per staging of its tokens;
// bf16 and fp32 rows are as large as the activation rows, and one pass per work-group
// (more work-groups, more loads in flight) measured faster.
template <class F>
constexpr int passes() { return F::EPC == 32 ? 4 : 1; }

struct StreamParams {
    const uint8_t *act;         // x [T][H] (gate/up) or h' [P][I] in sorted order (down)
    const uint8_t *w0, *w1;     // gate / up [E][I][H], or down [E][H][I] (w1 unused)
    const uint8_t *s0, *s1;     // MXFP4 / NVFP4 scales
    float ts0, ts1;             // NVFP4 tensor scales of w0 / w1 (1 otherwise)
    const int32_t *offsets, *sorted, *active;
    const float *wts;           // gate weight per slot (gate/up) or null
    uint8_t *out;               // h' [P][I] (act dtype) or o [P][H] fp32
    int N, K, topk, act_f32;    // N output rows per expert, K the contraction length
    int mt;                     // activation rows staged per pass
};

// GATEUP: h[p][i] = (wts ? wts[slot] : 1) * silu(Wg[e,i].x_t) * (Wu[e,i].x_t)
// DOWN  : o[p][n] = Wd[e,n].h[p]                       (p over the slots of expert e)
template <class F, int CPL, int LPR, bool GATEUP>
__global__ __launch_bounds__(SNT) void stream_ffn_kernel(StreamParams p) {
    constexpr int NPASS = passes<F>();                    // row passes per work-group
    constexpr int NMAT = GATEUP ? 2 : 1;
    constexpr int W = dec_words<F>();
    constexpr int RG = rows_per_group<F, CPL, NMAT>();   // rows per lane group
    constexpr int GPW = WAVE / LPR;                       // lane groups per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    const int a = blockIdx.y;
    if (a >= p.active[0]) return;
    const int e = p.active[1 + a];
    const int g0 = p.offsets[e], ne = p.offsets[e + 1] - g0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = lane / LPR, li = lane % LPR;
    const int nch = p.K / F::EPC;
    const size_t wrow = (size_t)nch * 16, srow = scale_row_bytes<F>(nch);
    const int ab = p.act_f32 ? 4 : 2;
    const size_t xrow = (size_t)p.K * ab;                 // bytes of one activation row

    // Pass q (< NPASS) covers rows base + q * RPP .. + RPP, RPP = RG * GPW * SWAVES; the
    // group's rows in a pass are row0 + q * RPP + r * GPW * SWAVES, r < RG.  The next
    // pass's weights are loaded (into the other register buffer) before this pass's
    // tokens are dotted, and the staged tokens serve every pass when they fit at once.
    constexpr int RPP = RG * GPW * SWAVES;
    const int row0 = blockIdx.x * (RPP * NPASS) + wave * GPW + grp;
    u32x4_t wq[2][NMAT][RG][CPL][W];
    auto load_pass = [&](int q, auto buf_c) __attribute__((always_inline)) {
        constexpr int b = decltype(buf_c)::value;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int row = row0 + q * RPP + r * GPW * SWAVES;
            const bool rok = row < p.N;
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const size_t rsel = (size_t)e * p.N + (rok ? row : 0);
                const uint8_t *wr = (m == 0 ? p.w0 : p.w1) + rsel * wrow;
                const uint8_t *sr = F::SCALED ? (m == 0 ? p.s0 : p.s1) + rsel * srow : nullptr;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = li + LPR * c;
                    load_chunk<F>(wr, sr, ch, rok && ch < nch, wq[b][m][r][c]);
                }
            }
        }
    };
    const int n16 = (int)(xrow / 16);
    auto stage = [&](int t0, int mt) __attribute__((always_inline)) {
        for (int idx = threadIdx.x; idx < mt * n16; idx += SNT) {
            const int t = idx / n16, q = idx % n16;
            const size_t src = GATEUP ? (size_t)(p.sorted[g0 + t0 + t] / p.topk) : (size_t)(g0 + t0 + t);
            *reinterpret_cast<u32x4_t *>(xs + (size_t)t * xrow + (size_t)q * 16) =
                *reinterpret_cast<const u32x4_t *>(p.act + src * xrow + (size_t)q * 16);
        }
    };
    auto compute = [&](int q, int t0, int mt, auto buf_c) __attribute__((always_inline)) {
        constexpr int b = decltype(buf_c)::value;
        for (int t = 0; t < mt; ++t) {
            const uint8_t *xt = xs + (size_t)t * xrow;
            float acc[NMAT][RG];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int r = 0; r < RG; ++r) acc[m][r] = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = li + LPR * c;
                if (ch < nch) {
                    const uint8_t *xp = xt + (size_t)ch * F::XB;
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int r = 0; r < RG; ++r) acc[m][r] = chunk_dot_dec<F>(wq[b][m][r][c], xp, acc[m][r]);
                }
            }
            const int pos = g0 + t0 + t;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const int row = row0 + q * RPP + r * GPW * SWAVES;
                const float s0 = group_sum<LPR>(acc[0][r]) * p.ts0;
                const float s1 = NMAT == 2 ? group_sum<LPR>(acc[NMAT - 1][r]) * p.ts1 : 0.f;
                if (li == LPR - 1 && row < p.N) {
                    if (GATEUP) {
                        const float sc = p.wts ? p.wts[p.sorted[pos]] : 1.f;
                        store_act(p.out, (size_t)pos * p.N + row, sc * swiglu(s0, s1), p.act_f32);
                    } else {
                        reinterpret_cast<float *>(p.out)[(size_t)pos * p.N + row] = s0;
                    }
                }
            }
        }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    const bool once = ne <= p.mt;   // all of the expert's rows staged at once
    load_pass(0, B0{});
    if (once) {
        stage(0, ne);
        __syncthreads();
    }
    auto run_pass = [&](int q, auto buf_c) __attribute__((always_inline)) {
        if (once) {
            compute(q, 0, ne, buf_c);
        } else {
            for (int t0 = 0; t0 < ne; t0 += p.mt) {
                const int mt = min(p.mt, ne - t0);
                __syncthreads();   // the previous chunk's reads of xs are done
                stage(t0, mt);
                __syncthreads();
                compute(q, t0, mt, buf_c);
            }
        }
    };
#pragma unroll
    for (int q = 0; q < NPASS; q += 2) {
        if (q + 1 < NPASS) load_pass(q + 1, B1{});
        run_pass(q, B0{});
        if (q + 1 < NPASS) {
            if (q + 2 < NPASS) load_pass(q + 2, B0{});
            run_pass(q + 1, B1{});
        }
    }
}

// 16-byte chunks per lane and lanes per row for rows of nch chunks
static void lane_shape(int nch, int &cpl, int &lpr) {
    lpr = nch <= 16 ? 16 : nch <= 32 ? 32 : 64;
    const int c = (nch + lpr - 1) / lpr;
    cpl = c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 16;
}

template <class F, bool GATEUP>
static hipError_t stream_launch(StreamParams prm, const moe_shape &s, hipStream_t st) {
    const int nch = prm.K / F::EPC;
    int cpl, lpr;
    lane_shape(nch, cpl, lpr);
    const size_t xrow = (size_t)prm.K * (prm.act_f32 ? 4 : 2);
    // an expert holds at most one slot per token, so at most T rows are ever staged
    prm.mt = (int)std::min<size_t>(std::min<size_t>(16, (size_t)std::max(1, s.num_tokens)), STAGE_BYTES / xrow);
    if (prm.mt < 1) return hipErrorInvalidValue;
    const size_t lds = (size_t)prm.mt * xrow;
    const int maxa = std::min(s.num_experts, s.num_tokens * s.top_k);
    constexpr int NMAT = GATEUP ? 2 : 1;
    auto go = [&](auto kern, int rg) {
        const int rows_per_block = rg * (WAVE / lpr) * SWAVES * passes<F>();
        dim3 grid((prm.N + rows_per_block - 1) / rows_per_block, maxa);
        hipLaunchKernelGGL(kern, grid, dim3(SNT), lds, st, prm);
        return hipGetLastError();
    };
#define MOE_SL(C, L) go(stream_ffn_kernel<F, C, L, GATEUP>, rows_per_group<F, C, NMAT>())
    if (lpr == 16) return MOE_SL(1, 16);
    if (lpr == 32) return MOE_SL(1, 32);
    if constexpr (F::EPC == 32) {   // MXFP4 rows of at most 8192 elements: <= 4 chunks per lane
        switch (cpl) {
            case 1: return MOE_SL(1, 64);
            case 2: return MOE_SL(2, 64);
            case 4: return MOE_SL(4, 64);
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (cpl) {
            case 1: return MOE_SL(1, 64);
            case 2: return MOE_SL(2, 64);
            case 4: return MOE_SL(4, 64);
            case 8: return MOE_SL(8, 64);
            default: return MOE_SL(16, 64);
        }
    }
#undef MOE_SL
}

}  // namespace

bool stream_ffn_supported(const moe_shape &s) {
    const size_t ab = act_bytes(s.act_dtype);
    const int epc = weight_chunk_elems(s.weight_dtype);
    // one activation row must fit the staging area; rows of at most 16 chunks per lane
    return (size_t)s.hidden * ab <= STAGE_BYTES && (size_t)s.intermediate * ab <= STAGE_BYTES &&
           s.hidden / epc <= 64 * 16 && s.intermediate / epc <= 64 * 16;
}

hipError_t launch_decode_gateup(const moe_shape &s, const void *x, const moe_expert_weights &w,
                                const int32_t *offsets, const int32_t *sorted, const int32_t *active,
                                const float *wts, void *h, hipStream_t st) {
    StreamParams prm{};
    prm.act = static_cast<const uint8_t *>(x);
    prm.w0 = static_cast<const uint8_t *>(w.w_gate);
    prm.w1 = static_cast<const uint8_t *>(w.w_up);
    prm.s0 = w.s_gate;
    prm.s1 = w.s_up;
    prm.ts0 = s.weight_dtype == MOE_NVFP4 ? w.ts_gate : 1.f;
    prm.ts1 = s.weight_dtype == MOE_NVFP4 ? w.ts_up : 1.f;
    prm.offsets = offsets;
    prm.sorted = sorted;
    prm.active = active;
    prm.wts = wts;
    prm.out = static_cast<uint8_t *>(h);
    prm.N = s.intermediate;
    prm.K = s.hidden;
    prm.topk = s.top_k;
    prm.act_f32 = s.act_dtype == MOE_F32;
    switch (s.weight_dtype) {
        case MOE_F32: return stream_launch<FmtF32, true>(prm, s, st);
        case MOE_BF16: return stream_launch<FmtBF16, true>(prm, s, st);
        case MOE_NVFP4: return stream_launch<FmtNV4, true>(prm, s, st);
        case MOE_MXINT8: return stream_launch<FmtI8, true>(prm, s, st);
        default: return stream_launch<FmtMX4, true>(prm, s, st);
    }
}

hipError_t launch_decode_down(const moe_shape &s, const moe_expert_weights &w, const int32_t *offsets,
                              const int32_t *active, const void *h, float *o, hipStream_t st) {
    StreamParams prm{};
    prm.act = static_cast<const uint8_t *>(h);
    prm.w0 = static_cast<const uint8_t *>(w.w_down);
    prm.s0 = w.s_down;
    prm.ts0 = s.weight_dtype == MOE_NVFP4 ? w.ts_down : 1.f;
    prm.ts1 = 1.f;
    prm.offsets = offsets;
    prm.active = active;
    prm.out = reinterpret_cast<uint8_t *>(o);
    prm.N = s.hidden;
    prm.K = s.intermediate;
    prm.topk = s.top_k;
    prm.act_f32 = s.act_dtype == MOE_F32;
    switch (s.weight_dtype) {
        case MOE_F32: return stream_launch<FmtF32, false>(prm, s, st);
        case MOE_BF16: return stream_launch<FmtBF16, false>(prm, s, st);
        case MOE_NVFP4: return stream_launch<FmtNV4, false>(prm, s, st);
        case MOE_MXINT8: return stream_launch<FmtI8, false>(prm, s, st);
        default: return stream_launch<FmtMX4, false>(prm, s, st);
    }
}

}  // namespace moe
