// grouped_gemm.hip -- MFMA (bf16, fp32 accumulate) grouped GEMM for prefill
// chunks: the dense contractions of the layer when each expert sees many
// tokens (the 8192-token chunks of "第 9 章 prefill：最大的瓶颈" §9.8, whose
// fused path groups tokens by expert on the device, §9.9).
//
// One kernel template, three uses:
//   ROUTER : logits[t][e] = x[t] . Wr[e] + bias[e]                  (fp32 out)
//   GATEUP : h'[p][i] = w_slot * silu(x_t . Wg[e][i]) * (x_t . Wu[e][i])
//            for sorted position p of expert e, token t = slot / k     (bf16 out)
//   DOWN   : o'[slot][n] = h'[p] . Wd[e][n]                          (bf16 out,
//            rows scattered to token-major slot order for the combine)
//   DOWN_F32: o[p][n] = h[p] . Wd[e][n] in sorted order, fp32 (the staged call)
//
// Tiling: a work-group computes a BM x BN output tile (two of them, gate and
// up, for GATEUP) with K steps of BK, from double-buffered LDS staged through
// registers; LDS rows padded by 16 bytes so the 16-byte MFMA operand reads of
// 16 consecutive rows hit 64 distinct banks.  Tiles are ordered m-tile major
// (the n-tiles of one m-tile share the gathered A rows) and the block id is
// remapped so each XCD works on a contiguous range of that order.
#include <hip/hip_ext.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int NXCD = 8;

enum { GM_ROUTER = 0, GM_GATEUP = 1, GM_DOWN = 2, GM_DOWN_F32 = 3 };
// 16-byte scale-table pieces per thread of the MXFP4 gate/up (K <= 6144 with 256 weight rows
// and 512 threads)
constexpr int kScaleTableChunks = 6;

#ifndef MOE_GEMM_GM
#define MOE_GEMM_GM 8   // m-tiles per ordering group of the tile order
#endif

struct GemmParams {
    const uint8_t *a;          // x [T][K] (ROUTER, GATEUP) or h' [P][K] (DOWN), bf16
    const int32_t *sorted;     // sorted slots [P]
    const int32_t *offsets;    // expert offsets [E+1]
    const int32_t *mtile_off;  // m-tile offsets [E+1] (tiles of BM rows per expert)
    const uint8_t *b0, *b1;    // weights [E][N][K] bf16, or MXFP4 codes [E][N][K/2] (b1: up, GATEUP only)
    const uint8_t *s0, *s1;    // MXFP4 E8M0 scales [E][N][K/32] or NVFP4 E4M3 scales [E][N][K/16]
    float ts0, ts1;            // NVFP4 tensor scales of b0 / b1
    const float *wts;          // gate weight per slot (GATEUP)
    const float *bias;         // router bias [N] or null
    uint8_t *out;
    int M, N, K, topk, E;
    int mt_max, nt;            // logical grid: nt n-tiles x mt_max m-tiles
};

__device__ __forceinline__ int find_expert(const int32_t *mtile_off, int E, int mt) {
    int lo = 0, hi = E;  // mtile_off[lo] <= mt < mtile_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (mtile_off[mid] <= mt) lo = mid;
        else hi = mid;
    }
    return lo;
}

// BM x BN output tile per matrix (NB = 2 matrices, gate and up, for GATEUP), K steps
// of BK, WM x WN waves, each wave MI x NJ blocks of 32x32 per matrix.  LDS rows are
// padded by 16 bytes so 16 consecutive rows read at one k offset hit distinct banks.
template <int MODE, int BM, int BN, int WM, int WN, int BK, int NS, bool MX, bool NV = false, bool I8 = false,
          bool ST = false>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(GemmParams p) {
    constexpr int NTH = WM * WN * 64;
    constexpr int NB = MODE == GM_GATEUP ? 2 : 1;
    constexpr int MI = BM / WM / 32, NJ = BN / WN / 32;
    constexpr int CPR = BK / 8;                       // 16-byte chunks per row
    constexpr int RPP = NTH / CPR;                    // rows staged per pass of all threads
    constexpr int AR = BM / RPP, BR = BN / RPP;       // staged rows per thread (A, each B)
    constexpr int GROW = BK * 2 + 16;                 // padded LDS row bytes
    constexpr int STAGE = (BM + NB * BN) * GROW;
    static_assert(AR * RPP == BM && BR * RPP == BN, "staging must tile the block");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int s_slot[BM];
    __shared__ float s_scale[BM];

    // ---- which tile ----------------------------------------------------------------------
    // Logical order: groups of MOE_GEMM_GM consecutive m-tiles, each group swept n-tile by
    // n-tile, so the tiles running together on one XCD share A rows and weight slices
    // in its L2; each XCD takes a contiguous range of that order.
    const int nblk = gridDim.x;
    const int per_xcd = nblk / NXCD;                 // grid is a multiple of NXCD
    const int L = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
    constexpr int GM = MOE_GEMM_GM;
    const int grp = L / (GM * p.nt), in_grp = L % (GM * p.nt);
    const int n_tile = in_grp / GM, mt = grp * GM + in_grp % GM;
    if (mt >= p.mt_max) return;
    int e = 0, m0, m_end;
    if (MODE == GM_ROUTER) {
        m0 = mt * BM;
        m_end = p.M;
        if (m0 >= m_end) return;
    } else {
        if (mt >= p.mtile_off[p.E]) return;
        e = find_expert(p.mtile_off, p.E, mt);
        m0 = p.offsets[e] + (mt - p.mtile_off[e]) * BM;
        m_end = p.offsets[e + 1];
    }
    const int n0 = n_tile * BN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t krow = (size_t)p.K * 2;   // bytes per A / B row

    if (MODE != GM_ROUTER) {
        for (int m = tid; m < BM; m += NTH) {
            const int pos = min(m0 + m, m_end - 1);
            const int slot = p.sorted[pos];
            s_slot[m] = slot;
            s_scale[m] = (MODE == GM_GATEUP && m0 + m < m_end) ? (p.wts ? p.wts[slot] : 1.f) : 0.f;
        }
    }
    __syncthreads();

    // ---- global sources of the rows this thread stages (CPR chunks of 16 B per row) ------
    const int sr = tid / CPR, sc = tid % CPR;
    const uint8_t *arow[AR];
#pragma unroll
    for (int i = 0; i < AR; ++i) {
        const int m = sr + RPP * i;
        const int pos = min(m0 + m, m_end - 1);
        const size_t row = MODE == GM_GATEUP ? (size_t)(s_slot[m] / p.topk) : (size_t)pos;
        arow[i] = p.a + row * krow + sc * 16;
    }
    const uint8_t *brow[NB][BR];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint8_t *base = (b == 0 ? p.b0 : p.b1) + ((size_t)e * p.N + n0) * krow;
#pragma unroll
        for (int i = 0; i < BR; ++i) brow[b][i] = MX ? nullptr : base + (size_t)(sr + RPP * i) * krow + sc * 16;
    }
    // MXFP4 / NVFP4 weights: a 16-byte chunk of E2M1 codes (32 K elements) per (weight row,
    // chunk); MXINT8 (I8): a 16-byte chunk of int8 codes (16 K elements, half a scale
    // block).  Dequantised to bf16 while it is written to LDS.
    static_assert(!I8 || (MX && !NV), "MXINT8 takes the coded-weight path");
    constexpr int QE = I8 ? 16 : 32;                              // K elements per code chunk
    constexpr int CQ = BK / QE;                                   // code chunks per row and K step
    constexpr int BQ = MX ? NB * BN * CQ / NTH : 1;               // code chunks staged per thread
    static_assert(!MX || BQ * NTH == NB * BN * CQ, "coded-weight staging must tile the block");
    // ST (MXFP4, MXINT8): the tile's E8M0 scales for the whole K ([NB*BN rows][K/32] bytes)
    // sit in LDS after the stages, loaded once per tile in 16-byte pieces (K % 512 == 0),
    // instead of one scale byte per thread and step from global memory (each such load
    // touches 32 rows' cache lines).  Step kt reads the bytes of the slice it writes to LDS
    // at its start.
    static_assert(!ST || (MX && !NV && (MODE == GM_GATEUP || MODE == GM_DOWN)), "scale table: E8M0 scales");
    const int srow = p.K / 32;               // scale bytes per weight row
    uint8_t *const sct = lds + NS * STAGE;   // the scale table
    int sidx[BQ];                            // this thread's row of the table, plus its chunk
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
        const int idx = tid + NTH * i;
        sidx[i] = (idx / CQ) * srow + (I8 ? idx % CQ / 2 : idx % CQ);   // MXINT8: two chunks a block
    }
    const uint8_t *bqrow[BQ], *bqsc[BQ];
    int bqlds[BQ];
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
        const int idx = tid + NTH * i, r = idx / CQ, c = idx % CQ;   // r: row over both matrices
        const int b = r / BN, rr = r % BN;
        const size_t grow = (size_t)e * p.N + n0 + rr;
        bqrow[i] = MX ? (b == 0 ? p.b0 : p.b1) + grow * (size_t)(I8 ? p.K : p.K / 2) + c * 16 : nullptr;
        bqsc[i] = MX ? (b == 0 ? p.s0 : p.s1) + grow * (size_t)(p.K / (NV ? 16 : 32)) + (I8 ? c / 2 : c * (NV ? 2 : 1))
                     : nullptr;
        bqlds[i] = (BM + r) * GROW + c * QE * 2;
    }

    // register sets of K slices in flight: a slice is loaded two steps before it is written
    // to LDS, three for the router (its one 4096-deep K loop per tile waits on memory).
    // Measured on the 4096-token chunks, layer time: MXFP4 1584 -> 1580 us, MXINT8 2402 ->
    // 2394, NVFP4 2091 -> 2082; three sets for the coded-weight gate/up made it slower
    // (MXFP4 1009 -> 1015 us, MXINT8 1483 -> 1604 us with 246 VGPRs).
    constexpr int BRX = MX ? 1 : BR;
    u32x4_t ra0[AR], rb0[NB][BRX], ra1[AR], rb1[NB][BRX], ra2[AR], rb2[NB][BRX];
    u32x4_t rq0[BQ], rq1[BQ], rq2[BQ];
    uint32_t rs0[BQ], rs1[BQ], rs2[BQ];
#define GG_GLOAD(RA, RB, RQ, RS, kt)                                                                      \
    do {                                                                                                  \
        const size_t ko_ = (size_t)(kt) * BK * 2;                                                         \
        _Pragma("unroll") for (int i = 0; i < AR; ++i) RA[i] = *reinterpret_cast<const u32x4_t *>(arow[i] + ko_); \
        if constexpr (MX) {                                                                               \
            _Pragma("unroll") for (int i = 0; i < BQ; ++i) {                                              \
                RQ[i] = *reinterpret_cast<const u32x4_t *>(bqrow[i] + (size_t)(kt) * (I8 ? BK : BK / 2)); \
                RS[i] = NV   ? (uint32_t) * reinterpret_cast<const uint16_t *>(bqsc[i] + (kt) * CQ * 2)    \
                        : ST ? 0u                                                                         \
                             : (uint32_t)bqsc[i][(kt) * (BK / 32)];                                        \
            }                                                                                             \
        } else {                                                                                          \
            _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                \
                _Pragma("unroll") for (int i = 0; i < BR; ++i) RB[b][i] =                                 \
                    *reinterpret_cast<const u32x4_t *>(brow[b][i] + ko_);                                  \
        }                                                                                                 \
    } while (0)
#define GG_LSTORE(RA, RB, RQ, RS, SX, stage)                                                              \
    do {                                                                                                  \
        uint8_t *base_ = lds + (stage) * STAGE;                                                           \
        _Pragma("unroll") for (int i = 0; i < AR; ++i)                                                    \
            *reinterpret_cast<u32x4_t *>(base_ + (sr + RPP * i) * GROW + sc * 16) = RA[i];                \
        if constexpr (MX && NV) {                                                                         \
            /* NVFP4: the power of two of each block's E4M3 scale in the convert, then the */              \
            /* remaining factor (exact in bf16) */                                                          \
            _Pragma("unroll") for (int i = 0; i < BQ; ++i) {                                              \
                float p2_[2], f_[2];                                                                      \
                e4m3_split(RS[i] & 0xffu, p2_[0], f_[0]);                                                 \
                e4m3_split(RS[i] >> 8, p2_[1], f_[1]);                                                    \
                _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                           \
                    const uint32_t cw = RQ[i][w];                                                         \
                    const float s_ = p2_[w >> 1], f2_ = f_[w >> 1];                                       \
                    u32x4_t o_;                                                                           \
                    o_[0] = bf16x2_mul_exact(fp4x2_to_bf16x2<0>(cw, s_), f2_);                            \
                    o_[1] = bf16x2_mul_exact(fp4x2_to_bf16x2<1>(cw, s_), f2_);                            \
                    o_[2] = bf16x2_mul_exact(fp4x2_to_bf16x2<2>(cw, s_), f2_);                            \
                    o_[3] = bf16x2_mul_exact(fp4x2_to_bf16x2<3>(cw, s_), f2_);                            \
                    *reinterpret_cast<u32x4_t *>(base_ + bqlds[i] + w * 16) = o_;                         \
                }                                                                                         \
            }                                                                                             \
        } else if constexpr (I8) {                                                                        \
            /* MXINT8: each code times the block's power of two (exact in bf16) */                        \
            _Pragma("unroll") for (int i = 0; i < BQ; ++i) {                                              \
                const float s_ = mxint8_scale(ST ? SX[i] : RS[i]);                                        \
                _Pragma("unroll") for (int w = 0; w < 2; ++w) {                                           \
                    u32x4_t o_;                                                                           \
                    o_[0] = i8x2_to_bf16x2<0>(RQ[i][2 * w], s_);                                          \
                    o_[1] = i8x2_to_bf16x2<1>(RQ[i][2 * w], s_);                                          \
                    o_[2] = i8x2_to_bf16x2<0>(RQ[i][2 * w + 1], s_);                                      \
                    o_[3] = i8x2_to_bf16x2<1>(RQ[i][2 * w + 1], s_);                                      \
                    *reinterpret_cast<u32x4_t *>(base_ + bqlds[i] + w * 16) = o_;                         \
                }                                                                                         \
            }                                                                                             \
        } else if constexpr (MX) {                                                                        \
            _Pragma("unroll") for (int i = 0; i < BQ; ++i) {                                              \
                const float s_ = e8m0_to_f32(ST ? SX[i] : RS[i]);                                         \
                _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                           \
                    const uint32_t cw = RQ[i][w];                                                         \
                    u32x4_t o_;                                                                           \
                    o_[0] = fp4x2_to_bf16x2<0>(cw, s_);                                                   \
                    o_[1] = fp4x2_to_bf16x2<1>(cw, s_);                                                   \
                    o_[2] = fp4x2_to_bf16x2<2>(cw, s_);                                                   \
                    o_[3] = fp4x2_to_bf16x2<3>(cw, s_);                                                   \
                    *reinterpret_cast<u32x4_t *>(base_ + bqlds[i] + w * 16) = o_;                         \
                }                                                                                         \
            }                                                                                             \
        } else {                                                                                          \
            _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                \
                _Pragma("unroll") for (int i = 0; i < BR; ++i)                                            \
                    *reinterpret_cast<u32x4_t *>(base_ + (BM + b * BN + sr + RPP * i) * GROW + sc * 16) = RB[b][i]; \
        }                                                                                                 \
    } while (0)

    // ---- MFMA main loop ----------------------------------------------------------------------
    const int wm = (wave / WN) * (BM / WM), wn = (wave % WN) * (BN / WN);
    const int lr = lane & 31, lk = (lane >> 5) * 16;          // operand row, k byte offset
    f32x16_t acc[NB][MI][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.f;

    // Double-buffered LDS, two register sets (three for the router).  Step kt computes
    // from LDS stage kt&1 while the global loads of slice kt+2 (kt+3) fill one register
    // set and slice kt+1 (loaded earlier) goes from another set into stage (kt+1)&1.  Inside a step the
    // operands of k-slice ks+1 are read from LDS while the MFMAs of slice ks run; the
    // scheduling hints interleave MFMA, DS-read and VMEM issue.
    static_assert(NS == 2, "two LDS stages");
    constexpr int KS = BK / 16;
    constexpr int NMF = NB * MI * NJ, NDS = MI + NB * NJ;
    const int KT = p.K / BK;
    bf16x8_t av[2][MI], bv[2][NB][NJ];
#define GG_OPLOAD(buf, base_, ks_)                                                                        \
    do {                                                                                                  \
        const int ko_ = (ks_) * 32 + lk;                                                                  \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) av[buf][i] =                                       \
            *reinterpret_cast<const bf16x8_t *>((base_) + (wm + 32 * i + lr) * GROW + ko_);               \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                    \
            _Pragma("unroll") for (int j = 0; j < NJ; ++j) bv[buf][b][j] =                                \
                *reinterpret_cast<const bf16x8_t *>((base_) + (BM + b * BN + wn + 32 * j + lr) * GROW + ko_); \
    } while (0)
#define GG_STEP(kt_, DIST, RA_LOAD, RB_LOAD, RQ_LOAD, RS_LOAD, RA_STORE, RB_STORE, RQ_STORE, RS_STORE)      \
    do {                                                                                                  \
        uint32_t sx_[BQ];                                                                                 \
        if constexpr (ST) {                                                                               \
            _Pragma("unroll") for (int i = 0; i < BQ; ++i) sx_[i] =                                       \
                sct[sidx[i] + min((kt_) + 1, KT - 1) * (BK / 32)];                                        \
        }                                                                                                 \
        GG_GLOAD(RA_LOAD, RB_LOAD, RQ_LOAD, RS_LOAD, min((kt_) + (DIST), KT - 1));                        \
        const uint8_t *base = lds + ((kt_) & 1) * STAGE;                                                  \
        if constexpr (ACT) {                                                                              \
            _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                           \
                const int cur = ks & 1;                                                                   \
                if (ks + 1 < KS) GG_OPLOAD(cur ^ 1, base, ks + 1);                                        \
                _Pragma("unroll") for (int b = 0; b < NB; ++b)                                            \
                    _Pragma("unroll") for (int i = 0; i < MI; ++i)                                        \
                        _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[b][i][j] =                     \
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][i], bv[cur][b][j], acc[b][i][j], 0, 0, 0); \
            }                                                                                             \
            _Pragma("unroll") for (int q = 0; q < KS * NMF; ++q) {                                        \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                        \
                if (q < (KS - 1) * NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                \
                if (q < AR + (MX ? 2 * BQ : NB * BR)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  \
            }                                                                                             \
        }                                                                                                 \
        GG_LSTORE(RA_STORE, RB_STORE, RQ_STORE, RS_STORE, sx_, ((kt_) + 1) & 1);                          \
        __syncthreads();                                                                                  \
        if constexpr (ACT) GG_OPLOAD(0, lds + (((kt_) + 1) & 1) * STAGE, 0);                              \
    } while (0)
    // A wave whose rows all lie past the tile's last row (an expert's tail m-tile) still
    // stages its share of every slice into LDS and takes every barrier, but reads no
    // operands and issues no MFMAs.  Not for NVFP4 weights: with the loop inside a lambda
    // their gate/up ran 5% slower on the 4096-token chunk (1249 -> 1312 us), against 3.5%
    // faster for MXFP4, so NVFP4 keeps the loop inline.
    if constexpr (NV) {
        constexpr bool ACT = true;
        GG_GLOAD(ra0, rb0, rq0, rs0, 0);
        GG_GLOAD(ra1, rb1, rq1, rs1, min(1, KT - 1));
        GG_LSTORE(ra0, rb0, rq0, rs0, rs0, 0);
        __syncthreads();
        GG_OPLOAD(0, lds, 0);
        for (int kt = 0; kt < KT; kt += 2) {
            GG_STEP(kt, 2, ra0, rb0, rq0, rs0, ra1, rb1, rq1, rs1);
            if (kt + 1 < KT) GG_STEP(kt + 1, 2, ra1, rb1, rq1, rs1, ra0, rb0, rq0, rs0);
        }
    } else {
        auto main_loop = [&](auto act_c) __attribute__((always_inline)) {
            constexpr bool ACT = decltype(act_c)::value;
            // the scale table's loads go first, so writing it to LDS waits for them only
            constexpr int TC = ST ? kScaleTableChunks : 1;
            const int tcr = srow / 16, ntc = NB * BN * tcr;
            u32x4_t tv[TC];
            if constexpr (ST) {
#pragma unroll
                for (int j = 0; j < TC; ++j) {
                    const int q = min(tid + NTH * j, ntc - 1), r = q / tcr, b = r / BN;
                    tv[j] = *reinterpret_cast<const u32x4_t *>((b == 0 ? p.s0 : p.s1) +
                                                               ((size_t)e * p.N + n0 + r % BN) * srow + (q % tcr) * 16);
                }
            }
            GG_GLOAD(ra0, rb0, rq0, rs0, 0);
            GG_GLOAD(ra1, rb1, rq1, rs1, min(1, KT - 1));
            uint32_t sx0[BQ];
            if constexpr (ST) {
#pragma unroll
                for (int j = 0; j < TC; ++j)
                    if (tid + NTH * j < ntc) *reinterpret_cast<u32x4_t *>(sct + (tid + NTH * j) * 16) = tv[j];
                __syncthreads();
#pragma unroll
                for (int i = 0; i < BQ; ++i) sx0[i] = sct[sidx[i]];
            }
            if constexpr (MODE == GM_ROUTER) {
                // slice s sits in register set s % 3: step kt loads slice kt + 3 into the set
                // that slice kt left (written to LDS the step before) and writes slice kt + 1
                GG_GLOAD(ra2, rb2, rq2, rs2, min(2, KT - 1));
                GG_LSTORE(ra0, rb0, rq0, rs0, sx0, 0);
                __syncthreads();
                if constexpr (ACT) GG_OPLOAD(0, lds, 0);
                for (int kt = 0; kt < KT; kt += 3) {
                    GG_STEP(kt, 3, ra0, rb0, rq0, rs0, ra1, rb1, rq1, rs1);
                    if (kt + 1 < KT) GG_STEP(kt + 1, 3, ra1, rb1, rq1, rs1, ra2, rb2, rq2, rs2);
                    if (kt + 2 < KT) GG_STEP(kt + 2, 3, ra2, rb2, rq2, rs2, ra0, rb0, rq0, rs0);
                }
            } else {
                GG_LSTORE(ra0, rb0, rq0, rs0, sx0, 0);
                __syncthreads();
                if constexpr (ACT) GG_OPLOAD(0, lds, 0);
                for (int kt = 0; kt < KT; kt += 2) {
                    GG_STEP(kt, 2, ra0, rb0, rq0, rs0, ra1, rb1, rq1, rs1);
                    if (kt + 1 < KT) GG_STEP(kt + 1, 2, ra1, rb1, rq1, rs1, ra0, rb0, rq0, rs0);
                }
            }
        };
        if (wm < m_end - m0)
            main_loop(std::true_type{});
        else
            main_loop(std::false_type{});
    }
#undef GG_STEP
#undef GG_GLOAD
#undef GG_LSTORE
#undef GG_OPLOAD

    // ---- epilogue ------------------------------------------------------------------------------
    // acc[.][i][j][r] holds C[row][col] with row = wm + 32i + 8(r/4) + 4(lane/32) + r%4,
    // col = wn + 32j + lane%32.
    if (MODE == GM_GATEUP || MODE == GM_DOWN) {
        // bf16 outputs: each wave transposes its tile through LDS and stores whole
        // 16-byte row pieces (the main loop is done with LDS after the last barrier)
        constexpr int TR = MI * 32, TC = NJ * 32, PITCH = TC + 8;
        uint16_t *ep = reinterpret_cast<uint16_t *>(lds) + wave * TR * PITCH;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    float v;
                    float g_ = acc[0][i][j][r], u_ = acc[NB - 1][i][j][r];
                    if constexpr (NV) {
                        g_ *= p.ts0;
                        u_ *= p.ts1;
                    }
                    if (MODE == GM_GATEUP) v = s_scale[wm + ml] * swiglu(g_, u_);
                    else v = g_;
                    ep[ml * PITCH + 32 * j + lr] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        constexpr int CPRow = TC / 8;   // 16-byte pieces per tile row
        for (int q = lane; q < TR * CPRow; q += 64) {
            const int ml = q / CPRow, ch = q % CPRow;
            const int m = wm + ml;
            if (m0 + m >= m_end) continue;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ep + ml * PITCH + ch * 8);
            const size_t row = MODE == GM_GATEUP ? (size_t)(m0 + m) : (size_t)s_slot[m];
            *reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(p.out) + row * p.N + n0 + wn + ch * 8) = v;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m0 + m >= m_end) continue;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int n = n0 + wn + 32 * j + lr;
                if (MODE == GM_ROUTER) {
                    const float b = p.bias ? p.bias[n] : 0.f;
                    reinterpret_cast<float *>(p.out)[(size_t)(m0 + m) * p.N + n] = acc[0][i][j][r] + b;
                } else {
                    reinterpret_cast<float *>(p.out)[(size_t)(m0 + m) * p.N + n] =
                        NV ? acc[0][i][j][r] * p.ts0 : acc[0][i][j][r];
                }
            }
        }
    }
}

// Tile shapes (rows per m-tile = the grouping's kGroupedTileM for the expert GEMMs,
// columns per n-tile and matrix, wave grid, K step).
#ifndef MOE_GU_CFG
#define MOE_GU_CFG 128, 128, 2, 4, 64   // gate/up: 128 x (128 + 128), 8 waves
#endif
#ifndef MOE_DN_CFG
#define MOE_DN_CFG 128, 256, 2, 4, 64   // down: 128 x 256, 8 waves
#endif
// router: x . Wr in 64 x 64 tiles, so 4096 tokens at E = 256 make 256 work-groups (64 with
// 128 x 128 tiles); measured on the 4096-token MXFP4, NVFP4 and MXINT8 chunks: layer 1598 ->
// 1587, 2118 -> 2104 and 2415 -> 2409 us.  An output's K order does not depend on the tile.
#define MOE_R_CFG 64, 64, 2, 2, 64
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_;
};
using CfgGU = TileCfg<MOE_GU_CFG>;
using CfgGU64 = TileCfg<64, 128, 2, 4, 64>;   // gate/up with the medium batches' 64-row m-tiles
using CfgDN = TileCfg<MOE_DN_CFG>;
using CfgR = TileCfg<MOE_R_CFG>;
static_assert(CfgGU::BM == kGroupedTileM && CfgDN::BM == kGroupedTileM && CfgGU64::BM == kWideSmallTileM,
              "m-tiles follow the grouping");

// m-tile offsets of the experts' groups: mtile_off[e] = sum over e' < e of ceil(cnt[e'] / rows),
// and the tile table: tiles[t] = {first row, end row of the expert, expert, 0}
__global__ __launch_bounds__(1024) void mtile_offsets_kernel(const int32_t *__restrict__ offsets, int E,
                                                             int32_t *__restrict__ mtile_off, int4 *__restrict__ tiles,
                                                             int rows) {
    __shared__ int s[1025];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) s[e] = (offsets[e + 1] - offsets[e] + rows - 1) / rows;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            const int c = s[e];
            s[e] = run;
            run += c;
        }
        s[E] = run;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += blockDim.x) mtile_off[e] = s[e];
    for (int e = tid; e < E; e += blockDim.x)
        for (int t = s[e]; t < s[e + 1]; ++t)
            tiles[t] = make_int4(offsets[e] + (t - s[e]) * rows, offsets[e + 1], e, 0);
}

// y[t][n] = sum_j o'[t*k + j][n]  (bf16 rows of one token, fp32 sum, one rounding)
__global__ __launch_bounds__(256) void combine_rows_kernel(const uint16_t *__restrict__ o, uint16_t *__restrict__ y,
                                                           int T, int H, int k) {
    const int t = blockIdx.x;
    const int n8 = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (t >= T || n8 >= H) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](const uint4 v) {
        acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
        acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
        acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
    };
    // the token's k rows are contiguous; up to eight loads in flight, summed in j order
    const uint16_t *src = o + (size_t)t * k * H + n8;
    int j = 0;
    for (; j + 8 <= k; j += 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4 *>(src + (size_t)(j + u) * H);
#pragma unroll
        for (int u = 0; u < 8; ++u) add(v[u]);
    }
    for (; j < k; ++j) add(*reinterpret_cast<const uint4 *>(src + (size_t)j * H));
    uint4 r;
    r.x = pack_bf16x2(acc[0], acc[1]);
    r.y = pack_bf16x2(acc[2], acc[3]);
    r.z = pack_bf16x2(acc[4], acc[5]);
    r.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4 *>(y + (size_t)t * H + n8) = r;
}

bool grouped_supported(const moe_shape &s) {
    return s.act_dtype == MOE_BF16 &&
           (s.weight_dtype == MOE_BF16 || s.weight_dtype == MOE_MXFP4 || s.weight_dtype == MOE_NVFP4 ||
            s.weight_dtype == MOE_MXINT8) &&
           s.hidden % CfgDN::BN == 0 && s.hidden % CfgGU::BK == 0 && s.intermediate % CfgGU::BN == 0 &&
           s.intermediate % CfgDN::BK == 0;
}

bool router_mfma_supported(const moe_shape &s) {
    return s.act_dtype == MOE_BF16 && s.num_experts % CfgR::BN == 0 && s.hidden % CfgR::BK == 0;
}

constexpr size_t kGemmLdsMax = 158 * 1024;
template <int MODE, class C>
constexpr size_t gemm_stage_bytes() {
    return C::NS * (size_t)(C::BM + (MODE == GM_GATEUP ? 2 : 1) * C::BN) * (C::BK * 2 + 16);
}
// an E8M0 scale table fits (whole 16-byte pieces, the LDS budget, the pieces per thread)
template <int MODE, class C>
static bool scale_table_fits(int K) {
    const size_t rows = (MODE == GM_GATEUP ? 2 : 1) * (size_t)C::BN;
    return K % 512 == 0 && gemm_stage_bytes<MODE, C>() + rows * (K / 32) <= kGemmLdsMax &&
           rows * (K / 512) <= (size_t)kScaleTableChunks * C::WM * C::WN * 64;
}

template <int MODE, class C, bool MX = false, bool NV = false, bool I8 = false, bool ST = false>
static hipError_t gemm_launch(GemmParams prm, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int NB = MODE == GM_GATEUP ? 2 : 1;
    constexpr size_t stage_bytes = gemm_stage_bytes<MODE, C>();
    constexpr size_t epi_bytes = (size_t)C::WM * C::WN * (C::BM / C::WM) * (C::BN / C::WN + 8) * 2;
    constexpr size_t lds_fixed = stage_bytes > epi_bytes ? stage_bytes : epi_bytes;
    static_assert(lds_fixed <= kGemmLdsMax, "LDS budget");
    const size_t lds = ST ? std::max(stage_bytes + (size_t)NB * C::BN * (prm.K / 32), epi_bytes) : lds_fixed;
    if (lds > kGemmLdsMax) return hipErrorInvalidValue;
    static bool attr_done = false;
    auto kern = grouped_gemm_kernel<MODE, C::BM, C::BN, C::WM, C::WN, C::BK, C::NS, MX, NV, I8, ST>;
    if (!attr_done) {
        hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(ST ? kGemmLdsMax : lds_fixed));
        if (r != hipSuccess) return r;
        attr_done = true;
    }
    int nblk = (prm.mt_max + MOE_GEMM_GM - 1) / MOE_GEMM_GM * MOE_GEMM_GM * prm.nt;
    nblk = (nblk + NXCD - 1) / NXCD * NXCD;
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(kern, dim3(nblk), dim3(C::WM * C::WN * 64), lds, st, ev0, ev1, 0, prm);
    else
        hipLaunchKernelGGL(kern, dim3(nblk), dim3(C::WM * C::WN * 64), lds, st, prm);
    return hipGetLastError();
}

hipError_t launch_router_mfma(const moe_shape &s, const void *x, const void *wr, const float *bias, float *logits,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    GemmParams prm{};
    prm.a = static_cast<const uint8_t *>(x);
    prm.b0 = static_cast<const uint8_t *>(wr);
    prm.bias = bias;
    prm.out = reinterpret_cast<uint8_t *>(logits);
    prm.M = s.num_tokens;
    prm.N = s.num_experts;
    prm.K = s.hidden;
    prm.topk = s.top_k;
    prm.E = 1;
    prm.mt_max = (s.num_tokens + CfgR::BM - 1) / CfgR::BM;
    prm.nt = s.num_experts / CfgR::BN;
    return gemm_launch<GM_ROUTER, CfgR>(prm, st, ev0, ev1);
}

hipError_t launch_mtile_offsets(const moe_shape &s, const int32_t *offsets, int32_t *mtile_off, int32_t *tiles,
                                int rows, hipStream_t st) {
    hipLaunchKernelGGL(mtile_offsets_kernel, dim3(1), dim3(1024), 0, st, offsets, s.num_experts, mtile_off,
                       reinterpret_cast<int4 *>(tiles), rows);
    return hipGetLastError();
}

static int mt_max_of(const moe_shape &s, int rows = kGroupedTileM) {
    const long P = (long)s.num_tokens * s.top_k;
    // sum over experts of ceil(cnt/rows) <= P/rows + (number of nonempty experts)
    return (int)(P / rows + std::min<long>(s.num_experts, P));
}

hipError_t launch_gateup_mfma(const moe_shape &s, const void *x, const moe_expert_weights &w, const int32_t *offsets,
                              const int32_t *sorted, const int32_t *mtile_off, const int32_t *tiles, const float *wts,
                              void *h, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (wide_gateup_supported(s)) return launch_gateup_wide(s, x, w, sorted, mtile_off, tiles, wts, h, st, ev0, ev1);
    GemmParams prm{};
    prm.a = static_cast<const uint8_t *>(x);
    prm.sorted = sorted;
    prm.offsets = offsets;
    prm.mtile_off = mtile_off;
    prm.b0 = static_cast<const uint8_t *>(w.w_gate);
    prm.b1 = static_cast<const uint8_t *>(w.w_up);
    prm.s0 = w.s_gate;
    prm.s1 = w.s_up;
    prm.ts0 = w.ts_gate;
    prm.ts1 = w.ts_up;
    prm.wts = wts;
    prm.out = static_cast<uint8_t *>(h);
    prm.M = s.num_tokens * s.top_k;
    prm.N = s.intermediate;
    prm.K = s.hidden;
    prm.topk = s.top_k;
    prm.E = s.num_experts;
    prm.mt_max = mt_max_of(s);
    prm.nt = s.intermediate / CfgGU::BN;
    if (s.weight_dtype == MOE_MXFP4 && grouped_tile_rows(s) == kWideSmallTileM) {
        prm.mt_max = mt_max_of(s, kWideSmallTileM);
        if (scale_table_fits<GM_GATEUP, CfgGU64>(s.hidden))
            return gemm_launch<GM_GATEUP, CfgGU64, true, false, false, true>(prm, st, ev0, ev1);
        return gemm_launch<GM_GATEUP, CfgGU64, true>(prm, st, ev0, ev1);
    }
    if (s.weight_dtype == MOE_MXFP4) {
        if (scale_table_fits<GM_GATEUP, CfgGU>(s.hidden))
            return gemm_launch<GM_GATEUP, CfgGU, true, false, false, true>(prm, st, ev0, ev1);
        return gemm_launch<GM_GATEUP, CfgGU, true>(prm, st, ev0, ev1);
    }
    if (s.weight_dtype == MOE_NVFP4) return gemm_launch<GM_GATEUP, CfgGU, true, true>(prm, st, ev0, ev1);
    if (s.weight_dtype == MOE_MXINT8) {
        if (scale_table_fits<GM_GATEUP, CfgGU>(s.hidden))
            return gemm_launch<GM_GATEUP, CfgGU, true, false, true, true>(prm, st, ev0, ev1);
        return gemm_launch<GM_GATEUP, CfgGU, true, false, true>(prm, st, ev0, ev1);
    }
    return gemm_launch<GM_GATEUP, CfgGU>(prm, st, ev0, ev1);
}

hipError_t launch_down_mfma(const moe_shape &s, const moe_expert_weights &w, const int32_t *offsets,
                            const int32_t *sorted, const int32_t *mtile_off, const int32_t *tiles, const void *h,
                            void *o, bool f32_sorted, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (!f32_sorted && wide_down_supported(s)) return launch_down_wide(s, w, sorted, mtile_off, tiles, h, o, st, ev0, ev1);
    GemmParams prm{};
    prm.a = static_cast<const uint8_t *>(h);
    prm.sorted = sorted;
    prm.offsets = offsets;
    prm.mtile_off = mtile_off;
    prm.b0 = static_cast<const uint8_t *>(w.w_down);
    prm.s0 = w.s_down;
    prm.ts0 = w.ts_down;
    prm.out = static_cast<uint8_t *>(o);
    prm.M = s.num_tokens * s.top_k;
    prm.N = s.hidden;
    prm.K = s.intermediate;
    prm.topk = s.top_k;
    prm.E = s.num_experts;
    prm.mt_max = mt_max_of(s);
    prm.nt = s.hidden / CfgDN::BN;
    const bool mx = s.weight_dtype == MOE_MXFP4, nv = s.weight_dtype == MOE_NVFP4, i8 = s.weight_dtype == MOE_MXINT8;
    if (f32_sorted) return nv ? gemm_launch<GM_DOWN_F32, CfgDN, true, true>(prm, st, ev0, ev1)
                         : i8 ? gemm_launch<GM_DOWN_F32, CfgDN, true, false, true>(prm, st, ev0, ev1)
                         : mx ? gemm_launch<GM_DOWN_F32, CfgDN, true>(prm, st, ev0, ev1)
                              : gemm_launch<GM_DOWN_F32, CfgDN>(prm, st, ev0, ev1);
    if (nv) return gemm_launch<GM_DOWN, CfgDN, true, true>(prm, st, ev0, ev1);
    const bool table = scale_table_fits<GM_DOWN, CfgDN>(s.intermediate);
    if (i8) return table ? gemm_launch<GM_DOWN, CfgDN, true, false, true, true>(prm, st, ev0, ev1)
                         : gemm_launch<GM_DOWN, CfgDN, true, false, true>(prm, st, ev0, ev1);
    if (mx) return table ? gemm_launch<GM_DOWN, CfgDN, true, false, false, true>(prm, st, ev0, ev1)
                         : gemm_launch<GM_DOWN, CfgDN, true>(prm, st, ev0, ev1);
    return gemm_launch<GM_DOWN, CfgDN>(prm, st, ev0, ev1);
}

hipError_t launch_combine_rows(const moe_shape &s, const void *o, void *y, hipStream_t st) {
    dim3 grid(s.num_tokens, (s.hidden / 8 + 255) / 256);
    hipLaunchKernelGGL(combine_rows_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t *>(o),
                       static_cast<uint16_t *>(y), s.num_tokens, s.hidden, s.top_k);
    return hipGetLastError();
}

}  // namespace moe
