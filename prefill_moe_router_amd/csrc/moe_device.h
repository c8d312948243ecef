// moe_device.h -- device-side helpers shared by the gfx950 kernels: element
// formats (fp32, bf16, MXFP4), 16-byte chunk dot products, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int WAVE = 64;

// ---- scalar conversions --------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even: the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32) in the default round-to-nearest-even mode
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// lo*lo' + hi*hi' + c on packed bf16 pairs, fp32 accumulate (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// E8M0 scale code -> fp32 multiplier 2^(code-127) (code 0 maps to 0, 255 to inf)
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) { return __uint_as_float(code << 23); }

// two E2M1 codes of byte `sel` of `packed` (low nibble first) times `scale`, as bf16x2
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t packed, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, SEL));
}

// silu(g) * u = g * u / (1 + e^-g), with the hardware reciprocal (v_rcp_f32, 1 ulp)
// instead of a correctly rounded division: the result is stored as bf16 (or compared at
// 1e-5 relative in fp32), far above that error.  g -> -inf gives g * rcp(inf) = -0.
__device__ __forceinline__ float swiglu(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// streaming (non-temporal) 16-byte load: weights are read once per call
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- bounded loads through a buffer resource --------------------------------------------
// A raw buffer resource over [base, base + bytes): a load at an offset past the end
// returns zero without touching memory.  Loads of a fixed count through it need no branch
// for the part of a row that does not exist, so the compiler's waits can count exactly
// the loads issued after the one a use depends on.  The base must be the same in every
// lane (it is taken from the first active one).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;   // an offset past the end of every resource

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    // word 3 (0x00020000): the gfx9 raw-buffer data format
    return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// 16 bytes at byte offset off, non-temporal (weights are read once per call)
__device__ __forceinline__ uint4 ld_rsrc16(rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// 16 bytes at byte offset off past the non-coherent caches (sc1: the load an agent-scope
// atomic load is), for data other work-groups wrote with agent-scope stores
__device__ __forceinline__ uint4 ld_rsrc16_agent(rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_rsrc_u8(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld_rsrc_u16(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---- waits, barriers and direct-to-LDS loads ----------------------------------------

typedef __attribute__((address_space(3))) void lds_ptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// one wave-wide direct load: 16 bytes per lane from g into LDS at l + 16 * lane (l
// wave-uniform).  A plain (non-template) function keeps the builtin out of the host
// pass's instantiation of the kernel template.
__device__ __forceinline__ void load_lds16(const void *g, uint8_t *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t *)l, 16, 0, 0);
}

// work-group barrier with no memory fence; "memory" keeps the compiler from moving
// memory accesses across it (the waits before it are explicit)
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// ---- wave64 reductions -----------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// DPP move of v (fp32 bits); lanes with no source read `fill`
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v, float fill) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                      false));
}

// Sums of groups of 16 / 32 / 64 consecutive lanes through DPP row shifts and
// row broadcasts (no LDS traffic).  The group's total lands in its last lane
// (lane 15 of each row, lanes 31 and 63, or lane 63).
__device__ __forceinline__ float dpp_sum16(float v) {
    v += dpp_f<0x111>(v, 0.f);  // row_shr:1
    v += dpp_f<0x112>(v, 0.f);  // row_shr:2
    v += dpp_f<0x114>(v, 0.f);  // row_shr:4
    v += dpp_f<0x118>(v, 0.f);  // row_shr:8
    return v;
}
__device__ __forceinline__ float dpp_sum32(float v) {
    v = dpp_sum16(v);
    return v + dpp_f<0x142, 0xa>(v, 0.f);  // row_bcast:15 into rows 1 and 3
}
__device__ __forceinline__ float dpp_sum64(float v) {
    v = dpp_sum32(v);
    return v + dpp_f<0x143, 0xc>(v, 0.f);  // row_bcast:31 into rows 2 and 3
}
// wave-uniform total of v over the 64 lanes
__device__ __forceinline__ float wave_sum_u(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dpp_sum64(v)), 63));
}
__device__ __forceinline__ float wave_max_u(float v) {
    const float ninf = -__builtin_inff();
    v = fmaxf(v, dpp_f<0x111>(v, ninf));
    v = fmaxf(v, dpp_f<0x112>(v, ninf));
    v = fmaxf(v, dpp_f<0x114>(v, ninf));
    v = fmaxf(v, dpp_f<0x118>(v, ninf));
    v = fmaxf(v, dpp_f<0x142, 0xa>(v, ninf));
    v = fmaxf(v, dpp_f<0x143, 0xc>(v, ninf));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// order-preserving map of fp32 to uint32 (-0 and +0 map to the same key)
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// lanes below this one
__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = threadIdx.x & 63;
    return l ? (~0ull >> (64 - l)) : 0ull;
}

// Top-k of one token's E (<= 1024) logits in one wave, by radix selection on
// order-preserving keys: the k-th largest key is found bit by bit from the
// top with ballot counts, keys above it are kept, and keys equal to it are
// kept in ascending expert id until k are kept (ties go to the lower id).
// Writes ids (ascending) and weights (softmax over all E at the kept ids,
// renormalised over the kept set when renorm) to ids[0..k) / w[0..k) (LDS) and
// ids_g / w_g (global), each when given, and ORs sel_bit into sel_mask[e] (LDS)
// for every kept expert e.
template <int NJ>
__device__ __forceinline__ void wave_topk(const float *lg, int E, int K, int renorm, int *ids, float *w,
                                          int32_t *ids_g, float *w_g, uint32_t *sel_mask = nullptr,
                                          uint32_t sel_bit = 0) {
    const int lane = threadIdx.x & 63;
    float v[NJ];
    uint32_t key[NJ];
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + 64 * j;
        const bool ok = e < E;
        v[j] = ok ? lg[e] : -__builtin_inff();
        key[j] = ok ? f32_order_key(v[j]) : 0u;
        m = fmaxf(m, v[j]);
    }
    m = wave_max_u(m);
    // Bit by bit from the top: `avail` keys share the prefix chosen so far, `need` of
    // them are still to be kept.  Once they are equal, every key sharing the prefix is
    // kept and the remaining bits need not be looked at (the common case after a dozen
    // bits); otherwise the walk ends at bit 0 with the threshold key itself.
    uint32_t prefix = 0;
    int need = K, avail = E;
    int b = 31;
    for (; b >= 0; --b) {
        const uint32_t cand = prefix | (1u << b);
        const uint32_t hi = cand >> b;   // odd, so the key 0 of a padding lane never matches
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot((key[j] >> b) == hi));
        if (cnt >= need) {
            prefix = cand;
            avail = cnt;
        } else {
            need -= cnt;
            avail -= cnt;
        }
        if (avail == need) break;
    }
    const int sh = b < 0 ? 0 : b;        // keys are compared on bits [sh, 32)
    const uint32_t pfx = prefix >> sh;
    // kept: top bits above the prefix, or equal to it among the first `need` such in id
    // order (all of them when the walk stopped early)
    const uint64_t lt = lanemask_lt();
    int eq_before = 0, sel_before = 0;
    float z = 0.f;
    float pe[NJ];
    bool sel[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool valid = key[j] != 0u;
        const uint32_t top = key[j] >> sh;
        const bool eq = valid && top == pfx;
        const uint64_t eqm = __ballot(eq);
        const int eq_rank = eq_before + __popcll(eqm & lt);
        eq_before += __popcll(eqm);
        sel[j] = valid && (top > pfx || (eq && eq_rank < need));
        pe[j] = valid ? __expf(v[j] - m) : 0.f;
        if (!renorm || sel[j]) z += pe[j];
    }
    const float denom = wave_sum_u(z);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const uint64_t sm = __ballot(sel[j]);
        const int pos = sel_before + __popcll(sm & lt);
        sel_before += __popcll(sm);
        if (sel[j]) {
            const int e = lane + 64 * j;
            const float wt = pe[j] / denom;
            if (ids) ids[pos] = e;
            if (w) w[pos] = wt;
            if (ids_g) ids_g[pos] = e;
            if (w_g) w_g[pos] = wt;
            if (sel_mask) atomicOr(sel_mask + e, sel_bit);
        }
    }
}

// DPP reductions of N independent values per lane at once, written step by step across
// the N values so that their chains interleave; each result is read from lane 63 and is
// wave-uniform.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v, uint32_t fill) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROW_MASK, 0xf, false);
}
// inclusive prefix sum over the 64 lanes: shifts within rows of 16 lanes, then the row
// totals through the row broadcasts (lane 63 ends with the total)
__device__ __forceinline__ uint32_t wave_incl_sum_u(uint32_t v) {
    v += dpp_u<0x111, 0xf>(v, 0u);   // row_shr:1
    v += dpp_u<0x112, 0xf>(v, 0u);   // row_shr:2
    v += dpp_u<0x114, 0xf>(v, 0u);   // row_shr:4
    v += dpp_u<0x118, 0xf>(v, 0u);   // row_shr:8
    v += dpp_u<0x142, 0xa>(v, 0u);   // row_bcast:15 into rows 1 and 3
    v += dpp_u<0x143, 0xc>(v, 0u);   // row_bcast:31 into rows 2 and 3
    return v;
}
template <int N>
__device__ __forceinline__ void wave_umax_n(uint32_t (&v)[N]) {
#define MOE_UMAX_STEP(CTRL, RM)                                                     \
    _Pragma("unroll") for (int i = 0; i < N; ++i) v[i] = max(v[i], dpp_u<CTRL, RM>(v[i], 0u));
    MOE_UMAX_STEP(0x111, 0xf)   // row_shr:1
    MOE_UMAX_STEP(0x112, 0xf)   // row_shr:2
    MOE_UMAX_STEP(0x114, 0xf)   // row_shr:4
    MOE_UMAX_STEP(0x118, 0xf)   // row_shr:8
    MOE_UMAX_STEP(0x142, 0xa)   // row_bcast:15 into rows 1 and 3
    MOE_UMAX_STEP(0x143, 0xc)   // row_bcast:31 into rows 2 and 3
#undef MOE_UMAX_STEP
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (uint32_t)__builtin_amdgcn_readlane((int)v[i], 63);
}
template <int N>
__device__ __forceinline__ void wave_fsum_n(float (&v)[N]) {
#define MOE_FSUM_STEP(CTRL, RM) _Pragma("unroll") for (int i = 0; i < N; ++i) v[i] += dpp_f<CTRL, RM>(v[i], 0.f);
    MOE_FSUM_STEP(0x111, 0xf)
    MOE_FSUM_STEP(0x112, 0xf)
    MOE_FSUM_STEP(0x114, 0xf)
    MOE_FSUM_STEP(0x118, 0xf)
    MOE_FSUM_STEP(0x142, 0xa)
    MOE_FSUM_STEP(0x143, 0xc)
#undef MOE_FSUM_STEP
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// inverse of f32_order_key
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Top-k of NTOK tokens at once in one wave (lg: the tokens' logits rows, E apart; E <=
// 64*NJ), with the selection and weights of wave_topk: the K largest logits, ties to the
// lower expert id, ids ascending, softmax weights (renormalised over the kept set when
// asked).  Logits are compared as order-preserving keys (-0 and +0 equal).  Two ways to
// select, both exact:
//  - ROUNDS (small K): K rounds of a wave arg-max over the keys not yet kept (DPP max,
//    then the lowest id holding it);
//  - otherwise the radix walk of wave_topk without its early exit: the K-th largest key
//    tau is built bit by bit (keep a bit when at least K keys are >= the candidate), keys
//    above tau are kept, keys equal to tau in ascending id.
// The tokens' chains run in lockstep with no branch, so they overlap.  Token tk's ids and
// weights go to s_ids / s_w + tk*K (LDS; the caller copies them out), and bit (bit0 + tk)
// is ORed into sel_mask[e] (LDS) for each kept expert of the tokens below nvalid.  s_trash:
// 64 words of LDS that lanes with nothing to write write to instead.
template <int NJ, int NTOK, bool ROUNDS>
__device__ __forceinline__ void wave_topk_multi(const float *lg, int E, int K, int renorm, int nvalid, int *s_ids,
                                                float *s_w, uint32_t *sel_mask, int bit0, uint32_t *s_trash) {
    const int lane = threadIdx.x & 63;
    float v[NTOK][NJ];
    uint32_t key[NTOK][NJ];
    bool sel[NTOK][NJ];
#pragma unroll
    for (int tk = 0; tk < NTOK; ++tk)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int e = lane + 64 * j;
            v[tk][j] = e < E ? lg[tk * E + e] : 0.f;
            key[tk][j] = e < E ? f32_order_key(v[tk][j]) : 0u;   // 0: no expert (below every key)
            sel[tk][j] = false;
        }
    uint32_t mkey[NTOK];
    if constexpr (ROUNDS) {
        uint32_t kt[NTOK][NJ];
#pragma unroll
        for (int tk = 0; tk < NTOK; ++tk)
#pragma unroll
            for (int j = 0; j < NJ; ++j) kt[tk][j] = key[tk][j];
        for (int round = 0; round < K; ++round) {
            uint32_t M[NTOK];
#pragma unroll
            for (int tk = 0; tk < NTOK; ++tk) {
                M[tk] = kt[tk][0];
#pragma unroll
                for (int j = 1; j < NJ; ++j) M[tk] = max(M[tk], kt[tk][j]);
            }
            wave_umax_n(M);
#pragma unroll
            for (int tk = 0; tk < NTOK; ++tk) {
                mkey[tk] = round == 0 ? M[tk] : mkey[tk];
                // lowest id holding M (ids lane + 64j: the first j with a hit, then its
                // lowest lane), by selects only
                uint64_t hit = __ballot(kt[tk][NJ - 1] == M[tk]);
                int wj = NJ - 1;
#pragma unroll
                for (int j = NJ - 2; j >= 0; --j) {
                    const uint64_t hj = __ballot(kt[tk][j] == M[tk]);
                    wj = hj ? j : wj;
                    hit = hj ? hj : hit;
                }
                const int wl = __builtin_ctzll(hit | (1ull << 63));
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const bool win = lane == wl && j == wj;
                    kt[tk][j] = win ? 0u : kt[tk][j];
                    sel[tk][j] = sel[tk][j] || win;
                }
            }
        }
    } else {
#pragma unroll
        for (int tk = 0; tk < NTOK; ++tk) {
            mkey[tk] = key[tk][0];
#pragma unroll
            for (int j = 1; j < NJ; ++j) mkey[tk] = max(mkey[tk], key[tk][j]);
        }
        wave_umax_n(mkey);
        uint32_t tau[NTOK];
#pragma unroll
        for (int tk = 0; tk < NTOK; ++tk) tau[tk] = 0u;
        for (int b = 31; b >= 0; --b) {
#pragma unroll
            for (int tk = 0; tk < NTOK; ++tk) {
                const uint32_t cand = tau[tk] | (1u << b);
                int cnt = 0;
#pragma unroll
                for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(key[tk][j] >= cand));
                tau[tk] = cnt >= K ? cand : tau[tk];
            }
        }
        const uint64_t lt = lanemask_lt();
#pragma unroll
        for (int tk = 0; tk < NTOK; ++tk) {
            int n_gt = 0;
#pragma unroll
            for (int j = 0; j < NJ; ++j) n_gt += __popcll(__ballot(key[tk][j] > tau[tk]));
            const int need = K - n_gt;
            int eq_before = 0;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bool eq = key[tk][j] != 0u && key[tk][j] == tau[tk];
                const uint64_t eqm = __ballot(eq);
                const int eq_rank = eq_before + __popcll(eqm & lt);
                eq_before += __popcll(eqm);
                sel[tk][j] = key[tk][j] != 0u && (key[tk][j] > tau[tk] || (eq && eq_rank < need));
            }
        }
    }
    const uint64_t lt = lanemask_lt();
    float pe[NTOK][NJ];
    float z[NTOK];
#pragma unroll
    for (int tk = 0; tk < NTOK; ++tk) {
        const float m = f32_from_order_key(mkey[tk]);
        z[tk] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            pe[tk][j] = key[tk][j] != 0u ? __expf(v[tk][j] - m) : 0.f;
            z[tk] += (!renorm || sel[tk][j]) ? pe[tk][j] : 0.f;
        }
    }
    wave_fsum_n(z);
#pragma unroll
    for (int tk = 0; tk < NTOK; ++tk) {
        int sel_before = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint64_t sm = __ballot(sel[tk][j]);
            const int pos = sel_before + __popcll(sm & lt);
            sel_before += __popcll(sm);
            const int e = lane + 64 * j;
            const bool s = sel[tk][j];
            *(s ? reinterpret_cast<uint32_t *>(s_ids + tk * K + pos) : s_trash + lane) = (uint32_t)e;
            *(s ? reinterpret_cast<uint32_t *>(s_w + tk * K + pos) : s_trash + lane) =
                __float_as_uint(pe[tk][j] / z[tk]);
            atomicOr(sel_mask + (e < E ? e : 0), s && tk < nvalid ? 1u << (bit0 + tk) : 0u);
        }
    }
}

// ---- element formats -------------------------------------------------------------
// A "chunk" is 16 bytes of a weight row: 4 fp32, 8 bf16 or 32 MXFP4 codes (one
// scale block).  Dot products are taken chunk by chunk against the matching
// activation elements.

struct FmtF32 {  // fp32 weights with fp32 activations
    static constexpr int EPC = 4;          // elements per 16-byte weight chunk
    static constexpr int XB = 16;          // activation bytes per chunk
    static constexpr bool SCALED = false;
    static constexpr int SB = 0;
};
struct FmtBF16 {  // bf16 weights with bf16 activations
    static constexpr int EPC = 8;
    static constexpr int XB = 16;
    static constexpr bool SCALED = false;
    static constexpr int SB = 0;
};
struct FmtMX4 {  // MXFP4 weights with bf16 activations
    static constexpr int EPC = 32;
    static constexpr int XB = 64;
    static constexpr bool SCALED = true;
    static constexpr int SB = 1;           // scale bytes per chunk: one E8M0 per 32 elements
};
struct FmtNV4 {  // NVFP4 weights (E2M1 codes, one E4M3 scale per 16 elements) with bf16 activations
    static constexpr int EPC = 32;
    static constexpr int XB = 64;
    static constexpr bool SCALED = true;
    static constexpr int SB = 2;           // two E4M3 scales per chunk (elements 0-15, 16-31)
};
struct FmtI8 {  // MXINT8 weights (OCP MX INT8 codes, one E8M0 scale per 32 elements), bf16 activations
    static constexpr int EPC = 16;
    static constexpr int XB = 32;
    static constexpr bool SCALED = true;
    static constexpr int SB = 1;           // one E8M0 scale per two chunks
};

// bytes of scales of a row of nch 16-byte chunks
template <class F>
__host__ __device__ constexpr size_t scale_row_bytes(size_t nch) {
    return !F::SCALED ? 0 : F::EPC == 16 ? nch / 2 : nch * F::SB;
}

// the scale code of chunk idx of a scale row: one byte (MXFP4), two (NVFP4, low byte
// for the chunk's first 16 elements), or the byte chunks 2j and 2j+1 share (MXINT8)
template <class F>
__device__ __forceinline__ uint32_t load_scale(const uint8_t *s, size_t idx) {
    if constexpr (F::SB == 2) return reinterpret_cast<const uint16_t *>(s)[idx];
    if constexpr (F::EPC == 16) return s[idx >> 1];
    return s[idx];
}

// the scale code of chunk ch through a resource over one scale row (zero past its end)
template <class F>
__device__ __forceinline__ uint32_t load_scale_r(rsrc_t r, uint32_t ch) {
    if constexpr (F::SB == 2) return ld_rsrc_u16(r, ch < 0x40000000u ? ch * 2 : kOutOfRange);
    if constexpr (F::EPC == 16) return ld_rsrc_u8(r, ch >> 1);
    return ld_rsrc_u8(r, ch);
}

// OCP MX INT8: an element is its int8 code times 2^-6, times the block's E8M0 scale
// 2^(code - 127): one power of two 2^(code - 133) for the block
__device__ __forceinline__ float mxint8_scale(uint32_t scale_code) {
    return __builtin_ldexpf(1.0f, (int)scale_code - 133);
}

// the signed bytes 2 SEL and 2 SEL + 1 of w times s, as a bf16 pair: exact while s is a
// power of two that keeps the products normal (an int8 needs 8 significant bits)
template <int SEL>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, float s) {
    const float lo = (float)(int8_t)(uint8_t)(w >> (16 * SEL)) * s;
    const float hi = (float)(int8_t)(uint8_t)(w >> (16 * SEL + 8)) * s;
    return pack_bf16x2(lo, hi);
}

// OCP FP8 E4M3 (bias 7, no infinities): normal codes (1 + m/8) * 2^(e-7), exponent field 0
// m/8 * 2^-6.  The NaN codes (S.1111.111) are not valid block scales.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// The same value as a power of two p2 times a factor f with at most 4 significant bits
// (1 + m/8, or m for exponent field 0, signed).  v_cvt_scalef32_pk_bf16_fp4 applies only
// the power-of-two part of its scale operand (measured on gfx950: a scale of 1.5 decodes
// as 1.0), so E4M3 scales are applied as the instruction's p2 and then f.
__device__ __forceinline__ void e4m3_split(uint32_t b, float &p2, float &f) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    p2 = e ? __uint_as_float((e + 120u) << 23) : 0.001953125f;
    f = e ? 1.0f + 0.125f * (float)m : (float)m;
    f = (b & 0x80u) ? -f : f;
}

// a bf16 pair times f, where each product is exact in bf16 (the repack truncates)
__device__ __forceinline__ uint32_t bf16x2_mul_exact(uint32_t v, float f) {
    const float lo = __uint_as_float(v << 16) * f, hi = __uint_as_float(v & 0xffff0000u) * f;
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// partial dot of one weight chunk with the activation chunk at xp (XB bytes)
template <class F>
__device__ __forceinline__ float chunk_dot(const uint4 &w, uint32_t scale_code, const uint8_t *xp, float acc);

template <>
__device__ __forceinline__ float chunk_dot<FmtF32>(const uint4 &w, uint32_t, const uint8_t *xp, float acc) {
    const float4 xv = *reinterpret_cast<const float4 *>(xp);
    acc = fmaf(__uint_as_float(w.x), xv.x, acc);
    acc = fmaf(__uint_as_float(w.y), xv.y, acc);
    acc = fmaf(__uint_as_float(w.z), xv.z, acc);
    acc = fmaf(__uint_as_float(w.w), xv.w, acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<FmtBF16>(const uint4 &w, uint32_t, const uint8_t *xp, float acc) {
    const uint4 xv = *reinterpret_cast<const uint4 *>(xp);
    acc = dot2_bf16(w.x, xv.x, acc);
    acc = dot2_bf16(w.y, xv.y, acc);
    acc = dot2_bf16(w.z, xv.z, acc);
    acc = dot2_bf16(w.w, xv.w, acc);
    return acc;
}

__device__ __forceinline__ float mx4_word_dot(uint32_t codes, float s, const uint4 &xv, float acc) {
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(codes, s), xv.x, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(codes, s), xv.y, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(codes, s), xv.z, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(codes, s), xv.w, acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<FmtMX4>(const uint4 &w, uint32_t scale_code, const uint8_t *xp, float acc) {
    const float s = e8m0_to_f32(scale_code);
    const uint4 *x4 = reinterpret_cast<const uint4 *>(xp);
    acc = mx4_word_dot(w.x, s, x4[0], acc);
    acc = mx4_word_dot(w.y, s, x4[1], acc);
    acc = mx4_word_dot(w.z, s, x4[2], acc);
    acc = mx4_word_dot(w.w, s, x4[3], acc);
    return acc;
}

// MXINT8: the 16 codes as bf16 (exact), dotted with 32 bytes of activations; the block's
// power of two multiplies the chunk's partial sum
template <>
__device__ __forceinline__ float chunk_dot<FmtI8>(const uint4 &w, uint32_t scale_code, const uint8_t *xp, float acc) {
    const uint4 *x4 = reinterpret_cast<const uint4 *>(xp);
    const uint4 xa = x4[0], xb = x4[1];
    float a = dot2_bf16(i8x2_to_bf16x2<0>(w.x, 1.0f), xa.x, 0.f);
    a = dot2_bf16(i8x2_to_bf16x2<1>(w.x, 1.0f), xa.y, a);
    a = dot2_bf16(i8x2_to_bf16x2<0>(w.y, 1.0f), xa.z, a);
    a = dot2_bf16(i8x2_to_bf16x2<1>(w.y, 1.0f), xa.w, a);
    a = dot2_bf16(i8x2_to_bf16x2<0>(w.z, 1.0f), xb.x, a);
    a = dot2_bf16(i8x2_to_bf16x2<1>(w.z, 1.0f), xb.y, a);
    a = dot2_bf16(i8x2_to_bf16x2<0>(w.w, 1.0f), xb.z, a);
    a = dot2_bf16(i8x2_to_bf16x2<1>(w.w, 1.0f), xb.w, a);
    return fmaf(mxint8_scale(scale_code), a, acc);
}

// NVFP4: each 16-element block is dotted with its codes' E2M1 values (decoded with a unit
// scale, exact) and the block's E4M3 scale multiplies the block's partial sum
template <>
__device__ __forceinline__ float chunk_dot<FmtNV4>(const uint4 &w, uint32_t scale_code, const uint8_t *xp, float acc) {
    const float s0 = e4m3_to_f32(scale_code & 0xffu), s1 = e4m3_to_f32(scale_code >> 8);
    const uint4 *x4 = reinterpret_cast<const uint4 *>(xp);
    float a0 = mx4_word_dot(w.x, 1.0f, x4[0], 0.f);
    a0 = mx4_word_dot(w.y, 1.0f, x4[1], a0);
    float a1 = mx4_word_dot(w.z, 1.0f, x4[2], 0.f);
    a1 = mx4_word_dot(w.w, 1.0f, x4[3], a1);
    return fmaf(s1, a1, fmaf(s0, a0, acc));
}

}  // namespace moe
