// grouped_gemm_wide.hip -- the large-tile MFMA grouped GEMM for bf16 experts in
// prefill chunks (the expert contractions of the 8192-token chunks in
// "第 9 章 prefill：最大的瓶颈" §9.8, tokens grouped on the device as in §9.9).
//
//   GATEUP : h'[p][i] = w_slot * silu(x_t . Wg[e][i]) * (x_t . Wu[e][i])   (bf16, sorted order)
//   DOWN   : o'[slot][n] = h'[p] . Wd[e][n]             (bf16, rows scattered to slot order)
//
// Design for gfx950:
//  * A work-group owns a 128-row m-tile of one expert (bf16 medium batches: 64 rows, which
//    the grouping then emits) and 256 weight rows (GATEUP: 128
//    intermediate columns of both gate and up; DOWN: 256 output columns).  bf16: 2 x 4
//    waves of 64 rows x 64 weight rows (4 independent 32x32 MFMA accumulators; a 16-deep
//    K slice reads 4 KB of operands from LDS per 4 MFMAs, against 5 KB for 32 x 128) in one
//    persistent work-group per CU, with 64-deep stages (below); it fetches each next
//    tile's rows under the K loop and its first stages under the epilogue.  MXFP4 down:
//    2 x 2 waves of 64 x 128 (8 accumulators, 128 registers), 72 KB of LDS, so two
//    work-groups share a CU and one group's tile start and epilogue hide under the
//    other's MFMAs.
//  * A wave whose rows all lie past the expert's last row (the tail m-tile of an expert)
//    skips its operand reads and MFMAs; it still issues its share of the stage loads and
//    takes every barrier, so the wait counts hold.
//  * Each m-tile's rows come from a tile table the grouping writes ({first row, end
//    row, expert} per tile): one load, no search over the m-tile offsets.
//  * Operands go from global memory straight into LDS (global_load_lds_dwordx4: no
//    staging registers, no VALU), in a ring of 3 stages, so two stages are in flight
//    while one is consumed.  A stage is 32 K elements (64-byte rows) or 64 (128-byte
//    rows: each staged row piece is a whole line of its source row, which L2 serves
//    faster per byte than half lines, at the price of 144 KB of ring).
//  * LDS rows hold 16-byte chunks with the chunk index XOR-swizzled by a few row bits,
//    so the 16-byte operand reads fall in distinct banks without padding (a direct LDS
//    load writes 1 KB contiguously, which rules padding out).
//  * Waits are explicit: vmcnt counts this wave's loads of the stages still in flight,
//    and the work-group barrier carries no memory fence (a fence would drain the
//    loads in flight).  The barrier that ends stage st lands after the next stage's
//    first operands are in registers, so the slot it frees is refilled three stages
//    ahead.
#include <hip/hip_ext.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int NXCD = 8;
constexpr int TBN = 256;                // weight rows per n-tile (all configurations)
constexpr int BK = 32;                  // K elements of one step (two 16-deep MFMA slices)
enum { WG_GATEUP = 0, WG_DOWN = 1 };

// m-tiles per group of the tile order.  Measured on the 8192-token chunk (bf16, same-box
// rounds of 4 / 8 / 16 / 32): gate/up 546-553 us at 4 against 555-559 at 8, down
// 325.5-326.3 us at 16 against 327.3-329.2 at 8; MXFP4 down keeps 8.
constexpr int group_m(int mode, bool mx) { return mx ? 8 : mode == WG_GATEUP ? 4 : 16; }


struct WideParams {
    const uint8_t *a;          // x [T][K] (GATEUP) or h' [P][K] (DOWN), bf16
    const int32_t *sorted;     // sorted slots [P]
    const int32_t *mtile_off;  // m-tile offsets [E+1] (only [E], the tile count, is read)
    const int4 *tiles;         // per m-tile {first row, end row of the expert, expert, 0}
    const uint8_t *b0, *b1;    // weights [E][N][K] bf16 or MXFP4 codes [E][N][K/2] (b1: up, GATEUP only)
    const uint8_t *s0, *s1;    // MXFP4 E8M0 scales [E][N][K/32]
    const float *wts;          // gate weight per slot (GATEUP) or null
    uint8_t *out;
    int N, K, topk, E;         // N: weight rows per expert (GATEUP: I, DOWN: H)
    int mt_max, nt;
};

// The 16-byte chunk kc of LDS row r sits at chunk slot kc ^ swz<KH>(r).  Measured on
// gfx950 (SQ_LDS_BANK_CONFLICT of an isolated read loop): with 64-byte rows, the
// 16-byte MFMA operand reads (32 rows, two chunks per row per half-wave) are
// conflict-free with bits 2..3 of the row as the XOR key, 2-way with bits 1..2,
// 4-way unswizzled.  That fits 64 four-byte banks with 16 lanes of a 16-byte read
// served together: the 16 rows a read pass touches must spread over the 16 chunk
// positions of 256 bytes.  With 128-byte rows (two steps per stage) two rows share a
// 256-byte span, so the key is bits 1..3 of the row over eight chunk slots.
template <int KH>
__device__ __forceinline__ int swz(int r) { return KH == 1 ? (r >> 2) & 3 : (r >> 1) & 7; }




#define WG_INLINE __attribute__((always_inline))

}  // namespace

// WM x WN waves (4 or 8); each wave owns BM/WM rows x 128 weight rows.
// KH: steps (32 K elements each) per LDS stage.  KH = 2 stages 64 K elements, so every
// staged row is one whole 128-byte line of the source row: L2 serves a CU's requests
// line by line, and half-line requests take about as long as whole ones.  NS: stages
// in the LDS ring.
// MX: the weights are MXFP4 (KH = 1).  A stage then holds each B row's 16 bytes of E2M1
// codes (32 K elements; row stride 16 bytes, which 4-byte operand reads of 16
// consecutive rows take without bank conflicts), the tile's E8M0 scales for the whole K
// sit in an LDS table loaded once, and each B operand is decoded to bf16 as it is read
// from LDS (v_cvt_scalef32_pk_bf16_fp4): a quarter of the LDS bytes of bf16 weights.
// PER: persistent work-groups (one per CU, with the 144 KB ring) that walk their XCD's
// share of tiles.  Under each K loop they fetch the next tile's rows; after it, the next
// tile's first two stages load into ring slots 0 and 1 while the epilogue transposes
// through slot 2, so a tile's start no longer waits on the tile table and row list.
template <int MODE, int BM, int WM, int WN, int OCC, bool MX, int KH, int NS, bool PER>
__global__ __launch_bounds__(WM * WN * 64, OCC) void grouped_gemm_wide_kernel(WideParams p) {
    constexpr int NTH = WM * WN * 64;
    static_assert(WM * WN == 4 || WM * WN == 8, "four or eight waves");
    static_assert(KH == 1 || (KH == 2 && !MX), "two-step stages are for bf16 weights");
    static_assert(NS >= 2, "at least two stages");
    static_assert(!PER || (NS == 3 && WM * WN * 64 >= BM), "persistent: three slots, a thread per tile row");
    constexpr int WROWS = TBN / WN;                  // weight rows per wave
    constexpr int BN = TBN;                          // weight rows per n-tile
    constexpr int RW = BM / WM;                      // rows per wave
    constexpr int MI = RW / 32, NJ = WROWS / 32;     // 32x32 blocks per wave
    constexpr int ROWB = 64 * KH;                    // bytes of one staged bf16 row
    constexpr int LPR = ROWB / 16;                   // lanes per staged row in a direct load
    constexpr int B_ROWB = MX ? BK / 2 : ROWB;       // bytes of one staged B row
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * B_ROWB;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_LOADS = A_BYTES / 16 / NTH, B_LOADS = B_BYTES / 16 / NTH;   // per thread and stage
    constexpr int LOADS = A_LOADS + B_LOADS;
    constexpr int NCOL = MODE == WG_GATEUP ? BN / 2 : BN;   // output columns per n-tile
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    __shared__ int s_slot[PER ? 2 : 1][BM];
    __shared__ float s_scale[BM];

    constexpr int GM = group_m(MODE, MX);
    // ---- which tile: groups of GM m-tiles swept n-tile by n-tile (the last group holds
    // the remaining m-tiles), each XCD a contiguous, equal share of that order (blocks are
    // dealt to XCDs round-robin).  The share comes from the tile count the grouping wrote,
    // so the grid's slack past it (sized for the worst case) exits at once; persistent
    // work-groups take every (grid / 8)-th tile of their XCD's share.
    const int n_mt = p.mtile_off[p.E];
    const int total = n_mt * p.nt;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int xcd = blockIdx.x % NXCD;
    const int wstride = PER ? (int)(gridDim.x / NXCD) : per_xcd;
    // tile idx of this XCD's share: its n-tile, rows [m0, m_end) and expert
    auto tile_at = [&](int idx, int &nt_, int &m0_, int &mend_, int &e_) WG_INLINE {
        const int L = xcd * per_xcd + idx;
        if (idx >= per_xcd || L >= total) return false;
        const int grp = L / (GM * p.nt), in_grp = L % (GM * p.nt);
        const int gm = min(GM, n_mt - grp * GM);          // m-tiles in this group
        nt_ = in_grp / gm;
        // through the constant address space: a scalar load, counted by lgkmcnt, so fetching
        // the next tile under a K loop does not wait for the stage loads in flight (the table
        // is written by an earlier launch and only read here)
        typedef int i32x4c __attribute__((ext_vector_type(4)));
        const i32x4c ti = ((const __attribute__((address_space(4))) i32x4c *)(uintptr_t)p.tiles)[grp * GM + in_grp % gm];
        m0_ = ti.x;
        mend_ = ti.y;
        e_ = ti.z;
        return true;
    };
    int idx = blockIdx.x / NXCD;
    int n_tile, m0, m_end, e;
    if (!tile_at(idx, n_tile, m0, m_end, e)) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const size_t krow = (size_t)p.K * 2;           // bytes of one A row
    const int NST = p.K / (BK * KH);   // stages; KH == 1: even and >= 4, KH == 2: >= 2 (wide_*_supported)

    int sb = 0;   // s_slot buffer of the current tile
    for (int m = tid; m < BM; m += NTH) {
        const int pos = min(m0 + m, m_end - 1);
        const int slot = p.sorted[pos];
        s_slot[0][m] = slot;
        if (!PER) s_scale[m] = (MODE == WG_GATEUP && m0 + m < m_end) ? (p.wts ? p.wts[slot] : 1.f) : 0.f;
    }
    __syncthreads();

    // ---- sources of this lane's direct loads.  One wave-wide load fills 1 KB of LDS,
    // 1024 / ROWB rows of LPR chunks; lane l lands in row (1024 / ROWB) g + l / LPR at
    // chunk slot l % LPR, which holds the row's logical chunk (l % LPR) ^ swz(row).
    constexpr int RPL = 1024 / ROWB;               // rows per wave-wide load
    const int lrow = lane / LPR;
    // B: LDS row q of the tile belongs to the waves of column wn = q / WROWS.  GATEUP: the
    // first half of a wave's range is gate columns c0 + (WROWS / 2) * wn + (0 .. WROWS/2-1),
    // the second half the same up columns (c0 = the n-tile's first intermediate column).
    // DOWN: output column n0 + q.
    // global weight row of LDS B row r of n-tile nt_ of expert e_, and whether it belongs
    // to the second matrix (up)
    auto brow_of = [&](int r, bool &second, int e_, int nt_) WG_INLINE {
        if (MODE == WG_GATEUP) {
            const int rl = r % WROWS;
            second = rl >= WROWS / 2;
            return (size_t)e_ * p.N + (size_t)nt_ * NCOL + (WROWS / 2) * (r / WROWS) + ((unsigned)rl % (WROWS / 2));
        }
        second = false;
        return (size_t)e_ * p.N + (size_t)nt_ * BN + r;
    };
    const size_t brow_bytes = MX ? (size_t)p.K / 2 : krow;   // bytes of one global B row
    const uint8_t *asrc[A_LOADS];
    const uint8_t *bsrc[B_LOADS];
    // sources of a tile whose row slots are in s_slot[sbuf]
    auto set_sources = [&](int sbuf, int e_, int nt_, int m0_, int mend_) WG_INLINE {
#pragma unroll
        for (int q = 0; q < A_LOADS; ++q) {
            const int r = RPL * (wave * A_LOADS + q) + lrow;
            const int kc = (lane % LPR) ^ swz<KH>(r);
            const size_t row = MODE == WG_GATEUP ? (size_t)(s_slot[sbuf][r] / p.topk) : (size_t)min(m0_ + r, mend_ - 1);
            asrc[q] = p.a + row * krow + kc * 16;
        }
#pragma unroll
        for (int q = 0; q < B_LOADS; ++q) {
            // bf16: RPL rows of LPR swizzled chunks per wave-wide load; MX: 64 rows of one chunk
            const int r = MX ? 64 * (wave * B_LOADS + q) + lane : RPL * (wave * B_LOADS + q) + lrow;
            const int kc = MX ? 0 : (lane % LPR) ^ swz<KH>(r);
            bool second;
            const size_t wrow = brow_of(r, second, e_, nt_);
            bsrc[q] = (second ? p.b1 : p.b0) + wrow * brow_bytes + kc * 16;
        }
    };
    set_sources(0, e, n_tile, m0, m_end);
    auto issue = [&](int st, int stage) WG_INLINE {
        uint8_t *sa = lds + stage * STAGE;
        const size_t ko = (size_t)st * ROWB;
#pragma unroll
        for (int q = 0; q < A_LOADS; ++q)
            load_lds16(asrc[q] + ko, sa + (wave * A_LOADS + q) * 1024);
#pragma unroll
        for (int q = 0; q < B_LOADS; ++q)
            load_lds16(bsrc[q] + (size_t)st * B_ROWB, sa + A_BYTES + (wave * B_LOADS + q) * 1024);
    };
    // MX: the tile's scale table [BN][K/32] bytes at SC_OFF, loaded once (K % 512 == 0)
    constexpr int SC_OFF = NS * STAGE;
    const int spr = p.K / 32;                       // scale bytes per B row
    auto issue_scales = [&]() WG_INLINE {
        const int cpr = spr / 16;                   // 16-byte chunks per row
        for (int c0 = wave * WAVE; c0 < BN * cpr; c0 += NTH) {
            const int c = c0 + lane, r = c / cpr, w = c - r * cpr;
            bool second;
            const size_t wrow = brow_of(r, second, e, n_tile);
            load_lds16((second ? p.s1 : p.s0) + wrow * spr + w * 16, lds + SC_OFF + (size_t)c0 * 16);
        }
    };

    // ---- operand reads: lane reads row (32 * blk + lane % 32), logical chunk 4h + 2s +
    // lane / 32 for step half h of the stage and K16 sub-step s.  The chunk bits 0..1 and
    // bit 2 do not mix under the key, so half h is the offset of half 0 with bit 6 flipped.
    const int lr = lane & 31, hh = lane >> 5;
    const int opoff0 = lr * ROWB + ((hh ^ swz<KH>(lr)) * 16);
    const int opoff1 = lr * ROWB + (((2 + hh) ^ swz<KH>(lr)) * 16);
    bf16x8_t av[2][2][MI], bv[2][2][NJ];   // [buffer][k16 sub-step][block]
    // kt: the step (32 K elements) whose operands are read, from ring slot `stage`.
    // buf is a compile-time constant (std::integral_constant) so the operand arrays stay
    // in registers; so is the step's half of its stage (KH == 2: the buffer).
    auto read_ops = [&](int kt, int stage, auto buf_c) WG_INLINE {
        constexpr int buf = decltype(buf_c)::value;
        constexpr int hoff = KH == 2 ? 64 * buf : 0;
        const uint8_t *sa = lds + stage * STAGE + wm * RW * ROWB;
        const uint8_t *sb = lds + stage * STAGE + A_BYTES + wn * WROWS * B_ROWB;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int o = (s ? opoff1 : opoff0) ^ hoff;
#pragma unroll
            for (int i = 0; i < MI; ++i) av[buf][s][i] = *reinterpret_cast<const bf16x8_t *>(sa + i * 32 * ROWB + o);
            if constexpr (!MX) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    bv[buf][s][j] = *reinterpret_cast<const bf16x8_t *>(sb + j * 32 * ROWB + o);
            }
        }
        if constexpr (MX) {
            // lane (lr, hh) of sub-step s takes K elements 16s + 8hh .. +8 of its row: bytes
            // 8s + 4hh of the row's 16 staged code bytes; one E8M0 scale per row and stage
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int q = wn * WROWS + 32 * j + lr;
                const float sc = e8m0_to_f32(lds[SC_OFF + (size_t)q * spr + kt]);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint32_t cw = *reinterpret_cast<const uint32_t *>(sb + (32 * j + lr) * B_ROWB + 8 * s + 4 * hh);
                    u32x4_t o4;
                    o4[0] = fp4x2_to_bf16x2<0>(cw, sc);
                    o4[1] = fp4x2_to_bf16x2<1>(cw, sc);
                    o4[2] = fp4x2_to_bf16x2<2>(cw, sc);
                    o4[3] = fp4x2_to_bf16x2<3>(cw, sc);
                    bv[buf][s][j] = __builtin_bit_cast(bf16x8_t, o4);
                }
            }
        }
    };

    f32x16_t acc[MI][NJ];

    auto mfma_sub = [&](auto buf_c, auto s_c) WG_INLINE {
        constexpr int buf = decltype(buf_c)::value, s = decltype(s_c)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[buf][s][i], bv[buf][s][j], acc[i][j], 0, 0, 0);
    };

    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    // prologue: stages 0..NS-1 in flight, stage 0 landed for every wave, its first step's
    // operands read
    if constexpr (MX) issue_scales();   // older than the stage loads: retired by the first wait
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(min(st, NST - 1), st);
    wait_vm<(NS - 1) * LOADS>();
    barrier_nofence();
    if (wm * RW < m_end - m0) read_ops(0, 0, C0{});

    // A step consumes the operands of one 32-deep K slice from register buffer `cur`
    // and reads the next slice's into the other buffer.  A step that ends a stage (every
    // step for KH == 1, the second of each pair for KH == 2): MFMAs of the first K16
    // half; wait until this wave's loads of the next stage landed and its LDS reads are
    // done; barrier (so every wave's loads of the next stage landed and every wave is
    // done reading this one); refill this stage's slot NS stages ahead; read the next
    // stage's first operands; MFMAs of the second half.  A step inside a stage (KH == 2,
    // the first of each pair) only reads the stage's second half between its MFMAs.  In
    // the last stage-ending step (vm 0) nothing is refilled.
    // Scheduling: the MFMAs of the first half stay before the barrier, and the loads,
    // LDS reads and MFMAs of the second half are interleaved after it.  The refill
    // index is clamped: near the end it reloads the last stage into a slot nobody
    // reads again, which keeps the step branch-free.
    constexpr int NMF = MI * NJ, NRD = MX ? 2 * MI + 3 * NJ : 2 * (MI + NJ);
    constexpr int VPM = (LOADS + NMF - 1) / NMF;   // refill loads placed per MFMA
    // ACT: the wave has rows of the tile's expert; a wave past the expert's last row only
    // loads its share of the stages and takes the barriers.
    auto step = [&](int kt, int st, auto cur_c, auto ends_c, auto vm_c, auto refill_c, auto act_c) WG_INLINE {
        using Next = std::integral_constant<int, 1 - decltype(cur_c)::value>;
        constexpr bool ends = decltype(ends_c)::value;
        constexpr bool refill = ends && decltype(refill_c)::value;
        constexpr bool act = decltype(act_c)::value;
        if constexpr (act) mfma_sub(cur_c, C0{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ends) {
            wait_vm<decltype(vm_c)::value>();
            wait_lgkm0();
            barrier_nofence();
            __builtin_amdgcn_sched_barrier(0);
            if (refill) issue(min(st + NS, NST - 1), st % NS);
            if constexpr (act) read_ops(kt + 1, (st + 1) % NS, Next{});
        } else {
            if constexpr (act) read_ops(kt + 1, st % NS, Next{});
        }
        if constexpr (!act) return;
        mfma_sub(cur_c, C1{});
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   // one MFMA
            if (refill && q * VPM < LOADS) __builtin_amdgcn_sched_group_barrier(0x020, VPM, 0);  // VMEM reads
            if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, NRD / NMF > 1 ? NRD / NMF : 1, 0);  // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    using VL = std::integral_constant<int, (NS - 2) * LOADS>;
    using V0 = std::integral_constant<int, 0>;
    using T = std::true_type;
    using F = std::false_type;
    for (;;) {
        // PER: the next tile's rows and this tile's gate weights, fetched under the K loop
        // (kept in registers until the epilogue, so the K loop's waits are not extended)
        int n_nt = 0, n_m0 = 0, n_mend = 0, n_e = 0, n_slot = 0;
        float c_scale = 0.f;
        bool have_next = false;
        if constexpr (PER) {
            have_next = tile_at(idx + wstride, n_nt, n_m0, n_mend, n_e);
            if (tid < BM) {
                if (have_next) n_slot = p.sorted[min(n_m0 + tid, n_mend - 1)];
                if (MODE == WG_GATEUP) c_scale = m0 + tid < m_end ? (p.wts ? p.wts[s_slot[sb][tid]] : 1.f) : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        auto kloop = [&](auto a) WG_INLINE {
            if constexpr (KH == 1) {
                for (int kt = 0; kt < NST - 2; kt += 2) {
                    step(kt, kt, C0{}, T{}, VL{}, T{}, a);
                    step(kt + 1, kt + 1, C1{}, T{}, VL{}, T{}, a);
                }
                step(NST - 2, NST - 2, C0{}, T{}, V0{}, F{}, a);
            } else {
                for (int st = 0; st < NST - 2; ++st) {
                    step(2 * st, st, C0{}, F{}, V0{}, F{}, a);
                    step(2 * st + 1, st, C1{}, T{}, VL{}, T{}, a);
                }
                step(2 * NST - 4, NST - 2, C0{}, F{}, V0{}, F{}, a);
                step(2 * NST - 3, NST - 2, C1{}, T{}, V0{}, F{}, a);
                step(2 * NST - 2, NST - 1, C0{}, F{}, V0{}, F{}, a);
            }
            if constexpr (decltype(a)::value) {
                mfma_sub(C1{}, C0{});
                mfma_sub(C1{}, C1{});
            }
        };
        if (wm * RW < m_end - m0)
            kloop(T{});
        else
            kloop(F{});

        // ---- epilogue: each wave transposes its tile through LDS (its own region) and
        // stores whole 16-byte row pieces.  All waves are past their last LDS operand read
        // once they pass this barrier.
        __builtin_amdgcn_s_waitcnt(0);
        barrier_nofence();
        uint8_t *epi = lds;
        if constexpr (PER) {
            // this tile's gate weights and the next tile's row slots into LDS, then the next
            // tile's first two stages into slots 0 and 1; the epilogue works in slot 2
            if (tid < BM) {
                s_scale[tid] = c_scale;
                if (have_next) s_slot[sb ^ 1][tid] = n_slot;
            }
            __syncthreads();
            if (have_next) {
                set_sources(sb ^ 1, n_e, n_nt, n_m0, n_mend);
                issue(0, 0);
                issue(min(1, NST - 1), 1);
            }
            epi = lds + 2 * STAGE;
        }
        // acc[i][j][r] holds C[row][col], row = 32i + 8(r/4) + 4(lane/32) + r%4, col = 32j + lane%32
        if (MODE == WG_GATEUP) {
            // wave's h' tile: RW rows x HC columns (gate blocks j < NJ / 2 pair with up blocks
            // NJ / 2 + j)
            constexpr int HC = WROWS / 2, CPR = HC / 8;
            constexpr int PITCH = HC + 8;   // bf16 elements per transposed row
            uint16_t *ep = reinterpret_cast<uint16_t *>(epi) + wave * RW * PITCH;
    #pragma unroll
            for (int i = 0; i < MI; ++i)
    #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ml = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const float sc = s_scale[wm * RW + ml];
    #pragma unroll
                    for (int j = 0; j < NJ / 2; ++j)
                        ep[ml * PITCH + 32 * j + lr] =
                            (uint16_t)f32_to_bf16_rne(sc * swiglu(acc[i][j][r], acc[i][NJ / 2 + j][r]));
                }
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
            const int col0 = n_tile * NCOL + HC * wn;
            for (int q = lane; q < RW * CPR; q += 64) {
                const int ml = (unsigned)q / CPR, ch = (unsigned)q % CPR;
                const int m = wm * RW + ml;
                if (m0 + m >= m_end) continue;
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ep + ml * PITCH + ch * 8);
                *reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(p.out) + (size_t)(m0 + m) * p.N + col0 + ch * 8) = v;
            }
        } else {
            // wave's o' tile: RW rows x WROWS columns, in passes of PR rows (16 when the
            // epilogue shares the ring with the next tile's loads: a third of it)
            constexpr int PITCH = WROWS + 8, CPR = WROWS / 8;
            constexpr int PR = PER ? 16 : 32;
            uint16_t *ep = reinterpret_cast<uint16_t *>(epi) + wave * PR * PITCH;
            const int col0 = n_tile * BN + WROWS * wn;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int h = 0; h < 32 / PR; ++h) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int ml = 8 * (r >> 2) + 4 * hh + (r & 3);   // ml / PR depends on r only
                        if ((8 * (r >> 2)) / PR != h) continue;
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            ep[(ml - h * PR) * PITCH + 32 * j + lr] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
                    }
                    wait_lgkm0();
                    __builtin_amdgcn_wave_barrier();
                    for (int q = lane; q < PR * CPR; q += 64) {
                        const int ml = (unsigned)q / CPR, ch = (unsigned)q % CPR;
                        const int m = wm * RW + 32 * i + h * PR + ml;
                        if (m0 + m >= m_end) continue;
                        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ep + ml * PITCH + ch * 8);
                        *reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(p.out) + (size_t)s_slot[sb][m] * p.N +
                                                     col0 + ch * 8) = v;
                    }
                    wait_lgkm0();
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }

        if (!PER || !have_next) break;
        // the next tile: its stages 0 and 1 landed (vm 0 also retires the epilogue's stores),
        // every wave is past the epilogue's use of slot 2, which now takes stage 2
        idx += wstride;
        n_tile = n_nt;
        m0 = n_m0;
        m_end = n_mend;
        e = n_e;
        sb ^= 1;
        wait_vm<0>();
        wait_lgkm0();
        barrier_nofence();
        issue(min(2, NST - 1), 2);
        if (wm * RW < m_end - m0) read_ops(0, 0, C0{});
    }
}

namespace {

// the configurations the launchers use (the 8192-token chunk, H=2048, E=128, k=8, I=768,
// same-box A/B):
//  * bf16 gate/up and down: 2 x 4 waves (64 x 64 per wave, 128 x 256 per work-group),
//    stages of 64 K elements (whole-line rows), 3 of them (144 KB), one persistent
//    work-group per CU;
//  * MXFP4 down: 2 x 2 waves (64 x 128 per wave), stages of 32 K elements (the codes of a
//    B row are 16 bytes per step either way), 3 of them (72 KB with the scale table), two
//    work-groups per CU.
constexpr int CBN = TBN;
constexpr int MX_MAX_K = 4096;   // MXFP4: the tile's scale table (CBN x K/32 bytes) stays <= 32 KB

template <int MODE, bool MX>
struct WideCfg {
    static constexpr bool wide_stage = !MX;
    static constexpr int WM = 2, KH = wide_stage ? 2 : 1, NS = 3, OCC = wide_stage ? 1 : 2;
    static constexpr bool PER = wide_stage;
    static constexpr int WN = wide_stage ? 4 : 2;
    static constexpr int NTH = WM * WN * 64;
};

template <int MODE, bool MX, int BM>
hipError_t wide_launch(const WideParams &prm, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    using C = WideCfg<MODE, MX>;
    constexpr size_t rowb = 64 * C::KH;
    constexpr size_t stage = BM * rowb + CBN * (MX ? BK / 2 : rowb);
    constexpr size_t ring = (size_t)C::NS * stage;
    // the epilogue's transposes: per wave, its rows x (half) its columns (GATEUP) or passes of
    // 16 / 32 rows (DOWN), padded by 8 bf16 per row; in ring slot 2 for persistent
    // work-groups, else from the start of the dynamic LDS
    constexpr size_t wrows = CBN / C::WN;
    constexpr size_t epi = (size_t)C::WM * C::WN * 2 *
                           (MODE == WG_GATEUP ? (size_t)(BM / C::WM) * (wrows / 2 + 8) : (C::PER ? 16 : 32) * (wrows + 8));
    static_assert(!C::PER || epi <= stage, "the epilogue fits ring slot 2");
    constexpr size_t lds_max = std::max(ring + (MX ? (size_t)CBN * MX_MAX_K / 32 : 0), C::PER ? 0 : epi);
    static_assert(lds_max <= 160 * 1024 - 2048, "LDS ring too large");
    static bool attr_done = false;
    auto kern = grouped_gemm_wide_kernel<MODE, BM, C::WM, C::WN, C::OCC, MX, C::KH, C::NS, C::PER>;
    if (!attr_done) {
        hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
        if (r != hipSuccess) return r;
        attr_done = true;
    }
    const size_t lds = std::max(ring + (MX ? (size_t)CBN * prm.K / 32 : 0), C::PER ? (size_t)0 : epi);
    constexpr int GM = group_m(MODE, MX);
    int nblk = (prm.mt_max + GM - 1) / GM * GM * prm.nt;
    nblk = (nblk + NXCD - 1) / NXCD * NXCD;
    if (C::PER) {
        // one work-group per CU (the ring takes most of a CU's LDS), a multiple of the XCD count
        int dev = 0, cus = 0;
        hipError_t r = hipGetDevice(&dev);
        if (r == hipSuccess) r = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (r != hipSuccess) return r;
        nblk = std::min(nblk, std::max(NXCD, cus / NXCD * NXCD));
    }
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(kern, dim3(nblk), dim3(C::NTH), lds, st, ev0, ev1, 0, prm);
    else
        hipLaunchKernelGGL(kern, dim3(nblk), dim3(C::NTH), lds, st, prm);
    return hipGetLastError();
}

int mt_max_wide(const moe_shape &s, int rows) {
    const long P = (long)s.num_tokens * s.top_k;
    return (int)(P / rows + std::min<long>(s.num_experts, P));
}

}  // namespace


// K must be a multiple of 64 and at least 128 (an even number of 32-deep steps, at least
// 4: two stages of 64); MXFP4 also wants K a multiple of 512 (whole 16-byte chunks of
// scales per row) and at most MX_MAX_K
static bool wide_k_ok(const moe_shape &s, int K) {
    if (K % (2 * BK) || K < 4 * BK) return false;
    return s.weight_dtype == MOE_BF16 || (K % 512 == 0 && K <= MX_MAX_K);
}
// MXFP4 gate/up stays on the register-staged kernel (grouped_gemm.hip): on the 4096-token
// chunk (H=4096, E=256, k=8, I=1024) it measured 1085-1092 us against 1196-1200 us here,
// while the MXFP4 down projection runs here (438-444 us against ~656 us)
bool wide_gateup_supported(const moe_shape &s) {
    return s.act_dtype == MOE_BF16 && s.weight_dtype == MOE_BF16 && s.intermediate % (CBN / 2) == 0 &&
           wide_k_ok(s, s.hidden);
}
bool wide_down_supported(const moe_shape &s) {
    return s.act_dtype == MOE_BF16 && (s.weight_dtype == MOE_BF16 || s.weight_dtype == MOE_MXFP4) &&
           s.hidden % CBN == 0 && wide_k_ok(s, s.intermediate);
}

// m-tile height of the grouped GEMMs of moe_forward on `s`: 64 rows while the pairs average
// at most 48 per expert for bf16 experts on the large-tile kernels, or at most 32 for MXFP4
// experts (register-staged gate/up, large-tile down); else 128.  The results are the same
// bits either way (an output's K order does not depend on the tile).  Measured, layer time
// with the grouped path forced:
//  - bf16 decode shape (H=2048, E=128, k=8, I=768): 3-6% faster at 2-32 pairs per expert
//    (T = 32..512), 4% slower at 64 (T = 1024);
//  - MXFP4 shape (H=4096, E=256, k=8, I=1024): 11-14% faster at 3-6 pairs per expert, 8% at
//    12, 3.5% at 24, 9% slower at 48 (T = 1536).
int grouped_tile_rows(const moe_shape &s) {
    const long P = (long)s.num_tokens * s.top_k, E = s.num_experts;
    if (s.weight_dtype == MOE_BF16 && wide_gateup_supported(s) && wide_down_supported(s))
        return P <= 48 * E ? kWideSmallTileM : kGroupedTileM;
    if (s.weight_dtype == MOE_MXFP4 && wide_down_supported(s)) return P <= 32 * E ? kWideSmallTileM : kGroupedTileM;
    return kGroupedTileM;
}

hipError_t launch_gateup_wide(const moe_shape &s, const void *x, const moe_expert_weights &w, const int32_t *sorted,
                              const int32_t *mtile_off, const int32_t *tiles, const float *wts, void *h,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    WideParams prm{};
    prm.a = static_cast<const uint8_t *>(x);
    prm.sorted = sorted;
    prm.mtile_off = mtile_off;
    prm.tiles = reinterpret_cast<const int4 *>(tiles);
    prm.b0 = static_cast<const uint8_t *>(w.w_gate);
    prm.b1 = static_cast<const uint8_t *>(w.w_up);
    prm.s0 = w.s_gate;
    prm.s1 = w.s_up;
    prm.wts = wts;
    prm.out = static_cast<uint8_t *>(h);
    prm.N = s.intermediate;
    prm.K = s.hidden;
    prm.topk = s.top_k;
    prm.E = s.num_experts;
    prm.nt = s.intermediate / (CBN / 2);
    if (s.weight_dtype == MOE_MXFP4) {
        prm.mt_max = mt_max_wide(s, kGroupedTileM);
        return wide_launch<WG_GATEUP, true, kGroupedTileM>(prm, st, ev0, ev1);
    }
    const int rows = grouped_tile_rows(s);
    prm.mt_max = mt_max_wide(s, rows);
    if (rows == kWideSmallTileM) return wide_launch<WG_GATEUP, false, kWideSmallTileM>(prm, st, ev0, ev1);
    return wide_launch<WG_GATEUP, false, kGroupedTileM>(prm, st, ev0, ev1);
}

hipError_t launch_down_wide(const moe_shape &s, const moe_expert_weights &w, const int32_t *sorted,
                            const int32_t *mtile_off, const int32_t *tiles, const void *h, void *o, hipStream_t st,
                            hipEvent_t ev0, hipEvent_t ev1) {
    WideParams prm{};
    prm.a = static_cast<const uint8_t *>(h);
    prm.sorted = sorted;
    prm.mtile_off = mtile_off;
    prm.tiles = reinterpret_cast<const int4 *>(tiles);
    prm.b0 = static_cast<const uint8_t *>(w.w_down);
    prm.s0 = w.s_down;
    prm.out = static_cast<uint8_t *>(o);
    prm.N = s.hidden;
    prm.K = s.intermediate;
    prm.topk = s.top_k;
    prm.E = s.num_experts;
    prm.nt = s.hidden / CBN;
    if (s.weight_dtype == MOE_MXFP4) {
        const int rows = grouped_tile_rows(s);
        prm.mt_max = mt_max_wide(s, rows);
        if (rows == kWideSmallTileM) return wide_launch<WG_DOWN, true, kWideSmallTileM>(prm, st, ev0, ev1);
        return wide_launch<WG_DOWN, true, kGroupedTileM>(prm, st, ev0, ev1);
    }
    const int rows = grouped_tile_rows(s);
    prm.mt_max = mt_max_wide(s, rows);
    if (rows == kWideSmallTileM) return wide_launch<WG_DOWN, false, kWideSmallTileM>(prm, st, ev0, ev1);
    return wide_launch<WG_DOWN, false, kGroupedTileM>(prm, st, ev0, ev1);
}

}  // namespace moe
