// prefill_bf16.hip -- fused GQA attention prefill, bf16 storage, fp32 state,
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) for both contractions, gfx950.
//
// Method (ADR-0060 page, "AHBM GQA Fused Attention kernel (Llama3-70B)"):
//  * GQA fold (TL;DR, section 5.2): the G query heads of KV head kv and the
//    T_q query tokens form M = T_q * G rows, ordered t-major (row r is token
//    r / G, query head kv * G + r % G), so one K/V tile serves all of them and
//    K/V are never broadcast.
//  * Per KV tile (section 3): S = scale * Q K^T, additive mask on boundary
//    tiles only, online softmax m_new = max(m, rowmax S), P = exp(S - m_new),
//    corr = exp(m - m_new), l = l * corr + rowsum P, O = O * corr + P V.
//    The kernel works in base 2: scores are multiplied by scale * log2(e)
//    and exp2 replaces exp; LSE is converted back to natural log at the end.
//  * Causal tile classes (section 5.4): a key tile wholly after the last
//    query of a block is skipped, a tile wholly at or before the first query
//    is computed without mask, anything else gets the element mask
//    key > q_offset + t  ->  -inf.
//
// MI355X mapping:
//  * Work-group = 8 waves x 32 query rows (256 rows), key tiles of 64; two
//    waves per SIMD.  blockIdx -> (kv head fastest, then batch, then row
//    block); causal row blocks are issued longest-first.  With 8 KV heads and
//    8 XCDs the round-robin dispatch keeps each KV head's K/V in one XCD's L2.
//  * The MFMA computes S^T = K Q^T: A = K tile rows from LDS, B = Q^T held in
//    registers for the whole sweep.  In the 32x32 output layout each lane
//    then owns one query column, so the running max / sum / rescale are
//    lane-local (only lanes l and l^32 share a query, joined with
//    v_permlane32_swap), and the fp32 P values of a lane, packed to bf16, are
//    exactly the B operand of O^T = V^T P^T.  K rows are loaded into the A
//    operand in a permuted order (bits 2 and 3 of the row index swapped) so
//    that the 8 keys a lane contributes to each P.V step are consecutive.
//  * K and V tiles go from HBM/L2 straight into LDS with buffer_load_dwordx4
//    ... lds (no staging registers) through a buffer resource per tile, so
//    the per-lane offset is a fixed register and rows past S_kv read as
//    zeros; a ring of four LDS stages holds the tiles being read (i - 1 for
//    P.V, i for QK) and loading (i + 1, i + 2).  Rows are not padded;
//    instead the 16-byte chunks of each row are XOR-swizzled (chunk c of row
//    r sits at c ^ f(r)), which makes the b128 K reads and the
//    ds_read_b64_tr_b16 V^T reads (each lane of a 16-lane group receives one
//    head-dim column of four key rows) bank-conflict free.
//  * Ping-pong: waves w and w + 4 share a SIMD.  Waves 0-3 and 4-7 run the
//    same per-tile work half a tile apart, separated by a barrier in the
//    middle of every tile, so on each SIMD one wave is in its MFMA phase
//    (P.V of the previous tile, then QK of this tile) while the other is in
//    its softmax phase (VALU).  The MFMA phase runs at raised wave priority,
//    and its LDS operands are read one group of MFMAs ahead.  The VALU work
//    per tile is kept small: row max as max3 chains, tile loads without
//    per-lane address arithmetic.
//  * Lazy rescaling: the running max used for the exponentials is only moved
//    when some row's tile max exceeds it by more than 8 (log2 units), so most
//    tiles skip the O rescale; exact, since O and l always share the same
//    reference max and P stays below 2^8.  The tile's row max itself is only
//    taken when needed: P is first computed against the current reference,
//    and only if some lane's sum of P over the tile exceeds 2^8 (which any
//    P above 2^8 implies) does the wave compute the row max, rescale if it
//    grew by more than 8 and recompute P.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;   // 256 query rows per work-group
constexpr int kBlockN = 64;                      // keys per tile
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 4;                       // LDS ring depth (tiles resident)
constexpr float kRescaleThreshold = 8.f;         // log2 units
constexpr int kCachePolicyNT = 2;                // buffer-load cache policy: non-temporal

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

template <int D>
struct Tile {
    static constexpr int ELEMS = kBlockN * D;            // one K or V tile, unpadded
    static constexpr int CPR = D / 8;                    // 16-byte chunks per row
    static constexpr int ROWS_PER_LOAD = 64 / CPR;       // rows per wave load instruction
    static constexpr int LOADS = kBlockN / ROWS_PER_LOAD / kWaves;   // per wave per tensor
};

// Physical 16-byte chunk of logical chunk c in row r is c ^ swz(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Row of the A operand that lane-row m loads: bits 2 and 3 swapped.
__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Issue this wave's direct-to-LDS loads of one K or V tile `tile` into the
// stage buffer dst: 64 LDS rows, which are the keys tile*64 .. of one KV head
// (HP = 1) or the keys tile*32 .. of two neighbouring KV heads, head-major
// (HP = 2).  The buffer resource spans only the tile's keys below S_kv: rows
// past it read as zeros, their scores are masked to -inf and their P is
// exactly 0.
template <int D, int HP>
__device__ __forceinline__ void issue_half(uint16_t* dst, const uint16_t* __restrict__ base,
                                           int64_t row_stride, int tile, int S_kv, int wave,
                                           int lane) {
    using T = Tile<D>;
    constexpr int TK = kBlockN / HP;   // keys per tile
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
        const int row0 = (wave * T::LOADS + i) * T::ROWS_PER_LOAD;
        const int r = row0 + lane / T::CPR;
        const int cc = (lane % T::CPR) ^ swz<D>(r);
        const int rows = min(TK, S_kv - tile * TK);
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(base + (int64_t)tile * TK * row_stride), (short)0,
            rows * (int)row_stride * 2, 0x00020000);
        // (r < 64: LDS row r is key r of the head, or key r % 32 of head r / 32)
        const int key = HP == 2 ? r & 31 : r;
        const int head = HP == 2 ? r >> 5 : 0;
        const int lo = (key * (int)row_stride + head * D + cc * 8) * 2;   // bytes
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + row0 * D), 16, lo, 0, 0, 0);
    }
}
template <int D, int HP>
__device__ __forceinline__ void issue_tile(uint16_t* kst, uint16_t* vst,
                                           const uint16_t* __restrict__ kbase,
                                           const uint16_t* __restrict__ vbase,
                                           int64_t row_stride, int tile, int S_kv, int wave,
                                           int lane) {
    issue_half<D, HP>(kst, kbase, row_stride, tile, S_kv, wave, lane);
    issue_half<D, HP>(vst, vbase, row_stride, tile, S_kv, wave, lane);
}

// Work-group barrier for LDS traffic only: this wave's LDS operations have
// completed, then all waves meet.  Unlike __syncthreads() it does not wait for
// outstanding global->LDS loads of later tiles (those are waited for
// explicitly with wait_vmcnt); the memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Barrier of the tile loop: all waves meet, without waiting for this wave's
// LDS reads first.  Every LDS read of a K/V stage in the loop feeds an MFMA
// of the same phase, except the first V^T step read at the end of a softmax
// phase for the next phase's P.V, and that stage is not refilled before two
// more iterations; so no read is pending on a stage a DMA load issued after
// the barrier writes (the Q rows staged before the loop are read before the
// full lds_barrier that precedes it).
__device__ __forceinline__ void loop_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N == 0 || N == 2 || N == 4 || N == 8, "vmcnt values used here");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

template <int D>
struct LaneOffsets {
    int k[D / 16];            // K operand read offset (elements) per k-step, key block 0
    int v[2][D / 32];         // V^T tr16 read offset per (half t, 32-dim block), key step 0
};

// SPLIT: the key tiles a row block sees are cut into n_split contiguous
// ranges, one work-group each, and every work-group writes the unnormalised
// partial (m in base-2 units, l, O) of its rows to the workspace instead of
// O and LSE (partial row ((b * n_split + split) * T_q + t) * H_q + h); the
// decode combine kernel merges them.
//
// MASK: kMaskNone (every key), kMaskCausal (key j visible to position p iff
// j <= p), kMaskWindow (causal, and j < sink or j > p - window: attention
// sinks plus a local window).  With the window, a row block's key tiles are
// the sink tiles followed by the window tiles; the tiles in between are
// never loaded.
constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2;

// PLAN: multi-token decode over a packed varlen cache.  The work-group's key
// range is one split of a decode plan (sequence sq, keys [kb, kb + L) of
// plan.len[sq]); the kernel sees that range as its own sequence of S keys
// with token 0 at position kv_len - T_q - kb (the causal rule of decode with
// T_q new tokens, shifted to the range), and writes partials as SPLIT does,
// at the plan's split index.  Blocks: KV head fastest, then row block, then
// plan unit.
//
// HP = 2 (plan ranges of at most 128 query rows per KV head): a work-group
// serves two neighbouring KV heads, waves 0-3 the rows of the first and
// waves 4-7 those of the second, so both wave groups have rows to compute;
// a tile is then 32 keys of both heads (the same 64 LDS rows), and each
// group reads its own head's half.
struct NoPlan {};
template <bool PLAN>
using PlanArg = typename std::conditional<PLAN, DecodePlanChunk, NoPlan>::type;

template <int D, int MASK, bool SPLIT, bool PLAN = false, int HP = 1>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int B,
    int T_q, int S_kv, int H_q, int H_kv, int G, float c, int q_offset, int n_mblk,
    int n_split, float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    int window, int sink, const PlanArg<PLAN> plan) {
    static_assert(!PLAN || (MASK == kMaskCausal && !SPLIT), "plan ranges are causal partials");
    static_assert(HP == 1 || (PLAN && HP == 2), "two KV heads per work-group: plan ranges only");
    constexpr int KB = 2 / HP;           // 32-key blocks of a tile per head
    constexpr int TK = 32 * KB;          // keys per tile
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool PARTIAL = SPLIT || PLAN;   // writes (m, l, O) partials
    constexpr bool WINDOW = MASK == kMaskWindow;
    using T = Tile<D>;
    constexpr int KSTEPS = D / 16;   // MFMA k-steps over the head dim
    constexpr int DBLK = D / 32;     // 32-row blocks of O^T
    constexpr int LOADS_PER_TILE = 2 * T::LOADS;   // vmem ops per wave per tile
    static_assert(LOADS_PER_TILE == 2 || LOADS_PER_TILE == 4, "wait_vmcnt covers 2 and 4");
    static_assert(kStages == 4, "the tile loop below is unrolled over four stages");
    __shared__ __attribute__((aligned(1024))) uint16_t ksm[kStages * T::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t vsm[kStages * T::ELEMS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int hh = lane >> 5;

    int bid = blockIdx.x;
    const int kvg = bid % (H_kv / HP);               // KV head (group) of the work-group
    bid /= H_kv / HP;
    const int kv = kvg * HP + (HP == 2 ? wave >> 2 : 0);   // this wave's KV head
    int split = 0, b, mb;
    int64_t prow;   // partial (split) index of the work-group's rows
    // K/V row 0 of the keys this work-group walks (their count is S_kv, and
    // q_offset the position of query token 0 relative to that row)
    int64_t key_row0;
    if constexpr (PLAN) {
        mb = bid % n_mblk;
        const int unit = bid / n_mblk;
        int sq = 0;
        while (sq + 1 < plan.nseq && plan.unit_base[sq + 1] <= unit) ++sq;
        const int L = plan.split_len[sq];
        const int len = plan.len[sq];
        const int kb = (unit - plan.unit_base[sq]) * L;
        b = plan.seq0 + sq;
        S_kv = min(L, len - kb);
        q_offset = len - T_q - kb;
        key_row0 = plan.key_off[sq] + kb;
        prow = (int64_t)plan.split_base + unit;
    } else {
        if (SPLIT) {
            split = bid % n_split;
            bid /= n_split;
        }
        b = bid % B;
        mb = bid / B;
        // causal row blocks run longest-first; window blocks (all about as
        // long) in ascending order, so a block's lowest window tiles, which
        // it processes first, were loaded into the XCD's L2 by the blocks
        // before it, and its new keys come last, behind the tile read-ahead
        if (CAUSAL && !WINDOW) mb = n_mblk - 1 - mb;
        key_row0 = (int64_t)b * S_kv;
        prow = (int64_t)b * n_split + split;
    }

    const int rows_total = T_q * G;
    const int r0 = mb * kBlockM;
    // first row of this wave
    const int rw0 = r0 + (HP == 2 ? wave & 3 : wave) * kRowsPerWave;
    const int row = rw0 + lq;
    const bool valid = row < rows_total;
    // rows past the end read the last row's Q (loads are never predicated);
    // their outputs are not written
    const int row_c = valid ? row : rows_total - 1;
    const int t = row_c / G;
    const int g = row_c % G;
    const int64_t qo_off = (((int64_t)b * T_q + t) * H_q + (int64_t)kv * G + g) * D;

    // Key range of the work-group and of this wave.
    // (wave- and block-uniform values are pinned to scalar registers so the
    // branches on them are scalar branches)
    const int t_hi = min(T_q - 1, (r0 + kBlockM / HP - 1) / G);
    // (a plan range can start after every key the block's tokens see)
    const int kend = CAUSAL ? max(0, min(S_kv, q_offset + t_hi + 1)) : S_kv;
    int wg_tiles = (kend + TK - 1) / TK;
    // window: tiles [0, sink_tiles) then [sink_tiles + gap, ...); the work-group
    // counts tiles in that compacted order (tile index = j + (j >= sink_tiles) * gap)
    int sink_tiles = 0, gap = 0;
    if (WINDOW) {
        const int t_lo = min(T_q - 1, r0 / G);
        const int p_lo = q_offset + t_lo;
        sink_tiles = (min(sink, kend) + TK - 1) / TK;
        const int w_tile0 = max(0, p_lo - window + 1) / TK;
        gap = max(0, w_tile0 - sink_tiles);
        wg_tiles -= gap;
        sink_tiles = __builtin_amdgcn_readfirstlane(sink_tiles);
        gap = __builtin_amdgcn_readfirstlane(gap);
    }
    // this work-group's tiles: [j_lo, j_lo + n_tiles)
    int j_lo = 0, n_tiles = wg_tiles;
    if (SPLIT) {
        const int per = (wg_tiles + n_split - 1) / n_split;
        j_lo = min(wg_tiles, split * per);
        n_tiles = min(wg_tiles - j_lo, per);
    }
    j_lo = __builtin_amdgcn_readfirstlane(j_lo);
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
    const bool wave_live = rw0 < rows_total;
    const int wt_lo = rw0 / G;
    const int wt_hi = min(T_q - 1, (rw0 + kRowsPerWave - 1) / G);
    const int wave_kend = __builtin_amdgcn_readfirstlane(
        wave_live ? (CAUSAL ? min(S_kv, q_offset + wt_hi + 1) : S_kv) : 0);
    // keys [0, wave_full) are visible to every row of this wave
    const int wave_full = __builtin_amdgcn_readfirstlane(
        CAUSAL ? min(S_kv, q_offset + wt_lo + 1) : S_kv);
    // last key this row may see (rows past the end see everything: their output is dropped)
    const int last_key = CAUSAL ? (valid ? min(q_offset + t, S_kv - 1) : S_kv - 1) : S_kv - 1;
    // window: keys in [sink, win_lo) are hidden from this row; the wave's rows
    // all see [0, sink) and [wave_win_all, wave_full); a tile is needed by some
    // row of the wave if it reaches wave_win_any
    const int win_lo = (WINDOW && valid) ? q_offset + t - window + 1 : -1;
    const int wave_win_any = __builtin_amdgcn_readfirstlane(WINDOW ? q_offset + wt_lo - window + 1 : 0);
    const int wave_win_all = __builtin_amdgcn_readfirstlane(WINDOW ? q_offset + wt_hi - window + 1 : 0);

    const int64_t row_stride = (int64_t)H_kv * D;
    const uint16_t* kbase = k + (key_row0 * H_kv + kvg * HP) * D;
    const uint16_t* vbase = v + (key_row0 * H_kv + kvg * HP) * D;

    // global tile of the work-group's compacted tile index j
    auto tile_of = [&](int j) { return WINDOW ? j + (j >= sink_tiles ? gap : 0) : j; };
    // loads of the work-group's tile j into LDS stage st; the first two tiles
    // start loading before anything else
    auto issue = [&](int j, int st) __attribute__((always_inline)) {
        issue_tile<D, HP>(ksm + st * T::ELEMS, vsm + st * T::ELEMS, kbase, vbase, row_stride,
                      tile_of(j_lo + j), S_kv, wave, lane);
    };
    // Q and O pass through LDS, each wave through its own 32-row area in the
    // stages tiles 2 and 3 use later (waves 0-3 in the K stages, 4-7 in the
    // V stages), so that global accesses move whole rows (a wave instruction
    // covers 64 / (D / 8) rows) instead of 8 bytes of 32 rows; the 16-byte
    // chunks of a row are XOR-swizzled as in the K/V tiles.
    uint16_t* qo_lds = (wave < 4 ? ksm : vsm) + 2 * T::ELEMS + (wave & 3) * kRowsPerWave * D;
    constexpr int QROWS = 64 / T::CPR;                   // rows per wave instruction
    // global element offset of row r of the work-group (clamped into range)
    auto row_off = [&](int r) {
        const int rc = min(r, rows_total - 1);
        return (((int64_t)b * T_q + rc / G) * H_q + (int64_t)kv * G + rc % G) * D;
    };
    {
        // rows of the first token of this work-group onwards, < 2^31 bytes away
        const int t0 = r0 / G;
        const uint16_t* qbase = q + (((int64_t)b * T_q + t0) * H_q + (int64_t)kv * G) * D;
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, (short)0,
                                                                      0x7ffffff0, 0x00020000);
#pragma unroll
        for (int i = 0; i < kRowsPerWave / QROWS; ++i) {
            const int lr = i * QROWS + lane / T::CPR;
            const int cc = (lane % T::CPR) ^ swz<D>(lr);
            const int rc = min(rw0 + lr, rows_total - 1);
            const int off = (int)((((int64_t)(rc / G - t0) * H_q + rc % G) * D + cc * 8) * 2);
            // (non-temporal: each Q row is read once, the L2 is kept for K/V)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(qo_lds + i * QROWS * D), 16,
                                                     off, 0, 0, kCachePolicyNT);
        }
    }
    if (n_tiles > 0) issue(0, 0);
    if (n_tiles > 1) issue(1, 1);

    // Q^T operand, resident for the whole key sweep (this wave's Q rows have
    // landed once at most the tile loads behind them are outstanding).
    if (n_tiles > 1) wait_vmcnt<2 * LOADS_PER_TILE>();
    else if (n_tiles > 0) wait_vmcnt<LOADS_PER_TILE>();
    else wait_vmcnt<0>();
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
        qf[ks] = *(const bf16x8*)(qo_lds + lq * D + (((2 * ks + hh) ^ swz<D>(lq)) << 3));

    // Per-lane LDS read offsets (elements), fixed for the whole sweep (with
    // two heads, this wave's head's 32 rows of every tile).
    LaneOffsets<D> off;
    {
        const int hofs = (HP == 2 ? wave >> 2 : 0) * 32 * D;
        const int kr = swap_bits23(lq);               // + 32 rows for the second key block
        const int kf = swz<D>(kr);
#pragma unroll
        for (int kst = 0; kst < KSTEPS; ++kst)
            off.k[kst] = hofs + kr * D + (((2 * kst + hh) ^ kf) << 3);
        const int L16 = lane & 15;
        const int dh = (lane >> 4) & 1;
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int vr = 8 * hh + 4 * th + (L16 >> 2);   // + 16 rows per key step
            const int vf = swz<D>(vr);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const int col = 32 * db + 16 * dh + 4 * (L16 & 3);
                off.v[th][db] = hofs + vr * D + (((col >> 3) ^ vf) << 3) + (col & 7);
            }
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // reference max (raw score units) used by P
    float l_run = 0.f;

    auto needs = [&](int j) __attribute__((always_inline)) {
        const int key0 = tile_of(j_lo + j) * TK;
        bool w = key0 < wave_kend;
        if (WINDOW) w = w && (key0 < sink || key0 + TK > wave_win_any);
        return w;
    };
    f32x16 s[KB];
    uint32_t pk[KB][8];
    // S^T = K Q^T of tile j (stage st); K operands read one group ahead
    auto qk = [&](int j, const uint16_t* kt) __attribute__((always_inline)) {
        if (!needs(j)) return;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
        // MFMA n: key block n % KB, head-dim step n / KB
        constexpr int NQ = KB * KSTEPS, QG = 4, NG = NQ / QG;
        auto kread = [&](int n) { return *(const bf16x8*)(kt + (n % KB) * 32 * D + off.k[n / KB]); };
        bf16x8 ka[2][QG];
#pragma unroll
        for (int i = 0; i < QG; ++i) ka[0][i] = kread(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) {
#pragma unroll
                for (int i = 0; i < QG; ++i) ka[(g + 1) & 1][i] = kread((g + 1) * QG + i);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < QG; ++i) {
                const int n = g * QG + i;
                s[n % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[g & 1][i], qf[n / KB],
                                                                   s[n % KB], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // mask, running max, lazy rescale, P (packed bf16) and its row sum
    auto softmax = [&](int j) __attribute__((always_inline)) {
        if (!needs(j)) return;
        const int key0 = tile_of(j_lo + j) * TK;
        // element i of s[kb] is key key0 + 32 kb + 16 (i / 8) + 8 hh + (i % 8)
        bool need_mask = key0 + TK > wave_full;
        if (WINDOW) need_mask = need_mask || (key0 + TK > sink && key0 < wave_win_all);
        if (need_mask) {
            if constexpr (WINDOW) {
                // element i of s[kb] is key key0 + 8 hh + cc, cc = 32 kb + 16
                // (i / 8) + i % 8: hidden past the row's last key or inside
                // [sink, win_lo) (one unsigned range compare), written
                // branch-free so that the compiler emits compares and selects
                // (the short-circuit form became a branch per element)
                const int lim = last_key - key0 - 8 * hh;
                const int wbase = key0 + 8 * hh - sink;
                const unsigned wlen = (unsigned)max(win_lo - sink, 0);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int cc = kb * 32 + (i >> 3) * 16 + (i & 7);
                        const bool hide = (cc > lim) | ((unsigned)(wbase + cc) < wlen);
                        s[kb][i] = hide ? -INFINITY : s[kb][i];
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + kb * 32 + (i >> 3) * 16 + hh * 8 + (i & 7);
                        if (key > last_key) s[kb][i] = -INFINITY;
                    }
            }
        }
        // exponentials against the current reference max first; a lane whose
        // P sum exceeds 2^8 (infinite while a row with visible keys has no
        // reference max yet) sends the wave through the row max and the
        // rescale, then P is recomputed
        auto expsum = [&](float mcv) __attribute__((always_inline)) {
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = fast_exp2(__builtin_fmaf(s[kb][i], c, -mcv));
                    const float p1 = fast_exp2(__builtin_fmaf(s[kb][i + 1], c, -mcv));
                    pk[kb][i >> 1] = pack_bf16x2(p0, p1);
                    ps += p0 + p1;
                }
            return ps;
        };
        // (the first tile has no reference max in any row: take the row max
        // directly; O and l are still zero, so there is nothing to rescale)
        // (window blocks are short: their first tile takes the row max
        // directly, with nothing to rescale since O and l are still zero)
        const bool first = WINDOW && j == 0;
        float psum = first ? 0.f : expsum(fmaxf(m_run * c, -1e30f));
        if (first || __builtin_amdgcn_ballot_w64(psum > 256.f) != 0) {
            float mt;
            if constexpr (KB == 2) {
                float mt0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
                float mt1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
                for (int i = 3; i < 15; i += 2) {
                    mt0 = fmaxf(fmaxf(mt0, s[0][i]), s[0][i + 1]);
                    mt1 = fmaxf(fmaxf(mt1, s[1][i]), s[1][i + 1]);
                }
                mt = fmaxf(fmaxf(mt0, s[0][15]), fmaxf(mt1, s[1][15]));
            } else {
                mt = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
                for (int i = 3; i < 15; i += 2) mt = fmaxf(fmaxf(mt, s[0][i]), s[0][i + 1]);
                mt = fmaxf(mt, s[0][15]);
            }
            {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                           false, false);
                mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            if (first) {
                m_run = mt;
            } else if (__builtin_amdgcn_ballot_w64(mt * c > m_run * c + kRescaleThreshold) != 0) {
                const float m_new = fmaxf(m_run, mt);
                // 0 for a row's first visible keys; a row with no visible key
                // so far keeps corr = 1
                const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * c);
                l_run *= corr;
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
                m_run = m_new;
            }
            // a window or a split can start past the keys a row sees: its m stays
            // -inf and P = 0
            const float mc = ((PARTIAL || WINDOW) && m_run == -INFINITY) ? 0.f : m_run * c;
            psum = expsum(mc);
        }
        l_run += psum;
    };
    // O^T += V^T P^T of tile j; V^T operands read one 16-key step ahead, the
    // first two steps' at the end of the preceding softmax phase (vpre): an
    // LDS read issued between the MFMAs of the MFMA phase delays the next
    // MFMA issue (the phase runs at ~42 cycles per 32-cycle MFMA with its
    // operand reads, ~33 with operands from registers), while the softmax
    // phase beside it on the SIMD has room for them.
    auto vread = [&](const uint16_t* vt, int kst, int db) __attribute__((always_inline)) {
        const s16x4 lo = lds_read_tr16(vt + kst * 16 * D + off.v[0][db]);
        const s16x4 hi = lds_read_tr16(vt + kst * 16 * D + off.v[1][db]);
        return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    constexpr int NPRE = 2;   // 16-key steps of V^T read ahead (32 VGPRs)
    s16x8 vpre[NPRE][DBLK];
    auto pv_pre = [&](int j, const uint16_t* vt) __attribute__((always_inline)) {
        if (!needs(j)) return;
#pragma unroll
        for (int ps = 0; ps < NPRE; ++ps)
#pragma unroll
            for (int db = 0; db < DBLK; ++db) vpre[ps][db] = vread(vt, ps, db);
    };
    auto pv = [&](int j, const uint16_t* vt) __attribute__((always_inline)) {
        if (!needs(j)) return;
        s16x8 va[2][DBLK];
#pragma unroll
        for (int db = 0; db < DBLK; ++db) va[0][db] = vpre[0][db];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kst = 0; kst < 2 * KB; ++kst) {   // 16-key steps
            if (kst + 1 < 2 * KB) {
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
                    va[(kst + 1) & 1][db] = kst + 1 < NPRE ? vpre[kst + 1 < NPRE ? kst + 1 : 0][db]
                                                           : vread(vt, kst + 1, db);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int kb = kst >> 1, half = kst & 1;
            const u32x4 pw = {pk[kb][half * 4 + 0], pk[kb][half * 4 + 1], pk[kb][half * 4 + 2],
                              pk[kb][half * 4 + 3]};
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va[kst & 1][db]), __builtin_bit_cast(bf16x8, pw),
                    oacc[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // tile i + 1 must be in LDS for every wave; tile i + 2 may stay in flight
    auto end_iter = [&](int i) __attribute__((always_inline)) {
        if (i + 2 < n_tiles) wait_vmcnt<LOADS_PER_TILE>();
        else wait_vmcnt<0>();
        loop_barrier();
    };
    // Iteration i (tile i in stage i & 3), i = 0 .. n_tiles: waves 0-3 run
    // [PV(i - 1), QK(i)] then [softmax(i)]; waves 4-7 run [softmax(i - 1)]
    // then [PV(i - 1), QK(i)]; both meet the mid-iteration barrier and the
    // end barrier.  Each wave issues its part of tile i + 2 at the start of
    // its softmax phase (the two groups' loads do not queue together), into
    // the stage of tile i - 2, free everywhere since the end of iteration
    // i - 1.
    auto iter0 = [&](int i, int st) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        if (i >= 1) pv(i - 1, vsm + ((st + 3) & 3) * T::ELEMS);
        if (i < n_tiles) qk(i, ksm + st * T::ELEMS);
        __builtin_amdgcn_s_setprio(0);
        loop_barrier();
        if (i + 2 < n_tiles) issue(i + 2, (st + 2) & 3);
        if (i < n_tiles) {
            softmax(i);
            pv_pre(i, vsm + st * T::ELEMS);
        }
        end_iter(i);
    };
    auto iter1 = [&](int i, int st) __attribute__((always_inline)) {
        if (i + 2 < n_tiles) issue(i + 2, (st + 2) & 3);
        if (i >= 1) {
            softmax(i - 1);
            pv_pre(i - 1, vsm + ((st + 3) & 3) * T::ELEMS);
        }
        loop_barrier();
        __builtin_amdgcn_s_setprio(1);
        if (i >= 1) pv(i - 1, vsm + ((st + 3) & 3) * T::ELEMS);
        if (i < n_tiles) qk(i, ksm + st * T::ELEMS);
        __builtin_amdgcn_s_setprio(0);
        end_iter(i);
    };

    if (n_tiles > 1) wait_vmcnt<LOADS_PER_TILE>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (n_tiles > 0) {
        if (wave < 4) {
            for (int i = 0; i <= n_tiles; i += 4) {
                iter0(i, 0);
                if (i + 1 <= n_tiles) iter0(i + 1, 1);
                if (i + 2 <= n_tiles) iter0(i + 2, 2);
                if (i + 3 <= n_tiles) iter0(i + 3, 3);
            }
        } else {
            for (int i = 0; i <= n_tiles; i += 4) {
                iter1(i, 0);
                if (i + 1 <= n_tiles) iter1(i + 1, 1);
                if (i + 2 <= n_tiles) iter1(i + 2, 2);
                if (i + 3 <= n_tiles) iter1(i + 3, 3);
            }
        }
    }

    // ---- epilogue: O / l, LSE ----
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                   false, false);
        l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (PARTIAL) {
        if (valid) {
            const int64_t hrow = (prow * T_q + t) * H_q + (int64_t)kv * G + g;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    *(f32x4*)(ws_o + hrow * D + db * 32 + u * 8 + hh * 4) =
                        f32x4{oacc[db][4 * u], oacc[db][4 * u + 1], oacc[db][4 * u + 2],
                              oacc[db][4 * u + 3]};
            if (hh == 0) {
                ws_m[hrow] = m_run * c;      // base-2 units (-inf: no visible key here)
                ws_l[hrow] = l_run;
            }
        }
        return;
    }
    // (every wave is past the last barrier: no LDS reads or loads remain)
    const float inv = 1.f / l_run;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            u32x2 w = {pack_bf16x2(oacc[db][4 * u] * inv, oacc[db][4 * u + 1] * inv),
                       pack_bf16x2(oacc[db][4 * u + 2] * inv, oacc[db][4 * u + 3] * inv)};
            *(u32x2*)(qo_lds + lq * D + (((db * 4 + u) ^ swz<D>(lq)) << 3) + hh * 4) = w;
        }
    if (valid && lse != nullptr && hh == 0)
        lse[qo_off / D] = (m_run * c + fast_log2(l_run)) * kLn2;
#pragma unroll
    for (int i = 0; i < kRowsPerWave / QROWS; ++i) {
        const int lr = i * QROWS + lane / T::CPR;
        const int cp = lane % T::CPR;
        const u32x4 val = *(const u32x4*)(qo_lds + lr * D + cp * 8);
        if (rw0 + lr < rows_total)   // (non-temporal, as the Q rows)
            __builtin_nontemporal_store(val, (u32x4*)(o + row_off(rw0 + lr) + ((cp ^ swz<D>(lr)) << 3)));
    }
}

}  // namespace

template <int D, int MASK, bool SPLIT>
static hipError_t launch_one(const PrefillArgs& a, int n_split, const DecodeWorkspace* ws,
                             hipStream_t stream) {
    const int64_t n_mblk = prefill_row_blocks(a.T_q, a.H_q / a.H_kv);
    const int64_t grid = n_mblk * a.B * a.H_kv * (SPLIT ? n_split : 1);
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, MASK, SPLIT>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.T_q, a.S_kv, a.H_q,
                       a.H_kv, a.H_q / a.H_kv, c, a.q_offset, (int)n_mblk, n_split,
                       SPLIT ? ws->m : nullptr, SPLIT ? ws->l : nullptr, SPLIT ? ws->o : nullptr,
                       a.window, a.sink, NoPlan{});
    return hipGetLastError();
}

int64_t prefill_row_blocks(int T_q, int G) { return ((int64_t)T_q * G + kBlockM - 1) / kBlockM; }

int decode_rows_heads_per_workgroup(int T_q, int G, int H_kv) {
    return ((int64_t)T_q * G <= kBlockM / 2 && H_kv % 2 == 0) ? 2 : 1;
}

template <bool SPLIT>
static hipError_t dispatch(const PrefillArgs& a, int n_split, const DecodeWorkspace* ws,
                           hipStream_t stream) {
    if (a.window > 0)
        return a.d == 128 ? launch_one<128, kMaskWindow, SPLIT>(a, n_split, ws, stream)
                          : launch_one<64, kMaskWindow, SPLIT>(a, n_split, ws, stream);
    if (a.d == 128)
        return a.causal ? launch_one<128, kMaskCausal, SPLIT>(a, n_split, ws, stream)
                        : launch_one<128, kMaskNone, SPLIT>(a, n_split, ws, stream);
    return a.causal ? launch_one<64, kMaskCausal, SPLIT>(a, n_split, ws, stream)
                    : launch_one<64, kMaskNone, SPLIT>(a, n_split, ws, stream);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    return dispatch<false>(a, 1, nullptr, stream);
}

hipError_t launch_prefill_split_bf16(const PrefillArgs& a, int n_split, const DecodeWorkspace& ws,
                                     hipStream_t stream) {
    return dispatch<true>(a, n_split, &ws, stream);
}

hipError_t launch_decode_rows_bf16(const void* q, const void* k, const void* v,
                                   const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                   int T_q, int H_q, int H_kv, int d, float scale,
                                   hipStream_t stream) {
    const int G = H_q / H_kv;
    const int hp = decode_rows_heads_per_workgroup(T_q, G, H_kv);
    const int64_t n_mblk = prefill_row_blocks(T_q, G);
    const int64_t grid = (int64_t)plan.units * n_mblk * (H_kv / hp);
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const float c = scale * kLog2e;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, nullptr,
                           nullptr, 1, T_q, 0, H_q, H_kv, G, c, 0, (int)n_mblk, 1, ws.m, ws.l,
                           ws.o, 0, 0, plan);
    };
    if (d == 128) {
        if (hp == 2) go(prefill_bf16_kernel<128, kMaskCausal, false, true, 2>);
        else go(prefill_bf16_kernel<128, kMaskCausal, false, true, 1>);
    } else {
        if (hp == 2) go(prefill_bf16_kernel<64, kMaskCausal, false, true, 2>);
        else go(prefill_bf16_kernel<64, kMaskCausal, false, true, 1>);
    }
    return hipGetLastError();
}

}  // namespace gqa
