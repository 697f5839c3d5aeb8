// decode.hip -- split-KV GQA decode (FlashDecoding) for gfx950: a split
// kernel writing unnormalised partials and a log-sum-exp combine kernel.
//
// Method (ADR-0060 page, "AHBM GQA Fused Attention kernel (Llama3-70B)"):
//  * Decode has one (or, for multi-token decode, T_q <= 16-ish) query token
//    per sequence; the G query heads of a KV head (times the T_q tokens) are
//    folded into the matmul M dimension so each K/V tile is read once for all
//    of them (section 5.2, "G * T_q" rows).  With one token there is no causal
//    mask, only a bounds mask on the ragged last tile of a split; with T_q new
//    tokens, token t at position len - T_q + t sees keys up to itself.
//  * The keys of a sequence are sharded; every shard produces the
//    unnormalised triplet (m_i, l_i, O_i) of the online softmax (sections 3
//    and 5.3), and the shards are reduced once, at the owner, with the
//    associative merge of section 4: m = max(m_a, m_b), s_a = exp(m_a - m),
//    s_b = exp(m_b - m), l = l_a s_a + l_b s_b, O = O_a s_a + O_b s_b, then
//    O / l.  Partials here are kept in base 2 (scores times log2(e)).
//
// MI355X mapping:
//  * Split kernel: one work-group of 4 waves per (split, KV head, group of 16
//    query heads).  The waves take interleaved 32-key tiles of the split;
//    each wave streams its K rows straight from HBM into MFMA A operands
//    (v_mfma_f32_16x16x32_bf16, S^T = K Q^T with the G heads as the 16 MFMA
//    columns), so each lane owns one query head and the softmax state is
//    lane-local.  V rows are loaded with 16-byte coalesced loads into a
//    per-wave row-major LDS tile and read back with ds_read_b64_tr_b16 as
//    the V^T A operand of O^T = V^T P^T.  The next tile's loads are issued before the current
//    tile's math.  At the end the four wave partials are merged through LDS
//    and one partial per (split, query head) is written.
//  * Combine kernel: one wave per (sequence, query head, 32 dims of O); the
//    partials of all splits are read in parallel and reduced in a fixed order
//    (no atomics: bitwise reproducible).
#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 32;       // keys per wave tile
constexpr int kCols = 16;       // query heads per MFMA column block

template <int D>
struct DecodeSmem {
    static constexpr int VS = D + 16;                 // V row stride (elements): tr16 reads 2-way
    static constexpr int VT_ELEMS = kTile * VS;       // per wave
};

// Key (within a 32-key tile) that A-operand row m of 16-key block blk loads.
// With it, P slot j (= 4 blk + i) of lane group g4 = m / 4 holds key g4 + 4 j,
// so each transposed V read of a 16-lane group touches 4 rows spaced by 4.
__device__ __forceinline__ int tile_key(int m, int blk) { return (m >> 2) + 16 * blk + 4 * (m & 3); }

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
}

// Storage formats of the K/V cache.  Quantised caches hold signed integer
// codes with one fp32 scale per (KV head, channel): K = code_k * k_scale,
// V = code_v * v_scale.  int4 packs two codes per byte, the even channel in
// the low nibble.
constexpr int kKvBf16 = 0, kKvInt8 = 1, kKvInt4 = 2;

// Loads are never predicated (a predicated load forces the compiler to wait
// for it on the spot): keys past the split end are clamped to its last key.
// Their scores are masked to -inf, so their P is exactly 0 and the clamped
// (finite) K/V values do not contribute.
// Cache row of walk index kk: the identity for a packed cache; for a ring
// cache, the sinks [0, s_end) and then the window positions, whose slots
// start at ring offset r0 and wrap at the ring length.
struct RowMap {
    int s_end, sink, r0, wrap;
    __device__ __forceinline__ int operator()(int kk) const {
        if (kk < s_end) return kk;
        int r = r0 + (kk - s_end);
        r = r >= wrap ? r - wrap : r;
        return sink + r;
    }
};
struct Identity {
    __device__ __forceinline__ int operator()(int kk) const { return kk; }
};

// int8 codes enter the MFMAs as their exact bf16 images.  int4 codes enter
// as offset values: flipping bit 3 of each nibble gives n = code + 8 in
// [0, 15], and the bf16 bit pattern 0x4300 | n is the number 128 + n = code
// + 136, so a pair of values costs one byte permute and one OR, with no
// conversion.  The offset is taken out exactly afterwards: from the scores as
// 136 * sum_x q'_x, from O as 136 * sum_j p_j (the same bf16 p the MFMA used).
template <int KVF>
constexpr float kCodeOffset = KVF == kKvInt4 ? 136.f : 0.f;

// Eight signed int8 codes (two words) -> eight bf16 values (exact: |code| <= 128).
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (__bf16)(float)(int)__builtin_amdgcn_sbfe(lo, 8 * i, 8);
        r[4 + i] = (__bf16)(float)(int)__builtin_amdgcn_sbfe(hi, 8 * i, 8);
    }
    return r;
}
// Eight int4 codes (one word, code i in bits 4i..4i+3) -> eight bf16 values code + 136.
__device__ __forceinline__ bf16x8 i4x8_to_bf16(uint32_t w) {
    w ^= 0x88888888u;
    const uint32_t even = w & 0x0f0f0f0fu;          // n of codes 0, 2, 4, 6 in bytes 0..3
    const uint32_t odd = (w >> 4) & 0x0f0f0f0fu;    // n of codes 1, 3, 5, 7
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)   // byte j of even -> bits 0..7, byte j of odd -> bits 16..23
        r[j] = __builtin_amdgcn_perm(odd, even, 0x0c000c00u | ((4u + j) << 16) | j) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, r);
}

// K/V cache bytes are read once per call, so the cache loads are
// non-temporal (streaming: the line is not kept for reuse).  Measured against
// plain loads: decode_128k 86.5 vs 99.6 us per call, the 16-sequence ragged
// batch 196 vs 207 us, int8 codes 106 vs 123 us.  The exceptions are the K
// code loads of quantised caches, where a 128-byte line is shared by two
// loads of one wave (int8) or by two KV heads in neighbouring work-groups
// (int4): non-temporal K loads measured 128 vs 106 us (int8), 88 vs 85 us
// (int4).  (int4 V rows share lines the same way; there the non-temporal
// loads fetch 12% more bytes but still run faster, 85 vs 87 us.)
template <typename V>
__device__ __forceinline__ V load_stream(const uint8_t* p) {
    return __builtin_nontemporal_load((const V*)p);
}

// One wave's 32-key tile in registers.  K: the A operands of two 16-key
// blocks (lane row m = lane % 16 of block blk holds key tile_key(m, blk));
// V: KPL 16-byte chunks of rows, later stored to LDS as bf16 row-major.
// bf16: k-step s of lane group g4 covers dims 32 s + 8 g4 .. + 7.  Quantised:
// lane group g4 owns the contiguous dims g4 * D / 4 .. + D / 4 - 1 and
// k-step s covers g4 * D / 4 + 8 s .. + 7 (one contiguous load per row); the
// Q operand is laid out to match.
template <int D, int KVF>
struct WaveTile {
    static constexpr int KSTEPS = D / 32;                        // MFMA k-steps over the head dim
    static constexpr int ROW_BYTES = KVF == kKvBf16 ? 2 * D : KVF == kKvInt8 ? D : D / 2;
    static constexpr int KWORDS = ROW_BYTES / 16;                // K words per lane per row
    static constexpr int CPR = ROW_BYTES / 16;                   // 16-byte V chunks per row
    static constexpr int RPI = 64 / CPR;                         // V rows per wave load
    static constexpr int KPL = kTile / RPI;                      // V loads per lane
    static constexpr int DPC = KVF == kKvBf16 ? 8 : KVF == kKvInt8 ? 16 : 32;   // dims per chunk
    uint32_t kw[2][KWORDS];
    u32x4 vr[KPL];

    template <typename Map>
    __device__ __forceinline__ void load(const uint8_t* __restrict__ kseq,
                                         const uint8_t* __restrict__ vseq, int64_t row_bytes,
                                         int key0, int key_end, int lane, const Map& row_of) {
        const int m = lane & 15, g4 = lane >> 4;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int kk = row_of(min(key0 + tile_key(m, blk), key_end - 1));
            const uint8_t* row = kseq + (int64_t)kk * row_bytes;
            if constexpr (KVF == kKvBf16) {
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    const u32x4 x = load_stream<u32x4>(row + 2 * (s * 32 + g4 * 8));
#pragma unroll
                    for (int i = 0; i < 4; ++i) kw[blk][4 * s + i] = x[i];
                }
            } else if constexpr (KWORDS >= 4) {
#pragma unroll
                for (int c4 = 0; c4 < KWORDS / 4; ++c4) {
                    const u32x4 x = *(const u32x4*)(row + g4 * (ROW_BYTES / 4) + 16 * c4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) kw[blk][4 * c4 + i] = x[i];
                }
            } else {
                const u32x2 x = *(const u32x2*)(row + g4 * (ROW_BYTES / 4));
                kw[blk][0] = x[0];
                kw[blk][1] = x[1];
            }
        }
        const int dc = lane % CPR, kg = lane / CPR;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const int kk = row_of(min(key0 + e * RPI + kg, key_end - 1));
            vr[e] = load_stream<u32x4>(vseq + (int64_t)kk * row_bytes + dc * 16);
        }
    }

    __device__ __forceinline__ bf16x8 k_operand(int blk, int s) const {
        if constexpr (KVF == kKvBf16) {
            const u32x4 x = {kw[blk][4 * s], kw[blk][4 * s + 1], kw[blk][4 * s + 2],
                             kw[blk][4 * s + 3]};
            return __builtin_bit_cast(bf16x8, x);
        } else if constexpr (KVF == kKvInt8) {
            return i8x8_to_bf16(kw[blk][2 * s], kw[blk][2 * s + 1]);
        } else {
            return i4x8_to_bf16(kw[blk][s]);
        }
    }

    // V tile into the wave's LDS area as bf16, row-major (key rows, head dims contiguous).
    __device__ __forceinline__ void store_v(uint16_t* __restrict__ vt, int lane) const {
        using SM = DecodeSmem<D>;
        const int dc = lane % CPR, kg = lane / CPR;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            uint16_t* dst = vt + (e * RPI + kg) * SM::VS + dc * DPC;
            if constexpr (KVF == kKvBf16) {
                *(u32x4*)dst = vr[e];
            } else if constexpr (KVF == kKvInt8) {
                *(bf16x8*)dst = i8x8_to_bf16(vr[e][0], vr[e][1]);
                *(bf16x8*)(dst + 8) = i8x8_to_bf16(vr[e][2], vr[e][3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) *(bf16x8*)(dst + 8 * i) = i4x8_to_bf16(vr[e][i]);
            }
        }
    }
};

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// RING: keys come from a ring-buffer cache (see RowMap); each new token t at
// position n - T_q + t sees the sinks and the `window` newest positions up
// to its own, which in walk order is [0, s_end) and [wbeg_t, vend_t).
// KVF: cache storage format.  For a quantised cache the K scale of each
// channel is folded into Q (q' = q * k_scale, split into a bf16 high and low
// part so the fold loses nothing: two MFMAs per k-step against the exact
// bf16 image of the offset codes), and the V scale multiplies the partial O
// once, since O[x] = v_scale[x] * sum_j p_j code_v[j, x].
// HP: KV heads per work-group (1 or 2).  With two, waves 0 and 2 serve KV
// head 2p and waves 1 and 3 head 2p + 1, each pair interleaving the split's
// tiles; a work-group then reads 512 contiguous bytes of every key row it
// touches instead of 256, which streams measurably faster (6.2 vs 5.7 TB/s
// for a pure read of a 512 MiB cache in this shape).
template <int D, int NH, bool RING, int KVF, int HP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, const DecodePlanChunk plan, int T_q, int H_q, int H_kv, int G,
    int n_hg, float c, RingArgs ring, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
    using SM = DecodeSmem<D>;
    using WT = WaveTile<D, KVF>;
    constexpr bool QUANT = KVF != kKvBf16;
    constexpr bool OFFSET = KVF == kKvInt4;   // codes enter the MFMAs as code + 136
    constexpr int KSTEPS = WT::KSTEPS;
    constexpr int DBLK = D / 16;             // 16-row blocks of O^T
    constexpr int WSTRIDE = kCols * (D + 2);        // per wave: O [16][D], then m[16], l[16]
    __shared__ __attribute__((aligned(16))) uint16_t vtiles[kWaves * SM::VT_ELEMS];
    __shared__ __attribute__((aligned(16))) float mrg[kWaves * WSTRIDE];

    static_assert(HP == 1 || HP == 2, "one or two KV heads per work-group");
    constexpr int TSTRIDE = kWaves / HP;     // tile stride of a wave within the split
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;               // MFMA column within a 16-column block
    const int g4 = lane >> 4;

    // Quantised caches: the KV heads of one key range run on one XCD, back to
    // back, because they share the cache's 128-byte lines (an int4 key row of
    // one head is 64 bytes) and each line then comes from HBM once.  (bf16
    // rows are 256 bytes per head; there the round-robin order measures
    // faster.)
    int bid = QUANT ? xcd_contiguous(blockIdx.x, gridDim.x) : (int)blockIdx.x;
    const int n_kvg = H_kv / HP;
    const int kvg = bid % n_kvg;             // KV heads kvg * HP .. kvg * HP + HP - 1
    bid /= n_kvg;
    const int kv = kvg * HP + wave % HP;     // this wave's KV head
    const int hg = bid % n_hg;
    const int unit = bid / n_hg;
    int sq = 0;                              // sequence (within this launch) owning the unit
    while (sq + 1 < plan.nseq && plan.unit_base[sq + 1] <= unit) ++sq;
    const int split = unit - plan.unit_base[sq];
    const int len = plan.len[sq];
    const int L = plan.split_len[sq];
    const int kbeg = split * L;
    const int kend = min(len, kbeg + L);
    const int b = plan.seq0 + sq;
    const int ncols = T_q * G;
    // walk index <-> position: [0, s_end) are positions 0.., then w_lo.. (ring);
    // a packed cache is the identity (s_end = w_lo = 0)
    int s_end = 0, w_lo = 0, pos0 = len - T_q;   // pos0: position of new token 0
    RowMap rmap{0, 0, 0, 1};
    if (RING) {
        const int n = plan.ntok[sq];
        pos0 = n - T_q;
        s_end = min(ring.sink, n);
        w_lo = max(s_end, pos0 - ring.window + 1);
        const int wrap = ring.capacity - ring.sink;
        rmap = RowMap{s_end, ring.sink, w_lo >= ring.sink ? (w_lo - ring.sink) % wrap : 0, wrap};
    }

    // MFMA columns: the G * T_q query rows (new token t, query head g) of a KV
    // head, in blocks of 16; this work-group takes blocks hg*NH .. hg*NH+NH-1,
    // so every K/V tile it loads serves up to 16*NH rows.
    // vis_end[h]: new token t sits at position len - T_q + t and sees keys up to it.
    int vis_end[NH];
    int wbeg[NH];                            // ring: window part of token t starts here
    bf16x8 qf[NH][KSTEPS];
    bf16x8 qlo[QUANT ? NH : 1][QUANT ? KSTEPS : 1];   // low part of q * k_scale
    float kc[NH];                            // int4: score offset of the offset codes
    float lb[NH];                            // int4: sum of the bf16 P fed to P.V
    const int64_t row_bytes = (int64_t)H_kv * WT::ROW_BYTES;
    const uint8_t* kseq = k + plan.key_off[sq] * row_bytes + (int64_t)kv * WT::ROW_BYTES;
    const uint8_t* vseq = v + plan.key_off[sq] * row_bytes + (int64_t)kv * WT::ROW_BYTES;
    const int n_tiles = (kend - kbeg + kTile - 1) / kTile;
    // One register tile per wave: the loads of the wave's next tile go out as
    // soon as the current tile's K has fed the MFMAs and its V is in LDS.
    // (Two tiles in flight per wave measured 1-4% slower on the long and the
    // quantised batches; bf16 caches with one column block use
    // decode_stream_kernel instead.)
    WT wt;
    const int tt = wave / HP;
    auto load = [&](WT& w, int tile) __attribute__((always_inline)) {
        const int key0 = kbeg + tile * kTile;
        if (RING) w.load(kseq, vseq, row_bytes, key0, kend, lane, rmap);
        else w.load(kseq, vseq, row_bytes, key0, kend, lane, Identity{});
    };

#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int f = (hg * NH + h) * kCols + col;
        // columns past the end read a valid row's Q; their outputs are never written
        const int fc = min(f, ncols - 1);
        const int tq = fc / G;
        const int hq = kv * G + fc % G;
        const int pos = pos0 + tq;
        if (RING) {
            vis_end[h] = min(kend, pos < s_end ? pos + 1 : s_end + (pos - w_lo + 1));
            wbeg[h] = s_end + max(0, pos - ring.window + 1 - w_lo);
        } else {
            vis_end[h] = min(kend, pos + 1);
            wbeg[h] = 0;
        }
        // Q^T operand: column = query row, k-group g4 = 8 dims per k-step
        // (the same dims as the K operand of that k-step).
        kc[h] = 0.f;
        if constexpr (!QUANT) {
            const uint16_t* qrow = q + (((int64_t)b * T_q + tq) * H_q + hq) * D + g4 * 8;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                qf[h][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + s * 32));
        } else {
            const int d0 = g4 * (D / 4);
            const uint16_t* qrow = q + (((int64_t)b * T_q + tq) * H_q + hq) * D + d0;
            const float* ks = k_scale + (int64_t)kv * D + d0;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const bf16x8 raw = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 8 * s));
                const f32x4 s0 = *(const f32x4*)(ks + 8 * s);
                const f32x4 s1 = *(const f32x4*)(ks + 8 * s + 4);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float qs = (float)raw[i] * (i < 4 ? s0[i] : s1[i - 4]);
                    const __bf16 hi = (__bf16)qs;
                    qf[h][s][i] = hi;
                    qlo[h][s][i] = (__bf16)(qs - (float)hi);
                }
            }
            // 136 * sum over all channels of the q' the MFMAs see (hi + lo)
            float qsum = 0.f;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i) qsum += (float)qf[h][s][i] + (float)qlo[h][s][i];
            qsum += xor16(qsum);
            qsum += xor32(qsum);
            kc[h] = kCodeOffset<KVF> * qsum;
        }
    }
    // walk indices before mask_from are visible to all tokens (apart from the
    // ring window starts, all below wbeg_max)
    const int mask_from = RING ? min(kend, pos0 < s_end ? pos0 + 1 : s_end + (pos0 - w_lo + 1))
                               : min(kend, len - T_q + 1);
    const int wbeg_max = RING ? s_end + max(0, pos0 + T_q - 1 - ring.window + 1 - w_lo) : 0;
    uint16_t* vt = vtiles + wave * SM::VT_ELEMS;
    // transposed-read source address: lane L of group g4 points at key row
    // g4 + 4 (L / 4) (+ 16 for the second read), dims 4 (L % 4) of each 16-dim block
    const uint16_t* vrd = vt + (g4 + 4 * ((lane & 15) >> 2)) * SM::VS + 4 * (lane & 3);

    f32x4 oacc[NH][DBLK];
    float m_run[NH], l_run[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[h][i] = f32x4{};
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
        lb[h] = 0.f;
    }

    load(wt, tt);

    // one tile: S^T = K Q^T, V into the wave's LDS tile (then, if `reload`,
    // the loads of tile `next` into the same registers), mask, online
    // softmax, O += P V
    auto process = [&](WT& tl, int tile, int next, bool reload) __attribute__((always_inline)) {
        const int key0 = kbeg + tile * kTile;
        // S^T for two 16-key blocks; element i of s[h][blk] is key key0 + g4 + 16 blk + 4 i
        f32x4 s[NH][2];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                s[h][blk] = f32x4{};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const bf16x8 ka = tl.k_operand(blk, ks);
                    s[h][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[h][ks], s[h][blk],
                                                                         0, 0, 0);
                    if constexpr (QUANT)
                        s[h][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qlo[h][ks],
                                                                             s[h][blk], 0, 0, 0);
                }
                if constexpr (OFFSET) s[h][blk] -= kc[h];
            }
        wave_lds_fence();                    // previous tile's V reads are done
        tl.store_v(vt, lane);
        if (reload) load(tl, next);
        if (key0 + kTile > mask_from || (RING && key0 + kTile > s_end && key0 < wbeg_max)) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key0 + g4 + 16 * blk + 4 * i;
                        if constexpr (RING) {
                            // branch-free: past the visible end, or in the ring's
                            // gap [s_end, wbeg) (one unsigned range compare)
                            const bool hide =
                                (key >= vis_end[h]) |
                                ((unsigned)(key - s_end) < (unsigned)max(wbeg[h] - s_end, 0));
                            s[h][blk][i] = hide ? -INFINITY : s[h][blk][i];
                        } else {
                            if (key >= vis_end[h]) s[h][blk][i] = -INFINITY;
                        }
                    }
        }
        float corr[NH];
        bf16x8 pb[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float mt = fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
                             fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
            mt = fmaxf(mt, xor16(mt));
            mt = fmaxf(mt, xor32(mt));
            const float m_new = fmaxf(m_run[h], mt);
            const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
            corr[h] = fast_exp2(m_run[h] * c - mc);
            float p[8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p[blk * 4 + i] = fast_exp2(__builtin_fmaf(s[h][blk][i], c, -mc));
            l_run[h] = l_run[h] * corr[h] +
                       (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
            m_run[h] = m_new;
            u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
            pb[h] = __builtin_bit_cast(bf16x8, pw);
            if constexpr (OFFSET) {
                float ps = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) ps += bf16_lo(pw[w]) + bf16_hi(pw[w]);
                lb[h] = lb[h] * corr[h] + ps;
            }
        }
        wave_lds_fence();                    // V of this tile is visible to the wave
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const s16x4 lo = lds_read_tr16(vrd + db * 16);
            const s16x4 hi = lds_read_tr16(vrd + 16 * SM::VS + db * 16);
            const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                oacc[h][db] *= corr[h];
                oacc[h][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a8), pb[h], oacc[h][db], 0, 0, 0);
            }
        }
    };

    int t = tt;
    for (; t + TSTRIDE < n_tiles; t += TSTRIDE) process(wt, t, t + TSTRIDE, true);
    if (t < n_tiles) process(wt, t, 0, false);

    // ---- merge the wave partials of each KV head through LDS, one column block at a time ----
    const int64_t pidx = (int64_t)plan.split_base + unit;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int fbase = (hg * NH + h) * kCols;
        if (fbase >= ncols) break;           // work-group uniform
        if (h > 0) __syncthreads();          // the previous block's merge reads are done
        float lr = l_run[h];
        lr += xor16(lr);
        lr += xor32(lr);
        float* mw_o = mrg + wave * WSTRIDE;
        if constexpr (OFFSET) {   // take the V code offset out: O -= 136 * sum_j p_j
            float lt = lb[h];
            lt += xor16(lt);
            lt += xor32(lt);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) oacc[h][db] -= kCodeOffset<KVF> * lt;
        }
#pragma unroll
        for (int db = 0; db < DBLK; ++db) *(f32x4*)(mw_o + col * D + db * 16 + g4 * 4) = oacc[h][db];
        if (g4 == 0) {
            mw_o[kCols * D + col] = m_run[h];
            mw_o[kCols * D + kCols + col] = lr;
        }
        __syncthreads();
        for (int e = tid; e < HP * kCols * (D / 4); e += kThreads) {
            const int hk = e / (kCols * (D / 4));    // head of the work-group's HP
            const int e2 = e % (kCols * (D / 4));
            const int cc = e2 / (D / 4), x = (e2 % (D / 4)) * 4;
            const int fo = fbase + cc;
            if (fo >= ncols) continue;
            const int kvh = kvg * HP + hk;
            float mx = -INFINITY;
#pragma unroll
            for (int w = hk; w < kWaves; w += HP) mx = fmaxf(mx, mrg[w * WSTRIDE + kCols * D + cc]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float lsum = 0.f;
#pragma unroll
            for (int w = hk; w < kWaves; w += HP) {
                const float* base = mrg + w * WSTRIDE;
                const float mwv = base[kCols * D + cc];
                const float sc = (mwv == -INFINITY) ? 0.f : fast_exp2((mwv - mx) * c);
                acc += sc * *(const f32x4*)(base + cc * D + x);
                lsum += sc * base[kCols * D + kCols + cc];
            }
            if constexpr (QUANT) acc *= *(const f32x4*)(v_scale + (int64_t)kvh * D + x);
            // partial row: (split, new token, query head)
            const int64_t hrow = (pidx * T_q + fo / G) * H_q + (int64_t)kvh * G + fo % G;
            *(f32x4*)(ws_o + hrow * D + x) = acc;
            if (x == 0) {
                ws_m[hrow] = mx * c;             // base-2 units
                ws_l[hrow] = lsum;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 caches (packed or ring) with at most 16 query rows per KV head (one new
// token of up to 16 query heads per KV head, or a few new tokens of fewer),
// one KV head per work-group: the split kernel's job with the K/V bytes
// streamed into LDS instead of registers.
//  * Every wave walks its 32-key tiles (tile w, w + 4, ... of the split)
//    through a ring of R LDS slots of its own: K and V rows go from HBM
//    straight into a slot with buffer_load ... lds, four whole 256-byte rows
//    per wave instruction (the register path fetches K as half cache lines of
//    16 rows per instruction, which streams measurably slower).  A slot is
//    refilled with the wave's tile i + R as soon as tile i is read, so R
//    tiles stay in flight per wave and no barrier is needed.
//  * K A-operands are read back with ds_read_b128, V^T with
//    ds_read_b64_tr_b16; the 16-byte chunks of each row are XOR-swizzled by
//    the row (chunk c of row r at c ^ (r mod CPR)), which keeps both reads
//    free of bank conflicts.
//  * One LDS array per slot: the compiler then waits for the DMA loads of the
//    slot being read, not for every DMA load in flight.
//  * The four wave partials meet once at the end: each wave leaves its
//    unnormalised partial in its own slot, one barrier, then every thread
//    merges four waves' values for its outputs.
//  * A launch of one sequence finds its plan entries with one round of
//    kernel-argument loads.
// With R = 2 a work-group holds 128 KiB of LDS (one per compute unit); with
// R = 1 (splits of at most 128 keys, one tile per wave) 64 KiB.
constexpr int kStreamOneSlotKeys = kWaves * kTile;   // 128: one tile per wave
// bf16 caches with up to 32 query rows per KV head take decode_stream_kernel
__host__ __device__ inline bool decode_is_stream(int T_q, int G) { return T_q * G <= 2 * kCols; }

// One wave-wide 16-byte-per-lane load from a buffer straight into LDS
// (lane l's 16 bytes at lds_byte + 16 l).  Written as inline assembly so that
// the compiler does not track it: it would otherwise wait for every LDS load
// in flight before any LDS read it cannot attribute to a particular one; the
// kernels that use it wait for these loads themselves (s_waitcnt vmcnt) and
// issue no other vector-memory loads.
typedef __attribute__((ext_vector_type(4))) int i32x4;
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int range) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xffff), range, 0x00020000};
}
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_byte, int voffset) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(lds_byte), "v"(voffset), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int D>
struct StreamSmem {
    static constexpr int TILE_ELEMS = kTile * D;              // one K or V tile
    static constexpr int SLOT_ELEMS = 2 * TILE_ELEMS;         // K then V
};

template <int D>
__device__ __forceinline__ int stream_swz(int r) { return r & (D / 8 - 1); }

// NH: 16-row column blocks of query rows per KV head (1, or 2 for 17-32 rows,
// which always takes two slots per wave: with the Q area of 32 rows the
// work-group holds 160 KiB of LDS).  Each K or V read from LDS feeds NH
// MFMAs.
template <int D, int R, bool RING, int NH = 1>
// The first sixteen argument dwords (pointers to Q, K and V, the first
// sequence's plan entry and the head counts) are everything a work-group of
// a one-sequence launch needs before it issues its loads; the library is
// built to preload them into scalar registers at dispatch, so those loads do
// not wait for a kernel-argument fetch.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, R == 1 ? 2 : 1))) void decode_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t key_off0, int nseq, int len0, int split_len0,
    int seq0, int T_q, int H_q, int H_kv, int G, float* __restrict__ ws_m,
    float* __restrict__ ws_l, float* __restrict__ ws_o, const DecodePlanChunk plan, float c,
    RingArgs ring) {
    using SM = StreamSmem<D>;
    constexpr int KSTEPS = D / 32;
    constexpr int DBLK = D / 16;
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int ROWS_PER_LOAD = 64 / CPR;        // rows per wave DMA instruction
    constexpr int LOADS = kTile / ROWS_PER_LOAD;   // DMA instructions per K or V tile
    constexpr int LPT = 2 * LOADS;                 // per tile (K and V)
    static_assert(R == 1 || R == 2, "one or two slots per wave");
    static_assert(NH == 1 || (NH == 2 && R == 2), "32 query rows: two slots per wave");
    __shared__ __attribute__((aligned(1024))) uint16_t slot0[kWaves * SM::SLOT_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t slot1[R > 1 ? kWaves * SM::SLOT_ELEMS : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t qlds[kWaves * NH * kCols * D];   // per wave

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int g4 = lane >> 4;

    const int kv = blockIdx.x % H_kv;
    const int unit = blockIdx.x / H_kv;
    // plan entries: index 0 comes with the leading arguments (unit_base[0]
    // is 0); a launch of several sequences looks its own up
    int sq = 0;
    int len = len0, L = split_len0, ub = 0;
    int ntok = RING ? plan.ntok[0] : len0;
    int64_t key_off = key_off0;
    if (nseq > 1) {
        while (sq + 1 < plan.nseq && plan.unit_base[sq + 1] <= unit) ++sq;
        len = plan.len[sq];
        L = plan.split_len[sq];
        ub = plan.unit_base[sq];
        ntok = plan.ntok[sq];
        key_off = plan.key_off[sq];
    }
    const int split = unit - ub;
    const int kbeg = split * L;
    const int kend = min(len, kbeg + L);
    const int b = seq0 + sq;
    const int ncols = T_q * G;
    // walk index <-> position: [0, s_end) are positions 0.., then w_lo.. (ring);
    // a packed cache is the identity (s_end = w_lo = 0)
    int s_end = 0, w_lo = 0, pos0 = len - T_q;    // pos0: position of new token 0
    RowMap rmap{0, 0, 0, 1};
    if (RING) {
        pos0 = ntok - T_q;
        s_end = min(ring.sink, ntok);
        w_lo = max(s_end, pos0 - ring.window + 1);
        const int wrap = ring.capacity - ring.sink;
        rmap = RowMap{s_end, ring.sink, w_lo >= ring.sink ? (w_lo - ring.sink) % wrap : 0, wrap};
    }

    // Q^T operand (column = query row; block h holds rows 16 h ..)
    int vis_end[NH], wbeg[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int fc = min(h * kCols + col, ncols - 1);   // columns past the end read a valid row
        const int pos = pos0 + fc / G;
        if (RING) {
            vis_end[h] = min(kend, pos < s_end ? pos + 1 : s_end + (pos - w_lo + 1));
            wbeg[h] = s_end + max(0, pos - ring.window + 1 - w_lo);
        } else {
            vis_end[h] = min(kend, pos + 1);
            wbeg[h] = 0;
        }
    }
    // Q rows of the 16 NH columns go into the wave's own Q area first (row c =
    // column c, chunks swizzled as the K rows), so that the wait for the
    // first tile covers them
    uint16_t* qw = qlds + wave * NH * kCols * D;
    {
        // based at the KV head's first query head of token 0; T_q * H_q * d * 2
        // bytes stay far below 2^31 (T_q <= 256)
        const i32x4 rs = buffer_rsrc(q + ((int64_t)b * T_q * H_q + (int64_t)kv * G) * D, 0x7ffffff0);
#pragma unroll
        for (int j = 0; j < NH * kCols / ROWS_PER_LOAD; ++j) {
            const int r = j * ROWS_PER_LOAD + lane / CPR;           // column
            const int rc = min(r, ncols - 1);
            const int cc = (lane % CPR) ^ stream_swz<D>(r);
            dma16(rs, lds_addr(qw + j * ROWS_PER_LOAD * D),
                  (((rc / G) * H_q + rc % G) * D + cc * 8) * 2);
        }
    }
    bf16x8 qf[NH][KSTEPS];                         // read once its loads have landed
    // walk indices before mask_from are visible to all tokens (apart from the
    // ring window starts, all below wbeg_max)
    const int mask_from = RING ? min(kend, pos0 < s_end ? pos0 + 1 : s_end + (pos0 - w_lo + 1))
                               : min(kend, pos0 + 1);
    const int wbeg_max = RING ? s_end + max(0, pos0 + T_q - 1 - ring.window + 1 - w_lo) : 0;

    const int64_t row_elems = (int64_t)H_kv * D;
    const uint16_t* kseq = k + key_off * row_elems + (int64_t)kv * D;
    const uint16_t* vseq = v + key_off * row_elems + (int64_t)kv * D;
    auto wslot = [&](int sl) { return (sl == 0 ? slot0 : slot1) + wave * SM::SLOT_ELEMS; };
    const int n_tiles = (kend - kbeg + kTile - 1) / kTile;
    const int n_w = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;   // this wave's tiles

    // DMA of the wave's tile i into slot sl; rows past the split end re-read
    // its last key
    auto issue = [&](int i, int sl) __attribute__((always_inline)) {
        const int key0 = kbeg + (wave + kWaves * i) * kTile;
        const int last = kend - 1;
        const int kfirst = RING ? 0 : min(key0, last);
        const int range = 0x7ffffff0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint16_t* src = h == 0 ? kseq : vseq;
            uint16_t* dst = wslot(sl) + h * SM::TILE_ELEMS;
            // packed: based at the tile's first row; ring: at the sequence's
            // first slot (the host keeps capacity * row bytes below 2^31)
            const i32x4 rs = buffer_rsrc(src + (int64_t)kfirst * row_elems, range);
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                const int r = j * ROWS_PER_LOAD + lane / CPR;
                const int cc = (lane % CPR) ^ stream_swz<D>(r);
                const int key = min(key0 + r, last);
                const int row = RING ? rmap(key) : key - kfirst;
                const int off = (int)(((int64_t)row * row_elems + cc * 8) * 2);
                dma16(rs, lds_addr(dst + j * ROWS_PER_LOAD * D), off);
            }
        }
    };
#pragma unroll
    for (int sl = 0; sl < R; ++sl)
        if (sl < n_w) issue(sl, sl);

    // per-lane LDS read offsets (elements within a tile)
    int koff[2][KSTEPS];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int r = tile_key(col, blk);
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) koff[blk][st] = r * D + (((st * 4 + g4) ^ stream_swz<D>(r)) << 3);
    }
    // V^T: lane L of group g4 reads key row g4 + 4 (L / 4) (+ 16), dims 4 (L % 4) of each 16-dim block
    int voff[2][DBLK];
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
        const int r = g4 + 4 * ((lane & 15) >> 2) + 16 * hi;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int x = db * 16 + 4 * (lane & 3);
            voff[hi][db] = r * D + (((x >> 3) ^ stream_swz<D>(r)) << 3) + (x & 7);
        }
    }

    f32x4 oacc[NH][DBLK];
    float m_run[NH], l_run[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int j = 0; j < DBLK; ++j) oacc[h][j] = f32x4{};
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
    }

    // one tile from slot sl: S^T = K Q^T, mask, online softmax, O += P V
    // (more: the wave's next tile is in flight behind this one; K is waited
    // for before the call, V only before the P.V step)
    auto process = [&](int i, int sl, bool more) __attribute__((always_inline)) {
        const int key0 = kbeg + (wave + kWaves * i) * kTile;
        const uint16_t* kt = wslot(sl);
        const uint16_t* vt = kt + SM::TILE_ELEMS;
        f32x4 s[NH][2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
            for (int h = 0; h < NH; ++h) s[h][blk] = f32x4{};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                const bf16x8 ka = *(const bf16x8*)(kt + koff[blk][st]);
#pragma unroll
                for (int h = 0; h < NH; ++h)
                    s[h][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[h][st], s[h][blk],
                                                                         0, 0, 0);
            }
        }
        if (key0 + kTile > mask_from || (RING && key0 + kTile > s_end && key0 < wbeg_max)) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = key0 + g4 + 16 * blk + 4 * e;
                        if constexpr (RING) {
                            // branch-free: past the visible end, or in the ring's
                            // gap [s_end, wbeg) (one unsigned range compare)
                            const bool hide =
                                (key >= vis_end[h]) |
                                ((unsigned)(key - s_end) < (unsigned)max(wbeg[h] - s_end, 0));
                            s[h][blk][e] = hide ? -INFINITY : s[h][blk][e];
                        } else {
                            if (key >= vis_end[h]) s[h][blk][e] = -INFINITY;
                        }
                    }
        }
        bf16x8 pb[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float mt = fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
                             fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
            mt = fmaxf(mt, xor16(mt));
            mt = fmaxf(mt, xor32(mt));
            // Lazy rescale: the reference max moves only when a column's tile
            // max exceeds it by more than 2^8 in the exponentials (then O and
            // l are rescaled); otherwise P <= 2^8 against the old reference,
            // which the fp32 sums carry exactly as well.  The wave's first
            // tile sets it.
            if (i == 0) {
                m_run[h] = mt;
            } else if (__builtin_amdgcn_ballot_w64(mt * c > m_run[h] * c + 8.f) != 0) {
                const float m_new = fmaxf(m_run[h], mt);
                const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run[h] - m_new) * c);
                l_run[h] *= corr;
#pragma unroll
                for (int db = 0; db < DBLK; ++db) oacc[h][db] *= corr;
                m_run[h] = m_new;
            }
            const float mc = (m_run[h] == -INFINITY) ? 0.f : m_run[h] * c;
            float p[8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p[blk * 4 + e] = fast_exp2(__builtin_fmaf(s[h][blk][e], c, -mc));
            l_run[h] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                              pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            pb[h] = __builtin_bit_cast(bf16x8, pw);
        }
        if (more) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LPT) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const s16x4 lo = lds_read_tr16(vt + voff[0][db]);
            const s16x4 hi = lds_read_tr16(vt + voff[1][db]);
            const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int h = 0; h < NH; ++h)
                oacc[h][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a8), pb[h], oacc[h][db], 0, 0, 0);
        }
    };

    // Q from the wave's Q area (its loads are older than every tile's)
    if (R == 2 && n_w >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LPT) : "memory");
    else if (n_w >= 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LPT) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int r = h * kCols + col;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
            qf[h][st] = *(const bf16x8*)(qw + r * D + (((st * 4 + g4) ^ stream_swz<D>(r)) << 3));
    }

    // Tile j sits in slot j mod R; when it is processed the loads in flight
    // are those of the wave's tiles j .. min(j + R, n_w) - 1, oldest first, so
    // the wait leaves the later tiles' loads outstanding.
    for (int i = 0; i < n_w; i += R) {
#pragma unroll
        for (int sl = 0; sl < R; ++sl) {
            const int j = i + sl;
            if (j >= n_w) break;                   // wave-uniform
            // this tile's K rows (issued before its V rows) have landed
            const bool more = R == 2 && j + 1 < n_w;
            if (more) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LPT + LOADS) : "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LOADS) : "memory");
            process(j, sl, more);
            if (j + R < n_w) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the slot's LDS reads are done
                issue(j + R, sl);
            }
        }
    }

    // ---- merge the four wave partials ----
    // Each wave puts its unnormalised partial (m, l, O) of column block h into
    // its own slot-h area, which no other wave reads before the barrier;
    // after it, every thread merges four waves' values for its outputs.
    // no DMA write into this wave's slots may still be pending
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // wave area: O [16][CS] (columns padded by 4 floats against bank
    // conflicts), then l [16], then m [16]
    constexpr int CS = D + 4;
    constexpr int AREA = kCols * CS + 2 * kCols;             // floats
    static_assert(AREA * 4 <= SM::SLOT_ELEMS * 2, "a wave's merge area fits its slot");
    constexpr int AREA_STRIDE = SM::SLOT_ELEMS / 2;          // floats between waves' areas
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        float lr = l_run[h];
        lr += xor16(lr);
        lr += xor32(lr);
        float* mw = (float*)((h == 0 ? slot0 : slot1) + wave * SM::SLOT_ELEMS);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) *(f32x4*)(mw + col * CS + db * 16 + g4 * 4) = oacc[h][db];
        if (g4 == 0) {
            mw[kCols * CS + col] = lr;
            mw[kCols * CS + kCols + col] = m_run[h];
        }
    }
    __syncthreads();
    const int64_t pidx = (int64_t)plan.split_base + unit;
    constexpr int PER = kCols * D / 4 / kThreads;  // f32x4 outputs per thread and block
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const float* mrg = (const float*)(h == 0 ? slot0 : slot1);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * kThreads;
            const int cl = e / (D / 4), x = (e % (D / 4)) * 4;
            const int cc = h * kCols + cl;         // query row of the KV head
            if (cc >= ncols) continue;
            float mwv[kWaves], mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                mwv[w] = mrg[w * AREA_STRIDE + kCols * CS + kCols + cl];
                mx = fmaxf(mx, mwv[w]);
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float lsum = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = (mwv[w] == -INFINITY) ? 0.f : fast_exp2((mwv[w] - mx) * c);
                acc += sc * *(const f32x4*)(mrg + w * AREA_STRIDE + cl * CS + x);
                lsum += sc * mrg[w * AREA_STRIDE + kCols * CS + cl];
            }
            const int64_t hrow = (pidx * T_q + cc / G) * H_q + (int64_t)kv * G + cc % G;
            *(f32x4*)(ws_o + hrow * D + x) = acc;
            if (x == 0) {
                ws_m[hrow] = mx * c;               // base-2 units
                ws_l[hrow] = lsum;
            }
        }
    }
}

// One wave per (sequence, query head, 32-dim chunk of O).  Lane (sg, dq):
// split group sg = lane / 8 takes splits sg, sg + 8, sg + 16, ...; dim quad
// dq = lane % 8 owns dims 4 dq .. 4 dq + 3 of the chunk.  A lane loads a
// batch of NB of its splits at once and folds them, in split order, into a
// running (m, l, O) with the section 4 merge; the eight split groups are then
// merged with a fixed butterfly, so the result does not depend on timing
// (bitwise reproducible for a given split plan, and the same for every NB: a
// missing split folds in as an exact no-op).  NB follows the launch's
// longest sequence, so short plans do not issue loads for absent splits.
// All in base 2.

__device__ __forceinline__ void merge_lse(float& m, float& l, f32x4& o, float m2, float l2,
                                          const f32x4& o2) {
    const float mm = fmaxf(m, m2);
    const float w1 = (m == -INFINITY) ? 0.f : fast_exp2(m - mm);
    const float w2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mm);
    l = l * w1 + l2 * w2;
    o = o * w1 + o2 * w2;
    m = mm;
}

template <int D, int NB>
// (leading arguments: what a one-sequence launch needs before its loads,
// preloaded into scalar registers like the stream kernel's)
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, int nseq, int split_base, int units0, int seq0, int T_q,
    int H_q, uint16_t* __restrict__ o, float* __restrict__ lse, const DecodePlanChunk plan) {
    constexpr int CHUNKS = D / 32;
    const int R = T_q * H_q;                                   // rows per sequence
    const int lane = threadIdx.x;
    const int item = blockIdx.x;   // (sequence, head, chunk)
    if (item >= nseq * R * CHUNKS) return;
    const int chunk = item % CHUNKS;
    const int sh = item / CHUNKS;
    const int sq = sh / R, r = sh % R;                         // r = t * H_q + h
    // one sequence: its splits are the launch's units
    const int n = nseq == 1 ? units0 : plan.unit_base[sq + 1] - plan.unit_base[sq];
    const int64_t p0 = (int64_t)split_base + (nseq == 1 ? 0 : plan.unit_base[sq]);

    const int sg = lane >> 3, dq = lane & 7;
    const int dim = chunk * 32 + dq * 4;
    float m = -INFINITY, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = sg; s0 < n; s0 += 8 * NB) {
        float mv[NB], lv[NB];
        f32x4 ov[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int s = s0 + 8 * u;
            const int64_t hrow = (p0 + (s < n ? s : 0)) * R + r;
            mv[u] = s < n ? ws_m[hrow] : -INFINITY;
            lv[u] = s < n ? ws_l[hrow] : 0.f;
            ov[u] = *(const f32x4*)(ws_o + hrow * D + dim);
            if (s >= n) ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) merge_lse(m, l, acc, mv[u], lv[u], ov[u]);
    }
#pragma unroll
    for (int step = 0; step < 3; ++step) {   // partner lanes l ^ 8, l ^ 16, l ^ 32
        auto other = [step](float x) { return step == 0 ? xor8(x) : step == 1 ? xor16(x) : xor32(x); };
        const float m2 = other(m);
        const float l2 = other(l);
        f32x4 o2;
#pragma unroll
        for (int i = 0; i < 4; ++i) o2[i] = other(acc[i]);
        merge_lse(m, l, acc, m2, l2, o2);
    }
    const float inv = 1.f / l;
    const int b = seq0 + sq;
    if (sg == 0) {
        u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *(u32x2*)(o + ((int64_t)b * R + r) * D + dim) = w;
    }
    if (lse != nullptr && chunk == 0 && lane == 0)
        lse[(int64_t)b * R + r] = (m + fast_log2(l)) * kLn2;
}

// Row-per-wave variant for launches of many rows with few splits each
// (multi-token decode: T_q * H_q rows per sequence): each wave merges one
// whole row.  Its lanes form SG = 256 / D split groups of D / 4 lanes, lane
// (sg, dq) owning dims 4 dq .. 4 dq + 3 and splits sg, sg + SG, ...; the
// groups then merge with a fixed butterfly as above (same merge order for
// every NB).  Four waves (four rows) per work-group.
constexpr int kCombineRowWaves = 4;
// launches with at least this many (sequence, row) pairs and at most four
// splits per lane group take the row-per-wave kernel
constexpr int64_t kCombineRowsMin = 4096;

template <int D, int NB>
__global__ __launch_bounds__(64 * kCombineRowWaves) void decode_combine_rows_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, uint16_t* __restrict__ o, float* __restrict__ lse,
    const DecodePlanChunk plan, int T_q, int H_q) {
    constexpr int LPG = D / 4;          // lanes per split group
    constexpr int SG = 64 / LPG;        // split groups per wave
    const int R = T_q * H_q;            // rows per sequence
    const int lane = threadIdx.x & 63;
    const int sh = blockIdx.x * kCombineRowWaves + (threadIdx.x >> 6);   // (sequence, row)
    if (sh >= plan.nseq * R) return;    // whole wave
    const int sq = sh / R, r = sh % R;  // r = t * H_q + h
    const int n = plan.unit_base[sq + 1] - plan.unit_base[sq];
    const int64_t p0 = (int64_t)plan.split_base + plan.unit_base[sq];
    const int sg = lane / LPG, dim = (lane % LPG) * 4;
    float m = -INFINITY, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = sg; s0 < n; s0 += SG * NB) {
        float mv[NB], lv[NB];
        f32x4 ov[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int s = s0 + SG * u;
            const int64_t hrow = (p0 + (s < n ? s : 0)) * R + r;
            mv[u] = s < n ? ws_m[hrow] : -INFINITY;
            lv[u] = s < n ? ws_l[hrow] : 0.f;
            ov[u] = *(const f32x4*)(ws_o + hrow * D + dim);
            if (s >= n) ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) merge_lse(m, l, acc, mv[u], lv[u], ov[u]);
    }
#pragma unroll
    for (int step = (SG == 2 ? 1 : 0); step < 2; ++step) {   // partners l ^ 16 (SG 4), l ^ 32
        auto other = [step](float x) { return step == 0 ? xor16(x) : xor32(x); };
        const float m2 = other(m);
        const float l2 = other(l);
        f32x4 o2;
#pragma unroll
        for (int i = 0; i < 4; ++i) o2[i] = other(acc[i]);
        merge_lse(m, l, acc, m2, l2, o2);
    }
    const float inv = 1.f / l;
    const int b = plan.seq0 + sq;
    if (sg == 0) {
        u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *(u32x2*)(o + ((int64_t)b * R + r) * D + dim) = w;
    }
    if (lse != nullptr && lane == 0)
        lse[(int64_t)b * R + r] = (m + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Wide variant for many query rows per KV head (G * T_q > 32, e.g. multi-token
// decode): the four waves of a work-group split the column blocks instead of
// the keys.  Every 128-key K/V tile of the split is loaded into LDS once per
// work-group (each thread moves eight 16-byte chunks of K and eight of V at
// D = 128; the next tile's loads are in flight in registers while a tile is
// computed, in four 32-key parts) and each
// wave reads it for its own NHW blocks of 16 query rows, so the tile feeds up
// to 4 * NHW * 16 rows; each wave keeps the softmax state of its rows over the
// whole split and writes its partials itself (no cross-wave merge).  K rows in
// LDS: 16-byte chunk c of row r at chunk position c ^ swz(r) (the A-operand
// reads of 16 rows x one chunk are then bank-conflict free); V rows
// row-major at stride VS as in the split kernel.

constexpr int kWideWaves = 4;

// Chunk permutation of K row r: distinct modulo 8 over the 8 rows that eight
// consecutive lanes read together, and below the chunks per row (16 at
// D = 128, 8 at D = 64).
template <int D>
__device__ __forceinline__ int wide_swz(int r) {
    const int f = ((r & 3) << 2) | ((r >> 2) & 3);
    return D == 128 ? f : (f & 7);
}

template <int D, int NHW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, const DecodePlanChunk plan, int T_q, int H_q, int H_kv, int G,
    int n_hg, float c) {
    using SM = DecodeSmem<D>;
    constexpr int KSTEPS = D / 32;
    constexpr int DBLK = D / 16;
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int NSUB = 4;                       // 32-key sub-tiles per tile
    constexpr int WT = NSUB * kTile;              // keys per tile
    constexpr int KT_ELEMS = WT * D;              // K tile (swizzled, unpadded)
    constexpr int VT_ELEMS = WT * SM::VS;
    constexpr int CH_PER_THREAD = WT * CPR / kThreads;   // 8 (D = 128) or 4 (D = 64)
    __shared__ __attribute__((aligned(16))) uint16_t kst[KT_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vst[VT_ELEMS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int g4 = lane >> 4;

    int bid = blockIdx.x;
    const int kv = bid % H_kv;
    bid /= H_kv;
    const int hg = bid % n_hg;
    const int unit = bid / n_hg;
    int sq = 0;
    while (sq + 1 < plan.nseq && plan.unit_base[sq + 1] <= unit) ++sq;
    const int split = unit - plan.unit_base[sq];
    const int len = plan.len[sq];
    const int L = plan.split_len[sq];
    const int kbeg = split * L;
    const int kend = min(len, kbeg + L);
    const int b = plan.seq0 + sq;
    const int ncols = T_q * G;
    const int pos0 = len - T_q;
    const int n_tiles = (kend - kbeg + WT - 1) / WT;

    const int64_t row_stride = (int64_t)H_kv * D;
    const uint16_t* kseq = k + (plan.key_off[sq] * H_kv + kv) * (int64_t)D;
    const uint16_t* vseq = v + (plan.key_off[sq] * H_kv + kv) * (int64_t)D;

    // tile loads: thread chunk ci = tid + kThreads * u -> row ci / CPR, chunk ci % CPR
    u32x4 kr[CH_PER_THREAD], vr[CH_PER_THREAD];
    auto load = [&](int t) {
        const int key0 = kbeg + t * WT;
#pragma unroll
        for (int u = 0; u < CH_PER_THREAD; ++u) {
            const int ci = tid + kThreads * u;
            const int key = min(key0 + ci / CPR, kend - 1);
            kr[u] = load_stream<u32x4>((const uint8_t*)(kseq + (int64_t)key * row_stride + (ci % CPR) * 8));
            vr[u] = load_stream<u32x4>((const uint8_t*)(vseq + (int64_t)key * row_stride + (ci % CPR) * 8));
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < CH_PER_THREAD; ++u) {
            const int ci = tid + kThreads * u;
            const int r = ci / CPR, ch = ci % CPR;
            *(u32x4*)(&kst[r * D + ((ch ^ wide_swz<D>(r)) << 3)]) = kr[u];
            *(u32x4*)(&vst[r * SM::VS + ch * 8]) = vr[u];
        }
    };

    // this wave's column blocks: (hg * kWideWaves + wave) * NHW + h
    int vis_end[NHW];
    bf16x8 qf[NHW][KSTEPS];
#pragma unroll
    for (int h = 0; h < NHW; ++h) {
        const int f = ((hg * kWideWaves + wave) * NHW + h) * kCols + col;
        const int fc = min(f, ncols - 1);
        const int tq = fc / G;
        const int hq = kv * G + fc % G;
        vis_end[h] = min(kend, pos0 + tq + 1);
        const uint16_t* qrow = q + (((int64_t)b * T_q + tq) * H_q + hq) * D + g4 * 8;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            qf[h][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + s * 32));
    }
    const int wave_cols = ((hg * kWideWaves + wave) * NHW) * kCols;
    const bool wave_live = wave_cols < ncols;     // wave-uniform
    const int mask_from = min(kend, pos0 + 1);

    // per-lane LDS read offsets: K A-operand row tile_key(col, blk), logical chunk 4 s + g4
    int koff[2][KSTEPS];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int r = tile_key(col, blk);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) koff[blk][s] = r * D + (((s * 4 + g4) ^ wide_swz<D>(r)) << 3);
    }
    const int vrd = (g4 + 4 * ((lane & 15) >> 2)) * SM::VS + 4 * (lane & 3);

    f32x4 oacc[NHW][DBLK];
    float m_run[NHW], l_run[NHW];
#pragma unroll
    for (int h = 0; h < NHW; ++h) {
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[h][i] = f32x4{};
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
    }

    // one LDS tile; the next tile waits in registers (its loads are in
    // flight while this one is computed)
    if (n_tiles > 0) {
        load(0);
        store();
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) load(t + 1);
#pragma unroll
        for (int half = 0; half < NSUB; ++half) {
          const int key0 = kbeg + t * WT + half * kTile;
          if (wave_live && key0 < kend) {
            const uint16_t* kt = kst + half * kTile * D;
            const uint16_t* vt = vst + half * kTile * SM::VS;
            f32x4 s[NHW][2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int h = 0; h < NHW; ++h) s[h][blk] = f32x4{};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const bf16x8 a = *(const bf16x8*)(kt + koff[blk][ks]);
#pragma unroll
                    for (int h = 0; h < NHW; ++h)
                        s[h][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[h][ks], s[h][blk],
                                                                             0, 0, 0);
                }
            }
            if (key0 + kTile > mask_from) {
#pragma unroll
                for (int h = 0; h < NHW; ++h)
#pragma unroll
                    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (key0 + g4 + 16 * blk + 4 * i >= vis_end[h]) s[h][blk][i] = -INFINITY;
            }
            float corr[NHW];
            bf16x8 pb[NHW];
#pragma unroll
            for (int h = 0; h < NHW; ++h) {
                float mt = fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
                                 fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
                mt = fmaxf(mt, xor16(mt));
                mt = fmaxf(mt, xor32(mt));
                const float m_new = fmaxf(m_run[h], mt);
                const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
                corr[h] = fast_exp2(m_run[h] * c - mc);
                float p[8];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p[blk * 4 + i] = fast_exp2(__builtin_fmaf(s[h][blk][i], c, -mc));
                l_run[h] = l_run[h] * corr[h] +
                           (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
                m_run[h] = m_new;
                u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
                pb[h] = __builtin_bit_cast(bf16x8, pw);
            }
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const s16x4 lo = lds_read_tr16(vt + vrd + db * 16);
                const s16x4 hi = lds_read_tr16(vt + vrd + 16 * SM::VS + db * 16);
                const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int h = 0; h < NHW; ++h) {
                    oacc[h][db] *= corr[h];
                    oacc[h][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a8), pb[h], oacc[h][db], 0, 0, 0);
                }
            }
          }
        }
        if (t + 1 < n_tiles) {
            __syncthreads();                  // every wave is done with tile t
            store();
        }
        __syncthreads();
    }

    // ---- each wave writes the partials of its own rows ----
    const int64_t pidx = (int64_t)plan.split_base + unit;
#pragma unroll
    for (int h = 0; h < NHW; ++h) {
        float lr = l_run[h];
        lr += xor16(lr);
        lr += xor32(lr);
        const int fo = ((hg * kWideWaves + wave) * NHW + h) * kCols + col;
        if (fo < ncols) {
            const int64_t hrow = (pidx * T_q + fo / G) * H_q + (int64_t)kv * G + fo % G;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) *(f32x4*)(ws_o + hrow * D + db * 16 + g4 * 4) = oacc[h][db];
            if (g4 == 0) {
                ws_m[hrow] = m_run[h] * c;      // base-2 units
                ws_l[hrow] = lr;
            }
        }
    }
}

}  // namespace

int decode_column_blocks_per_group(int T_q, int G) { return T_q * G > kCols ? 2 : 1; }

// from kDecodeRowsMin rows: the prefill tile loop (launch_decode_rows_bf16);
// more than two 16-row column blocks below that: the wide kernel (bf16,
// packed cache)
static bool decode_use_rows(int T_q, int G) { return T_q * G >= kDecodeRowsMin; }
static bool decode_use_wide(int T_q, int G) { return T_q * G > 2 * kCols && !decode_use_rows(T_q, G); }
static int decode_wide_nhw(int T_q, int G) { return T_q * G > kWideWaves * kCols ? 2 : 1; }

// bf16 splits of at least this many keys take two KV heads per work-group
// (each wave then walks at least eight 32-key tiles); shorter splits keep one
// head per work-group and four waves on its tiles, which keeps more waves busy.
constexpr int kPairMinSplitLen = 512;

int64_t decode_workgroups_per_split(DecodeKind kind, int T_q, int G, int H_kv, int split_len) {
    int64_t n_hg;
    bool pairs = false;
    if (kind == DecodeKind::Bf16 && decode_use_rows(T_q, G)) {
        // 512 threads and 128 KiB of LDS: one work-group per compute unit
        return prefill_row_blocks(T_q, G) * (H_kv / decode_rows_heads_per_workgroup(T_q, G, H_kv)) *
               kDecodeWorkgroupsPerCu;
    }
    if (kind == DecodeKind::Bf16 && decode_use_wide(T_q, G)) {
        n_hg = decode_column_groups(T_q, G);
    } else {
        const int nh = decode_column_blocks_per_group(T_q, G);
        n_hg = (((int64_t)T_q * G + kCols - 1) / kCols + nh - 1) / nh;
        pairs = kind == DecodeKind::Bf16 || kind == DecodeKind::Ring;
    }
    int hp = (pairs && H_kv % 2 == 0 && split_len >= kPairMinSplitLen) ? 2 : 1;
    // bf16 caches with up to two column blocks stream K/V into LDS one KV
    // head per work-group (decode_stream_kernel); with two slots per wave a
    // work-group holds the LDS of two, so it counts twice
    int occ = 1;
    if ((kind == DecodeKind::Bf16 || kind == DecodeKind::Ring) && decode_is_stream(T_q, G)) {
        hp = 1;
        occ = (T_q * G > kCols || split_len > kStreamOneSlotKeys) ? 2 : 1;
    }
    return n_hg * (H_kv / hp) * occ;
}

int decode_column_groups(int T_q, int G) {
    if (decode_use_rows(T_q, G)) return (int)prefill_row_blocks(T_q, G);
    const int blocks = (T_q * G + kCols - 1) / kCols;
    const int per = decode_use_wide(T_q, G) ? kWideWaves * decode_wide_nhw(T_q, G)
                                            : decode_column_blocks_per_group(T_q, G);
    return (blocks + per - 1) / per;
}

template <int D, int NHW>
static hipError_t launch_wide(const void* q, const void* k, const void* v,
                              const DecodeWorkspace& ws, const DecodePlanChunk& plan, int T_q,
                              int H_q, int H_kv, float c, hipStream_t stream) {
    const int G = H_q / H_kv;
    const int blocks = (T_q * G + kCols - 1) / kCols;
    const int n_hg = (blocks + kWideWaves * NHW - 1) / (kWideWaves * NHW);
    const int64_t grid = (int64_t)plan.units * n_hg * H_kv;
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_wide_kernel<D, NHW>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, ws.m,
                       ws.l, ws.o, plan, T_q, H_q, H_kv, G, n_hg, c);
    return hipGetLastError();
}

struct KvScales {
    const float* k = nullptr;
    const float* v = nullptr;
};

template <int D, int NH, bool RING, int KVF>
static void launch_split(int hp, int64_t units_hg, const void* q, const void* k, const void* v,
                         const DecodeWorkspace& ws, const DecodePlanChunk& plan, int T_q, int H_q,
                         int H_kv, int G, int n_hg, float c, const RingArgs& ring,
                         const KvScales& sc, hipStream_t stream) {
    const dim3 grid((unsigned)(units_hg * (H_kv / hp)));
    if (hp == 2)
        hipLaunchKernelGGL((decode_split_kernel<D, NH, RING, KVF, 2>), grid, dim3(kThreads), 0,
                           stream, (const uint16_t*)q, (const uint8_t*)k, (const uint8_t*)v, ws.m,
                           ws.l, ws.o, plan, T_q, H_q, H_kv, G, n_hg, c, ring, sc.k, sc.v);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, NH, RING, KVF, 1>), grid, dim3(kThreads), 0,
                           stream, (const uint16_t*)q, (const uint8_t*)k, (const uint8_t*)v, ws.m,
                           ws.l, ws.o, plan, T_q, H_q, H_kv, G, n_hg, c, ring, sc.k, sc.v);
}


template <bool RING, int KVF = kKvBf16>
static hipError_t split_dispatch(const void* q, const void* k, const void* v,
                                 const DecodeWorkspace& ws, const DecodePlanChunk& plan, int T_q,
                                 int H_q, int H_kv, int d, float scale, const RingArgs& ring,
                                 hipStream_t stream, const KvScales& sc = KvScales{}) {
    const int G = H_q / H_kv;
    // this kernel covers nh column blocks per work-group (not the wide kernel's count)
    const int nh = decode_column_blocks_per_group(T_q, G);
    const int n_hg = ((T_q * G + kCols - 1) / kCols + nh - 1) / nh;
    const int64_t grid = (int64_t)plan.units * n_hg * H_kv;
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (RING && (ring.sink < 0 || ring.capacity - ring.sink < 1 || ring.window < 1))
        return hipErrorInvalidValue;
    int min_len = plan.split_len[0];
    for (int i = 1; i < plan.nseq; ++i) min_len = std::min(min_len, (int)plan.split_len[i]);
    // (quantised caches keep one head per work-group: their rows are 64 or 128
    // bytes per head and the XCD-contiguous order already keeps a key range's
    // heads together; pairing measured 13-20% slower there)
    const int hp = (KVF == kKvBf16 && H_kv % 2 == 0 && min_len >= kPairMinSplitLen) ? 2 : 1;
    const float c = scale * kLog2e;
    const int64_t uh = (int64_t)plan.units * n_hg;
    if (KVF == kKvBf16 && decode_is_stream(T_q, G) &&
        (!RING || (int64_t)ring.capacity * H_kv * d * 2 < 0x7fff0000)) {
        // one KV head per work-group, K/V streamed into LDS (decode_stream_kernel)
        int max_len = 0;
        for (int i = 0; i < plan.nseq; ++i)
            max_len = std::max(max_len, std::min((int)plan.split_len[i], (int)plan.len[i]));
        const dim3 sgrid((unsigned)(plan.units * H_kv));
        const bool wide = T_q * G > kCols;          // two column blocks (always two slots)
        const bool two = wide || max_len > kStreamOneSlotKeys;
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, sgrid, dim3(kThreads), 0, stream, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v, plan.key_off[0], plan.nseq,
                               (int)plan.len[0], (int)plan.split_len[0], plan.seq0, T_q, H_q, H_kv,
                               G, ws.m, ws.l, ws.o, plan, c, ring);
        };
        if (d == 128) {
            if (wide) go(decode_stream_kernel<128, 2, RING, 2>);
            else if (two) go(decode_stream_kernel<128, 2, RING, 1>);
            else go(decode_stream_kernel<128, 1, RING, 1>);
        } else {
            if (wide) go(decode_stream_kernel<64, 2, RING, 2>);
            else if (two) go(decode_stream_kernel<64, 2, RING, 1>);
            else go(decode_stream_kernel<64, 1, RING, 1>);
        }
        return hipGetLastError();
    }
    if (d == 128 && nh == 1)
        launch_split<128, 1, RING, KVF>(hp, uh, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, sc, stream);
    else if (d == 128)
        launch_split<128, 2, RING, KVF>(hp, uh, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, sc, stream);
    else if (nh == 1)
        launch_split<64, 1, RING, KVF>(hp, uh, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, sc, stream);
    else
        launch_split<64, 2, RING, KVF>(hp, uh, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, sc, stream);
    return hipGetLastError();
}

hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v,
                                    const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                    int T_q, int H_q, int H_kv, int d, float scale,
                                    hipStream_t stream) {
    const int G = H_q / H_kv;
    if (decode_use_rows(T_q, G))
        return launch_decode_rows_bf16(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, stream);
    if (decode_use_wide(T_q, G)) {
        const float c = scale * kLog2e;
        const bool two = decode_wide_nhw(T_q, G) == 2;
        if (d == 128)
            return two ? launch_wide<128, 2>(q, k, v, ws, plan, T_q, H_q, H_kv, c, stream)
                       : launch_wide<128, 1>(q, k, v, ws, plan, T_q, H_q, H_kv, c, stream);
        return two ? launch_wide<64, 2>(q, k, v, ws, plan, T_q, H_q, H_kv, c, stream)
                   : launch_wide<64, 1>(q, k, v, ws, plan, T_q, H_q, H_kv, c, stream);
    }
    return split_dispatch<false>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, RingArgs{1, 0, 1},
                                 stream);
}

hipError_t launch_decode_quant_split(const void* q, const void* k, const void* v,
                                     const float* k_scale, const float* v_scale, int bits,
                                     const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                     int T_q, int H_q, int H_kv, int d, float scale,
                                     hipStream_t stream) {
    const KvScales sc{k_scale, v_scale};
    const RingArgs none{1, 0, 1};
    if (bits == 8)
        return split_dispatch<false, kKvInt8>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, none,
                                              stream, sc);
    if (bits == 4)
        return split_dispatch<false, kKvInt4>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, none,
                                              stream, sc);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_ring_split(const void* q, const void* k, const void* v,
                                    const float* k_scale, const float* v_scale, int bits,
                                    const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                    int T_q, int H_q, int H_kv, int d, float scale,
                                    const RingArgs& ring, hipStream_t stream) {
    const KvScales sc{k_scale, v_scale};
    if (bits == 16)
        return split_dispatch<true>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, ring, stream);
    if (bits == 8)
        return split_dispatch<true, kKvInt8>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, ring,
                                             stream, sc);
    if (bits == 4)
        return split_dispatch<true, kKvInt4>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, ring,
                                             stream, sc);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine_bf16(const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                      void* o, float* lse, int T_q, int H_q, int d,
                                      hipStream_t stream) {
    const int64_t grid = (int64_t)plan.nseq * T_q * H_q * (d / 32);   // one wave per item
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    int max_n = 1;
    for (int i = 0; i < plan.nseq; ++i)
        max_n = std::max(max_n, (int)(plan.unit_base[i + 1] - plan.unit_base[i]));
    const int64_t rows = (int64_t)plan.nseq * T_q * H_q;
    const int sg = 256 / d;   // split groups of the row-per-wave kernel
    if (rows >= kCombineRowsMin && max_n <= 4 * sg) {
        const int per = (max_n + sg - 1) / sg;
        const int nb = per <= 1 ? 1 : per <= 2 ? 2 : 4;
        const dim3 rgrid((unsigned)((rows + kCombineRowWaves - 1) / kCombineRowWaves));
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, rgrid, dim3(64 * kCombineRowWaves), 0, stream, ws.m, ws.l,
                               ws.o, (uint16_t*)o, lse, plan, T_q, H_q);
        };
        if (d == 128) {
            if (nb == 1) go(decode_combine_rows_kernel<128, 1>);
            else if (nb == 2) go(decode_combine_rows_kernel<128, 2>);
            else go(decode_combine_rows_kernel<128, 4>);
        } else {
            if (nb == 1) go(decode_combine_rows_kernel<64, 1>);
            else if (nb == 2) go(decode_combine_rows_kernel<64, 2>);
            else go(decode_combine_rows_kernel<64, 4>);
        }
        return hipGetLastError();
    }
    const int per_lane = (max_n + 7) / 8;   // splits of one lane group
    const int nb = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64), 0, stream, ws.m, ws.l, ws.o,
                           plan.nseq, plan.split_base, plan.units, plan.seq0, T_q, H_q,
                           (uint16_t*)o, lse, plan);
    };
    if (d == 128) {
        if (nb == 1) go(decode_combine_kernel<128, 1>);
        else if (nb == 2) go(decode_combine_kernel<128, 2>);
        else if (nb == 4) go(decode_combine_kernel<128, 4>);
        else go(decode_combine_kernel<128, 8>);
    } else {
        if (nb == 1) go(decode_combine_kernel<64, 1>);
        else if (nb == 2) go(decode_combine_kernel<64, 2>);
        else if (nb == 4) go(decode_combine_kernel<64, 4>);
        else go(decode_combine_kernel<64, 8>);
    }
    return hipGetLastError();
}

}  // namespace gqa
