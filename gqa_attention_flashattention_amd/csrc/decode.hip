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

template <int D>
struct WaveTile {
    static constexpr int KSTEPS = D / 32;     // MFMA k-steps over the head dim
    static constexpr int KPL = D / 16;        // V rows per lane (8 for D = 128, 4 for D = 64)
    u32x4 kf[2][KSTEPS];                      // K A operands, two 16-key blocks
    u32x4 vr[KPL];                            // V chunks: KPL rows x 8 dims
};

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

template <int D, typename Map>
__device__ __forceinline__ void load_wave_tile(WaveTile<D>& w, const uint16_t* __restrict__ kseq,
                                               const uint16_t* __restrict__ vseq,
                                               int64_t row_stride, int key0, int key_end,
                                               int lane, const Map& row_of) {
    const int m = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int kk = row_of(min(key0 + tile_key(m, blk), key_end - 1));
#pragma unroll
        for (int s = 0; s < WaveTile<D>::KSTEPS; ++s)
            w.kf[blk][s] = *(const u32x4*)(kseq + (int64_t)kk * row_stride + s * 32 + g4 * 8);
    }
    constexpr int CPR = D / 8;                // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;             // rows per wave instruction
    const int dc = lane % CPR, kg = lane / CPR;
#pragma unroll
    for (int e = 0; e < WaveTile<D>::KPL; ++e) {
        const int kk = row_of(min(key0 + e * RPI + kg, key_end - 1));
        w.vr[e] = *(const u32x4*)(vseq + (int64_t)kk * row_stride + dc * 8);
    }
}

// V tile into the wave's LDS area, row-major (key rows, head dims contiguous).
template <int D>
__device__ __forceinline__ void store_v(const WaveTile<D>& w, uint16_t* __restrict__ vt, int lane) {
    using SM = DecodeSmem<D>;
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;
    const int dc = lane % CPR, kg = lane / CPR;
#pragma unroll
    for (int e = 0; e < WaveTile<D>::KPL; ++e)
        *(u32x4*)(vt + (e * RPI + kg) * SM::VS + dc * 8) = w.vr[e];
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// RING: keys come from a ring-buffer cache (see RowMap); each new token t at
// position n - T_q + t sees the sinks and the `window` newest positions up
// to its own, which in walk order is [0, s_end) and [wbeg_t, vend_t).
template <int D, int NH, bool RING>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, const DecodePlanChunk plan, int T_q, int H_q, int H_kv, int G,
    int n_hg, float c, RingArgs ring) {
    using SM = DecodeSmem<D>;
    constexpr int KSTEPS = WaveTile<D>::KSTEPS;
    constexpr int DBLK = D / 16;             // 16-row blocks of O^T
    constexpr int WSTRIDE = kCols * (D + 2);        // per wave: O [16][D], then m[16], l[16]
    __shared__ __attribute__((aligned(16))) uint16_t vtiles[kWaves * SM::VT_ELEMS];
    __shared__ __attribute__((aligned(16))) float mrg[kWaves * WSTRIDE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;               // MFMA column within a 16-column block
    const int g4 = lane >> 4;

    int bid = blockIdx.x;
    const int kv = bid % H_kv;
    bid /= H_kv;
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
    const int64_t row_stride = (int64_t)H_kv * D;
    const uint16_t* kseq = k + (plan.key_off[sq] * H_kv + kv) * (int64_t)D;
    const uint16_t* vseq = v + (plan.key_off[sq] * H_kv + kv) * (int64_t)D;
    const int n_tiles = (kend - kbeg + kTile - 1) / kTile;
    // the first tile's K/V loads go out before anything else
    WaveTile<D> wt;
    int tt = wave;
    auto load = [&](int key0) {
        if (RING) load_wave_tile<D>(wt, kseq, vseq, row_stride, key0, kend, lane, rmap);
        else load_wave_tile<D>(wt, kseq, vseq, row_stride, key0, kend, lane, Identity{});
    };
    if (tt < n_tiles) load(kbeg + tt * kTile);

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
        // Q^T operand: column = query row, k-group g4 = 8 dims per k-step.
        const uint16_t* qrow = q + (((int64_t)b * T_q + tq) * H_q + hq) * D + g4 * 8;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            qf[h][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + s * 32));
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
    }

    for (; tt < n_tiles; tt += kWaves) {
        const int key0 = kbeg + tt * kTile;
        // S^T for two 16-key blocks; element i of s[h][blk] is key key0 + g4 + 16 blk + 4 i
        f32x4 s[NH][2];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                s[h][blk] = f32x4{};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    s[h][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wt.kf[blk][ks]), qf[h][ks], s[h][blk], 0, 0, 0);
            }
        wave_lds_fence();                    // previous tile's V reads are done
        store_v<D>(wt, vt, lane);
        const int nt = tt + kWaves;
        if (nt < n_tiles) load(kbeg + nt * kTile);
        if (key0 + kTile > mask_from || (RING && key0 + kTile > s_end && key0 < wbeg_max)) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key0 + g4 + 16 * blk + 4 * i;
                        bool hide = key >= vis_end[h];
                        if (RING) hide = hide || (key >= s_end && key < wbeg[h]);
                        if (hide) s[h][blk][i] = -INFINITY;
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
    }

    // ---- merge the four wave partials through LDS, one column block at a time ----
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
#pragma unroll
        for (int db = 0; db < DBLK; ++db) *(f32x4*)(mw_o + col * D + db * 16 + g4 * 4) = oacc[h][db];
        if (g4 == 0) {
            mw_o[kCols * D + col] = m_run[h];
            mw_o[kCols * D + kCols + col] = lr;
        }
        __syncthreads();
        for (int e = tid; e < kCols * (D / 4); e += kThreads) {
            const int cc = e / (D / 4), x = (e % (D / 4)) * 4;
            const int fo = fbase + cc;
            if (fo >= ncols) continue;
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, mrg[w * WSTRIDE + kCols * D + cc]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float lsum = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float* base = mrg + w * WSTRIDE;
                const float mwv = base[kCols * D + cc];
                const float sc = (mwv == -INFINITY) ? 0.f : fast_exp2((mwv - mx) * c);
                acc += sc * *(const f32x4*)(base + cc * D + x);
                lsum += sc * base[kCols * D + kCols + cc];
            }
            // partial row: (split, new token, query head)
            const int64_t hrow = (pidx * T_q + fo / G) * H_q + (int64_t)kv * G + fo % G;
            *(f32x4*)(ws_o + hrow * D + x) = acc;
            if (x == 0) {
                ws_m[hrow] = mx * c;             // base-2 units
                ws_l[hrow] = lsum;
            }
        }
    }
}

// One wave per (sequence, query head, 32-dim chunk of O).  Lane (sg, dq):
// split group sg = lane / 8 takes splits sg, sg + 8, sg + 16, ...; dim quad
// dq = lane % 8 owns dims 4 dq .. 4 dq + 3 of the chunk.  A lane loads a
// batch of its splits at once and folds them into a running (m, l, O) with
// the section 4 merge; the eight split groups are then merged with a fixed
// butterfly, so the result does not depend on timing (bitwise reproducible
// for a given split plan).  All in base 2.
constexpr int kCombineBatch = 8;

__device__ __forceinline__ void merge_lse(float& m, float& l, f32x4& o, float m2, float l2,
                                          const f32x4& o2) {
    const float mm = fmaxf(m, m2);
    const float w1 = (m == -INFINITY) ? 0.f : fast_exp2(m - mm);
    const float w2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mm);
    l = l * w1 + l2 * w2;
    o = o * w1 + o2 * w2;
    m = mm;
}

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, uint16_t* __restrict__ o, float* __restrict__ lse,
    const DecodePlanChunk plan, int T_q, int H_q) {
    constexpr int CHUNKS = D / 32;
    const int R = T_q * H_q;                                   // rows per sequence
    const int lane = threadIdx.x;
    const int item = blockIdx.x;   // (sequence, head, chunk)
    if (item >= plan.nseq * R * CHUNKS) return;
    const int chunk = item % CHUNKS;
    const int sh = item / CHUNKS;
    const int sq = sh / R, r = sh % R;                         // r = t * H_q + h
    const int n = plan.unit_base[sq + 1] - plan.unit_base[sq];
    const int64_t p0 = (int64_t)plan.split_base + plan.unit_base[sq];

    const int sg = lane >> 3, dq = lane & 7;
    const int dim = chunk * 32 + dq * 4;
    float m = -INFINITY, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = sg; s0 < n; s0 += 8 * kCombineBatch) {
        float mv[kCombineBatch], lv[kCombineBatch];
        f32x4 ov[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int s = s0 + 8 * u;
            const int64_t hrow = (p0 + (s < n ? s : 0)) * R + r;
            mv[u] = s < n ? ws_m[hrow] : -INFINITY;
            lv[u] = s < n ? ws_l[hrow] : 0.f;
            ov[u] = *(const f32x4*)(ws_o + hrow * D + dim);
            if (s >= n) ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) merge_lse(m, l, acc, mv[u], lv[u], ov[u]);
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
    const int b = plan.seq0 + sq;
    if (sg == 0) {
        u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *(u32x2*)(o + ((int64_t)b * R + r) * D + dim) = w;
    }
    if (lse != nullptr && chunk == 0 && lane == 0)
        lse[(int64_t)b * R + r] = (m + fast_log2(l)) * kLn2;
}

}  // namespace

int decode_column_blocks_per_group(int T_q, int G) { return T_q * G > kCols ? 2 : 1; }

int decode_column_groups(int T_q, int G) {
    const int blocks = (T_q * G + kCols - 1) / kCols;
    const int nh = decode_column_blocks_per_group(T_q, G);
    return (blocks + nh - 1) / nh;
}

template <int D, int NH, bool RING>
static void launch_split(dim3 grid, const void* q, const void* k, const void* v,
                         const DecodeWorkspace& ws, const DecodePlanChunk& plan, int T_q, int H_q,
                         int H_kv, int G, int n_hg, float c, const RingArgs& ring,
                         hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<D, NH, RING>), grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, ws.m, ws.l,
                       ws.o, plan, T_q, H_q, H_kv, G, n_hg, c, ring);
}

template <bool RING>
static hipError_t split_dispatch(const void* q, const void* k, const void* v,
                                 const DecodeWorkspace& ws, const DecodePlanChunk& plan, int T_q,
                                 int H_q, int H_kv, int d, float scale, const RingArgs& ring,
                                 hipStream_t stream) {
    const int G = H_q / H_kv;
    const int n_hg = decode_column_groups(T_q, G);
    const int nh = decode_column_blocks_per_group(T_q, G);
    const int64_t grid = (int64_t)plan.units * n_hg * H_kv;
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (RING && (ring.sink < 0 || ring.capacity - ring.sink < 1 || ring.window < 1))
        return hipErrorInvalidValue;
    const float c = scale * kLog2e;
    const dim3 g((unsigned)grid);
    if (d == 128 && nh == 1)
        launch_split<128, 1, RING>(g, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, stream);
    else if (d == 128)
        launch_split<128, 2, RING>(g, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, stream);
    else if (nh == 1)
        launch_split<64, 1, RING>(g, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, stream);
    else
        launch_split<64, 2, RING>(g, q, k, v, ws, plan, T_q, H_q, H_kv, G, n_hg, c, ring, stream);
    return hipGetLastError();
}

hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v,
                                    const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                    int T_q, int H_q, int H_kv, int d, float scale,
                                    hipStream_t stream) {
    return split_dispatch<false>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, RingArgs{1, 0, 1},
                                 stream);
}

hipError_t launch_decode_ring_split_bf16(const void* q, const void* k, const void* v,
                                         const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                         int T_q, int H_q, int H_kv, int d, float scale,
                                         const RingArgs& ring, hipStream_t stream) {
    return split_dispatch<true>(q, k, v, ws, plan, T_q, H_q, H_kv, d, scale, ring, stream);
}

hipError_t launch_decode_combine_bf16(const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                      void* o, float* lse, int T_q, int H_q, int d,
                                      hipStream_t stream) {
    const int64_t grid = (int64_t)plan.nseq * T_q * H_q * (d / 32);   // one wave per item
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (d == 128)
        hipLaunchKernelGGL((decode_combine_kernel<128>), dim3((unsigned)grid), dim3(64), 0, stream,
                           ws.m, ws.l, ws.o, (uint16_t*)o, lse, plan, T_q, H_q);
    else
        hipLaunchKernelGGL((decode_combine_kernel<64>), dim3((unsigned)grid), dim3(64), 0, stream,
                           ws.m, ws.l, ws.o, (uint16_t*)o, lse, plan, T_q, H_q);
    return hipGetLastError();
}

}  // namespace gqa
