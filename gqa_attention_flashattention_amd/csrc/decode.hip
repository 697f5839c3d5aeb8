// decode.hip -- split-KV GQA decode (FlashDecoding) for gfx950: a split
// kernel writing unnormalised partials and a log-sum-exp combine kernel.
//
// Method (ADR-0060 page, "AHBM GQA Fused Attention kernel (Llama3-70B)"):
//  * Decode has one query token per sequence; the G query heads of a KV head
//    are folded into the matmul M dimension so each K/V tile is read once for
//    all of them (section 5.2).  There is no causal mask, only a bounds mask
//    on the ragged last tile of a split.
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
//    lane-local.  V rows are loaded with 16-byte coalesced loads and
//    transposed into a per-wave LDS tile (V^T), the A operand of
//    O^T = V^T P^T.  The next tile's loads are issued before the current
//    tile's math.  At the end the four wave partials are merged through LDS
//    and one partial per (split, query head) is written.
//  * Combine kernel: one wave per (sequence, query head); partials are read
//    in split order (fixed order, no atomics: bitwise reproducible).
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
    static constexpr int VS = kTile + 8;              // V^T row stride (elements)
    static constexpr int VT_ELEMS = D * VS;            // per wave
};

// Key (within a 32-key tile) that A-operand row m of 16-key block blk loads,
// chosen so that the 8 P values a lane holds are keys 8 * (lane / 16) + 0..7.
__device__ __forceinline__ int tile_key(int m, int blk) { return (m >> 2) * 8 + blk * 4 + (m & 3); }

template <int D>
struct WaveTile {
    static constexpr int KSTEPS = D / 32;     // MFMA k-steps over the head dim
    static constexpr int KPL = D / 16;        // V keys per lane (8 for D = 128, 4 for D = 64)
    u32x4 kf[2][KSTEPS];                      // K A operands, two 16-key blocks
    u32x4 vr[KPL];                            // V rows: KPL keys x 8 dims
};

template <int D>
__device__ __forceinline__ void load_wave_tile(WaveTile<D>& w, const uint16_t* __restrict__ kseq,
                                               const uint16_t* __restrict__ vseq,
                                               int64_t row_stride, int key0, int key_end,
                                               int lane) {
    const int m = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int kk = key0 + tile_key(m, blk);
#pragma unroll
        for (int s = 0; s < WaveTile<D>::KSTEPS; ++s) {
            u32x4 val = {0u, 0u, 0u, 0u};
            if (kk < key_end) val = *(const u32x4*)(kseq + (int64_t)kk * row_stride + s * 32 + g4 * 8);
            w.kf[blk][s] = val;
        }
    }
    constexpr int CPR = D / 8;                // 16-byte chunks per row
    const int dc = lane % CPR, kg = lane / CPR;
#pragma unroll
    for (int e = 0; e < WaveTile<D>::KPL; ++e) {
        const int kk = key0 + kg * WaveTile<D>::KPL + e;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (kk < key_end) val = *(const u32x4*)(vseq + (int64_t)kk * row_stride + dc * 8);
        w.vr[e] = val;
    }
}

// Transpose the lane's KPL keys x 8 dims into V^T[dim][key] in LDS.
template <int D>
__device__ __forceinline__ void store_vt(const WaveTile<D>& w, uint16_t* __restrict__ vt, int lane) {
    using SM = DecodeSmem<D>;
    constexpr int KPL = WaveTile<D>::KPL;
    constexpr int CPR = D / 8;
    const int dc = lane % CPR, kg = lane / CPR;
#pragma unroll
    for (int p = 0; p < 4; ++p) {            // dim pair (2p, 2p + 1)
        uint32_t lo[KPL / 2], hi[KPL / 2];
#pragma unroll
        for (int e = 0; e < KPL; e += 2) {
            lo[e / 2] = __builtin_amdgcn_perm(w.vr[e + 1][p], w.vr[e][p], 0x05040100u);
            hi[e / 2] = __builtin_amdgcn_perm(w.vr[e + 1][p], w.vr[e][p], 0x07060302u);
        }
        uint16_t* d0 = vt + (dc * 8 + 2 * p) * SM::VS + kg * KPL;
        uint16_t* d1 = d0 + SM::VS;
        if constexpr (KPL == 8) {
            *(u32x4*)d0 = u32x4{lo[0], lo[1], lo[2], lo[3]};
            *(u32x4*)d1 = u32x4{hi[0], hi[1], hi[2], hi[3]};
        } else {
            *(u32x2*)d0 = u32x2{lo[0], lo[1]};
            *(u32x2*)d1 = u32x2{hi[0], hi[1]};
        }
    }
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, const DecodePlanChunk plan, int H_q, int H_kv, int G, int n_hg,
    float c) {
    using SM = DecodeSmem<D>;
    constexpr int KSTEPS = WaveTile<D>::KSTEPS;
    constexpr int DBLK = D / 16;             // 16-row blocks of O^T
    constexpr int MERGE_FLOATS = kWaves * kCols * (D + 2);
    constexpr int VT_BYTES = kWaves * SM::VT_ELEMS * 2;
    constexpr int SMEM_BYTES = VT_BYTES > MERGE_FLOATS * 4 ? VT_BYTES : MERGE_FLOATS * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;               // query head within the 16-head block
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

    const int head = hg * kCols + col;       // head within the KV group
    const bool col_valid = head < G;
    const int hq = kv * G + (col_valid ? head : 0);

    // Q^T operand: column = query head, k-group g4 = 8 dims per k-step.
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (col_valid) val = *(const u32x4*)(q + ((int64_t)b * H_q + hq) * D + s * 32 + g4 * 8);
        qf[s] = __builtin_bit_cast(bf16x8, val);
    }

    const int64_t row_stride = (int64_t)H_kv * D;
    const uint16_t* kseq = k + (plan.key_off[sq] * H_kv + kv) * (int64_t)D;
    const uint16_t* vseq = v + (plan.key_off[sq] * H_kv + kv) * (int64_t)D;
    uint16_t* vt = (uint16_t*)smem + wave * SM::VT_ELEMS;

    f32x4 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

    const int n_tiles = (kend - kbeg + kTile - 1) / kTile;
    WaveTile<D> wt;
    int tt = wave;
    if (tt < n_tiles) load_wave_tile<D>(wt, kseq, vseq, row_stride, kbeg + tt * kTile, kend, lane);
    for (; tt < n_tiles; tt += kWaves) {
        const int key0 = kbeg + tt * kTile;
        // S^T for two 16-key blocks; element i of s[blk] is key key0 + 8 g4 + 4 blk + i
        f32x4 s[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, wt.kf[blk][ks]), qf[ks], s[blk], 0, 0, 0);
        }
        wave_lds_fence();                    // previous tile's V^T reads are done
        store_vt<D>(wt, vt, lane);
        const int nt = tt + kWaves;
        if (nt < n_tiles) load_wave_tile<D>(wt, kseq, vseq, row_stride, kbeg + nt * kTile, kend, lane);
        if (key0 + kTile > kend) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (key0 + 8 * g4 + 4 * blk + i >= kend) s[blk][i] = -INFINITY;
        }
        float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
        const float corr = fast_exp2(m_run * c - mc);
        float p[8];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[blk * 4 + i] = fast_exp2(__builtin_fmaf(s[blk][i], c, -mc));
        l_run = l_run * corr + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        m_run = m_new;
        u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                    pack_bf16x2(p[6], p[7])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        wave_lds_fence();                    // V^T of this tile is visible to the wave
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            oacc[db] *= corr;
            bf16x8 a = *(const bf16x8*)(vt + (db * 16 + col) * SM::VS + g4 * 8);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[db], 0, 0, 0);
        }
    }

    // ---- merge the four wave partials through LDS ----
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();                         // every wave is done with its V^T tile
    float* mrg = (float*)smem;
    float* mw_o = mrg + wave * kCols * (D + 2);     // [16][D] then m[16], l[16]
    float* mw_m = mw_o + kCols * D;
    float* mw_l = mw_m + kCols;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) mw_o[col * D + db * 16 + g4 * 4 + i] = oacc[db][i];
    if (g4 == 0) {
        mw_m[col] = m_run;
        mw_l[col] = l_run;
    }
    __syncthreads();
    const int64_t pidx = (int64_t)plan.split_base + unit;
    for (int e = tid; e < kCols * D; e += kThreads) {
        const int cc = e / D, x = e % D;
        if (hg * kCols + cc >= G) continue;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, mrg[w * kCols * (D + 2) + kCols * D + cc]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* base = mrg + w * kCols * (D + 2);
            const float mwv = base[kCols * D + cc];
            const float sc = (mwv == -INFINITY) ? 0.f : fast_exp2((mwv - mx) * c);
            acc += sc * base[cc * D + x];
            lsum += sc * base[kCols * D + kCols + cc];
        }
        const int64_t hrow = pidx * H_q + (int64_t)kv * G + hg * kCols + cc;
        ws_o[hrow * D + x] = acc;
        if (x == 0) {
            ws_m[hrow] = mx * c;             // base-2 units
            ws_l[hrow] = lsum;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, uint16_t* __restrict__ o, float* __restrict__ lse,
    const DecodePlanChunk plan, int H_q) {
    constexpr int VPL = D / 64;              // values per lane
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);     // (sequence, head) in this launch
    if (item >= plan.nseq * H_q) return;
    const int sq = item / H_q, h = item % H_q;
    const int n = plan.unit_base[sq + 1] - plan.unit_base[sq];
    const int64_t p0 = (int64_t)plan.split_base + plan.unit_base[sq];

    float mx = -INFINITY;
    for (int s = lane; s < n; s += 64) mx = fmaxf(mx, ws_m[(p0 + s) * H_q + h]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));

    float acc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc[i] = 0.f;
    float lsum = 0.f;
    for (int s = 0; s < n; ++s) {
        const int64_t hrow = (p0 + s) * H_q + h;
        const float w = fast_exp2(ws_m[hrow] - mx);
        lsum += w * ws_l[hrow];
        const float* src = ws_o + hrow * D + lane * VPL;
        if constexpr (VPL == 2) {
            float2 val = *(const float2*)src;
            acc[0] += w * val.x;
            acc[1] += w * val.y;
        } else {
            acc[0] += w * src[0];
        }
    }
    const float inv = 1.f / lsum;
    const int b = plan.seq0 + sq;
    uint16_t* dst = o + ((int64_t)b * H_q + h) * D + lane * VPL;
    if constexpr (VPL == 2) {
        *(uint32_t*)dst = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
        dst[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
    }
    if (lse != nullptr && lane == 0) lse[(int64_t)b * H_q + h] = (mx + fast_log2(lsum)) * kLn2;
}

}  // namespace

hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v,
                                    const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                    int H_q, int H_kv, int d, float scale, hipStream_t stream) {
    const int G = H_q / H_kv;
    const int n_hg = (G + kCols - 1) / kCols;
    const int64_t grid = (int64_t)plan.units * n_hg * H_kv;
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const float c = scale * kLog2e;
    if (d == 128)
        hipLaunchKernelGGL((decode_split_kernel<128>), dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           ws.m, ws.l, ws.o, plan, H_q, H_kv, G, n_hg, c);
    else
        hipLaunchKernelGGL((decode_split_kernel<64>), dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           ws.m, ws.l, ws.o, plan, H_q, H_kv, G, n_hg, c);
    return hipGetLastError();
}

hipError_t launch_decode_combine_bf16(const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                      void* o, float* lse, int H_q, int d, hipStream_t stream) {
    const int64_t items = (int64_t)plan.nseq * H_q;
    const int64_t grid = (items + 3) / 4;
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (d == 128)
        hipLaunchKernelGGL((decode_combine_kernel<128>), dim3((unsigned)grid), dim3(256), 0, stream,
                           ws.m, ws.l, ws.o, (uint16_t*)o, lse, plan, H_q);
    else
        hipLaunchKernelGGL((decode_combine_kernel<64>), dim3((unsigned)grid), dim3(256), 0, stream,
                           ws.m, ws.l, ws.o, (uint16_t*)o, lse, plan, H_q);
    return hipGetLastError();
}

}  // namespace gqa
