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
//  * Work-group = 4 waves x 32 query rows (128 rows), key tiles of 64.
//    blockIdx -> (kv head fastest, then batch, then row block); causal row
//    blocks are issued longest-first.  With 8 KV heads and 8 XCDs the
//    round-robin dispatch keeps each KV head's K/V in one XCD's L2.
//  * The MFMA computes S^T = K Q^T: A = K tile rows from LDS, B = Q^T held in
//    registers for the whole sweep.  In the 32x32 output layout each lane
//    then owns one query column, so the running max / sum / rescale are
//    lane-local (only lanes l and l^32 share a query), and the fp32 P values
//    of a lane are exactly the B operand of O^T = V^T P^T after packing to
//    bf16.  The K rows are loaded into the A operand in a permuted order
//    (bits 2 and 3 of the row index swapped) so that the 8 keys a lane
//    contributes to each P.V step are consecutive.
//  * K tiles are stored row-major in LDS (row padded by 16 B, conflict-free
//    b128 reads); V tiles are transposed on the way into LDS (V^T rows = head
//    dims) so the P.V A operand is one b128 read per lane.  LDS is double
//    buffered; the next tile's global loads are issued before the current
//    tile's math.
#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;   // 128 query rows per work-group
constexpr int kBlockN = 64;                      // keys per tile
constexpr int kThreads = kWaves * 64;

template <int D>
struct PrefillSmem {
    static constexpr int KS = D + 8;             // K row stride (elements)
    static constexpr int VS = kBlockN + 8;       // V^T row stride (elements)
    static constexpr int K_ELEMS = kBlockN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
};

// Row of the A operand that lane-row m loads: bits 2 and 3 swapped.
__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
struct TileRegs {
    static constexpr int K_CHUNKS = kBlockN * D / 8 / kThreads;    // 16-byte chunks per thread
    static constexpr int V_TOTAL = (kBlockN / 4) * (D / 8);  // items of 4 keys x 8 dims
    static constexpr int V_ITEMS = (V_TOTAL + kThreads - 1) / kThreads;
    u32x4 kc[K_CHUNKS];
    u32x4 vc[V_ITEMS][4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int64_t row_stride,
                                          int key0, int S_kv, int tid) {
    constexpr int CPR = D / 8;   // chunks per key row
#pragma unroll
    for (int i = 0; i < TileRegs<D>::K_CHUNKS; ++i) {
        int c = tid + i * kThreads;
        int key = c / CPR, dc = c % CPR;
        int kk = key0 + key;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (kk < S_kv) val = *(const u32x4*)(kbase + (int64_t)kk * row_stride + dc * 8);
        r.kc[i] = val;
    }
#pragma unroll
    for (int i = 0; i < TileRegs<D>::V_ITEMS; ++i) {
        int it = tid + i * kThreads;
        int dc = it % CPR, kq = it / CPR;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int kk = key0 + kq * 4 + e;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (it < TileRegs<D>::V_TOTAL && kk < S_kv) val = *(const u32x4*)(vbase + (int64_t)kk * row_stride + dc * 8);
            r.vc[i][e] = val;
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, uint16_t* __restrict__ buf,
                                           int tid) {
    using SM = PrefillSmem<D>;
    constexpr int CPR = D / 8;
    uint16_t* ks = buf;
    uint16_t* vt = buf + SM::K_ELEMS;
#pragma unroll
    for (int i = 0; i < TileRegs<D>::K_CHUNKS; ++i) {
        int c = tid + i * kThreads;
        int key = c / CPR, dc = c % CPR;
        *(u32x4*)(ks + key * SM::KS + dc * 8) = r.kc[i];
    }
#pragma unroll
    for (int i = 0; i < TileRegs<D>::V_ITEMS; ++i) {
        int it = tid + i * kThreads;
        if (it >= TileRegs<D>::V_TOTAL) break;
        int dc = it % CPR, kq = it / CPR;
#pragma unroll
        for (int p = 0; p < 4; ++p) {   // dim pair (2p, 2p+1) of this chunk
            uint32_t w0 = r.vc[i][0][p], w1 = r.vc[i][1][p];
            uint32_t w2 = r.vc[i][2][p], w3 = r.vc[i][3][p];
            u32x2 lo = {__builtin_amdgcn_perm(w1, w0, 0x05040100u),
                        __builtin_amdgcn_perm(w3, w2, 0x05040100u)};
            u32x2 hi = {__builtin_amdgcn_perm(w1, w0, 0x07060302u),
                        __builtin_amdgcn_perm(w3, w2, 0x07060302u)};
            *(u32x2*)(vt + (dc * 8 + 2 * p) * SM::VS + kq * 4) = lo;
            *(u32x2*)(vt + (dc * 8 + 2 * p + 1) * SM::VS + kq * 4) = hi;
        }
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int B,
    int T_q, int S_kv, int H_q, int H_kv, int G, float c, int q_offset, int n_mblk) {
    using SM = PrefillSmem<D>;
    constexpr int KSTEPS = D / 16;   // MFMA k-steps over the head dim
    constexpr int DBLK = D / 32;     // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SM::BUF_ELEMS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int hh = lane >> 5;

    int bid = blockIdx.x;
    const int kv = bid % H_kv;
    bid /= H_kv;
    const int b = bid % B;
    int mb = bid / B;
    if (CAUSAL) mb = n_mblk - 1 - mb;

    const int rows_total = T_q * G;
    const int r0 = mb * kBlockM;
    const int rw0 = r0 + wave * kRowsPerWave;          // first row of this wave
    const int row = rw0 + lq;
    const bool valid = row < rows_total;
    const int t = valid ? row / G : 0;
    const int g = valid ? row % G : 0;
    const int64_t qo_off = (((int64_t)b * T_q + t) * H_q + (int64_t)kv * G + g) * D;

    // Q^T operand, resident for the whole key sweep.
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (valid) val = *(const u32x4*)(q + qo_off + ks * 16 + hh * 8);
        qf[ks] = __builtin_bit_cast(bf16x8, val);
    }

    // Key range of the work-group and of this wave.
    const int t_lo = r0 / G;
    const int t_hi = min(T_q - 1, (r0 + kBlockM - 1) / G);
    const int kend = CAUSAL ? min(S_kv, q_offset + t_hi + 1) : S_kv;
    const int n_tiles = (kend + kBlockN - 1) / kBlockN;
    const bool wave_live = rw0 < rows_total;
    const int wt_lo = rw0 / G;
    const int wt_hi = min(T_q - 1, (rw0 + kRowsPerWave - 1) / G);
    const int wave_kend = CAUSAL ? min(S_kv, q_offset + wt_hi + 1) : S_kv;
    // keys [0, wave_full) are visible to every row of this wave
    const int wave_full = CAUSAL ? min(S_kv, q_offset + wt_lo + 1) : S_kv;
    const int pos = CAUSAL ? (valid ? q_offset + t : S_kv) : S_kv;   // last visible key + 1 - 1

    const int64_t row_stride = (int64_t)H_kv * D;
    const uint16_t* kbase = k + ((int64_t)b * S_kv * H_kv + kv) * D;
    const uint16_t* vbase = v + ((int64_t)b * S_kv * H_kv + kv) * D;

    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    TileRegs<D> regs;
    load_tile<D>(regs, kbase, vbase, row_stride, 0, S_kv, tid);
    store_tile<D>(regs, smem, tid);
    __syncthreads();

    const int arow0 = swap_bits23(lq);

    for (int j = 0; j < n_tiles; ++j) {
        const bool has_next = j + 1 < n_tiles;
        if (has_next) load_tile<D>(regs, kbase, vbase, row_stride, (j + 1) * kBlockN, S_kv, tid);

        const int key0 = j * kBlockN;
        if (wave_live && key0 < wave_kend) {
            const uint16_t* ks = smem + (j & 1) * SM::BUF_ELEMS;
            const uint16_t* vt = ks + SM::K_ELEMS;
            // ---- S^T = K Q^T (two 32-key blocks) ----
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{};
                const uint16_t* krow = ks + (kb * 32 + arow0) * SM::KS + hh * 8;
#pragma unroll
                for (int kst = 0; kst < KSTEPS; ++kst) {
                    bf16x8 a = *(const bf16x8*)(krow + kst * 16);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kst], s[kb], 0, 0, 0);
                }
            }
            // element i of s[kb] is key key0 + 32 kb + 16 (i / 8) + 8 hh + (i % 8)
            const bool need_mask = (key0 + kBlockN > wave_full);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        int key = key0 + kb * 32 + (i >> 3) * 16 + hh * 8 + (i & 7);
                        if (key > pos || key >= S_kv) s[kb][i] = -INFINITY;
                    }
            }
            // ---- online softmax (base 2) ----
            float mt = s[0][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[0][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[1][i]);
            mt = max_xor32(mt);
            const float m_new = fmaxf(m_run, mt);
            const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
            const float corr = fast_exp2(m_run * c - mc);
            float psum = 0.f;
            uint32_t pk[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    float p0 = fast_exp2(__builtin_fmaf(s[kb][i], c, -mc));
                    float p1 = fast_exp2(__builtin_fmaf(s[kb][i + 1], c, -mc));
                    psum += p0 + p1;
                    pk[kb][i >> 1] = pack_bf16x2(p0, p1);
                }
            l_run = l_run * corr + psum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
            // ---- O^T += V^T P^T, four 16-key steps ----
#pragma unroll
            for (int kst = 0; kst < 4; ++kst) {
                const int kb = kst >> 1, half = kst & 1;
                u32x4 pw = {pk[kb][half * 4 + 0], pk[kb][half * 4 + 1], pk[kb][half * 4 + 2],
                            pk[kb][half * 4 + 3]};
                bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int db = 0; db < DBLK; ++db) {
                    bf16x8 a = *(const bf16x8*)(vt + (db * 32 + lq) * SM::VS + kst * 16 + hh * 8);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
                }
            }
        }
        if (has_next) store_tile<D>(regs, smem + ((j + 1) & 1) * SM::BUF_ELEMS, tid);
        __syncthreads();
    }

    // ---- epilogue: O / l, LSE ----
    const float l_tot = sum_xor32(l_run);
    if (valid) {
        const float inv = 1.f / l_tot;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 w = {pack_bf16x2(oacc[db][4 * u] * inv, oacc[db][4 * u + 1] * inv),
                           pack_bf16x2(oacc[db][4 * u + 2] * inv, oacc[db][4 * u + 3] * inv)};
                *(u32x2*)(o + qo_off + db * 32 + u * 8 + hh * 4) = w;
            }
        if (lse != nullptr && hh == 0)
            lse[qo_off / D] = (m_run * c + fast_log2(l_tot)) * kLn2;
    }
}

}  // namespace

template <int D, bool CAUSAL>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
    const int rows_total = a.T_q * (a.H_q / a.H_kv);
    const int n_mblk = (rows_total + kBlockM - 1) / kBlockM;
    const int64_t grid = (int64_t)n_mblk * a.B * a.H_kv;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.B, a.T_q, a.S_kv, a.H_q, a.H_kv, a.H_q / a.H_kv, c,
                       a.q_offset, n_mblk);
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
    return a.causal ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
}

}  // namespace gqa
