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
//  * K and V tiles are both stored row-major in LDS with 16-byte writes.  The
//    V^T operand is read with ds_read_b64_tr_b16 (each lane of a 16-lane group
//    receives one head-dim column of four key rows), so V is never transposed
//    in registers.  Row paddings make the b128 K reads and the transposed V
//    reads bank-conflict free.  LDS is double buffered; the next tile's global
//    loads are issued before the current tile's math.
//  * Lazy rescaling: the running max used for the exponentials is only moved
//    when some row's tile max exceeds it by more than 8 (log2 units), so most
//    tiles skip the O rescale; exact, since O and l always share the same
//    reference max and P stays below 2^8.
#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;   // 256 query rows per work-group
constexpr int kBlockN = 64;                      // keys per tile
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleThreshold = 8.f;         // log2 units

template <int D>
struct PrefillSmem {
    static constexpr int KS = D + 8;             // K row stride (elements): b128 reads conflict-free
    static constexpr int VS = D + 32;            // V row stride (elements): tr16 reads conflict-free
    static constexpr int K_ELEMS = kBlockN * KS;
    static constexpr int V_ELEMS = kBlockN * VS;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int CHUNKS = kBlockN * D / 8 / kThreads;   // 16-byte chunks per thread per tensor
};

// Row of the A operand that lane-row m loads: bits 2 and 3 swapped.
__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
}

template <int D>
struct TileRegs {
    u32x4 kc[PrefillSmem<D>::CHUNKS];
    u32x4 vc[PrefillSmem<D>::CHUNKS];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int64_t row_stride,
                                          int key0, int S_kv, int tid) {
    constexpr int CPR = D / 8;   // chunks per key row
#pragma unroll
    for (int i = 0; i < PrefillSmem<D>::CHUNKS; ++i) {
        const int c = tid + i * kThreads;
        const int kk = key0 + c / CPR;
        const int64_t off = (int64_t)kk * row_stride + (c % CPR) * 8;
        u32x4 kval = {0u, 0u, 0u, 0u}, vval = {0u, 0u, 0u, 0u};
        if (kk < S_kv) {
            kval = *(const u32x4*)(kbase + off);
            vval = *(const u32x4*)(vbase + off);
        }
        r.kc[i] = kval;
        r.vc[i] = vval;
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, uint16_t* __restrict__ buf,
                                           int tid) {
    using SM = PrefillSmem<D>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < SM::CHUNKS; ++i) {
        const int c = tid + i * kThreads;
        const int key = c / CPR, dc = c % CPR;
        *(u32x4*)(buf + key * SM::KS + dc * 8) = r.kc[i];
        *(u32x4*)(buf + SM::K_ELEMS + key * SM::VS + dc * 8) = r.vc[i];
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(
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
    const int t_hi = min(T_q - 1, (r0 + kBlockM - 1) / G);
    const int kend = CAUSAL ? min(S_kv, q_offset + t_hi + 1) : S_kv;
    const int n_tiles = (kend + kBlockN - 1) / kBlockN;
    const bool wave_live = rw0 < rows_total;
    const int wt_lo = rw0 / G;
    const int wt_hi = min(T_q - 1, (rw0 + kRowsPerWave - 1) / G);
    const int wave_kend = CAUSAL ? min(S_kv, q_offset + wt_hi + 1) : S_kv;
    // keys [0, wave_full) are visible to every row of this wave
    const int wave_full = CAUSAL ? min(S_kv, q_offset + wt_lo + 1) : S_kv;
    const int pos = CAUSAL ? (valid ? q_offset + t : S_kv) : S_kv;

    const int64_t row_stride = (int64_t)H_kv * D;
    const uint16_t* kbase = k + ((int64_t)b * S_kv * H_kv + kv) * D;
    const uint16_t* vbase = v + ((int64_t)b * S_kv * H_kv + kv) * D;

    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // reference max (raw score units) used by P
    float l_run = 0.f;

    TileRegs<D> regs;
    load_tile<D>(regs, kbase, vbase, row_stride, 0, S_kv, tid);
    store_tile<D>(regs, smem, tid);
    __syncthreads();

    // K operand rows and V^T transposed-read addresses (per lane, per buffer offset 0)
    const int krow_off = swap_bits23(lq) * SM::KS + hh * 8;
    // tr16 source lane L = lane % 16 of group (dh = (lane/16) % 2, hh): key row 8 hh + 4 t + L / 4,
    // columns 16 dh + 4 (L % 4) of each 32-dim block
    const int L16 = lane & 15;
    const int dh = (lane >> 4) & 1;
    const int vrow_off = (hh * 8 + (L16 >> 2)) * SM::VS + dh * 16 + (L16 & 3) * 4;

    for (int j = 0; j < n_tiles; ++j) {
        const bool has_next = j + 1 < n_tiles;
        if (has_next) load_tile<D>(regs, kbase, vbase, row_stride, (j + 1) * kBlockN, S_kv, tid);

        const int key0 = j * kBlockN;
        if (wave_live && key0 < wave_kend) {
            const uint16_t* ks = smem + (j & 1) * SM::BUF_ELEMS;
            const uint16_t* vs = ks + SM::K_ELEMS;
            // ---- S^T = K Q^T (two 32-key blocks) ----
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{};
                const uint16_t* krow = ks + kb * 32 * SM::KS + krow_off;
#pragma unroll
                for (int kst = 0; kst < KSTEPS; ++kst) {
                    bf16x8 a = *(const bf16x8*)(krow + kst * 16);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kst], s[kb], 0, 0, 0);
                }
            }
            // element i of s[kb] is key key0 + 32 kb + 16 (i / 8) + 8 hh + (i % 8)
            if (key0 + kBlockN > wave_full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + kb * 32 + (i >> 3) * 16 + hh * 8 + (i & 7);
                        if (key > pos || key >= S_kv) s[kb][i] = -INFINITY;
                    }
            }
            // ---- online softmax (base 2), lazy rescale ----
            float mt = fmaxf(s[0][0], s[1][0]);
#pragma unroll
            for (int i = 1; i < 16; ++i) mt = fmaxf(mt, fmaxf(s[0][i], s[1][i]));
            {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                           false, false);
                mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const bool grow = mt * c > m_run * c + kRescaleThreshold;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = fmaxf(m_run, mt);
                // 0 on the first tile; a row with no visible key so far keeps corr = 1
                const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * c);
                l_run *= corr;
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
                m_run = m_new;
            }
            const float mc = m_run * c;
            float psum = 0.f;
            uint32_t pk[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = fast_exp2(__builtin_fmaf(s[kb][i], c, -mc));
                    const float p1 = fast_exp2(__builtin_fmaf(s[kb][i + 1], c, -mc));
                    psum += p0 + p1;
                    pk[kb][i >> 1] = pack_bf16x2(p0, p1);
                }
            l_run += psum;
            // ---- O^T += V^T P^T, four 16-key steps ----
#pragma unroll
            for (int kst = 0; kst < 4; ++kst) {
                const int kb = kst >> 1, half = kst & 1;
                u32x4 pw = {pk[kb][half * 4 + 0], pk[kb][half * 4 + 1], pk[kb][half * 4 + 2],
                            pk[kb][half * 4 + 3]};
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
                const uint16_t* vp = vs + kst * 16 * SM::VS + vrow_off;
#pragma unroll
                for (int db = 0; db < DBLK; ++db) {
                    s16x4 lo = lds_read_tr16(vp + db * 32);
                    s16x4 hi = lds_read_tr16(vp + 4 * SM::VS + db * 32);
                    typedef __attribute__((ext_vector_type(8))) short s16x8;
                    s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a8), pb, oacc[db], 0, 0, 0);
                }
            }
        }
        if (has_next) store_tile<D>(regs, smem + ((j + 1) & 1) * SM::BUF_ELEMS, tid);
        __syncthreads();
    }

    // ---- epilogue: O / l, LSE ----
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                   false, false);
        l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (valid) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 w = {pack_bf16x2(oacc[db][4 * u] * inv, oacc[db][4 * u + 1] * inv),
                           pack_bf16x2(oacc[db][4 * u + 2] * inv, oacc[db][4 * u + 3] * inv)};
                *(u32x2*)(o + qo_off + db * 32 + u * 8 + hh * 4) = w;
            }
        if (lse != nullptr && hh == 0)
            lse[qo_off / D] = (m_run * c + fast_log2(l_run)) * kLn2;
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
