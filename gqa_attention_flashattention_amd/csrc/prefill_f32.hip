// prefill_f32.hip -- fused GQA attention prefill in fp32 throughout (fp32
// storage, fp32 products and softmax state, no reduced-precision matrix
// instructions), gfx950 VALU.
//
// Same method as the bf16 kernel (ADR-0060 page, "AHBM GQA Fused Attention
// kernel (Llama3-70B)": GQA fold of section 5.2, per-tile online softmax of
// section 3, causal tile classes of section 5.4), kept deliberately simple:
// it serves small fp32 problems where exactness to ~1e-6 relative matters
// more than speed.  One thread owns one query row (t-major fold of the G
// query heads of a KV head); a work-group of 128 rows streams K/V tiles of
// 32 keys through LDS, every thread reading the same K/V element at a time
// (LDS broadcast).  Per tile: 32 scores, tile max, exp, running merge.
#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kRows = 128;     // query rows (threads) per work-group
constexpr int kTileN = 32;     // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int B, int T_q, int S_kv, int H_q, int H_kv,
    int G, float scale, int q_offset, int n_mblk) {
    __shared__ __attribute__((aligned(16))) float ks[kTileN][D];
    __shared__ __attribute__((aligned(16))) float vs[kTileN][D];

    const int tid = threadIdx.x;
    int bid = blockIdx.x;
    const int kv = bid % H_kv;
    bid /= H_kv;
    const int b = bid % B;
    int mb = bid / B;
    if (CAUSAL) mb = n_mblk - 1 - mb;

    const int rows_total = T_q * G;
    const int r0 = mb * kRows;
    const int row = r0 + tid;
    const bool valid = row < rows_total;
    const int t = valid ? row / G : 0;
    const int g = valid ? row % G : 0;
    const int64_t qo_off = (((int64_t)b * T_q + t) * H_q + (int64_t)kv * G + g) * D;
    const int pos = CAUSAL ? (valid ? q_offset + t : S_kv) : S_kv;

    float qr[D];
#pragma unroll
    for (int x = 0; x < D; x += 4) {
        float4 val = valid ? *(const float4*)(q + qo_off + x) : make_float4(0.f, 0.f, 0.f, 0.f);
        qr[x] = val.x;
        qr[x + 1] = val.y;
        qr[x + 2] = val.z;
        qr[x + 3] = val.w;
    }
    float acc[D];
#pragma unroll
    for (int x = 0; x < D; ++x) acc[x] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int t_hi = min(T_q - 1, (r0 + kRows - 1) / G);
    const int kend = CAUSAL ? min(S_kv, q_offset + t_hi + 1) : S_kv;
    const int64_t row_stride = (int64_t)H_kv * D;
    const float* kbase = k + ((int64_t)b * S_kv * H_kv + kv) * D;
    const float* vbase = v + ((int64_t)b * S_kv * H_kv + kv) * D;

    for (int key0 = 0; key0 < kend; key0 += kTileN) {
        // cooperative tile load: kTileN * D / 4 float4 per tensor
        for (int i = tid; i < kTileN * D / 4; i += kRows) {
            int kk = i / (D / 4), x = (i % (D / 4)) * 4;
            float4 kvv = make_float4(0.f, 0.f, 0.f, 0.f), vvv = kvv;
            if (key0 + kk < S_kv) {
                kvv = *(const float4*)(kbase + (int64_t)(key0 + kk) * row_stride + x);
                vvv = *(const float4*)(vbase + (int64_t)(key0 + kk) * row_stride + x);
            }
            *(float4*)&ks[kk][x] = kvv;
            *(float4*)&vs[kk][x] = vvv;
        }
        __syncthreads();
        float s[kTileN];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < kTileN; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int x = 0; x < D; ++x) dot = __builtin_fmaf(qr[x], ks[j][x], dot);
            const int key = key0 + j;
            s[j] = (key > pos || key >= S_kv) ? -INFINITY : dot * scale;
            mt = fmaxf(mt, s[j]);
        }
        const float m_new = fmaxf(m_run, mt);
        if (m_new != -INFINITY) {
            const float corr = expf(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int x = 0; x < D; ++x) acc[x] *= corr;
#pragma unroll
            for (int j = 0; j < kTileN; ++j) {
                const float p = expf(s[j] - m_new);
                l_run += p;
#pragma unroll
                for (int x = 0; x < D; ++x) acc[x] = __builtin_fmaf(p, vs[j][x], acc[x]);
            }
            m_run = m_new;
        }
        __syncthreads();
    }
    if (valid) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int x = 0; x < D; x += 4)
            *(float4*)(o + qo_off + x) =
                make_float4(acc[x] * inv, acc[x + 1] * inv, acc[x + 2] * inv, acc[x + 3] * inv);
        if (lse != nullptr) lse[qo_off / D] = m_run + logf(l_run);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
    const int G = a.H_q / a.H_kv;
    const int rows_total = a.T_q * G;
    const int n_mblk = (rows_total + kRows - 1) / kRows;
    const int64_t grid = (int64_t)n_mblk * a.B * a.H_kv;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kRows), 0,
                       stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (float*)a.o, a.lse, a.B, a.T_q, a.S_kv, a.H_q, a.H_kv, G, a.scale,
                       a.q_offset, n_mblk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
    return a.causal ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
}

}  // namespace gqa
