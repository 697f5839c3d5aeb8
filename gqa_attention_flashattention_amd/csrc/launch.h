// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/gqa_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, T_q, S_kv, H_q, H_kv, d;
    float scale;
    int causal;
    int q_offset;
    int window = 0;   // > 0: causal with attention sinks + local window (bf16 kernel only)
    int sink = 0;
};

// Sequences described per decode launch (kernel-argument plan).
constexpr int kDecodeSeqPerLaunch = 64;

struct DecodePlanChunk {
    int nseq;                                // sequences in this launch
    int split_base;                          // global split index of this launch's first split
    int units;                               // sum of splits over this launch's sequences
    int64_t key_off[kDecodeSeqPerLaunch];    // first key row of each sequence
    int32_t len[kDecodeSeqPerLaunch];        // keys the kernel walks (kv_len; ring: resident visible keys)
    int32_t ntok[kDecodeSeqPerLaunch];       // ring cache only: tokens written so far
    int32_t split_len[kDecodeSeqPerLaunch];  // L_b
    int32_t unit_base[kDecodeSeqPerLaunch + 1];  // prefix of splits within the launch
    int32_t seq0;                            // batch index of the first sequence
};

struct DecodeWorkspace {
    float* m;   // [total_splits][H_q]
    float* l;   // [total_splits][H_q]
    float* o;   // [total_splits][H_q][d]
};


hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

// Row blocks (work-groups per batch entry and KV head) of the bf16 prefill
// kernel for T_q * G query rows.
int64_t prefill_row_blocks(int T_q, int G);

// KV-split prefill, step 1: partials of n_split key ranges per row block into
// ws (partial row ((b * n_split + split) * T_q + t) * H_q + h); step 2 is
// launch_decode_combine_bf16 with a chunk whose sequence sq owns splits
// sq * n_split .. sq * n_split + n_split - 1.
hipError_t launch_prefill_split_bf16(const PrefillArgs& a, int n_split, const DecodeWorkspace& ws,
                                     hipStream_t stream);

// Work-groups per (split, KV head) that the split kernel uses for T_q * G
// query rows (each covers up to 32 rows).
int decode_column_groups(int T_q, int G);

// Work-groups one split of split_len keys occupies, over all KV heads, for
// the kernel a decode entry point launches: packed bf16 cache (split or wide
// kernel), quantised cache, or ring cache.  Two such work-groups are
// resident per compute unit.
enum class DecodeKind { Bf16, Quant, QuantInt4, Ring };
int64_t decode_workgroups_per_split(DecodeKind kind, int T_q, int G, int H_kv, int split_len);
constexpr int kDecodeWorkgroupsPerCu = 2;

// T_q new tokens per sequence (1 for plain decode); partial and output rows are
// (sequence, token, query head).
hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v,
                                    const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                    int T_q, int H_q, int H_kv, int d, float scale,
                                    hipStream_t stream);

// Quantised cache (bits = 8 or 4): k, v packed [sum kv_len, H_kv, d] signed
// int8 codes, or int4 codes two per byte (even channel in the low nibble);
// k_scale, v_scale fp32 [H_kv, d]; the value is code * scale.
hipError_t launch_decode_quant_split(const void* q, const void* k, const void* v,
                                     const float* k_scale, const float* v_scale, int bits,
                                     const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                     int T_q, int H_q, int H_kv, int d, float scale,
                                     hipStream_t stream);

// Ring-buffer cache (capacity slots per sequence, key_off = b * capacity): the
// first `sink` positions stay in slots 0..sink-1, position j >= sink lives in
// slot sink + (j - sink) mod (capacity - sink).  The kernel walks plan.len[sq]
// keys: the resident sinks, then the window positions in order.
struct RingArgs {
    int capacity;
    int sink;
    int window;
};
// bits = 16: bf16 cache; 8 / 4: quantised codes as launch_decode_quant_split
// (k_scale, v_scale fp32 [H_kv, d]), [B, capacity, H_kv, d or d/2] bytes.
hipError_t launch_decode_ring_split(const void* q, const void* k, const void* v,
                                    const float* k_scale, const float* v_scale, int bits,
                                    const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                    int T_q, int H_q, int H_kv, int d, float scale,
                                    const RingArgs& ring, hipStream_t stream);
// Multi-token decode with at least kDecodeRowsMin query rows per KV head
// (T_q * G) over a packed bf16 cache: each (split, row block of 256 rows, KV
// head) runs the prefill kernel's tile loop (32x32 MFMAs, 64-key tiles) on
// the split's key range and writes partials like launch_decode_split_bf16.
constexpr int kDecodeRowsMin = 128;
// KV heads per work-group of that path: two when a head has at most 128 rows
// (and H_kv is even), so both wave groups of the work-group have rows.
int decode_rows_heads_per_workgroup(int T_q, int G, int H_kv);
hipError_t launch_decode_rows_bf16(const void* q, const void* k, const void* v,
                                   const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                   int T_q, int H_q, int H_kv, int d, float scale,
                                   hipStream_t stream);

hipError_t launch_decode_combine_bf16(const DecodeWorkspace& ws, const DecodePlanChunk& plan,
                                      void* o, float* lse, int T_q, int H_q, int d,
                                      hipStream_t stream);

}  // namespace gqa
