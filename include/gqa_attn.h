/*
 * gqa_attn.h -- C ABI of libgqa_attn.so: grouped-query fused attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (ADR-0060 page, "AHBM GQA Fused Attention kernel
 * (Llama3-70B)"): every KV head serves G = H_q / H_kv query heads, query
 * head h reading KV head h / G (TL;DR pseudocode and section 5.2: the G
 * query heads are folded into the M dimension of both matrix products, K and
 * V are never broadcast).  Per query row the result is
 *     O = softmax(scale * q K^T + mask) V,   LSE = ln sum_j exp(scale * q.k_j)
 * over the keys the row may see, computed FlashAttention-style: K/V tiles
 * are streamed, an online softmax keeps a running max m, running sum l and
 * running output O (section 3, per-tile op sequence) and the score matrix is
 * never stored.  Causal prefill skips key tiles that lie wholly in the future
 * and masks only boundary tiles (section 5.4).  Decode splits each sequence's
 * keys across work-groups, each returning an unnormalised partial (m, l, O),
 * and a log-sum-exp merge reduces them (section 4, FlashDecoding).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers (HIP global memory) unless marked
 *    HOST.  All tensors are dense, row-major, with no padding.  The caller
 *    allocates and owns every buffer passed in; the library never frees or
 *    retains them after the call returns.  q, k, v are only read.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued on it and the call returns without synchronising; outputs are
 *    valid once the stream has reached that point.
 *  - Return value: GQA_OK (0) or a gqa_status code.  Argument errors are
 *    detected on the host before anything is enqueued, so a failed call has
 *    no effect on device memory.  No entry point aborts, throws or prints.
 *  - dtype: GQA_BF16 (storage bf16, fp32 accumulation and softmax state) or
 *    GQA_F32 (fp32 storage and arithmetic throughout, no reduced-precision
 *    matrix instructions).  Head dim d must be 64 or 128.
 *  - Threads.  Entry points that take only caller-owned buffers
 *    (gqa_attn_prefill, gqa_attn_prefill_window, gqa_attn_decode_split,
 *    gqa_attn_decode_combine and the host-only queries) may be called from
 *    any number of host threads at once.  The others (gqa_attn_decode,
 *    _multi, _quant, _ring, _ring_quant and the KV-parallel prefills) share
 *    one library-owned workspace per device and process.  Each such call
 *    holds a lock on it from the moment it takes the buffer until its last
 *    kernel is queued, so calls from several host threads on ONE stream of
 *    a device are safe: a call that has to grow the buffer allocates a new
 *    one (at least twice the size) and keeps the old one allocated for the
 *    kernels already queued against it.  Such calls on
 *    DIFFERENT streams of one device may run their kernels at the same time
 *    and overwrite each other's partials: serialise them (e.g. with events)
 *    or use gqa_attn_decode_split / gqa_attn_decode_combine with a
 *    caller-owned workspace per stream.
 *  - HIP graphs: every entry point enqueues only kernel launches (no
 *    memset, copy or host synchronisation), so a call may be captured.  The
 *    library-owned workspace (gqa_attn_decode, _multi, _quant, _ring,
 *    _ring_quant and the KV-parallel prefills) grows on demand: a call that
 *    needs more than it holds calls hipMalloc (which a capture may refuse),
 *    never waits for the device and frees nothing, so graphs captured
 *    earlier keep a valid buffer until gqa_attn_release_workspace.  Make the
 *    largest such call once before capturing, or capture
 *    gqa_attn_decode_split / gqa_attn_decode_combine with a caller-owned
 *    workspace, or gqa_attn_decode_noalloc.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_OK = 0,
    GQA_ERR_NULL = 1,        /* a required pointer is NULL */
    GQA_ERR_SHAPE = 2,       /* sizes < 1, H_q % H_kv != 0, kv_len[b] < 1, too large */
    GQA_ERR_UNSUPPORTED = 3, /* head dim / dtype combination not built */
    GQA_ERR_RANGE = 4,       /* causal q_offset out of range, workspace too small */
    GQA_ERR_HIP = 5          /* the HIP runtime reported an error (launch, alloc) */
} gqa_status;

typedef enum { GQA_BF16 = 0, GQA_F32 = 1 } gqa_dtype;

/* Human-readable text for a gqa_status value (static storage, never NULL). */
const char *gqa_attn_status_string(int status);

/* Library version as an integer MAJOR*10000 + MINOR*100 + PATCH. */
int gqa_attn_version(void);

/*
 * Prefill / chunked prefill (ADR-0060 sections 3, 5.4).
 *   q   [B, T_q, H_q, d]     o [B, T_q, H_q, d]        (dtype)
 *   k,v [B, S_kv, H_kv, d]                              (dtype)
 *   lse [B, T_q, H_q] fp32, natural log of sum_j exp(scale q.k_j); may be NULL.
 * causal != 0: the query at row t sits at absolute position q_offset + t and
 * sees key j iff j <= q_offset + t (diagonal included; requires
 * 0 <= q_offset and q_offset + T_q <= S_kv).  causal == 0: every query sees
 * all S_kv keys and q_offset is ignored.  `scale` multiplies q.k before the
 * softmax (1/sqrt(d) for standard attention).
 * Errors: GQA_ERR_NULL (q, k, v or o NULL), GQA_ERR_SHAPE (also for
 * H_q * d * 514 > 2^31 - 1: a work-group addresses its Q rows with 32-bit
 * byte offsets), GQA_ERR_UNSUPPORTED, GQA_ERR_RANGE (bad q_offset),
 * GQA_ERR_HIP.
 */
int gqa_attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int T_q, int S_kv, int H_q, int H_kv, int d, float scale,
                     int causal, int q_offset, int dtype, void *stream);

/*
 * KV-parallel prefill (ADR-0060 section 5.5, sequence-parallel prefill, on one
 * GPU): same operation, arguments and layouts as gqa_attn_prefill (bf16 only),
 * but the key tiles that each block of query rows sees are cut into
 * `n` contiguous ranges processed by separate work-groups; each writes the
 * unnormalised partial (m, l, O) of its rows and the log-sum-exp merge of
 * section 4 (the decode combine kernel) produces O and LSE.  This raises the
 * number of work-groups when B * H_kv * row blocks is small (short chunks over
 * long caches).  num_splits > 0 asks for that many ranges, num_splits <= 0 lets
 * the library choose: with one work-group resident per compute unit, the n in
 * [1, min(64, T / 4)] (T = 64-key tiles of the longest row block) minimising
 * ceil(blocks * n / CUs) * (ceil(T / n) + 4), ties to the smaller n.  n is
 * then clamped to [1, 64], to T and so that the partials fit in 4 GiB.  n == 1 runs gqa_attn_prefill's kernel.
 * Uses the library-owned workspace of gqa_attn_decode (same concurrency rule),
 * n * B * T_q * H_q * (d + 2) * 4 bytes.
 * Errors: as gqa_attn_prefill; GQA_ERR_UNSUPPORTED for dtype != GQA_BF16.
 */
int gqa_attn_prefill_kvsplit(const void *q, const void *k, const void *v, void *o, float *lse,
                             int B, int T_q, int S_kv, int H_q, int H_kv, int d, float scale,
                             int causal, int q_offset, int num_splits, int dtype, void *stream);

/*
 * Causal prefill with attention sinks and a local window (the sink +
 * local-window policy of the hard-cap ring-buffer KV cache, pccx page "Gemma
 * 3N E4B on pccx v002 -- Execution / Scheduling", section 4; ADR-0060 section
 * 5.4 tile classes extended to it): the query at position p = q_offset + t
 * sees key j iff j <= p and (j < sink or j > p - window).  Arguments and
 * layouts as gqa_attn_prefill with causal = 1 (bf16 only).  Key tiles that
 * no row of a block sees (between the sink tiles and the block's window) are
 * never loaded.  Requires window >= 1 and sink >= 0 (sink >= S_kv means every
 * earlier key is a sink, i.e. plain causal).
 * Errors: as gqa_attn_prefill; GQA_ERR_RANGE for window < 1 or sink < 0;
 * GQA_ERR_UNSUPPORTED for dtype != GQA_BF16.
 */
int gqa_attn_prefill_window(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int T_q, int S_kv, int H_q, int H_kv, int d, float scale,
                            int q_offset, int window, int sink, int dtype, void *stream);

/*
 * KV-parallel form of gqa_attn_prefill_window (the two prefill variants
 * above combined): the sink + window tiles each row block sees are cut into
 * n contiguous ranges on separate work-groups and merged by the log-sum-exp
 * combine, as gqa_attn_prefill_kvsplit; for short chunks under long windows.
 * num_splits > 0 asks for that many ranges; num_splits <= 0 lets the library
 * choose by gqa_attn_prefill_kvsplit's rule with T = the sink tiles plus the
 * window tiles of a row block.  Arguments, layouts, requirements and errors
 * as gqa_attn_prefill_window; workspace as gqa_attn_prefill_kvsplit.
 */
int gqa_attn_prefill_window_kvsplit(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int T_q, int S_kv, int H_q, int H_kv,
                                    int d, float scale, int q_offset, int window, int sink,
                                    int num_splits, int dtype, void *stream);

/*
 * Host only: the number of key ranges n that gqa_attn_prefill_kvsplit uses for
 * these arguments (>= 1), or minus a gqa_status code for invalid sizes.
 */
int gqa_attn_prefill_kvsplit_count(int B, int T_q, int S_kv, int H_q, int H_kv, int d,
                                   int causal, int q_offset, int num_splits);

/*
 * Decode, one new token per sequence (ADR-0060 sections 4, 5.2, 5.3).
 *   q   [B, H_q, d]            o [B, H_q, d]            (dtype)
 *   k,v [sum_b kv_len[b], H_kv, d], sequences packed back to back: sequence b
 *       occupies rows off_b .. off_b + kv_len[b] - 1, off_b = sum_{b'<b} kv_len[b'].
 *   kv_len: HOST array [B] of int32, every entry >= 1.
 * Each query attends to all keys of its sequence (no mask).  The keys of each
 * (sequence, KV head) are cut into contiguous splits as gqa_attn_decode_plan
 * describes: num_splits > 0 caps the splits per sequence at that number,
 * num_splits <= 0 lets the library choose.  Launches the
 * split kernel then the combine kernel on `stream`, using a workspace that the
 * library allocates on first use per device and grows on demand (a hipMalloc
 * may therefore happen inside this call, never a device synchronisation or a
 * free; use gqa_attn_decode_split/_combine with a caller-owned workspace, or
 * gqa_attn_decode_noalloc, to avoid the allocation).
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED, GQA_ERR_HIP.
 */
int gqa_attn_decode(const void *q, const void *k, const void *v, void *o, int B, int H_q,
                    int H_kv, int d, const int32_t *kv_len, float scale, int num_splits,
                    int dtype, void *stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same operation, arguments, layouts, split plan and
 * result as gqa_attn_decode (the same kernels; results are bitwise those of
 * gqa_attn_decode with the same arguments), but the split partials go to a
 * fixed scratch array inside the library, GQA_ATTN_NOALLOC_SCRATCH_BYTES per
 * device, held by every device the library runs on until the process ends.
 * The call makes no hipMalloc / hipFree and no allocating library call; the
 * first call on a device looks up that device's scratch address
 * (hipGetSymbolAddress), so make one call per device before capturing.
 * The plan's partials, total_splits * H_q * (d + 2) * 4 bytes (see
 * gqa_attn_decode_plan), must fit in the scratch: larger requests return
 * GQA_ERR_RANGE before anything is enqueued (e.g. 64 query heads at d = 128
 * allow 504 splits in total; pass num_splits to stay below).
 * Every call on a device shares that device's scratch: calls whose kernels
 * may overlap (different streams, or several host threads without ordering
 * between their streams) race on it and must be serialised by the caller.
 * Errors: as gqa_attn_decode, plus GQA_ERR_RANGE (scratch too small).
 */
#define GQA_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
/*
 * Workspace housekeeping, for callers that want the device memory of the
 * library-owned workspace back (long-running servers after a burst of long
 * sequences): waits for the current device (hipDeviceSynchronize), then
 * frees the current workspace buffer and every buffer retired by growth.
 * The next call that needs a workspace allocates a new one.  Graphs captured
 * from calls that used the freed buffers must not be replayed afterwards.
 * Errors: GQA_ERR_HIP.
 */
int gqa_attn_release_workspace(void);
int gqa_attn_decode_noalloc(const void *q, const void *k, const void *v, void *o, int B,
                            int H_q, int H_kv, int d, const int32_t *kv_len, float scale,
                            int num_splits, int dtype, void *stream);

/*
 * Split plan (host only, no device access).  Sequence b is cut into
 * n_b = ceil(kv_len[b] / L_b) splits of L_b keys (the last may be shorter),
 * split s covering keys [s*L_b, min((s+1)*L_b, kv_len[b])):
 *   num_splits > 0:  L_b = ceil(kv_len[b] / min(num_splits, kv_len[b])), so
 *                    n_b <= num_splits (fewer when the division rounds up);
 *   num_splits <= 0: L_b = L for all b, a multiple of 64 between 128 and
 *                    8192.  For B <= 256 (bf16 and ring caches, and int4
 *                    codes in gqa_attn_decode_quant / _ring_quant) L is the
 *                    multiple of 64 (up to 1024), of 128 (up to 2048) or of
 *                    256 (beyond) that minimises
 *                    ceil(W / R) * (L + 256) summed over the launches of 64
 *                    sequences, plus 8 * max_b n_b, W being the split
 *                    work-groups of a launch and R the number resident at
 *                    once (two per compute unit).  A bf16 or ring cache
 *                    with at most 32 query rows per KV head (G * T_q <= 32)
 *                    takes one work-group per (split, KV head), which counts
 *                    twice above 128 keys or above 16 rows (it holds the LDS
 *                    of two); a
 *                    bf16 packed cache with at least 128 query rows per KV
 *                    head (G * T_q >= 128, gqa_attn_decode_multi) takes one
 *                    work-group per (split, block of 256 rows, KV head),
 *                    counted twice; other cases pair KV heads from 512
 *                    keys on.  Otherwise W is
 *                    about four per compute unit.  A positive integer in the
 *                    environment variable GQA_ATTN_SPLIT_LEN (read once per
 *                    process) replaces the automatic L for every decode entry
 *                    point (a tuning and measurement override).  The plan
 *                    of the device current at the call.
 * Writes (every output pointer may be NULL):
 *   splits[b]        n_b (HOST array [B]),
 *   *split_len       L_b of the longest split over all sequences,
 *   *total_splits    sum_b n_b,
 *   *max_splits      max_b n_b,
 *   *workspace_bytes total_splits * H_q * (d + 2) * 4, the partials workspace
 *                    gqa_attn_decode_split needs.
 * Errors: GQA_ERR_NULL (kv_len NULL), GQA_ERR_SHAPE.
 */
int gqa_attn_decode_plan(int B, int H_q, int H_kv, int d, const int32_t *kv_len,
                         int num_splits, int32_t *splits, int *split_len,
                         int64_t *total_splits, int *max_splits, size_t *workspace_bytes);

/*
 * Decode step 1 of 2 (FlashDecoding split, ADR-0060 section 5.3): for every
 * (sequence b, KV head, split) writes the unnormalised partial of its G query
 * heads into `workspace` (device, fp32, at least workspace_bytes of
 * gqa_attn_decode_plan for the same arguments, 256-byte aligned):
 *   m [total_splits][H_q], l [total_splits][H_q], O [total_splits][H_q][d]
 * where split p = (sum_{b'<b} n_b') + s runs over sequences in order and
 * splits in key order (gqa_attn_decode_plan gives n_b);
 * m is the running max of scale * q.k in base-2 units (scores multiplied by
 * log2(e)), l = sum 2^(s2 - m), O = sum 2^(s2 - m) v.
 * Errors: as gqa_attn_decode, plus GQA_ERR_RANGE if workspace_bytes is too small.
 */
int gqa_attn_decode_split(const void *q, const void *k, const void *v, void *workspace,
                          size_t workspace_bytes, int B, int H_q, int H_kv, int d,
                          const int32_t *kv_len, float scale, int num_splits, int dtype,
                          void *stream);

/*
 * Decode step 2 of 2 (log-sum-exp combine, ADR-0060 section 4 merge): for
 * every (b, query head) merges the partials of its splits, in split order,
 * normalises once and writes o [B, H_q, d] (dtype) and, if lse != NULL,
 * lse [B, H_q] fp32 (natural log).  `workspace` must hold what
 * gqa_attn_decode_split wrote for the same B, H_q, H_kv, d, kv_len, num_splits.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED, GQA_ERR_RANGE,
 * GQA_ERR_HIP.
 */
int gqa_attn_decode_combine(const void *workspace, size_t workspace_bytes, void *o,
                            float *lse, int B, int H_q, int H_kv, int d,
                            const int32_t *kv_len, int num_splits, int dtype, void *stream);

/*
 * Multi-token decode (speculative verification, batched new tokens): T_q new
 * tokens per sequence whose K/V rows are already the last T_q rows of the
 * sequence in the cache.  The G query heads times the T_q tokens of a KV head
 * are folded into the matmul M dimension (ADR-0060 section 5.2: G * T_q rows
 * per KV tile), keys are split across work-groups and merged as in
 * gqa_attn_decode.  New token t of sequence b sits at position
 * kv_len[b] - T_q + t and attends to keys 0 .. kv_len[b] - T_q + t (causal
 * among the new tokens, bottom-right aligned, as in gqa_attn_prefill with
 * q_offset = kv_len[b] - T_q).
 *   q, o [B, T_q, H_q, d] (dtype)        lse [B, T_q, H_q] fp32, may be NULL
 *   k, v packed [sum_b kv_len[b], H_kv, d], kv_len HOST array [B]
 * Requires 1 <= T_q <= 256 and kv_len[b] >= T_q.  Uses the library-owned
 * workspace like gqa_attn_decode (same concurrency rule).
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED, GQA_ERR_RANGE,
 * GQA_ERR_HIP.
 */
int gqa_attn_decode_multi(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int T_q, int H_q, int H_kv, int d, const int32_t *kv_len,
                          float scale, int num_splits, int dtype, void *stream);

/*
 * Decode over a quantised KV cache (pccx page "Gemma 3N E4B on pccx v002 --
 * Execution / Scheduling", section 4 item 3: optional INT4 / INT8 KV cache,
 * the default for long contexts; section 6: INT4 KV cache in the base
 * configuration).  Symmetric per-channel quantisation: the value of K at
 * (key j, KV head kv, channel x) is code_k[j, kv, x] * k_scale[kv, x], and
 * likewise for V with v_scale.
 *   k, v packed [sum_b kv_len[b], H_kv, d] codes (same packing as
 *        gqa_attn_decode): kv_bits = 8: int8 in [-128, 127], one byte per
 *        channel; kv_bits = 4: two's-complement int4 in [-8, 7], two per byte,
 *        channel 2i in the low nibble of byte i.
 *   k_scale, v_scale fp32 [H_kv, d] (device).
 *   q, o [B, T_q, H_q, d] bf16; lse [B, T_q, H_q] fp32, may be NULL.
 * T_q new tokens per sequence with the causal rule of gqa_attn_decode_multi
 * (T_q = 1: plain decode).  The result is attention over the dequantised
 * K and V; fp32 accumulation as gqa_attn_decode.  Scale precision: each
 * k_scale multiplies the query in fp32 and enters the MFMA as a bf16 high
 * plus low pair (about 16 significant bits); v_scale multiplies the fp32
 * partial output exactly.  Scales are arbitrary finite fp32 values; parity
 * against the fp64 oracle is tested both with bf16-valued scales (where code
 * * scale is exact) and with scales that are not bf16 values.
 * Library-owned workspace.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED (kv_bits, d),
 * GQA_ERR_RANGE, GQA_ERR_HIP.
 */
int gqa_attn_decode_quant(const void *q, const void *k, const void *v, const float *k_scale,
                          const float *v_scale, void *o, float *lse, int B, int T_q, int H_q,
                          int H_kv, int d, const int32_t *kv_len, int kv_bits, float scale,
                          int num_splits, void *stream);

/*
 * Decode over a hard-cap ring-buffer KV cache with attention sinks and a local
 * window (pccx page "Gemma 3N E4B on pccx v002 -- Execution / Scheduling":
 * the KV ring buffer sized by max_tokens at init, and section 4, KV cache
 * management, where a wrapped ring keeps the sink positions and a local
 * window of the newest ones).  T_q >= 1 new tokens per sequence, already written to the cache.
 *   k, v [B, capacity, H_kv, d] (dtype): the first `sink` positions of
 *        sequence b stay in slots 0 .. sink-1; position j >= sink is in slot
 *        sink + (j - sink) mod (capacity - sink), so the ring keeps the
 *        capacity - sink newest positions.
 *   kv_len HOST [B]: tokens written so far (positions 0 .. kv_len[b]-1; may
 *        exceed capacity).  Requires kv_len[b] >= T_q.
 *   q, o [B, T_q, H_q, d]; lse [B, T_q, H_q] fp32, may be NULL.
 * New token t (position p = kv_len[b] - T_q + t) attends to key j iff j <= p
 * and (j < sink or j > p - window), as gqa_attn_prefill_window.  Requires
 * 0 <= sink < capacity, window >= 1 and window + T_q - 1 <= capacity - sink
 * (every key a new token sees is still resident).  Only the resident keys
 * that some new token sees are read; the split plan (num_splits as in
 * gqa_attn_decode) runs over them.  Library-owned workspace as
 * gqa_attn_decode.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED, GQA_ERR_RANGE
 * (sink/window/capacity), GQA_ERR_HIP.
 */
int gqa_attn_decode_ring(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                         int T_q, int H_q, int H_kv, int d, int capacity, const int32_t *kv_len,
                         int window, int sink, float scale, int num_splits, int dtype,
                         void *stream);

/*
 * Decode over a quantised hard-cap ring-buffer cache: the base configuration
 * of the pccx page ("Gemma 3N E4B on pccx v002 -- Execution / Scheduling",
 * section 6: INT4 KV cache with an 8192-token hard cap; section 4 items 2
 * and 3).  The ring layout, kv_len, window, sink and their requirements are
 * those of gqa_attn_decode_ring; the codes and scales those of
 * gqa_attn_decode_quant:
 *   k, v [B, capacity, H_kv, d] int8 codes (kv_bits = 8) or
 *        [B, capacity, H_kv, d/2] bytes of two int4 codes (kv_bits = 4,
 *        channel 2i in the low nibble of byte i);
 *   k_scale, v_scale fp32 [H_kv, d] (device);
 *   q, o [B, T_q, H_q, d] bf16; lse [B, T_q, H_q] fp32, may be NULL.
 * The result is gqa_attn_decode_ring's over the dequantised cache (value =
 * code * scale).  Library-owned workspace as gqa_attn_decode.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED (kv_bits, d),
 * GQA_ERR_RANGE (sink/window/capacity, scale), GQA_ERR_HIP.
 */
int gqa_attn_decode_ring_quant(const void *q, const void *k, const void *v, const float *k_scale,
                               const float *v_scale, void *o, float *lse, int B, int T_q,
                               int H_q, int H_kv, int d, int capacity, const int32_t *kv_len,
                               int window, int sink, int kv_bits, float scale, int num_splits,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
