// api.cpp -- the C ABI of libgqa_attn.so (declared in include/gqa_attn.h):
// argument validation, the decode split plan, the decode workspace cache and
// kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "gqa_attn.h"
#include "launch.h"

namespace {

using gqa::DecodePlanChunk;
using gqa::DecodeWorkspace;

constexpr int kTargetSplitWorkgroups = 1024;   // about four per compute unit on MI355X
constexpr int kMinSplitLen = 128;
constexpr int kMaxSplitLen = 8192;
constexpr int kSplitAlign = 64;
constexpr int kMaxDecodeTokens = 256;   // new tokens per sequence in gqa_attn_decode_multi
constexpr int kMaxPrefillSplits = 64;
constexpr int kMinPrefillSplitTiles = 4;          // 64-key tiles per split, at least
constexpr size_t kMaxPrefillWorkspace = (size_t)4 << 30;

bool finite_positive(float x) { return isfinite(x) && x > 0.f; }

int check_heads(int H_q, int H_kv, int d) {
    if (H_q < 1 || H_kv < 1 || (H_q % H_kv) != 0) return GQA_ERR_SHAPE;
    if (d != 64 && d != 128) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

// Per-sequence split lengths L_b and counts n_b (see gqa_attn_decode_plan).
struct Plan {
    int64_t total = 0;
    int max_splits = 0;
    int max_len = 0;
};

int env_split_len() {
    static int cached = -1;
    if (cached < 0) {
        const char* s = getenv("GQA_ATTN_SPLIT_LEN");
        int v = s ? atoi(s) : 0;
        cached = v > 0 ? v : 0;
    }
    return cached;
}

int device_cus();

// Automatic split length.  Two split work-groups are resident per compute
// unit; with W work-groups in a launch and `slots` resident at once, a slot
// runs about ceil(W / slots) splits one after another, each of up to L keys
// plus a fixed cost per work-group (Q load, merge, partial writes) counted as
// kSplitFixedKeys keys.  The length chosen is the candidate in [kMinSplitLen,
// kMaxSplitLen] that minimises ceil(W / slots) * (L + kSplitFixedKeys) summed
// over the launches (64 sequences each); ties go to the longer split (fewer
// partials).  Candidates: multiples of 64 up to 1024, of 128 up to 2048, of
// 256 beyond (47 at most; the search costs ~10 us of host time at 64
// sequences).  A launch a few work-groups over one
// round of slots pays a second round: on the 16-sequence ragged batch, 132
// splits of 2176 keys (528 work-groups) measured 196 us, 127 splits of 2304
// keys (508) 190 us and 129 splits of 2240 keys (516) 222 us.  With the search
// that batch runs 189 vs 196 us, four new tokens per sequence 211 vs 220 us
// and the ring batch 84.9 vs 86.8 us; int4 codes: the ragged batch 76 vs 84
// us, the 8192-slot ring 39.4 vs 47.7 us.  int8 codes and batches above
// kSearchMaxBatch take the length that gives about kTargetSplitWorkgroups
// work-groups (the search picked 4864-key splits for the ragged int8 batch:
// 116 vs 105 us).  The combine then reads every split of a sequence, so each
// split of the longest sequence adds kCombineKeysPerSplit keys: decode_8k
// takes 32 splits of 256 keys (one work-group per compute unit), 12.95 us per
// call, rather than 64 of 128 (two per compute unit), 13.33 us -- the split
// kernel runs 9.9-10.0 us either way, the combine has half the partials.
constexpr int kSearchMaxBatch = 256;
constexpr int kSplitFixedKeys = 256;
constexpr int kCombineKeysPerSplit = 8;
int64_t auto_split_len(int B, const int32_t* kv_len, int T_q, int G, int H_kv,
                       gqa::DecodeKind kind, int64_t total_keys, int n_hg) {
    if (B > kSearchMaxBatch || kind == gqa::DecodeKind::Quant) {
        int64_t per = (total_keys * H_kv * n_hg + kTargetSplitWorkgroups - 1) /
                      kTargetSplitWorkgroups;
        per = (per + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
        return per < kMinSplitLen ? kMinSplitLen : per > kMaxSplitLen ? kMaxSplitLen : per;
    }
    int64_t max_len = 0;
    for (int b = 0; b < B; ++b) max_len = kv_len[b] > max_len ? kv_len[b] : max_len;
    int64_t hi = (max_len + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    if (hi > kMaxSplitLen) hi = kMaxSplitLen;
    if (hi < kMinSplitLen) hi = kMinSplitLen;
    const int64_t slots = (int64_t)gqa::kDecodeWorkgroupsPerCu * device_cus();
    int64_t best = kMinSplitLen, best_cost = INT64_MAX;
    for (int64_t L = kMinSplitLen; L <= hi; L += L < 1024 ? 64 : L < 2048 ? 128 : 256) {
        const int64_t per_split = gqa::decode_workgroups_per_split(kind, T_q, G, H_kv, (int)L);
        int64_t cost = 0, max_n = 0;
        for (int b0 = 0; b0 < B; b0 += gqa::kDecodeSeqPerLaunch) {
            const int b1 = B - b0 < gqa::kDecodeSeqPerLaunch ? B : b0 + gqa::kDecodeSeqPerLaunch;
            int64_t n = 0;
            for (int b = b0; b < b1; ++b) {
                const int64_t nb = (kv_len[b] + L - 1) / L;
                n += nb;
                max_n = nb > max_n ? nb : max_n;
            }
            cost += (n * per_split + slots - 1) / slots * (L + kSplitFixedKeys);
        }
        cost += kCombineKeysPerSplit * max_n;
        if (cost <= best_cost) {
            best_cost = cost;
            best = L;
        }
    }
    return best;
}

int make_plan(int B, int T_q, int H_q, int H_kv, const int32_t* kv_len, int num_splits,
              int32_t* splits, int32_t* lens, Plan* out,
              gqa::DecodeKind kind = gqa::DecodeKind::Bf16) {
    if (kv_len == nullptr) return GQA_ERR_NULL;
    if (B < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv) return GQA_ERR_SHAPE;
    int64_t total_keys = 0;
    for (int b = 0; b < B; ++b) {
        if (kv_len[b] < 1) return GQA_ERR_SHAPE;
        total_keys += kv_len[b];
    }
    const int G = H_q / H_kv;
    const int n_hg = gqa::decode_column_groups(T_q, G);
    int64_t auto_len = 0;
    if (num_splits <= 0) {
        int forced = env_split_len();
        auto_len = forced > 0 ? forced
                              : auto_split_len(B, kv_len, T_q, G, H_kv, kind, total_keys, n_hg);
    }
    Plan p;
    for (int b = 0; b < B; ++b) {
        const int64_t len = kv_len[b];
        int64_t L;
        if (num_splits > 0) {
            const int64_t ns = num_splits < len ? num_splits : len;
            L = (len + ns - 1) / ns;
        } else {
            L = auto_len;
        }
        const int64_t n = (len + L - 1) / L;
        if (splits) splits[b] = (int32_t)n;
        if (lens) lens[b] = (int32_t)L;
        p.total += n;
        if (n > p.max_splits) p.max_splits = (int)n;
        const int64_t longest = L < len ? L : len;   // this sequence's longest split
        if (longest > p.max_len) p.max_len = (int)longest;
    }
    if (p.total > (int64_t)1 << 30) return GQA_ERR_SHAPE;
    *out = p;
    return GQA_OK;
}

// rows = partial rows per split: T_q * H_q
size_t workspace_bytes_for(int64_t total, int rows, int d) {
    return (size_t)total * (size_t)rows * (size_t)(d + 2) * sizeof(float);
}

DecodeWorkspace carve(void* base, int64_t total, int rows) {
    float* f = (float*)base;
    DecodeWorkspace ws;
    ws.m = f;
    ws.l = f + total * rows;
    ws.o = f + 2 * total * rows;
    return ws;
}

int check_decode_args(const void* q, const void* k, const void* v, int B, int H_q, int H_kv,
                      int d, const int32_t* kv_len, float scale, int dtype) {
    if (!q || !k || !v || !kv_len) return GQA_ERR_NULL;
    if (B < 1) return GQA_ERR_SHAPE;
    int rc = check_heads(H_q, H_kv, d);
    if (rc) return rc;
    if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
    if (!finite_positive(scale)) return GQA_ERR_RANGE;
    return GQA_OK;
}

// Split the batch into launches of at most kDecodeSeqPerLaunch sequences and
// call fn(chunk) for each.
// ring_cap > 0: a ring-buffer cache of ring_cap slots per sequence (sequence
// b starts at row b * ring_cap); kv_len are then the walked key counts and
// ntok the tokens written.
template <typename Fn>
int for_each_chunk(int B, const int32_t* kv_len, const int32_t* splits, const int32_t* lens,
                   Fn fn, int ring_cap = 0, const int32_t* ntok = nullptr) {
    int64_t key_off = 0, split_base = 0;
    for (int b0 = 0; b0 < B; b0 += gqa::kDecodeSeqPerLaunch) {
        DecodePlanChunk c;
        memset(&c, 0, sizeof(c));
        c.nseq = B - b0 < gqa::kDecodeSeqPerLaunch ? B - b0 : gqa::kDecodeSeqPerLaunch;
        c.seq0 = b0;
        if (split_base > 0x7fffffff) return GQA_ERR_SHAPE;
        c.split_base = (int)split_base;
        int units = 0;
        for (int i = 0; i < c.nseq; ++i) {
            c.key_off[i] = ring_cap > 0 ? (int64_t)(b0 + i) * ring_cap : key_off;
            c.len[i] = kv_len[b0 + i];
            c.ntok[i] = ntok ? ntok[b0 + i] : kv_len[b0 + i];
            c.split_len[i] = lens[b0 + i];
            c.unit_base[i] = units;
            units += splits[b0 + i];
            key_off += kv_len[b0 + i];
        }
        c.unit_base[c.nseq] = units;
        c.units = units;
        split_base += units;
        hipError_t e = fn(c);
        if (e != hipSuccess) return GQA_ERR_HIP;
    }
    return GQA_OK;
}

struct HostPlan {
    int32_t* splits = nullptr;
    int32_t* lens = nullptr;
    Plan p;
    ~HostPlan() {
        free(splits);
        free(lens);
    }
    int build(int B, int H_q, int H_kv, const int32_t* kv_len, int num_splits, int T_q = 1,
              gqa::DecodeKind kind = gqa::DecodeKind::Bf16) {
        splits = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
        lens = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
        if (!splits || !lens) return GQA_ERR_SHAPE;
        return make_plan(B, T_q, H_q, H_kv, kv_len, num_splits, splits, lens, &p, kind);
    }
};

// Per-device workspace owned by the library (the one-call decode entry
// points and the KV-parallel prefills).  A call holds the workspace lock from
// the moment it takes the buffer until its last kernel is queued (the
// WorkspaceLease lives to the end of the entry point), so two calls never
// swap buffers under each other.  A call that needs a larger buffer allocates
// one at least twice the size and retires the old one without freeing it:
// kernels queued by earlier calls, and graphs captured from them, keep a
// valid buffer, and growth neither waits for the device nor frees memory in
// the middle of an asynchronous call.  Retired buffers (at most about the
// size of the current one in total, by the doubling) are freed only by
// gqa_attn_release_workspace.  Calls on different streams of one device
// still share the current buffer's contents and must be serialised by the
// caller.
constexpr int kMaxDevices = 64;
struct CachedWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    std::vector<void*> retired;
};
std::mutex g_ws_mutex;
CachedWorkspace g_ws[kMaxDevices];

struct WorkspaceLease {
    std::unique_lock<std::mutex> lock;
    void* ptr = nullptr;
};

int get_workspace(size_t bytes, WorkspaceLease* lease) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
    std::unique_lock<std::mutex> lock(g_ws_mutex);
    CachedWorkspace& w = g_ws[dev];
    if (w.bytes < bytes) {
        size_t want = bytes < (1u << 20) ? (1u << 20) : bytes;
        if (want < 2 * w.bytes) want = 2 * w.bytes;
        void* p = nullptr;
        if (hipMalloc(&p, want) != hipSuccess) {
            // the doubled size may not fit where the exact one does
            (void)hipGetLastError();
            want = bytes;
            if (hipMalloc(&p, want) != hipSuccess) return GQA_ERR_HIP;
        }
        if (w.ptr) w.retired.push_back(w.ptr);   // still read by queued kernels and graphs
        w.ptr = p;
        w.bytes = want;
    }
    lease->ptr = w.ptr;
    lease->lock = std::move(lock);
    return GQA_OK;
}

}  // namespace

extern "C" int gqa_attn_release_workspace(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    CachedWorkspace& w = g_ws[dev];
    if (!w.ptr && w.retired.empty()) return GQA_OK;
    if (hipDeviceSynchronize() != hipSuccess) return GQA_ERR_HIP;
    int rc = GQA_OK;
    for (void* p : w.retired)
        if (hipFree(p) != hipSuccess) rc = GQA_ERR_HIP;
    w.retired.clear();
    if (w.ptr && hipFree(w.ptr) != hipSuccess) rc = GQA_ERR_HIP;
    w.ptr = nullptr;
    w.bytes = 0;
    return rc;
}

namespace {

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        return 256;
    return n;
}

int check_prefill_args(const void* q, const void* k, const void* v, const void* o, int B,
                       int T_q, int S_kv, int H_q, int H_kv, int d, float scale, int causal,
                       int q_offset) {
    if (!q || !k || !v || !o) return GQA_ERR_NULL;
    if (B < 1 || T_q < 1 || S_kv < 1) return GQA_ERR_SHAPE;
    int rc = check_heads(H_q, H_kv, d);
    if (rc) return rc;
    if (!finite_positive(scale)) return GQA_ERR_RANGE;
    if (causal && (q_offset < 0 || (int64_t)q_offset + T_q > S_kv)) return GQA_ERR_RANGE;
    if ((int64_t)T_q * (H_q / H_kv) > 0x7fffffff - 256) return GQA_ERR_SHAPE;
    // a work-group addresses its Q rows (at most 257 tokens) with 32-bit byte offsets
    if ((int64_t)H_q * d * 2 * 257 > 0x7fffffff) return GQA_ERR_SHAPE;
    return GQA_OK;
}

// Key splits per row block for the KV-parallel prefill (see gqa_attn_prefill_kvsplit).
// One prefill work-group is resident per compute unit (128 KiB of LDS), so
// W = blocks * n work-groups run in ceil(W / CUs) rounds, each about
// tiles / n tiles plus a fixed cost per work-group (Q load, epilogue) of
// kPrefillFixedTiles tiles; the automatic n minimises that product (ties to
// the smaller n: fewer partials).  On the 256-token chunk over 64k keys (64
// row blocks) that is n = 4, one round: 482 us, against 500 us for n = 8 (two
// rounds, the previous "two work-groups per compute unit" rule) and 650 us
// for n = 5.
constexpr int kPrefillFixedTiles = 4;
int prefill_splits(int B, int T_q, int S_kv, int H_q, int H_kv, int d, int causal, int q_offset,
                   int num_splits, int window = 0, int sink = 0) {
    const int64_t blocks = gqa::prefill_row_blocks(T_q, H_q / H_kv) * B * H_kv;
    // the longest row block sees keys up to its last query
    const int64_t keys = causal ? (int64_t)q_offset + T_q : S_kv;
    int64_t tiles = (keys + 63) / 64;
    if (window > 0) {   // a row block loads its sink tiles and the tiles of its window
        const int64_t tokens = (256 + H_q / H_kv - 1) / (H_q / H_kv);   // per row block
        const int64_t win = (sink + 63) / 64 + (window + tokens + 63) / 64 + 1;
        if (win < tiles) tiles = win;
    }
    int64_t ns;
    if (num_splits > 0) {
        ns = num_splits;
    } else {
        const int64_t cus = device_cus();
        int64_t hi = tiles / kMinPrefillSplitTiles;
        if (hi > kMaxPrefillSplits) hi = kMaxPrefillSplits;
        ns = 1;
        int64_t best = INT64_MAX;
        for (int64_t n = 1; n <= (hi < 1 ? 1 : hi); ++n) {
            const int64_t cost = (blocks * n + cus - 1) / cus * ((tiles + n - 1) / n + kPrefillFixedTiles);
            if (cost < best) {
                best = cost;
                ns = n;
            }
        }
    }
    if (ns > tiles) ns = tiles;
    if (ns > kMaxPrefillSplits) ns = kMaxPrefillSplits;
    const size_t row_bytes = (size_t)B * T_q * H_q * (size_t)(d + 2) * sizeof(float);
    while (ns > 1 && row_bytes * (size_t)ns > kMaxPrefillWorkspace) --ns;
    return ns < 1 ? 1 : (int)ns;
}

}  // namespace

extern "C" {

const char* gqa_attn_status_string(int status) {
    switch (status) {
        case GQA_OK: return "ok";
        case GQA_ERR_NULL: return "a required pointer is NULL";
        case GQA_ERR_SHAPE: return "invalid sizes (B, T_q, S_kv, heads, kv_len)";
        case GQA_ERR_UNSUPPORTED: return "unsupported head dim or dtype";
        case GQA_ERR_RANGE: return "argument out of range (q_offset, scale, workspace size)";
        case GQA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int gqa_attn_version(void) { return 100; }

int gqa_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int T_q, int S_kv, int H_q, int H_kv, int d, float scale, int causal,
                     int q_offset, int dtype, void* stream) {
    int rc = check_prefill_args(q, k, v, o, B, T_q, S_kv, H_q, H_kv, d, scale, causal, q_offset);
    if (rc) return rc;
    if (dtype != GQA_BF16 && dtype != GQA_F32) return GQA_ERR_UNSUPPORTED;
    gqa::PrefillArgs a{q, k, v, o, lse, B, T_q, S_kv, H_q, H_kv, d, scale, causal ? 1 : 0,
                       causal ? q_offset : 0};
    (void)hipGetLastError();
    hipError_t e = dtype == GQA_BF16 ? gqa::launch_prefill_bf16(a, (hipStream_t)stream)
                                     : gqa::launch_prefill_f32(a, (hipStream_t)stream);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_decode_plan(int B, int H_q, int H_kv, int d, const int32_t* kv_len, int num_splits,
                         int32_t* splits, int* split_len, int64_t* total_splits, int* max_splits,
                         size_t* workspace_bytes) {
    if (kv_len == nullptr) return GQA_ERR_NULL;
    if (B < 1) return GQA_ERR_SHAPE;
    int rc = check_heads(H_q, H_kv, d);
    if (rc) return rc;
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits);
    if (rc) return rc;
    if (splits) memcpy(splits, hp.splits, sizeof(int32_t) * (size_t)B);
    if (split_len) *split_len = hp.p.max_len;
    if (total_splits) *total_splits = hp.p.total;
    if (max_splits) *max_splits = hp.p.max_splits;
    if (workspace_bytes) *workspace_bytes = workspace_bytes_for(hp.p.total, H_q, d);
    return GQA_OK;
}

int gqa_attn_decode_split(const void* q, const void* k, const void* v, void* workspace,
                          size_t workspace_bytes, int B, int H_q, int H_kv, int d,
                          const int32_t* kv_len, float scale, int num_splits, int dtype,
                          void* stream) {
    int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, dtype);
    if (rc) return rc;
    if (!workspace) return GQA_ERR_NULL;
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits);
    if (rc) return rc;
    if (workspace_bytes < workspace_bytes_for(hp.p.total, H_q, d)) return GQA_ERR_RANGE;
    DecodeWorkspace ws = carve(workspace, hp.p.total, H_q);
    (void)hipGetLastError();
    return for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_split_bf16(q, k, v, ws, c, 1, H_q, H_kv, d, scale,
                                             (hipStream_t)stream);
    });
}

int gqa_attn_decode_combine(const void* workspace, size_t workspace_bytes, void* o, float* lse,
                            int B, int H_q, int H_kv, int d, const int32_t* kv_len,
                            int num_splits, int dtype, void* stream) {
    if (!workspace || !o || !kv_len) return GQA_ERR_NULL;
    if (B < 1) return GQA_ERR_SHAPE;
    int rc = check_heads(H_q, H_kv, d);
    if (rc) return rc;
    if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits);
    if (rc) return rc;
    if (workspace_bytes < workspace_bytes_for(hp.p.total, H_q, d)) return GQA_ERR_RANGE;
    DecodeWorkspace ws = carve((void*)workspace, hp.p.total, H_q);
    (void)hipGetLastError();
    return for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_combine_bf16(ws, c, o, lse, 1, H_q, d, (hipStream_t)stream);
    });
}

int gqa_attn_decode(const void* q, const void* k, const void* v, void* o, int B, int H_q,
                    int H_kv, int d, const int32_t* kv_len, float scale, int num_splits,
                    int dtype, void* stream) {
    int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, dtype);
    if (rc) return rc;
    if (!o) return GQA_ERR_NULL;
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits);
    if (rc) return rc;
    const size_t need = workspace_bytes_for(hp.p.total, H_q, d);
    WorkspaceLease lease;
    rc = get_workspace(need, &lease);
    if (rc) return rc;
    DecodeWorkspace ws = carve(lease.ptr, hp.p.total, H_q);
    (void)hipGetLastError();
    rc = for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_split_bf16(q, k, v, ws, c, 1, H_q, H_kv, d, scale,
                                             (hipStream_t)stream);
    });
    if (rc) return rc;
    return for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_combine_bf16(ws, c, o, nullptr, 1, H_q, d, (hipStream_t)stream);
    });
}

}  // extern "C"

namespace {

// Scratch of gqa_attn_decode_noalloc: the split partials live in this fixed
// device array instead of an allocated workspace.  Each device that the
// library runs on holds its own copy for the life of the process.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the first call on a device, with that device
// current, looks the device address up with hipGetSymbolAddress and keeps
// it per device; kernels receive that pointer.  Every partial the combine
// reads is written by the split kernel of the same call, so nothing in it
// has to start at zero.
static __device__ __align__(256) unsigned char scratch[GQA_ATTN_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return GQA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H_q,
                            int H_kv, int d, const int32_t* kv_len, float scale, int num_splits,
                            int dtype, void* stream) {
    int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, dtype);
    if (rc) return rc;
    if (!o) return GQA_ERR_NULL;
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits);
    if (rc) return rc;
    if (workspace_bytes_for(hp.p.total, H_q, d) > (size_t)GQA_ATTN_NOALLOC_SCRATCH_BYTES)
        return GQA_ERR_RANGE;
    void* base = nullptr;
    rc = scratch_address(&base);
    if (rc) return rc;
    DecodeWorkspace ws = carve(base, hp.p.total, H_q);
    (void)hipGetLastError();
    rc = for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_split_bf16(q, k, v, ws, c, 1, H_q, H_kv, d, scale,
                                             (hipStream_t)stream);
    });
    if (rc) return rc;
    return for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_combine_bf16(ws, c, o, nullptr, 1, H_q, d, (hipStream_t)stream);
    });
}

}  // extern "C"

namespace {

// KV-parallel prefill for an already checked argument set (a.window > 0: sink
// + local-window mask).
int prefill_kvsplit_impl(const gqa::PrefillArgs& a, int num_splits, void* stream) {
    const int ns = prefill_splits(a.B, a.T_q, a.S_kv, a.H_q, a.H_kv, a.d, a.causal, a.q_offset,
                                  num_splits, a.window, a.sink);
    (void)hipGetLastError();
    if (ns == 1)
        return gqa::launch_prefill_bf16(a, (hipStream_t)stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
    const int64_t total = (int64_t)a.B * ns;             // partials per (t, h)
    const int rows = a.T_q * a.H_q;
    WorkspaceLease lease;
    int rc = get_workspace(workspace_bytes_for(total, rows, a.d), &lease);
    if (rc) return rc;
    DecodeWorkspace ws = carve(lease.ptr, total, rows);
    if (gqa::launch_prefill_split_bf16(a, ns, ws, (hipStream_t)stream) != hipSuccess)
        return GQA_ERR_HIP;
    for (int b0 = 0; b0 < a.B; b0 += gqa::kDecodeSeqPerLaunch) {
        DecodePlanChunk c;
        memset(&c, 0, sizeof(c));
        c.nseq = a.B - b0 < gqa::kDecodeSeqPerLaunch ? a.B - b0 : gqa::kDecodeSeqPerLaunch;
        c.seq0 = b0;
        c.split_base = b0 * ns;
        for (int i = 0; i <= c.nseq; ++i) c.unit_base[i] = i * ns;
        c.units = c.nseq * ns;
        if (gqa::launch_decode_combine_bf16(ws, c, a.o, a.lse, a.T_q, a.H_q, a.d,
                                            (hipStream_t)stream) != hipSuccess)
            return GQA_ERR_HIP;
    }
    return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_attn_prefill_kvsplit(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int T_q, int S_kv, int H_q, int H_kv, int d, float scale,
                             int causal, int q_offset, int num_splits, int dtype, void* stream) {
    int rc = check_prefill_args(q, k, v, o, B, T_q, S_kv, H_q, H_kv, d, scale, causal, q_offset);
    if (rc) return rc;
    if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
    if (!causal) q_offset = 0;
    gqa::PrefillArgs a{q, k, v, o, lse, B, T_q, S_kv, H_q, H_kv, d, scale, causal ? 1 : 0,
                       q_offset};
    return prefill_kvsplit_impl(a, num_splits, stream);
}

int gqa_attn_prefill_window_kvsplit(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int T_q, int S_kv, int H_q, int H_kv,
                                    int d, float scale, int q_offset, int window, int sink,
                                    int num_splits, int dtype, void* stream) {
    int rc = check_prefill_args(q, k, v, o, B, T_q, S_kv, H_q, H_kv, d, scale, 1, q_offset);
    if (rc) return rc;
    if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
    if (window < 1 || sink < 0) return GQA_ERR_RANGE;
    gqa::PrefillArgs a{q, k, v, o, lse, B, T_q, S_kv, H_q, H_kv, d, scale, 1, q_offset};
    a.window = window;
    a.sink = sink < S_kv ? sink : S_kv;
    return prefill_kvsplit_impl(a, num_splits, stream);
}

int gqa_attn_prefill_window(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int T_q, int S_kv, int H_q, int H_kv, int d, float scale,
                            int q_offset, int window, int sink, int dtype, void* stream) {
    int rc = check_prefill_args(q, k, v, o, B, T_q, S_kv, H_q, H_kv, d, scale, 1, q_offset);
    if (rc) return rc;
    if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
    if (window < 1 || sink < 0) return GQA_ERR_RANGE;
    gqa::PrefillArgs a{q, k, v, o, lse, B, T_q, S_kv, H_q, H_kv, d, scale, 1, q_offset};
    a.window = window;
    a.sink = sink < S_kv ? sink : S_kv;
    (void)hipGetLastError();
    return gqa::launch_prefill_bf16(a, (hipStream_t)stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_prefill_kvsplit_count(int B, int T_q, int S_kv, int H_q, int H_kv, int d, int causal,
                                   int q_offset, int num_splits) {
    if (B < 1 || T_q < 1 || S_kv < 1 || check_heads(H_q, H_kv, d)) return -GQA_ERR_SHAPE;
    if (causal && (q_offset < 0 || (int64_t)q_offset + T_q > S_kv)) return -GQA_ERR_RANGE;
    return prefill_splits(B, T_q, S_kv, H_q, H_kv, d, causal, causal ? q_offset : 0, num_splits);
}

}  // extern "C"

namespace {

// Ring-buffer decode over a bf16 cache (bits = 16) or int8 / int4 codes.
int decode_ring_impl(const void* q, const void* k, const void* v, const float* k_scale,
                     const float* v_scale, int bits, void* o, float* lse, int B, int T_q,
                     int H_q, int H_kv, int d, int capacity, const int32_t* kv_len, int window,
                     int sink, float scale, int num_splits, void* stream) {
    if (!o) return GQA_ERR_NULL;
    if (T_q < 1 || T_q > kMaxDecodeTokens || capacity < 1) return GQA_ERR_SHAPE;
    // every key a new token may see must still be resident
    if (sink < 0 || sink >= capacity || window < 1 ||
        (int64_t)window + T_q - 1 > (int64_t)capacity - sink)
        return GQA_ERR_RANGE;
    int32_t* walk = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    if (!walk) return GQA_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        const int64_t n = kv_len[b];
        if (n < T_q) {
            free(walk);
            return GQA_ERR_SHAPE;
        }
        const int64_t s_end = n < sink ? n : sink;
        int64_t w_lo = n - T_q - window + 1;
        if (w_lo < s_end) w_lo = s_end;
        walk[b] = (int32_t)(s_end + (n - w_lo));
    }
    HostPlan hp;
    int rc = hp.build(B, H_q, H_kv, walk, num_splits, T_q,
                      bits == 16  ? gqa::DecodeKind::Ring
                      : bits == 4 ? gqa::DecodeKind::QuantInt4
                                  : gqa::DecodeKind::Quant);
    if (rc) {
        free(walk);
        return rc;
    }
    const int rows = T_q * H_q;
    WorkspaceLease lease;
    rc = get_workspace(workspace_bytes_for(hp.p.total, rows, d), &lease);
    if (rc) {
        free(walk);
        return rc;
    }
    DecodeWorkspace ws = carve(lease.ptr, hp.p.total, rows);
    const gqa::RingArgs ring{capacity, sink, window};
    (void)hipGetLastError();
    rc = for_each_chunk(B, walk, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_ring_split(q, k, v, k_scale, v_scale, bits, ws, c, T_q, H_q,
                                             H_kv, d, scale, ring, (hipStream_t)stream);
    }, capacity, kv_len);
    if (!rc)
        rc = for_each_chunk(B, walk, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
            return gqa::launch_decode_combine_bf16(ws, c, o, lse, T_q, H_q, d, (hipStream_t)stream);
        }, capacity, kv_len);
    free(walk);
    return rc;
}

}  // namespace

extern "C" {

int gqa_attn_decode_ring(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int T_q, int H_q, int H_kv, int d, int capacity, const int32_t* kv_len,
                         int window, int sink, float scale, int num_splits, int dtype,
                         void* stream) {
    const int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, dtype);
    if (rc) return rc;
    return decode_ring_impl(q, k, v, nullptr, nullptr, 16, o, lse, B, T_q, H_q, H_kv, d, capacity,
                            kv_len, window, sink, scale, num_splits, stream);
}

int gqa_attn_decode_ring_quant(const void* q, const void* k, const void* v, const float* k_scale,
                               const float* v_scale, void* o, float* lse, int B, int T_q,
                               int H_q, int H_kv, int d, int capacity, const int32_t* kv_len,
                               int window, int sink, int kv_bits, float scale, int num_splits,
                               void* stream) {
    const int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, GQA_BF16);
    if (rc) return rc;
    if (!k_scale || !v_scale) return GQA_ERR_NULL;
    if (kv_bits != 8 && kv_bits != 4) return GQA_ERR_UNSUPPORTED;
    return decode_ring_impl(q, k, v, k_scale, v_scale, kv_bits, o, lse, B, T_q, H_q, H_kv, d,
                            capacity, kv_len, window, sink, scale, num_splits, stream);
}

int gqa_attn_decode_quant(const void* q, const void* k, const void* v, const float* k_scale,
                          const float* v_scale, void* o, float* lse, int B, int T_q, int H_q,
                          int H_kv, int d, const int32_t* kv_len, int kv_bits, float scale,
                          int num_splits, void* stream) {
    int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, GQA_BF16);
    if (rc) return rc;
    if (!o || !k_scale || !v_scale) return GQA_ERR_NULL;
    if (kv_bits != 8 && kv_bits != 4) return GQA_ERR_UNSUPPORTED;
    if (T_q < 1 || T_q > kMaxDecodeTokens) return GQA_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
        if (kv_len[b] < T_q) return GQA_ERR_SHAPE;
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits, T_q,
                  kv_bits == 4 ? gqa::DecodeKind::QuantInt4 : gqa::DecodeKind::Quant);
    if (rc) return rc;
    const int rows = T_q * H_q;
    WorkspaceLease lease;
    rc = get_workspace(workspace_bytes_for(hp.p.total, rows, d), &lease);
    if (rc) return rc;
    DecodeWorkspace ws = carve(lease.ptr, hp.p.total, rows);
    (void)hipGetLastError();
    rc = for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_quant_split(q, k, v, k_scale, v_scale, kv_bits, ws, c, T_q, H_q,
                                              H_kv, d, scale, (hipStream_t)stream);
    });
    if (rc) return rc;
    return for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_combine_bf16(ws, c, o, lse, T_q, H_q, d, (hipStream_t)stream);
    });
}

int gqa_attn_decode_multi(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int T_q, int H_q, int H_kv, int d, const int32_t* kv_len,
                          float scale, int num_splits, int dtype, void* stream) {
    int rc = check_decode_args(q, k, v, B, H_q, H_kv, d, kv_len, scale, dtype);
    if (rc) return rc;
    if (!o) return GQA_ERR_NULL;
    if (T_q < 1 || T_q > kMaxDecodeTokens) return GQA_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
        if (kv_len[b] < T_q) return GQA_ERR_SHAPE;   // the new tokens are in the cache
    HostPlan hp;
    rc = hp.build(B, H_q, H_kv, kv_len, num_splits, T_q);
    if (rc) return rc;
    const int rows = T_q * H_q;
    const size_t need = workspace_bytes_for(hp.p.total, rows, d);
    WorkspaceLease lease;
    rc = get_workspace(need, &lease);
    if (rc) return rc;
    DecodeWorkspace ws = carve(lease.ptr, hp.p.total, rows);
    (void)hipGetLastError();
    rc = for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_split_bf16(q, k, v, ws, c, T_q, H_q, H_kv, d, scale,
                                             (hipStream_t)stream);
    });
    if (rc) return rc;
    return for_each_chunk(B, kv_len, hp.splits, hp.lens, [&](const DecodePlanChunk& c) {
        return gqa::launch_decode_combine_bf16(ws, c, o, lse, T_q, H_q, d, (hipStream_t)stream);
    });
}

}  // extern "C"
