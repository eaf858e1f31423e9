// gqa_api.hip -- the C ABI declared in include/gqa.h: argument validation, work
// map selection and kernel launch.  Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include <atomic>

#include "gqa.h"
#include "gqa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up_256(size_t x) { return (x + 255) & ~(size_t)255; }

gqa_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GQA_ERR_DEVICE;
    if (dev < kMaxDevices) {
        int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known == 1) return GQA_OK;
        if (known == 2) return GQA_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GQA_ERR_DEVICE;
    bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? GQA_OK : GQA_ERR_DEVICE;
}

// Largest power of two that divides G, capped at 8: the number of query heads
// of one group that share a prefill work-group.
int heads_per_workgroup(int G) {
    int gw = 1;
    while (gw < 8 && G % (2 * gw) == 0) gw *= 2;
    return gw;
}

constexpr int kDefaultSplits = 256 * gqa::kDecodeWaves;  // every wave of the split pass resident on 256 CUs

// The decode workspace of gqa_decode_noalloc: a fixed array in device memory,
// one copy per GPU, held until the process ends.  In host code `scratch` is
// only a stand-in for the symbol; the array's device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
std::atomic<void *> g_scratch[kMaxDevices];

// The current device's scratch address, or nullptr if it cannot be had.
void *device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);  // every thread finds the same address
    return q;
}
constexpr int kMaxSplits = 1 << 20;

bool splits_valid(int n) { return n >= 0 && n <= kMaxSplits; }

}  // namespace

extern "C" {

const char *gqa_status_string(gqa_status s) {
    switch (s) {
        case GQA_OK: return "ok";
        case GQA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case GQA_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
        case GQA_ERR_SIZE: return "a size, scale or split-count argument is out of range";
        case GQA_ERR_HEADS: return "h_q is not a multiple of h_kv";
        case GQA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
        case GQA_ERR_DTYPE: return "dtype not supported by this entry point";
        case GQA_ERR_WORKSPACE: return "a workspace is NULL, misaligned or too small";
        case GQA_ERR_LAUNCH: return "the HIP runtime reported a launch error";
        case GQA_ERR_DEVICE: return "the current device is not a gfx950 GPU";
        case GQA_ERR_SCRATCH: return "the call needs more than the fixed decode scratch holds";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Bytes of one row of the keep-mask summary: a byte per 64-key tile, rounded
// up to a multiple of 8.
int mask_summary_stride(int Lk) { return ((Lk + 63) / 64 + 7) / 8 * 8; }

// Shared by both prefill entry points: Lq query positions per sequence attend
// to Lk >= Lq keys, query row i sitting at position Lk - Lq + i.
// The rotary form passes tables cos, sin [Lk][d/2] and the k_rot output: the
// keys are rotated into k_rot first and the prefill reads them from there.
gqa_status prefill_impl(const void *q, const void *k, const void *v, void *o, int B, int Lq,
                        int Lk, int h_q, int h_kv, int d, gqa_dtype dt, int causal, float scale,
                        void *hip_stream, const float *rope_cos = nullptr,
                        const float *rope_sin = nullptr, void *k_rot = nullptr,
                        bool rope = false, const int32_t *kv_lens = nullptr,
                        bool varlen = false, const uint8_t *mask = nullptr,
                        long long mask_row = 0, long long mask_batch = 0,
                        bool masked = false, void *workspace = nullptr,
                        size_t workspace_bytes = 0) {
    if (!q || !k || !v || !o) return GQA_ERR_NULL_POINTER;
    if (masked) {
        if (!mask) return GQA_ERR_NULL_POINTER;
        if (!aligned16(mask)) return GQA_ERR_ALIGNMENT;
        // rows of 16-byte pieces covering the L_k keys; one batch's rows
        // addressed with 32-bit byte offsets
        if (mask_row < Lk || mask_row % 16 != 0 || mask_batch < 0 || mask_batch % 16 != 0)
            return GQA_ERR_SIZE;
        if (Lq > 0 && mask_row > (long long)0xffffffff / Lq) return GQA_ERR_SIZE;
    }
    if (varlen) {
        if (!kv_lens) return GQA_ERR_NULL_POINTER;
        if ((reinterpret_cast<uintptr_t>(kv_lens) & 3u) != 0) return GQA_ERR_ALIGNMENT;
    }
    if (rope) {
        if (!rope_cos || !rope_sin || !k_rot) return GQA_ERR_NULL_POINTER;
        if (!aligned16(rope_cos) || !aligned16(rope_sin) || !aligned16(k_rot))
            return GQA_ERR_ALIGNMENT;
        if (dt != GQA_BF16) return GQA_ERR_DTYPE;
        if (k_rot == k) return GQA_ERR_SIZE;  // rotated in place would race
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GQA_ERR_ALIGNMENT;
    if (B <= 0 || Lq <= 0 || Lk < Lq || h_q <= 0 || h_kv <= 0) return GQA_ERR_SIZE;
    if (h_q % h_kv != 0) return GQA_ERR_HEADS;
    if (d != 64 && d != 128) return GQA_ERR_HEAD_DIM;
    if (dt != GQA_F32 && dt != GQA_BF16) return GQA_ERR_DTYPE;
    if (!(scale > 0.f) || !isfinite(scale)) return GQA_ERR_SIZE;
    const int64_t rows_q = (int64_t)B * Lq * h_q, rows_kv = (int64_t)B * Lk * h_kv;
    if (rows_q > (int64_t)1 << 31 || rows_kv > (int64_t)1 << 31) return GQA_ERR_SIZE;
    // the bf16 kernel addresses one sequence's key/value rows of a head with
    // 32-bit byte offsets: Lk rows at a stride of h_kv * d elements
    if (dt == GQA_BF16 && (int64_t)Lk * h_kv * d * 2 > (int64_t)0xffffffff) return GQA_ERR_SIZE;

    gqa::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.L = Lq;
    a.Lk = Lk;
    a.off = Lk - Lq;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.G = h_q / h_kv;
    a.GW = heads_per_workgroup(a.G);
    a.nsub = a.G / a.GW;
    a.BM = 32 * (8 / a.GW);
    a.n_units = B * h_kv * a.nsub;
    a.n_qtiles = (Lq + a.BM - 1) / a.BM;
    a.c = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    a.rope_cos = rope ? rope_cos : nullptr;
    a.rope_sin = rope ? rope_sin : nullptr;
    a.kv_lens = varlen ? kv_lens : nullptr;
    a.mask = masked ? mask : nullptr;
    a.mask_row = masked ? mask_row : 0;
    a.mask_batch = masked ? mask_batch : 0;
    {
        // an exact power of two may be folded into q (q * 2^e is exact in bf16)
        int e = 0;
        a.fold = frexpf(a.c, &e) == 0.5f ? 1 : 0;
    }
    if ((int64_t)a.n_units * a.n_qtiles > 0x7fffffff) return GQA_ERR_SIZE;
    a.mcodes = nullptr;
    a.morder = nullptr;
    a.mwork = nullptr;
    a.mc_stride = 0;
    if (masked) {
        const size_t need = gqa_prefill_mask_workspace_bytes(B, Lq, Lk);
        if (need == 0) return GQA_ERR_SIZE;
        if (!workspace || !aligned16(workspace) || workspace_bytes < need)
            return GQA_ERR_WORKSPACE;
        // laid out for the most query tiles any head count gives (32 rows each)
        a.mcodes = static_cast<uint8_t *>(workspace);
        a.mc_stride = mask_summary_stride(Lk);
        const size_t tiles = (size_t)B * ((Lq + 31) / 32);
        char *ws = static_cast<char *>(workspace);
        a.morder = reinterpret_cast<int32_t *>(ws + round_up_256(tiles * (size_t)a.mc_stride));
        a.mwork = reinterpret_cast<int *>(ws + round_up_256(tiles * (size_t)a.mc_stride) +
                                          round_up_256(tiles * 4));
    }

    gqa_status st = check_device();
    if (st != GQA_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (rope) {
        gqa::RopeArgs r;
        r.x = k;
        r.out = k_rot;
        r.cos = rope_cos;
        r.sin = rope_sin;
        r.rows = (long long)B * Lk * h_kv;
        r.L = Lk;
        r.h = h_kv;
        r.pos = nullptr;
        r.x2 = nullptr;
        r.out2 = nullptr;
        r.rows2 = 0;
        r.h2 = 1;
        if (gqa::launch_rope_k_bf16(r, d, stream) != 0) return GQA_ERR_LAUNCH;
        a.k = k_rot;
    }
    int rc = dt == GQA_BF16 ? gqa::launch_prefill_bf16(a, d, causal != 0, stream)
                            : gqa::launch_prefill_f32(a, d, causal != 0, stream);
    return rc == 0 ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

gqa_status gqa_prefill(const void *q, const void *k, const void *v, void *o, int B, int L,
                       int h_q, int h_kv, int d, gqa_dtype dt, int causal, float scale,
                       void *hip_stream) {
    return prefill_impl(q, k, v, o, B, L, L, h_q, h_kv, d, dt, causal, scale, hip_stream);
}

gqa_status gqa_prefill_chunk(const void *q, const void *k, const void *v, void *o, int B,
                             int L_q, int L_k, int h_q, int h_kv, int d, gqa_dtype dt,
                             int causal, float scale, void *hip_stream) {
    return prefill_impl(q, k, v, o, B, L_q, L_k, h_q, h_kv, d, dt, causal, scale, hip_stream);
}

gqa_status gqa_prefill_rope(const void *q, const void *k, const void *v, const float *cos_table,
                            const float *sin_table, void *o, void *k_rot, int B, int L, int h_q,
                            int h_kv, int d, gqa_dtype dt, int causal, float scale,
                            void *hip_stream) {
    return prefill_impl(q, k, v, o, B, L, L, h_q, h_kv, d, dt, causal, scale, hip_stream,
                        cos_table, sin_table, k_rot, true);
}

gqa_status gqa_prefill_varlen(const void *q, const void *k, const void *v, void *o,
                              const int32_t *kv_lens, int B, int L, int h_q, int h_kv, int d,
                              gqa_dtype dt, int causal, float scale, void *hip_stream) {
    return prefill_impl(q, k, v, o, B, L, L, h_q, h_kv, d, dt, causal, scale, hip_stream, nullptr,
                        nullptr, nullptr, false, kv_lens, true);
}

gqa_status gqa_prefill_mask(const void *q, const void *k, const void *v, const uint8_t *mask,
                            long long mask_row_stride, long long mask_batch_stride, void *o,
                            int B, int L_q, int L_k, int h_q, int h_kv, int d, gqa_dtype dt,
                            int causal, float scale, void *workspace, size_t workspace_bytes,
                            void *hip_stream) {
    return prefill_impl(q, k, v, o, B, L_q, L_k, h_q, h_kv, d, dt, causal, scale, hip_stream,
                        nullptr, nullptr, nullptr, false, nullptr, false, mask, mask_row_stride,
                        mask_batch_stride, true, workspace, workspace_bytes);
}

size_t gqa_prefill_mask_workspace_bytes(int B, int L_q, int L_k) {
    if (B <= 0 || L_q <= 0 || L_k < L_q) return 0;
    const size_t tiles = (size_t)B * (size_t)((L_q + 31) / 32);  // at most, 32 rows a tile
    return round_up_256(tiles * (size_t)mask_summary_stride(L_k)) + round_up_256(tiles * 4) + 256;
}

int gqa_decode_default_splits(void) { return kDefaultSplits; }

size_t gqa_decode_workspace_bytes(int B, int h_q, int h_kv, int d, int num_splits) {
    if (B <= 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0 || (d != 64 && d != 128) ||
        !splits_valid(num_splits))
        return 0;
    const int nw = num_splits == 0 ? kDefaultSplits : num_splits;
    const int n_qsub = (h_q / h_kv + 15) / 16;
    const size_t slots = (size_t)nw + (size_t)B * h_kv * n_qsub;
    return round_up_256(slots * 16 * d * sizeof(float)) + round_up_256(slots * 16 * sizeof(float));
}

}  // extern "C"

namespace {

// Shared by both decode entry points; k_new/v_new non-null selects the append
// form (the new rows are written at seqlens[b] and attended as well).
// Paged caches pass layout kLayoutPaged, the block table and its shape, and
// S = 0 (the logical capacity is max_blocks * page_size).
gqa_status decode_impl(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                       const void *v_cache, const int32_t *seqlens, void *o, int B, int h_q,
                       int h_kv, int S, int d, gqa_dtype dt, int num_splits, void *workspace,
                       size_t workspace_bytes, void *hip_stream, int layout = gqa::kLayoutHeadMajor,
                       const int32_t *block_table = nullptr, int page_size = 0,
                       int max_blocks = 0, bool use_scratch = false) {
    // use_scratch: the workspace is the library's fixed scratch of this device
    // (gqa_decode_noalloc); a call needing more is refused
    const bool append = k_new != nullptr || v_new != nullptr;
    if (!q || !k_cache || !v_cache || !seqlens || !o) return GQA_ERR_NULL_POINTER;
    if (layout == gqa::kLayoutPaged) {
        if (!block_table) return GQA_ERR_NULL_POINTER;
        if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0) return GQA_ERR_ALIGNMENT;
        if (page_size <= 0 || page_size % 32 != 0 || max_blocks <= 0) return GQA_ERR_SIZE;
        if ((int64_t)max_blocks * page_size > 0x7fffffff) return GQA_ERR_SIZE;
        if ((int64_t)B * max_blocks > 0x7fffffff) return GQA_ERR_SIZE;
        S = max_blocks * page_size;
    }
    if (append && (!k_new || !v_new)) return GQA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
        return GQA_ERR_ALIGNMENT;
    if (append && (!aligned16(k_new) || !aligned16(v_new))) return GQA_ERR_ALIGNMENT;
    if (B <= 0 || h_q <= 0 || h_kv <= 0 || S <= 0) return GQA_ERR_SIZE;
    if (h_q % h_kv != 0) return GQA_ERR_HEADS;
    if (d != 64 && d != 128) return GQA_ERR_HEAD_DIM;
    if (dt != GQA_BF16) return GQA_ERR_DTYPE;
    if (!splits_valid(num_splits)) return GQA_ERR_SIZE;
    if ((int64_t)B * h_q > 0x7fffffff / 4) return GQA_ERR_SIZE;
    const size_t need = gqa_decode_workspace_bytes(B, h_q, h_kv, d, num_splits);
    if (use_scratch) {
        if (need > kScratchBytes) return GQA_ERR_SCRATCH;
    } else if (!workspace || !aligned16(workspace) || workspace_bytes < need) {
        return GQA_ERR_WORKSPACE;
    }

    gqa::DecodeArgs a;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_new = k_new;
    a.v_new = v_new;
    a.extra = append ? 1 : 0;
    a.seqlens = seqlens;
    a.o = o;
    a.B = B;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.G = h_q / h_kv;
    a.S = S;
    a.NW = num_splits == 0 ? kDefaultSplits : num_splits;
    a.n_qsub = (a.G + 15) / 16;
    const size_t slots = (size_t)a.NW + (size_t)B * h_kv * a.n_qsub;
    a.c = (float)(1.4426950408889634 / sqrt((double)d));
    a.layout = layout;
    a.block_table = block_table;
    a.page_size = page_size;
    a.max_blocks = max_blocks;

    gqa_status st = check_device();
    if (st != GQA_OK) return st;
    if (use_scratch) {
        workspace = device_scratch();
        if (!workspace) return GQA_ERR_DEVICE;
    }
    a.opart = static_cast<float *>(workspace);
    a.lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                      round_up_256(slots * 16 * d * sizeof(float)));
    int rc = gqa::launch_decode_bf16(a, d, static_cast<hipStream_t>(hip_stream));
    return rc == 0 ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *seqlens, void *o, int B, int h_q, int h_kv, int S, int d,
                      gqa_dtype dt, int num_splits, void *workspace, size_t workspace_bytes,
                      void *hip_stream) {
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, dt,
                       num_splits, workspace, workspace_bytes, hip_stream);
}

size_t gqa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *seqlens, void *o, int B, int h_q, int h_kv, int S,
                              int d, gqa_dtype dt, int num_splits, void *hip_stream) {
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, dt,
                       num_splits, nullptr, 0, hip_stream, gqa::kLayoutHeadMajor, nullptr, 0, 0,
                       true);
}

gqa_status gqa_decode_token_major(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *seqlens, void *o, int B, int h_q, int h_kv, int S,
                                  int d, gqa_dtype dt, int num_splits, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, dt,
                       num_splits, workspace, workspace_bytes, hip_stream, gqa::kLayoutTokenMajor);
}

gqa_status gqa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                            const int32_t *block_table, const int32_t *seqlens, void *o, int B,
                            int h_q, int h_kv, int page_size, int max_blocks, int d, gqa_dtype dt,
                            int num_splits, void *workspace, size_t workspace_bytes,
                            void *hip_stream) {
    return decode_impl(q, nullptr, nullptr, k_pages, v_pages, seqlens, o, B, h_q, h_kv, 0, d, dt,
                       num_splits, workspace, workspace_bytes, hip_stream, gqa::kLayoutPaged,
                       block_table, page_size, max_blocks);
}

size_t gqa_decode_rope_workspace_bytes(int B, int h_q, int h_kv, int d, int num_splits) {
    const size_t base = gqa_decode_workspace_bytes(B, h_q, h_kv, d, num_splits);
    if (base == 0) return 0;
    return base + round_up_256((size_t)B * h_q * d * 2) + round_up_256((size_t)B * h_kv * d * 2);
}

gqa_status gqa_decode_append_rope(const void *q, const void *k_new, const void *v_new,
                                  void *k_cache, void *v_cache, const int32_t *seqlens,
                                  const float *cos_table, const float *sin_table, void *o, int B,
                                  int h_q, int h_kv, int S, int d, gqa_dtype dt, int num_splits,
                                  void *workspace, size_t workspace_bytes, void *hip_stream) {
    // everything the decode checks, checked here too: nothing is enqueued
    // unless the whole call is valid
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !seqlens || !o || !cos_table ||
        !sin_table)
        return GQA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(o) || !aligned16(cos_table) || !aligned16(sin_table) ||
        (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
        return GQA_ERR_ALIGNMENT;
    if (B <= 0 || h_q <= 0 || h_kv <= 0 || S <= 0) return GQA_ERR_SIZE;
    if (h_q % h_kv != 0) return GQA_ERR_HEADS;
    if (d != 64 && d != 128) return GQA_ERR_HEAD_DIM;
    if (dt != GQA_BF16) return GQA_ERR_DTYPE;
    if (!splits_valid(num_splits)) return GQA_ERR_SIZE;
    if ((int64_t)B * h_q > 0x7fffffff / 4) return GQA_ERR_SIZE;
    const size_t base = gqa_decode_workspace_bytes(B, h_q, h_kv, d, num_splits);
    const size_t need = gqa_decode_rope_workspace_bytes(B, h_q, h_kv, d, num_splits);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return GQA_ERR_WORKSPACE;
    gqa_status st = check_device();
    if (st != GQA_OK) return st;

    // the rotated q and k_new rows go to the workspace after the decode's part
    char *q_rot = static_cast<char *>(workspace) + base;
    char *k_rot = q_rot + round_up_256((size_t)B * h_q * d * 2);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    gqa::RopeArgs r;
    r.cos = cos_table;
    r.sin = sin_table;
    r.L = S;
    r.pos = seqlens;
    r.x = q;  // q rows, then k_new rows, in one launch
    r.out = q_rot;
    r.rows = (long long)B * h_q;
    r.h = h_q;
    r.x2 = k_new;
    r.out2 = k_rot;
    r.rows2 = (long long)B * h_kv;
    r.h2 = h_kv;
    if (gqa::launch_rope_k_bf16(r, d, stream) != 0) return GQA_ERR_LAUNCH;
    return decode_impl(q_rot, k_rot, v_new, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, dt,
                       num_splits, workspace, base, hip_stream);
}

gqa_status gqa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                             void *v_cache, const int32_t *seqlens, void *o, int B, int h_q,
                             int h_kv, int S, int d, gqa_dtype dt, int num_splits,
                             void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (!k_new || !v_new) return GQA_ERR_NULL_POINTER;
    return decode_impl(q, k_new, v_new, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, dt,
                       num_splits, workspace, workspace_bytes, hip_stream);
}

}  // extern "C"
