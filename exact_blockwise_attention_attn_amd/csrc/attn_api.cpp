// Host side of the C ABI declared in include/attn.h: argument checks, kernel
// selection and the launch on the caller's stream.  No allocation, no
// synchronisation, no state.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn_launch.h"

namespace {

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

}  // namespace

extern "C" int attn_check_args(const void* q, const void* k, const void* v, const void* out, const float* lse,
                               int B, int H, int N, int d, float scale, int mask_kind, int window, int dtype) {
    if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_PTR;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_BAD_DTYPE;
    if (B <= 0 || H <= 0 || N <= 0) return ATTN_ERR_BAD_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    const uint64_t rows = bh * (uint64_t)N;
    // per-head offsets are 32-bit, the workgroup count stays far below the grid limit
    if ((uint64_t)N * (uint64_t)d >= (1ull << 31) || rows >= (1ull << 31) ||
        bh * (((uint64_t)N + 63) / 64) > (1ull << 24))
        return ATTN_ERR_BAD_SHAPE;
    if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_CAUSAL && mask_kind != ATTN_MASK_WINDOW &&
        mask_kind != ATTN_MASK_CAUSAL_WINDOW)
        return ATTN_ERR_BAD_MASK;
    if ((mask_kind == ATTN_MASK_WINDOW || mask_kind == ATTN_MASK_CAUSAL_WINDOW) && window < 0) return ATTN_ERR_BAD_MASK;
    if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(lse))
        return ATTN_ERR_MISALIGNED;
    const uint64_t eb = dtype == ATTN_DTYPE_F32 ? 4 : 2;
    const uint64_t tb = rows * (uint64_t)d * eb;   // bytes of one [B, H, N, d] tensor
    const uint64_t lb = rows * 4;
    if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) ||
        overlaps(lse, lb, q, tb) || overlaps(lse, lb, k, tb) || overlaps(lse, lb, v, tb) ||
        overlaps(lse, lb, out, tb))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int N, int d, float scale, int mask_kind, int window,
                        int dtype, void* stream) {
    const int st = attn_check_args(q, k, v, out, lse, B, H, N, d, scale, mask_kind, window, dtype);
    if (st != ATTN_OK) return st;

    AttnLaunch a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.d = d;
    const double c = std::fabs((double)scale) * 1.4426950408889634074;   // log2(e)
    a.c_log2 = (float)(c > 1e-30 ? c : 1e-30);
    a.negate_q = scale < 0.f ? 1 : 0;
    a.mask_kind = mask_kind;
    a.window = (mask_kind == ATTN_MASK_WINDOW || mask_kind == ATTN_MASK_CAUSAL_WINDOW) ? (window < N - 1 ? window : N - 1) : 0;
    a.stream = stream;

    (void)hipGetLastError();   // clear a stale error so the check below sees only this launch
    if (dtype == ATTN_DTYPE_BF16)
        attn_launch_bf16(a);
    else
        attn_launch_f32(a);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_bwd_check_args(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                   const float* lse, const void* dq, const void* dk, const void* dv, int B, int H,
                                   int N, int d, float scale, int mask_kind, int window, int dtype) {
    if (!dout || !dq || !dk || !dv) return ATTN_ERR_NULL_PTR;
    const int st = attn_check_args(q, k, v, out, lse, B, H, N, d, scale, mask_kind, window, dtype);
    if (st != ATTN_OK) return st;
    if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_BAD_DTYPE;
    if (misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv)) return ATTN_ERR_MISALIGNED;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t tb = rows * (uint64_t)d * 2;
    const uint64_t lb = rows * 4;
    const void* ins[5] = {q, k, v, out, dout};
    const void* outs[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], tb, ins[j], tb)) return ATTN_ERR_ALIAS;
        if (overlaps(outs[i], tb, lse, lb)) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], tb, outs[j], tb)) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int mask_kind, int window, int dtype, void* stream) {
    const int st = attn_bwd_check_args(q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, scale, mask_kind, window,
                                       dtype);
    if (st != ATTN_OK) return st;
    AttnBwdLaunch a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.H = H; a.N = N; a.d = d;
    const double c = std::fabs((double)scale) * 1.4426950408889634074;
    a.c_log2 = (float)(c > 1e-30 ? c : 1e-30);
    a.negate_q = scale < 0.f ? 1 : 0;
    a.scale = scale;
    a.mask_kind = mask_kind;
    a.window = (mask_kind == ATTN_MASK_WINDOW || mask_kind == ATTN_MASK_CAUSAL_WINDOW) ? (window < N - 1 ? window : N - 1) : 0;
    a.stream = stream;
    (void)hipGetLastError();
    attn_launch_bwd_bf16(a);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

namespace {

// shape check of the split-KV entry points; fills the workspace need when valid
int kv_shape(int B, int H, int Nq, int Nk, int d, int q_offset, int* n_split, uint64_t* ws_bytes) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || q_offset < 0 || (int64_t)q_offset + Nq > Nk)
        return ATTN_ERR_BAD_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    if ((uint64_t)Nk * (uint64_t)d >= (1ull << 31) || bh * (uint64_t)Nk >= (1ull << 31) ||
        bh * (((uint64_t)Nq + 127) / 128) > (1ull << 24))
        return ATTN_ERR_BAD_SHAPE;
    // fp32 partial O [BH, splits, Nq, d], then fp32 partial LSE [BH, splits, Nq], for the
    // most ranges a launch of this shape can use
    *n_split = attn_kv_max_splits(B, H, Nq, Nk, d);
    const uint64_t parts = bh * (uint64_t)*n_split * (uint64_t)Nq;
    *ws_bytes = *n_split > 1 ? parts * (uint64_t)d * 4 + parts * 4 : 0;
    return ATTN_OK;
}

}  // namespace

extern "C" unsigned long long attn_fwd_kv_workspace_size(int B, int H, int Nq, int Nk, int d) {
    int ns;
    uint64_t ws;
    if (kv_shape(B, H, Nq, Nk, d, 0, &ns, &ws) != ATTN_OK) return 0;
    return ws;
}

extern "C" int attn_fwd_kv_check_args(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                      int B, int H, int Nq, int Nk, int d, float scale, int mask_kind, int window,
                                      int q_offset, int dtype, const void* workspace,
                                      unsigned long long workspace_bytes) {
    if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_PTR;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_BAD_DTYPE;
    int ns;
    uint64_t need;
    const int st = kv_shape(B, H, Nq, Nk, d, q_offset, &ns, &need);
    if (st != ATTN_OK) return st;
    if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_CAUSAL && mask_kind != ATTN_MASK_WINDOW &&
        mask_kind != ATTN_MASK_CAUSAL_WINDOW)
        return ATTN_ERR_BAD_MASK;
    if ((mask_kind == ATTN_MASK_WINDOW || mask_kind == ATTN_MASK_CAUSAL_WINDOW) && window < 0) return ATTN_ERR_BAD_MASK;
    if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
    if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_BAD_DTYPE;
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(lse) ||
        (need > 0 && misaligned(workspace)))
        return ATTN_ERR_MISALIGNED;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    const uint64_t qb = bh * (uint64_t)Nq * (uint64_t)d * 2, kb = bh * (uint64_t)Nk * (uint64_t)d * 2;
    const uint64_t lb = bh * (uint64_t)Nq * 4;
    const void* ins[3] = {q, k, v};
    const uint64_t in_b[3] = {qb, kb, kb};
    for (int j = 0; j < 3; ++j) {
        if (overlaps(out, qb, ins[j], in_b[j]) || overlaps(lse, lb, ins[j], in_b[j])) return ATTN_ERR_ALIAS;
        if (need > 0 && overlaps(workspace, need, ins[j], in_b[j])) return ATTN_ERR_ALIAS;
    }
    if (overlaps(lse, lb, out, qb)) return ATTN_ERR_ALIAS;
    if (need > 0 && (overlaps(workspace, need, out, qb) || overlaps(workspace, need, lse, lb))) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

extern "C" int attn_fwd_kv(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq,
                           int Nk, int d, float scale, int mask_kind, int window, int q_offset, int dtype,
                           void* workspace, unsigned long long workspace_bytes, void* stream) {
    const int st = attn_fwd_kv_check_args(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset,
                                          dtype, workspace, workspace_bytes);
    if (st != ATTN_OK) return st;
    int n_split;
    uint64_t need;
    kv_shape(B, H, Nq, Nk, d, q_offset, &n_split, &need);
    AttnLaunch a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.B = B; a.H = H; a.N = Nq; a.d = d;
    const double c = std::fabs((double)scale) * 1.4426950408889634074;
    a.c_log2 = (float)(c > 1e-30 ? c : 1e-30);
    a.negate_q = scale < 0.f ? 1 : 0;
    a.mask_kind = mask_kind;
    a.window = (mask_kind == ATTN_MASK_WINDOW || mask_kind == ATTN_MASK_CAUSAL_WINDOW) ? (window < Nk - 1 ? window : Nk - 1) : 0;
    a.stream = stream;
    float* part_o = need > 0 ? (float*)workspace : nullptr;
    float* part_lse = need > 0 ? part_o + (uint64_t)B * H * n_split * Nq * d : nullptr;
    (void)hipGetLastError();
    attn_launch_kv_bf16(a, Nk, q_offset, part_o, part_lse);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_block_sparse_check_args(const void* q, const void* k, const void* v, const void* out,
                                                const float* lse, int B, int H, int N, int d, float scale, int causal,
                                                const unsigned char* layout, int dtype) {
    const int st = attn_check_args(q, k, v, out, lse, B, H, N, d, scale, ATTN_MASK_NONE, 0, dtype);
    if (st != ATTN_OK) return st;
    if (!layout) return ATTN_ERR_NULL_PTR;
    if (causal != 0 && causal != 1) return ATTN_ERR_BAD_MASK;
    if (dtype != ATTN_DTYPE_BF16) return ATTN_ERR_BAD_DTYPE;
    const uint64_t nb = ((uint64_t)N + ATTN_BLOCK_SPARSE_BLOCK - 1) / ATTN_BLOCK_SPARSE_BLOCK;
    if (nb > ATTN_BLOCK_SPARSE_MAX_BLOCKS) return ATTN_ERR_BAD_SHAPE;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t lay = (uint64_t)H * nb * nb;
    if (overlaps(out, rows * (uint64_t)d * 2, layout, lay) || overlaps(lse, rows * 4, layout, lay))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

extern "C" int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                                     int N, int d, float scale, int causal, const unsigned char* layout, int dtype,
                                     void* stream) {
    const int st = attn_fwd_block_sparse_check_args(q, k, v, out, lse, B, H, N, d, scale, causal, layout, dtype);
    if (st != ATTN_OK) return st;
    AttnLaunch a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.d = d;
    const double c = std::fabs((double)scale) * 1.4426950408889634074;
    a.c_log2 = (float)(c > 1e-30 ? c : 1e-30);
    a.negate_q = scale < 0.f ? 1 : 0;
    a.mask_kind = causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE;
    a.window = 0;
    a.stream = stream;
    (void)hipGetLastError();
    attn_launch_block_bf16(a, layout, causal);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Schedule overrides (attn_set_schedule): process-wide, read at every launch.
static std::atomic<int> g_rows_per_wave{0};
static std::atomic<int> g_head_group{-1};

static std::atomic<int> g_key_groups{-1};
static std::atomic<int> g_work_queue{-1};

int attn_sched_rows_per_wave() { return g_rows_per_wave.load(std::memory_order_relaxed); }
int attn_sched_head_group() { return g_head_group.load(std::memory_order_relaxed); }
int attn_sched_key_groups() { return g_key_groups.load(std::memory_order_relaxed); }
int attn_sched_work_queue() { return g_work_queue.load(std::memory_order_relaxed); }

// Work-queue slots of the forward launches (wq_take in attn_tile.h): a device array,
// one copy per device, whose device address is taken once per device with
// hipGetSymbolAddress (host code never hands the array's name to a kernel); each
// launch that uses the queue takes the next of WQ_SLOTS slots in turn.  A slot is
// left at zero by the last claiming workgroup of the launch that used it, so two
// launches share a slot only if WQ_SLOTS of them run at once on one device.
__device__ __align__(256) unsigned attn_wq_pool[WQ_SLOTS * WQ_SLOT_WORDS];

namespace {
constexpr int WQ_MAX_DEVICES = 64;
std::mutex g_wq_mu;
unsigned* g_wq_base[WQ_MAX_DEVICES];
std::atomic<unsigned> g_wq_next{0};
}  // namespace

unsigned* attn_wq_slot() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= WQ_MAX_DEVICES) return nullptr;
    unsigned* base;
    {
        std::lock_guard<std::mutex> lock(g_wq_mu);
        if (!g_wq_base[dev]) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(attn_wq_pool)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return nullptr;
            }
            g_wq_base[dev] = static_cast<unsigned*>(p);
        }
        base = g_wq_base[dev];
    }
    const unsigned slot = g_wq_next.fetch_add(1u, std::memory_order_relaxed) % WQ_SLOTS;
    return base + slot * WQ_SLOT_WORDS;
}

extern "C" int attn_set_work_queue(int mode) {
    if (mode < -1 || mode > 1) return ATTN_ERR_BAD_SHAPE;
    g_work_queue.store(mode, std::memory_order_relaxed);
    return ATTN_OK;
}

extern "C" int attn_set_schedule(int rows_per_wave, int head_group) {
    if (rows_per_wave != 0 && rows_per_wave != 32 && rows_per_wave != 64) return ATTN_ERR_BAD_SHAPE;
    if (head_group < -1) return ATTN_ERR_BAD_SHAPE;
    g_rows_per_wave.store(rows_per_wave, std::memory_order_relaxed);
    g_head_group.store(head_group, std::memory_order_relaxed);
    return ATTN_OK;
}

extern "C" int attn_set_key_groups(int key_groups) {
    if (key_groups != -1 && key_groups != 1 && key_groups != 2 && key_groups != 4) return ATTN_ERR_BAD_SHAPE;
    g_key_groups.store(key_groups, std::memory_order_relaxed);
    return ATTN_OK;
}

extern "C" const char* attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL_PTR: return "a tensor pointer is NULL";
        case ATTN_ERR_BAD_SHAPE: return "bad shape: B, H, N must be >= 1 and within the size limits";
        case ATTN_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dimension (d must be 64 or 128)";
        case ATTN_ERR_BAD_MASK: return "bad mask: unknown mask kind or negative window";
        case ATTN_ERR_BAD_DTYPE: return "bad dtype (0 = fp32, 1 = bf16; the backward and attn_fwd_kv take bf16 only)";
        case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
        case ATTN_ERR_BAD_SCALE: return "scale is not finite";
        case ATTN_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
        case ATTN_ERR_HIP: return "the HIP runtime reported an error at launch";
        case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than attn_fwd_kv_workspace_size()";
        case ATTN_ERR_SCRATCH_LIMIT:
            return "attn_fwd_kv_noalloc: the shape needs more scratch than ATTN_NOALLOC_SCRATCH_BYTES (64 MiB)";
        default: return "unknown status";
    }
}

extern "C" const char* attn_version(void) {
    return "attn 0.5.0 (gfx950; forward bf16 v_mfma_f32_32x32x16_bf16 and fp32 VALU; block-sparse forward bf16; "
           "split-KV forward and decode bf16; backward bf16)";
}
