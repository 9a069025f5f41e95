// Exact blockwise attention forward, bf16 inputs, fp32 accumulation, gfx950 (CDNA4).
//
// What is computed: softmax(scale * Q K^T) V per (batch, head), with masked keys
// excluded, plus the natural-log log-sum-exp of every row ("Transformer多头注意力8头并行
// 计算PyTorch实现与CUDA核函数优化", §1 and §2.2).  How: the blockwise method of the
// "Blockwise Parallel Transformer in PyTorch" page (every query block sees every
// key, so the result is exact) fused into one kernel in the spirit of the fused
// kernel of the Mosaic long-sequence attention page, §3.2 (K/V tiles staged on
// chip, score, softmax and the V product fused, one division by the running sum at
// the end), with the running maximum that sketch leaves out (its §5.1: exp
// overflow is the source of NaN; work relative to the maximum, in log space).
//
// Work decomposition.  One workgroup per (batch*head, block of BR = 32*NW query
// rows); wave w of the workgroup owns 32 query rows.  The workgroup walks the key
// tiles (BC = 64 keys) that hold an allowed key for one of its rows; whole tiles
// outside the mask are never visited, and element masking runs only on tiles that
// straddle the mask or the sequence end.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 64-wide wavefront).  Each wave
// computes the transposed score block S^T = K_tile Q_w^T (keys x queries), so a
// lane holds scores of ONE query (column n = lane % 32) for 32 of the 64 keys; the
// row max and row sum are in-lane reductions plus one exchange with lane ^ 32
// (v_permlane32_swap).  The probabilities stay in registers: the C layout of S^T
// is reused directly as the B operand of O^T += V^T P^T after packing to bf16, with
// the key order of each 16-key slab permuted identically on the V^T side (a
// contraction index may be permuted freely).  V^T is stored in LDS transposed and
// in that permuted key order, so the A operand is one 16-byte LDS read per lane.
//
// Data in HBM: q, k, v, out are contiguous [B, H, N, d] bf16, lse is [B, H, N] fp32.
// Q is read once into registers, K and V once per query block (served mostly from
// L2/MALL), O and LSE written once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn_bf16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BC = 64;              // keys per tile
constexpr float TAU = 8.0f;         // lazy rescale threshold (log2 domain)

template <int D, int NW>
struct Cfg {
    static constexpr int NT = 64 * NW;          // threads per workgroup
    static constexpr int BR = 32 * NW;          // query rows per workgroup
    static constexpr int KST = D + 8;           // K tile row stride (elements), keeps 16 B reads conflict-free
    static constexpr int VST = BC + 8;          // V^T tile row stride (elements)
    static constexpr int K_ELEMS = BC * KST;
    static constexpr int V_ELEMS = D * VST;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;       // two buffers of bf16
    static constexpr int K_CHUNKS = BC * D / 8;               // 16-byte chunks in a K tile
    static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
    static constexpr int V_UNITS = (BC / 4) * (D / 8);        // (4 keys x 8 dims) units of a V tile
    static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 workgroup");
    static_assert(D % 32 == 0, "head dim must be a multiple of 32");
};

// Position of key k (0..15) of a 16-key slab inside the permuted V^T row: lane half
// h of the P^T operand holds keys {4h..4h+3, 8+4h..8+4h+3} (the S^T C layout), and
// those 8 keys must sit contiguously at positions 8h..8h+7.
__device__ __forceinline__ int slab_pos(int k) {
    return ((k >> 2) & 1) * 8 + (k >> 3) * 4 + (k & 3);
}

__device__ __forceinline__ float wave_swap32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_swap32_add(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int MASK>
__device__ __forceinline__ bool key_allowed(int qi, int kj, int N, int window) {
    if (kj >= N) return false;
    if (MASK == ATTN_MASK_CAUSAL) return kj <= qi;
    if (MASK == ATTN_MASK_WINDOW) return (qi - kj <= window) && (kj - qi <= window);
    return true;
}

// Inclusive key-tile range holding an allowed key for some row of [r0, r1].
template <int MASK>
__device__ __forceinline__ void tile_range(int r0, int r1, int N, int window, int& lo, int& hi) {
    const int last = (N - 1) / BC;
    if (MASK == ATTN_MASK_CAUSAL) {
        lo = 0;
        hi = min(last, r1 / BC);
    } else if (MASK == ATTN_MASK_WINDOW) {
        lo = max(0, r0 - window) / BC;
        hi = min(N - 1, r1 + window) / BC;
    } else {
        lo = 0;
        hi = last;
    }
}

template <int D, int NW>
struct TileRegs {
    u32x4 k[Cfg<D, NW>::K_PER_T];
    u32x4 v[Cfg<D, NW>::V_PER_T][4];
};

template <int D, int NW>
__device__ __forceinline__ void load_tile(TileRegs<D, NW>& tr, const __bf16* __restrict__ Kh,
                                          const __bf16* __restrict__ Vh, int key0, int N, int tid) {
    using C = Cfg<D, NW>;
    constexpr int CPR = D / 8;                        // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
        const int c = tid + i * C::NT;
        const int row = c / CPR, col = (c % CPR) * 8;
        u32x4 val = {0u, 0u, 0u, 0u};
        if ((C::K_CHUNKS % C::NT == 0 || c < C::K_CHUNKS) && key0 + row < N)
            val = *reinterpret_cast<const u32x4*>(Kh + (size_t)(key0 + row) * D + col);
        tr.k[i] = val;
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
        const int u = tid + i * C::NT;
        const int grp = u / CPR, col = (u % CPR) * 8;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + grp * 4 + r;
            u32x4 val = {0u, 0u, 0u, 0u};
            if ((C::V_UNITS % C::NT == 0 || u < C::V_UNITS) && key < N)
                val = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + col);
            tr.v[i][r] = val;
        }
    }
}

template <int D, int NW>
__device__ __forceinline__ void store_tile(const TileRegs<D, NW>& tr, __bf16* Ks, __bf16* Vt, int tid) {
    using C = Cfg<D, NW>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
        const int c = tid + i * C::NT;
        if (C::K_CHUNKS % C::NT == 0 || c < C::K_CHUNKS) {
            const int row = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<u32x4*>(Ks + row * C::KST + col) = tr.k[i];
        }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
        const int u = tid + i * C::NT;
        if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
            const int grp = u / CPR, col = (u % CPR) * 8;
            const int key = grp * 4;                                  // first of 4 keys
            const int pos = (key >> 4) * 16 + slab_pos(key & 15);    // 4 consecutive positions
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // dword w of each row holds dims (col+2w, col+2w+1)
                const uint32_t a0 = tr.v[i][0][w], a1 = tr.v[i][1][w];
                const uint32_t a2 = tr.v[i][2][w], a3 = tr.v[i][3][w];
                const uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
                const uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
                const uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
                u32x2 even = {lo01, lo23}, odd = {hi01, hi23};
                *reinterpret_cast<u32x2*>(Vt + (col + 2 * w) * C::VST + pos) = even;
                *reinterpret_cast<u32x2*>(Vt + (col + 2 * w + 1) * C::VST + pos) = odd;
            }
        }
    }
}

template <int D, int NW, int MASK>
__global__ __launch_bounds__(64 * NW, 2)
void fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                int BH, int N, int nqt, float c_log2, int negate_q, int window) {
    using C = Cfg<D, NW>;
    constexpr int NS = D / 16;       // 16-dim slabs of the contraction over d
    constexpr int ND = D / 32;       // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * C::BUF_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;        // lane half
    const int ln = lane & 31;

    // Heaviest query blocks first for the causal mask; the (batch, head) index
    // varies fastest, so with BH a multiple of 8 every block of a head lands on the
    // same XCD (workgroups are dealt to the 8 XCDs round robin) and shares its L2.
    const int id = blockIdx.x;
    const int rank = id / BH;
    const int bh = id - rank * BH;
    const int qt = (MASK == ATTN_MASK_CAUSAL) ? (nqt - 1 - rank) : rank;
    const int q0 = qt * C::BR;

    const size_t head = (size_t)bh * N * D;
    const __bf16* Qh = Q + head;
    const __bf16* Kh = K + head;
    const __bf16* Vh = V + head;

    const int qw0 = q0 + wave * 32;              // first row of this wave
    const int my_q = qw0 + ln;                   // the query this lane's column holds
    const int qrow = min(my_q, N - 1);

    // Q operand (B of S^T = K Q^T): lane holds Q[my_q][16 s + 8 hl .. +8].
    bf16x8 qreg[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + s * 16 + hl * 8);
        if (negate_q) raw ^= 0x80008000u;        // exact sign flip: scale < 0 runs as -q with |scale|
        qreg[s] = __builtin_bit_cast(bf16x8, raw);
    }

    int t_lo, t_hi;
    tile_range<MASK>(q0, min(q0 + C::BR, N) - 1, N, window, t_lo, t_hi);
    int w_lo = 1, w_hi = 0;                      // this wave's own tile range (empty if no rows)
    if (qw0 < N) tile_range<MASK>(qw0, min(qw0 + 31, N - 1), N, window, w_lo, w_hi);

    f32x16 o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
    float m_run = -INFINITY;     // running max of c_log2 * s (log2 domain), lazily updated
    float l_run = 0.f;           // this lane's share of the running sum

    TileRegs<D, NW> tr;
    load_tile<D, NW>(tr, Kh, Vh, t_lo * BC, N, tid);
    store_tile<D, NW>(tr, lds, lds + C::K_ELEMS, tid);
    __syncthreads();

    for (int t = t_lo; t <= t_hi; ++t) {
        const int cur = (t - t_lo) & 1;
        __bf16* Ks = lds + cur * C::BUF_ELEMS;
        __bf16* Vt = Ks + C::K_ELEMS;
        if (t < t_hi) load_tile<D, NW>(tr, Kh, Vh, (t + 1) * BC, N, tid);

        if (t >= w_lo && t <= w_hi) {
            const int key0 = t * BC;
            // ---- S^T = K_tile Q^T : two 32-key blocks x 32 queries
            f32x16 s0, s1;
#pragma unroll
            for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + ln * C::KST + s * 16 + hl * 8);
                const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ks + (32 + ln) * C::KST + s * 16 + hl * 8);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qreg[s], s1, 0, 0, 0);
            }

            // ---- element mask, only where the tile straddles the mask or the end
            bool need_mask = key0 + BC > N;
            if (MASK == ATTN_MASK_CAUSAL) need_mask |= key0 + BC - 1 > qw0;
            if (MASK == ATTN_MASK_WINDOW) need_mask |= (key0 < qw0 + 31 - window) || (key0 + BC - 1 > qw0 + window);
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (!key_allowed<MASK>(my_q, kk, N, window)) s0[r] = -INFINITY;
                    if (!key_allowed<MASK>(my_q, kk + 32, N, window)) s1[r] = -INFINITY;
                }
            }

            // ---- online softmax (log2 domain, lazy rescale)
            float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
            mx = wave_swap32_max(mx) * c_log2;               // full row max, scaled (c_log2 > 0)
            const float m_new = fmaxf(m_run, mx);
            if (__any(m_new > m_run + TAU)) {
                const float base_new = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - base_new);   // 0 when m_run = -inf
                l_run *= alpha;
#pragma unroll
                for (int j = 0; j < ND; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
                m_run = m_new;
            }
            const float base = (m_run == -INFINITY) ? 0.f : m_run;
            bf16x8 p[4];
            float lsum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c_log2, -base));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c_log2, -base));
                lsum += e0 + e1;
                p[r >> 3][r & 7] = (__bf16)e0;
                p[2 + (r >> 3)][r & 7] = (__bf16)e1;
            }
            l_run += lsum;

            // ---- O^T += V^T P^T : 4 slabs of 16 keys x ND blocks of 32 dims
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int j = 0; j < ND; ++j) {
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + (j * 32 + ln) * C::VST + ks * 16 + hl * 8);
                    o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[ks], o[j], 0, 0, 0);
                }
            }
        }

        if (t < t_hi) store_tile<D, NW>(tr, lds + (cur ^ 1) * C::BUF_ELEMS, lds + (cur ^ 1) * C::BUF_ELEMS + C::K_ELEMS, tid);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l (bf16, nearest even), LSE = (m + log2 l) ln 2
    const float l_tot = wave_swap32_add(l_run);
    if (my_q < N) {
        const float inv = 1.0f / l_tot;
        __bf16* Orow = O + head + (size_t)my_q * D;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[j][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(Orow + j * 32 + 8 * g + 4 * hl) = val;
            }
        }
        if (hl == 0) LSE[(size_t)bh * N + my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    }
}

template <int D, int NW, int MASK>
static int launch(const AttnLaunch& a) {
    using C = Cfg<D, NW>;
    const int nqt = (a.N + C::BR - 1) / C::BR;
    const long long grid = (long long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd_kernel<D, NW, MASK>), dim3((unsigned)grid), dim3(C::NT), 0, (hipStream_t)a.stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.out, a.lse,
                       a.B * a.H, a.N, nqt, a.c_log2, a.negate_q, a.window);
    return 0;
}

template <int D, int NW>
static int by_mask(const AttnLaunch& a) {
    switch (a.mask_kind) {
        case ATTN_MASK_CAUSAL: return launch<D, NW, ATTN_MASK_CAUSAL>(a);
        case ATTN_MASK_WINDOW: return launch<D, NW, ATTN_MASK_WINDOW>(a);
        default: return launch<D, NW, ATTN_MASK_NONE>(a);
    }
}

}  // namespace attn_bf16

int attn_launch_bf16(const AttnLaunch& a) {
    using namespace attn_bf16;
    if (a.d == 128) return by_mask<128, 4>(a);
    return by_mask<64, 4>(a);
}
