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
// rows); wave w owns 32 query rows.  The workgroup walks the key tiles (BC = 64
// keys) that hold an allowed key for one of its rows; tiles wholly outside the
// mask are never visited and element masking runs only on tiles that straddle the
// mask or the sequence end.  A wave skips the matrix work of tiles that hold no
// allowed key for its own 32 rows.
//
// K/V staging.  Each K and V tile goes HBM -> LDS directly (global_load_lds_dwordx4,
// no VGPR round trip), row-major with the 16-byte chunks of a row XOR-swizzled by
// the row index, into one of two buffers: tile t+1 streams in while tile t is
// consumed, one barrier per tile.  The two buffers are distinct LDS arrays and the
// tile loop is unrolled by two, so every LDS read names its buffer statically and
// the compiler can see it never aliases the load in flight into the other one.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 64-wide wavefront).  Each wave
// computes the transposed score block S^T = K_tile Q_w^T (keys x queries), so a
// lane holds scores of ONE query (column n = lane % 32) for 32 of the 64 keys: row
// max and sums are in-lane plus one exchange with lane ^ 32 (v_permlane32_swap).
// The probabilities never leave registers: the C layout of S^T, packed to bf16, is
// the B operand of O^T += V^T P^T, where the 8 keys a lane holds per 16-key slab
// are {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); the A operand V^T is read from the
// row-major V tile with the transposing LDS read ds_read_b64_tr_b16 in exactly
// that key order (a contraction index may be permuted, as long as both operands
// agree).
//
// Softmax bookkeeping (log2 domain, c = |scale| log2 e): the running maximum is
// raised only when some row of the wave grows by more than TAU (then the O
// accumulator and sums are rescaled), so most tiles skip the rescale.  Two sums
// are kept: the fp32 sum of the probabilities (for LSE) and the sum of the same
// probabilities rounded to bf16 (v_dot2 with ones), which normalises O: O is then
// an exact convex combination of V rows with the rounded weights, and the bf16
// rounding of P perturbs relative weights only.
//
// Data in HBM: q, k, v, out are contiguous [B, H, N, d] bf16, lse is [B, H, N] fp32.
// Q is read once into registers, K and V once per query block (mostly L2/MALL
// hits), O and LSE written once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn_bf16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BC = 64;              // keys per tile

template <int V>
struct IntC { static constexpr int value = V; };
constexpr float TAU = 8.0f;         // lazy rescale threshold (log2 domain)

template <int D, int NW>
struct Cfg {
    static constexpr int NT = 64 * NW;              // threads per workgroup
    static constexpr int BR = 32 * NW;              // query rows per workgroup
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int TILE_BYTES = BC * D * 2;   // one K or V tile
    static constexpr int BUF_BYTES = 2 * TILE_BYTES;             // K tile + V tile
    static constexpr int LDS_BYTES = 2 * BUF_BYTES;              // both buffers
    static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / NW;  // 1 KB per wave instruction
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 workgroup");
    static_assert(TILE_BYTES % (1024 * NW) == 0, "tile must split evenly over the waves");
    static_assert(D == 64 || D == 128, "head dim");
};

// XOR applied to the chunk index of a row.  It makes both LDS read patterns
// conflict-free on 64 banks: 16 consecutive rows at one chunk (K operand, 16-byte
// reads) and 4 consecutive rows x 4 consecutive chunks (V operand, transposing
// 8-byte reads).
template <int D>
__device__ __forceinline__ int swz(int row) {
    if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

__device__ __forceinline__ float swap32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap32_add(float x) {
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

__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds_base, int byte_off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_base + byte_off));
    return __builtin_bit_cast(bf16x4, r);
}

template <int D, int NW, int MASK>
__global__ __launch_bounds__(64 * NW, 2)
void fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                int BH, int N, int nqt, float c_log2, int negate_q, int window) {
    using C = Cfg<D, NW>;
    constexpr int NS = D / 16;       // 16-dim slabs of the contraction over d
    constexpr int ND = D / 32;       // 32-row blocks of O^T
    constexpr int CPR = C::CPR;
    __shared__ __attribute__((aligned(1024))) char lds0[C::BUF_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds1[C::BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // ---- per-lane LDS addresses (byte offsets within a K or V tile)
    // loader: wave instruction i fills 1 KB block b = wave * LPW + i; lane -> slot
    int ld_row[C::LOADS_PER_WAVE], ld_col[C::LOADS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
        const int slot = (wave * C::LOADS_PER_WAVE + i) * 64 + lane;
        const int row = slot / CPR;
        ld_row[i] = row;
        ld_col[i] = ((slot % CPR) ^ swz<D>(row)) * 8;
    }
    // K operand: row ln (and 32 + ln, same swizzle), chunk 2 s + hl
    int kaddr[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kaddr[s] = (ln * CPR + ((2 * s + hl) ^ swz<D>(ln))) * 16;
    // V operand: transposing reads; read r of d-block j, supplier lane (g, s16)
    int vaddr[2][ND];
    {
        const int g = lane >> 4, s16 = lane & 15;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < ND; ++j) {
                const int rr = 8 * r + 4 * hl + (s16 >> 2);                 // key within a 16-key slab
                const int chunk = 4 * j + 2 * (g & 1) + ((s16 & 3) >> 1);
                vaddr[r][j] = (rr * CPR + (chunk ^ swz<D>(rr))) * 16 + (s16 & 1) * 8;
            }
    }

    int t_lo, t_hi;
    tile_range<MASK>(q0, min(q0 + C::BR, N) - 1, N, window, t_lo, t_hi);
    int w_lo = 1, w_hi = 0;                      // this wave's own tile range (empty if no rows)
    if (qw0 < N) tile_range<MASK>(qw0, min(qw0 + 31, N - 1), N, window, w_lo, w_hi);

    // issue the direct HBM -> LDS loads of key tile t into buffer `kb`
    auto load_tile = [&](int t, char* kb) {
        const int key0 = t * BC;
        char* vb = kb + C::TILE_BYTES;
#pragma unroll
        for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
            const int row = min(key0 + ld_row[i], N - 1);       // rows past the end: any valid row, masked later
            const size_t off = (size_t)row * D + ld_col[i];
            const int blk = (wave * C::LOADS_PER_WAVE + i) * 1024;
            __builtin_amdgcn_global_load_lds((const void*)(Kh + off), (lds_void*)(kb + blk), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(Vh + off), (lds_void*)(vb + blk), 16, 0, 0);
        }
    };

    f32x16 o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
    float m_run = -INFINITY;     // running max of c_log2 * s (log2 domain), lazily raised
    float l_exp = 0.f;           // this lane's share of sum p (fp32)
    float l_rnd = 0.f;           // this lane's share of sum bf16(p)

    // one tile: consume buffer B (tile t), stream tile t+1 into the other buffer
    auto step = [&](auto bufc, int t) {
        constexpr int B = decltype(bufc)::value;
        const char* kb = B ? lds1 : lds0;
        const char* vb = kb + C::TILE_BYTES;
        if (t < t_hi) load_tile(t + 1, B ? lds0 : lds1);

        if (t >= w_lo && t <= w_hi) {
            const int key0 = t * BC;
            // ---- S^T = K_tile Q^T : two 32-key blocks x 32 queries
            f32x16 s0, s1;
#pragma unroll
            for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb + kaddr[s]);
                const bf16x8 kc = *reinterpret_cast<const bf16x8*>(kb + kaddr[s] + 32 * CPR * 16);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qreg[s], s1, 0, 0, 0);
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
            mx = swap32_max(mx) * c_log2;                    // full row max, scaled (c_log2 > 0)
            const float m_new = fmaxf(m_run, mx);
            if (__any(m_new > m_run + TAU)) {
                const float base_new = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - base_new);   // 0 when m_run = -inf
                l_exp *= alpha;
                l_rnd *= alpha;
#pragma unroll
                for (int j = 0; j < ND; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
                m_run = m_new;
            }
            const float base = (m_run == -INFINITY) ? 0.f : m_run;
            bf16x8 p[4];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c_log2, -base));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r + 1], c_log2, -base));
                const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c_log2, -base));
                const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r + 1], c_log2, -base));
                l_exp += (e0 + e1) + (e2 + e3);
                bf16x2 pa, pb;
                pa[0] = (__bf16)e0; pa[1] = (__bf16)e1;
                pb[0] = (__bf16)e2; pb[1] = (__bf16)e3;
                l_rnd = __builtin_amdgcn_fdot2_f32_bf16(pa, (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, l_rnd, false);
                l_rnd = __builtin_amdgcn_fdot2_f32_bf16(pb, (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, l_rnd, false);
                p[r >> 3][r & 7] = pa[0]; p[r >> 3][(r & 7) + 1] = pa[1];
                p[2 + (r >> 3)][r & 7] = pb[0]; p[2 + (r >> 3)][(r & 7) + 1] = pb[1];
            }

            // ---- O^T += V^T P^T : 4 slabs of 16 keys x ND blocks of 32 dims
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int j = 0; j < ND; ++j) {
                    const bf16x4 lo = lds_read_tr(vb, vaddr[0][j] + ks * 16 * CPR * 16);
                    const bf16x4 hi = lds_read_tr(vb, vaddr[1][j] + ks * 16 * CPR * 16);
                    const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[ks], o[j], 0, 0, 0);
                }
            }
        }

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    load_tile(t_lo, lds0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int t = t_lo; t <= t_hi; t += 2) {
        step(IntC<0>{}, t);
        if (t + 1 <= t_hi) step(IntC<1>{}, t + 1);
    }

    // ---- epilogue: O = acc / sum bf16(p) (bf16, nearest even), LSE = (m + log2 sum p) ln 2
    const float le = swap32_add(l_exp);
    const float lr = swap32_add(l_rnd);
    if (my_q < N) {
        const float inv = 1.0f / lr;
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
        if (hl == 0) LSE[(size_t)bh * N + my_q] = (m_run + __builtin_amdgcn_logf(le)) * 0.69314718055994531f;
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
