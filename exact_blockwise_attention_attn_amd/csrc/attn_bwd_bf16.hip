// Exact attention backward, bf16 inputs, fp32 accumulation, gfx950 (CDNA4).
//
// What is computed: for O = softmax(scale Q K^T) V (masked keys excluded) and an
// upstream gradient dO, the exact gradients
//     dV = P^T dO,   dP = dO V^T,   D_i = <dO_i, O_i>,   dS = P o (dP - D),
//     dQ = scale dS K,   dK = scale dS^T Q,
// with P recomputed from Q, K and the forward's log-sum-exp (P_ij =
// exp(S_ij - LSE_i)) instead of stored: the recomputation the
// "长序列推理中的注意力机制优化策略与实践" page describes for FlashAttention (§3.1), so the
// N x N matrix never exists in the backward either.
//
// Three launches on the caller's stream:
//   prep   D_i = <dO_i, O_i> for every row, parked in the first 4 bytes of dq row i
//          (dq is written last, so it doubles as the scratch for D);
//   dkdv   one workgroup per (batch*head, block of 128 keys); each wave owns 32 keys
//          and walks the query tiles that see them: S and dP (its K and V rows sit
//          in registers, the Q and dO tiles stream through LDS), then
//          dV^T += dO^T P and dK^T += Q^T dS with P and dS straight from registers;
//   dq     one workgroup per (batch*head, block of 128 queries); each wave owns 32
//          queries and walks the key tiles they see: S^T and dP^T (Q and dO rows in
//          registers, K and V tiles in LDS), then dQ^T += K^T dS^T.  It reads D of
//          its own rows before it writes them.
// The matrix-core mapping is the forward's (v_mfma_f32_32x32x16_bf16): products
// whose C layout puts one row (or one column) per lane, so the per-row terms (LSE,
// D) are per lane or per register, and the bf16 P and dS packed from the C layout
// are directly the B operands of the next products; the transposed A operands
// (dO^T, Q^T, K^T) come from the row-major LDS tiles through transposing reads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"
#include "attn_tile.h"

namespace attn_bwd_bf16 {

using namespace attn_tile;

constexpr int NW = 4;                      // waves per workgroup
constexpr int BT = 32;                     // rows of an LDS tile, rows per wave
constexpr int BW = BT * NW;                // rows owned by a workgroup
constexpr float LOG2E = 1.4426950408889634f;

template <int D>
struct Shape {
    static constexpr int NS = D / 16;                  // 16-column slabs of a row
    static constexpr int ND = D / 32;                  // 32-column blocks of an output row
    static constexpr int TILE = BT * D * 2;            // bytes of one tile
    static constexpr int LPW = TILE / 1024 / NW;       // 1 KB direct loads per wave per tile
    static_assert(D == 64 || D == 128, "head dim");
};

// ---- D_i = <dO_i, O_i> (fp32), written into the first 4 bytes of dq row i
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
                                                   char* __restrict__ dq, long long rows) {
    constexpr int LPR = D / 8;                         // lanes per row, 8 elements each
    constexpr int RPW = 64 / LPR;                      // rows per wave
    const int lane = threadIdx.x & 63;
    const long long row = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const int c = lane % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 o = *reinterpret_cast<const u32x4*>(O + row * D + c * 8);
        const u32x4 g = *reinterpret_cast<const u32x4*>(dO + row * D + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = __builtin_fmaf(__uint_as_float(o[w] << 16), __uint_as_float(g[w] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(o[w] & 0xffff0000u), __uint_as_float(g[w] & 0xffff0000u), acc);
        }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (row < rows && c == 0) *reinterpret_cast<float*>(dq + row * D * 2) = acc;
}

// per-lane offsets of this wave's direct loads of a tile (see the layout in attn_tile.h)
template <int D>
struct Loader {
    uint32_t off[Shape<D>::LPW];
    int row[Shape<D>::LPW];
    __device__ __forceinline__ Loader(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < Shape<D>::LPW; ++i) {
            const int b = wave * Shape<D>::LPW + i;
            const int r = 16 * (b % (BT / 16)) + (lane >> 2);
            const int c = 4 * (b / (BT / 16)) + ((lane & 3) ^ ((r >> 2) & 3));
            off[i] = (uint32_t)(r * D + c * 8) * 2u;
            row[i] = r;
        }
    }
    // rows t*BT .. t*BT+BT-1 of a [N, D] head (buffer resource `rs`, head_rsrc) into
    // dst; rows past the end reload row N-1
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int t, int N, char* dst, int wave) const {
        const int r0 = t * BT;
        const uint32_t soff = (uint32_t)r0 * (uint32_t)(2 * D);
#pragma unroll
        for (int i = 0; i < Shape<D>::LPW; ++i) {
            const uint32_t o = off[i] - (uint32_t)max(0, row[i] - (N - 1 - r0)) * (2 * D);
            dma16(rs, (lds_void*)(dst + (wave * Shape<D>::LPW + i) * 1024), o, soff);
        }
    }
};

__device__ __forceinline__ bf16x8 load_row8(const __bf16* p, bool negate) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(p);
    if (negate) raw ^= 0x80008000u;                    // exact sign flip
    return __builtin_bit_cast(bf16x8, raw);
}

// allowed interval [lo, hi] of the other index for index x under the mask (n = N)
template <int MASK, bool X_IS_KEY>
__device__ __forceinline__ void allowed_interval(int x, int N, int window, int& lo, int& hi) {
    lo = 0;
    hi = N - 1;
    if (MASK == ATTN_MASK_CAUSAL) {
        if (X_IS_KEY) lo = x;        // queries i >= key j
        else hi = x;                 // keys j <= query i
    } else if (MASK == ATTN_MASK_WINDOW) {
        lo = max(0, x - window);
        hi = min(N - 1, x + window);
    } else if (MASK == ATTN_MASK_CAUSAL_WINDOW) {
        if (X_IS_KEY) { lo = x; hi = min(N - 1, x + window); }     // queries j <= i <= j + w
        else { lo = max(0, x - window); hi = x; }                   // keys i - w <= j <= i
    }
}

// =====================================================================================
// dK, dV: a workgroup owns 128 keys, a wave 32 of them; the query tiles stream by.
//
// Per query tile the wave runs S = Q_t K^T and dP = dO_t V^T (matrix cores), then
// P = exp2(c S - LSE) and dS = P (dP - D) (vector ALUs), then dV^T += dO_t^T P and
// dK^T += Q_t^T dS (matrix cores); each step depends on the one before.  Two waves per
// SIMD (the register file capped at 256 per wave) let one wave's vector step run
// under the other's matrix products.  That measured faster (+25% on a causal
// 8192-token backward) than software-pipelining the tiles within one wave, which
// needs a second set of S and dP and three LDS stages and so only fits one wave per
// SIMD.  LSE and D are read from LDS four rows at a time, right before use, to stay
// within the cap.
template <int D, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 8)))
void dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                 const __bf16* __restrict__ dO, const float* __restrict__ LSE, const char* __restrict__ dscratch,
                 __bf16* __restrict__ dK, __bf16* __restrict__ dV, int BH, int N, float c_log2, int negate,
                 float scale, int window, int hg) {
    using S_ = Shape<D>;
    constexpr int NS = S_::NS, ND = S_::ND, TILE = S_::TILE;
    __shared__ __attribute__((aligned(1024))) char qbuf0[TILE];
    __shared__ __attribute__((aligned(1024))) char qbuf1[TILE];
    __shared__ __attribute__((aligned(1024))) char gbuf0[TILE];
    __shared__ __attribute__((aligned(1024))) char gbuf1[TILE];
    __shared__ __attribute__((aligned(16))) float lbuf0[BT], lbuf1[BT], dbuf0[BT], dbuf1[BT];
    // at d = 128 the last four of the eight K and V operand slabs of each lane wait in
    // LDS (8 KB per wave) instead of registers: under the 256-register cap the compiler
    // would otherwise reload spilled operands from scratch on every tile, and the
    // unmasked copy of the probability block below would not fit
    constexpr int NL = D == 128 ? 4 : 0;               // slabs kept in LDS
    __shared__ __attribute__((aligned(16))) bf16x8 kvl[NL ? NW * NL * 2 * 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ln = lane & 31;
    const int id = blockIdx.x;
    int kt, bh;                                        // key block: the early ones see the most queries
    grouped_order(id, BH, (N + BW - 1) / BW, hg, kt, bh);
    const int k0 = kt * BW;
    const int k1 = min(k0 + BW, N) - 1;
    const size_t head = (size_t)bh * N * D;
    const int my_key = k0 + BT * wave + ln;
    const int kk = min(my_key, N - 1);

    // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T
    bf16x8 kop[NS], vop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        kop[s] = load_row8(K + head + (size_t)kk * D + 16 * s + 8 * hl, negate);
        vop[s] = load_row8(V + head + (size_t)kk * D + 16 * s + 8 * hl, false);
    }
    if constexpr (NL) {                                // each lane reads back only its own slots
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            kvl[((wave * NL + j) * 2 + 0) * 64 + lane] = kop[NS - NL + j];
            kvl[((wave * NL + j) * 2 + 1) * 64 + lane] = vop[NS - NL + j];
        }
    }
    int q_lo, q_hi;                                    // queries that see this key
    allowed_interval<MASK, true>(kk, N, window, q_lo, q_hi);
    const unsigned q_span = (unsigned)(q_hi - q_lo);

    // query tiles holding a query that sees one of the workgroup's keys
    int t_lo = 0, t_hi = (N - 1) / BT;
    if (MASK == ATTN_MASK_CAUSAL) t_lo = k0 / BT;
    if (MASK == ATTN_MASK_WINDOW) { t_lo = max(0, k0 - window) / BT; t_hi = min(N - 1, k1 + window) / BT; }
    if (MASK == ATTN_MASK_CAUSAL_WINDOW) { t_lo = k0 / BT; t_hi = min(N - 1, k1 + window) / BT; }
    const int n_tiles = t_hi - t_lo + 1;

    const TileOffsets off(lane);
    const Loader<D> ld(wave, lane);
    const float* lse_h = LSE + (size_t)bh * N;

    f32x16 dk[ND], dv[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[j][r] = 0.f; dv[j][r] = 0.f; }

    // LSE and D of the tile's rows: wave 0, one row per lane.  The LSE goes to the log2
    // domain only where it is written to LDS, so nothing waits on these loads early.
    auto stage_load = [&](int t, float& l2, float& dd) __attribute__((always_inline)) {
        const int row = min(t * BT + (lane & 31), N - 1);
        l2 = lse_h[row];
        dd = *reinterpret_cast<const float*>(dscratch + ((size_t)bh * N + row) * D * 2);
    };

    const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(Q + head, (uint32_t)N * (uint32_t)(2 * D));
    const __amdgpu_buffer_rsrc_t grs = buffer_rsrc(dO + head, (uint32_t)N * (uint32_t)(2 * D));
    ld.load(qrs, t_lo, N, qbuf0, wave);
    ld.load(grs, t_lo, N, gbuf0, wave);
    if (wave == 0 && lane < BT) {
        float l2, dd;
        stage_load(t_lo, l2, dd);
        lbuf0[lane] = l2 * LOG2E;
        dbuf0[lane] = dd;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    auto iter = [&](auto parity, int u) __attribute__((always_inline)) {
        constexpr int B = decltype(parity)::value;
        const int t = t_lo + u;
        const char* qb = B ? qbuf1 : qbuf0;
        const char* gb = B ? gbuf1 : gbuf0;
        const float* lb = B ? lbuf1 : lbuf0;
        const float* db = B ? dbuf1 : dbuf0;
        char* qn = B ? qbuf0 : qbuf1;
        char* gn = B ? gbuf0 : gbuf1;
        float* ln_ = B ? lbuf0 : lbuf1;
        float* dn = B ? dbuf0 : dbuf1;
        const bool more = u + 1 < n_tiles;
        float l2n = 0.f, ddn = 0.f;
        // the next tile's loads go out first in the step, after wave 0's LSE and D loads:
        // loads complete in order, so a wait for those (the compiler may place one early)
        // then never waits for the tile as well.  Nothing else in the step reads memory
        // (no register spills), so the tile has the whole step to arrive.
        if (more && wave == 0 && lane < BT) stage_load(t + 1, l2n, ddn);
        if (more) {
            ld.load(qrs, t + 1, N, qn, wave);
            ld.load(grs, t + 1, N, gn, wave);
        }
        // S = Q_t K^T and dP = dO_t V^T: rows = the tile's queries, columns = keys (lanes)
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int o = (k >> 1) * (4 * BT * 16) + ((k & 1) ? off.row_odd : off.row_even);
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qb + o);
            const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gb + o);
            const bool in_lds = k >= NS - NL;
            const int j = in_lds ? k - (NS - NL) : 0;
            const bf16x8 kb_ = in_lds ? kvl[((wave * NL + j) * 2 + 0) * 64 + lane] : kop[k];
            const bf16x8 vb_ = in_lds ? kvl[((wave * NL + j) * 2 + 1) * 64 + lane] : vop[k];
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb_, s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vb_, dp, 0, 0, 0);
        }
        // per row r of the C layout: query 8 (r/4) + 4 hl + r%4 of the tile; LSE and D
        // read four rows at a time, right before use.  The element mask runs only when the
        // tile's queries are not all allowed for every key of the wave.
        bf16x8 pp[2], dsp[2];
        const int rel0 = t * BT + 4 * hl - q_lo;
        auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 a = *reinterpret_cast<const float4*>(lb + 8 * g + 4 * hl);
                const float4 b = *reinterpret_cast<const float4*>(db + 8 * g + 4 * hl);
                const float l2[4] = {a.x, a.y, a.z, a.w}, dd[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int r = 4 * g + e4;
                    const int qoff = 8 * g + e4;
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2[e4]));
                    float p = e;
                    if constexpr (decltype(masked)::value) p = (unsigned)(rel0 + qoff) <= q_span ? e : 0.f;
                    const float ds = p * (dp[r] - dd[e4]);
                    pp[r >> 3][r & 7] = (__bf16)p;
                    dsp[r >> 3][r & 7] = (__bf16)ds;
                }
            }
        };
        {
            const int a0 = t * BT - q_lo;              // the whole tile inside this key's queries?
            if (__any(!(a0 >= 0 && a0 + (BT - 1) <= (int)q_span))) {
                asm volatile("" ::: "memory");
                probs(IntC<1>{});
            } else {
                probs(IntC<0>{});
            }
        }
        // dV^T += dO_t^T P and dK^T += Q_t^T dS (A operands: transposing reads of the tiles)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int j = 0; j < ND; ++j) {
                const int o = j * (4 * BT * 16) + ks * (16 * 4 * 16);
                const bf16x4 g0 = lds_read_tr(gb, o + off.tr[0]);
                const bf16x4 g1 = lds_read_tr(gb, o + off.tr[1]);
                const bf16x4 q0 = lds_read_tr(qb, o + off.tr[0]);
                const bf16x4 q1 = lds_read_tr(qb, o + off.tr[1]);
                dv[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                pp[ks], dv[j], 0, 0, 0);
                dk[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                dsp[ks], dk[j], 0, 0, 0);
            }
        }
        if (more && wave == 0 && lane < BT) {
            // (the empty asm keeps the multiply, and so the wait for the load, here)
            asm volatile("" : "+v"(l2n));
            ln_[lane] = l2n * LOG2E;
            dn[lane] = ddn;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    int u = 0;
    for (; u + 1 < n_tiles; u += 2) {
        iter(IntC<0>{}, u);
        iter(IntC<1>{}, u + 1);
    }
    if (u < n_tiles) iter(IntC<0>{}, u);

    if (my_key < N) {
        __bf16* dkr = dK + head + (size_t)my_key * D;
        __bf16* dvr = dV + head + (size_t)my_key * D;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 a, b;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = (__bf16)(dk[j][4 * g + e] * scale);
                    b[e] = (__bf16)dv[j][4 * g + e];
                }
                *reinterpret_cast<bf16x4*>(dkr + j * 32 + 8 * g + 4 * hl) = a;
                *reinterpret_cast<bf16x4*>(dvr + j * 32 + 8 * g + 4 * hl) = b;
            }
        }
    }
}

// =====================================================================================
// dQ: a workgroup owns 128 queries, a wave 32 of them; the key tiles stream by.
template <int D, int MASK>
__global__ __launch_bounds__(256, 1)
void dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
               const __bf16* __restrict__ dO, const float* __restrict__ LSE, char* __restrict__ dq_io,
               int BH, int N, int nqt, float c_log2, int negate, float scale, int window, int hg) {
    using S_ = Shape<D>;
    constexpr int NS = S_::NS, ND = S_::ND, TILE = S_::TILE;
    __shared__ __attribute__((aligned(1024))) char kbuf0[TILE];
    __shared__ __attribute__((aligned(1024))) char kbuf1[TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf0[TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ln = lane & 31;
    const int id = blockIdx.x;
    int rank, bh;
    grouped_order(id, BH, nqt, hg, rank, bh);
    const int qt = (MASK == ATTN_MASK_CAUSAL) ? (nqt - 1 - rank) : rank;   // heaviest first
    const int q0 = qt * BW;
    const size_t head = (size_t)bh * N * D;
    const int my_q = q0 + BT * wave + ln;
    const int qi = min(my_q, N - 1);

    // Q and dO rows of this lane's query: B operands of S^T = K Q^T and dP^T = V dO^T
    bf16x8 qop[NS], gop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        qop[s] = load_row8(Q + head + (size_t)qi * D + 16 * s + 8 * hl, negate);
        gop[s] = load_row8(dO + head + (size_t)qi * D + 16 * s + 8 * hl, false);
    }
    const float l2 = LSE[(size_t)bh * N + qi] * LOG2E;
    // D of this row, parked in its own dq row, read before the row is written
    const float dd = *reinterpret_cast<const float*>(dq_io + ((size_t)bh * N + qi) * D * 2);
    int k_lo, k_hi;
    allowed_interval<MASK, false>(qi, N, window, k_lo, k_hi);
    const unsigned k_span = (unsigned)(k_hi - k_lo);

    const int r1 = min(q0 + BW, N) - 1;
    int t_lo = 0, t_hi = (N - 1) / BT;
    if (MASK == ATTN_MASK_CAUSAL) t_hi = min(t_hi, r1 / BT);
    if (MASK == ATTN_MASK_WINDOW) { t_lo = max(0, q0 - window) / BT; t_hi = min(N - 1, r1 + window) / BT; }
    if (MASK == ATTN_MASK_CAUSAL_WINDOW) { t_lo = max(0, q0 - window) / BT; t_hi = min(t_hi, r1 / BT); }
    const int n_tiles = t_hi - t_lo + 1;

    const TileOffsets off(lane);
    const Loader<D> ld(wave, lane);

    f32x16 dqa[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[j][r] = 0.f;

    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(K + head, (uint32_t)N * (uint32_t)(2 * D));
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(V + head, (uint32_t)N * (uint32_t)(2 * D));
    ld.load(krs, t_lo, N, kbuf0, wave);
    ld.load(vrs, t_lo, N, vbuf0, wave);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    auto iter = [&](auto parity, int u) __attribute__((always_inline)) {
        constexpr int B = decltype(parity)::value;
        const int t = t_lo + u;
        const char* kb = B ? kbuf1 : kbuf0;
        const char* vb = B ? vbuf1 : vbuf0;
        if (u + 1 < n_tiles) {
            ld.load(krs, t + 1, N, B ? kbuf0 : kbuf1, wave);
            ld.load(vrs, t + 1, N, B ? vbuf0 : vbuf1, wave);
        }
        // S^T = K_t Q^T and dP^T = V_t dO^T: rows = the tile's keys, columns = queries (lanes)
        f32x16 st, dpt;
#pragma unroll
        for (int r = 0; r < 16; ++r) { st[r] = 0.f; dpt[r] = 0.f; }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int o = (k >> 1) * (4 * BT * 16) + ((k & 1) ? off.row_odd : off.row_even);
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb + o);
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(vb + o);
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[k], st, 0, 0, 0);
            dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gop[k], dpt, 0, 0, 0);
        }
        // the element mask runs only when the tile's keys are not all allowed for every
        // query of the wave
        bf16x8 dsp[2];
        const int rel0 = t * BT + 4 * hl - k_lo;
        auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int koff = 8 * (r >> 2) + (r & 3);
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c_log2, -l2));
                float p = e;
                if constexpr (decltype(masked)::value) p = (unsigned)(rel0 + koff) <= k_span ? e : 0.f;
                dsp[r >> 3][r & 7] = (__bf16)(p * (dpt[r] - dd));
            }
        };
        const int a0 = t * BT - k_lo;                  // the whole tile inside this query's keys?
        if (__any(!(a0 >= 0 && a0 + (BT - 1) <= (int)k_span))) {
            asm volatile("" ::: "memory");
            probs(IntC<1>{});
        } else {
            probs(IntC<0>{});
        }
        // dQ^T += K_t^T dS^T (A operand: transposing reads of the K tile)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int j = 0; j < ND; ++j) {
                const int o = j * (4 * BT * 16) + ks * (16 * 4 * 16);
                const bf16x4 a0 = lds_read_tr(kb, o + off.tr[0]);
                const bf16x4 a1 = lds_read_tr(kb, o + off.tr[1]);
                dqa[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                                 dsp[ks], dqa[j], 0, 0, 0);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    int u = 0;
    for (; u + 1 < n_tiles; u += 2) {
        iter(IntC<0>{}, u);
        iter(IntC<1>{}, u + 1);
    }
    if (u < n_tiles) iter(IntC<0>{}, u);

    if (my_q < N) {
        __bf16* dqr = reinterpret_cast<__bf16*>(dq_io) + head + (size_t)my_q * D;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (__bf16)(dqa[j][4 * g + e] * scale);
                *reinterpret_cast<bf16x4*>(dqr + j * 32 + 8 * g + 4 * hl) = a;
            }
        }
    }
}

template <int D, int MASK>
static int launch(const AttnBwdLaunch& a) {
    // head groups (grouped_order) for the full and causal masks: causal B4 H32 N16384
    // d128 +11%, B2 H32 N8192 +2%; a window's blocks read a narrow band, where the
    // grouping measured 3% slower
    const bool band = MASK == ATTN_MASK_WINDOW || MASK == ATTN_MASK_CAUSAL_WINDOW;
    int hg = attn_sched_head_group();
    if (hg < 0) hg = band ? 0 : head_group(a.N, a.d);
    const long long rows = (long long)a.B * a.H * a.N;
    constexpr int RPB = 4 * (64 / (D / 8));            // rows per prep workgroup
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL((prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       (const __bf16*)a.out, (const __bf16*)a.dout, (char*)a.dq, rows);
    const int BH = a.B * a.H;
    const int nblk = (a.N + BW - 1) / BW;
    hipLaunchKernelGGL((dkdv_kernel<D, MASK>), dim3((unsigned)((long long)nblk * BH)), dim3(256), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       (const char*)a.dq, (__bf16*)a.dk, (__bf16*)a.dv, BH, a.N, a.c_log2, a.negate_q, a.scale,
                       a.window, hg);
    hipLaunchKernelGGL((dq_kernel<D, MASK>), dim3((unsigned)((long long)nblk * BH)), dim3(256), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       (char*)a.dq, BH, a.N, nblk, a.c_log2, a.negate_q, a.scale, a.window, hg);
    return 0;
}

template <int D>
static int by_mask(const AttnBwdLaunch& a) {
    switch (a.mask_kind) {
        case ATTN_MASK_CAUSAL: return launch<D, ATTN_MASK_CAUSAL>(a);
        case ATTN_MASK_WINDOW: return launch<D, ATTN_MASK_WINDOW>(a);
        case ATTN_MASK_CAUSAL_WINDOW: return launch<D, ATTN_MASK_CAUSAL_WINDOW>(a);
        default: return launch<D, ATTN_MASK_NONE>(a);
    }
}

}  // namespace attn_bwd_bf16

int attn_launch_bwd_bf16(const AttnBwdLaunch& a) {
    if (a.d == 128) return attn_bwd_bf16::by_mask<128>(a);
    return attn_bwd_bf16::by_mask<64>(a);
}
