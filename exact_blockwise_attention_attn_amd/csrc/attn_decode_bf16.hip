// Decode: one new query per (batch, head) against a key/value cache, bf16 in,
// fp32 arithmetic, gfx950 (CDNA4).
//
// For one query at sequence position p, every mask allows one interval of keys
// [lo, hi] (causal: 0..p; window: p-w..p+w; causal window: p-w..p; none: all),
// computed on the host, so a key outside it is never read.  The interval is cut
// into ranges, one per workgroup, and each of the four waves of a workgroup
// streams a quarter of its range straight from HBM into registers: this work is
// bound by HBM bandwidth (the KV-cache decode of "万亿参数大模型Day-0适配实践与稀疏
// 注意力优化", §二, item 2), not by arithmetic, so there is no LDS staging and no
// matrix-core product, only enough loads in flight.
//
// Lane layout: a key row of D bf16 is read by D/8 lanes, 16 bytes each, so one
// wave load instruction covers 64/(D/8) keys; a chunk of CH keys (16 KB of K and V
// for either head dimension) is NL = 8 such loads per tensor per lane, and the
// next chunk is in flight while the current one is computed.
//   score  q.k: four v_dot2_f32_bf16 per lane (bf16 products are exact in fp32),
//          then a sum over the key's lanes with DPP row operations;
//   softmax per lane group (the lanes of one key slot): running maximum m in the
//          log2 domain, p = exp2(c s - m), running sum l, O scaled by
//          exp2(m_old - m_new) when the maximum grows (the online softmax of the
//          Mosaic long-sequence attention page, §3.2, with its maximum made
//          explicit);
//   O      fp32 FMAs of p with the unpacked V row, D/(D/8) = 8 dims per lane.
// At the end the groups of a wave, then the four waves (through LDS), are merged
// by their maxima and sums, and the workgroup writes either the final O and LSE
// (one range) or its range's normalised O and LSE to the workspace for the
// log-sum-exp merge of the split-KV path.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"
#include "attn_tile.h"

namespace attn_decode {

using namespace attn_tile;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct Shape {
    static constexpr int LPK = D / 8;       // lanes per key row
    static constexpr int KPL = 64 / LPK;    // keys per wave load instruction
    static constexpr int CH = 4096 / D;     // keys per chunk: 16 KB of K and V
    static constexpr int NL = CH / KPL;     // loads per tensor per lane per chunk
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(NL == 8, "chunk shape");
};

// sum over the D/8 lanes of a key slot (a quad, then half rows, then rows of 16);
// every lane of the slot gets the total
template <int LPK>
__device__ __forceinline__ float slot_sum(float x) {
    auto dpp = [](float v, auto ctrl) __attribute__((always_inline)) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    x += dpp(x, IntC<0xB1>{});     // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp(x, IntC<0x4E>{});     // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp(x, IntC<0x141>{});    // row_half_mirror: the other quad of the 8
    if constexpr (LPK == 16) x += dpp(x, IntC<0x140>{});   // row_mirror: the other half of the 16
    return x;
}

// q.k over a lane's 8 dims.  Each word is copied to a scalar before the bit cast:
// a bit cast applied directly to an element of a vector reference compiles to a
// read of element 0 (seen in the ISA of this file).
__device__ __forceinline__ float dot8(const u32x4& k, const u32x4& q) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t kw = k[w], qw = q[w];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw), __builtin_bit_cast(bf16x2_t, qw), s, false);
    }
    return s;
}

struct DecodeArgs {
    int lo, hi;          // allowed keys of the query: [lo, hi], 0 <= lo <= hi < Nk
    int n_split;         // ranges of the interval, one per workgroup
    int split_len;       // keys per range, a multiple of 4 chunks
    float* part_o;       // [BH, n_split, D] fp32 (n_split > 1)
    float* part_lse;     // [BH, n_split] fp32
};

template <int D>
__global__ __launch_bounds__(256) void decode_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                     const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                     float* __restrict__ LSE, int BH, int Nk, float c_log2,
                                                     int negate_q, DecodeArgs a) {
    using S = Shape<D>;
    constexpr int LPK = S::LPK, KPL = S::KPL, CH = S::CH, NL = S::NL;
    __shared__ float s_acc[4][D];
    __shared__ float s_m[4], s_l[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane / LPK, sub = lane % LPK;
    const int split = blockIdx.x / BH, bh = blockIdx.x - split * BH;

    // keys of this workgroup and of this wave
    const int kb = a.lo + split * a.split_len;
    const int ke = min(a.hi + 1, kb + a.split_len);
    const int wlen = a.split_len / 4;
    const int wkb = kb + wave * wlen;
    const int wke = min(ke, wkb + wlen);

    const __bf16* Kh = K + (size_t)bh * Nk * D + sub * 8;
    const __bf16* Vh = V + (size_t)bh * Nk * D + sub * 8;
    u32x4 q = *reinterpret_cast<const u32x4*>(Q + (size_t)bh * D + sub * 8);
    if (negate_q) q ^= 0x80008000u;      // exact sign flip: scale < 0 runs as -q with |scale|

    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    // keys c0 + i KPL + g (i < NL) of a chunk; rows past the wave's end reload its last key
    auto load = [&](int c0, u32x4* kr, u32x4* vr) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const size_t row = (size_t)min(c0 + i * KPL + g, wke - 1) * D;
            kr[i] = *reinterpret_cast<const u32x4*>(Kh + row);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const size_t row = (size_t)min(c0 + i * KPL + g, wke - 1) * D;
            vr[i] = *reinterpret_cast<const u32x4*>(Vh + row);
        }
    };
    auto compute = [&](int c0, const u32x4* kr, const u32x4* vr) __attribute__((always_inline)) {
        float s[NL];
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            s[i] = slot_sum<LPK>(dot8(kr[i], q));
            if (c0 + i * KPL + g >= wke) s[i] = -INFINITY;
            cm = fmaxf(cm, s[i]);
        }
        const float m_new = fmaxf(m, cm * c_log2);
        if (m_new > m) {                  // the maximum grew: rescale (rare after the first chunks)
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // 0 while m = -inf
            l *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= alpha;
            m = m_new;
        }
        const float base = (m == -INFINITY) ? 0.f : m;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c_log2, -base));
            l += p;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x = vr[i][w];
                acc[2 * w] = __builtin_fmaf(p, __uint_as_float(x << 16), acc[2 * w]);
                acc[2 * w + 1] = __builtin_fmaf(p, __uint_as_float(x & 0xffff0000u), acc[2 * w + 1]);
            }
        }
    };

    if (wkb < wke) {
        // two chunks in flight: the loads of the next chunk are issued before the
        // current one is computed.  Loads past the end are clamped to the last key
        // (one cached row) and their keys masked, so the loop needs no branch on them.
        u32x4 ka[NL], va[NL], kb2[NL], vb2[NL];
        load(wkb, ka, va);
        for (int c = wkb; c < wke; c += 2 * CH) {
            load(c + CH, kb2, vb2);
            compute(c, ka, va);
            load(c + 2 * CH, ka, va);
            compute(c + CH, kb2, vb2);
        }
    }

    // merge the key slots of the wave (lanes sub, sub + LPK, ...), then the waves
    float M = m;
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
    const float wgt = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
    l *= wgt;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= wgt;
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
        l += __shfl_xor(l, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], x);
    }
    if (g == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[wave][sub * 8 + e] = acc[e];
    }
    if (lane == 0) {
        s_m[wave] = M;
        s_l[wave] = l;
    }
    __syncthreads();
    if (tid < D) {
        float Mw = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float ww = (s_m[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w] - Mw);
            L = __builtin_fmaf(ww, s_l[w], L);
            o = __builtin_fmaf(ww, s_acc[w][tid], o);
        }
        const float lse = L > 0.f ? (Mw + __builtin_amdgcn_logf(L)) * 0.69314718055994531f : -INFINITY;
        if (a.n_split == 1) {
            O[(size_t)bh * D + tid] = (__bf16)(o / L);
            if (tid == 0) LSE[bh] = lse;
        } else {
            const size_t pr = (size_t)bh * a.n_split + split;
            a.part_o[pr * D + tid] = L > 0.f ? o / L : 0.f;
            if (tid == 0) a.part_lse[pr] = lse;
        }
    }
}

}  // namespace attn_decode

// Ranges of a decode launch over an interval of L keys: one full round of
// workgroups (the kernel fits three per CU, 256 CUs: 768; measured best against 1024
// to 3072, where a partial second round leaves CUs idle at the end), at least four
// chunks per wave, ranges a multiple of four chunks.  The count never exceeds
// attn_decode_max_splits(B, H, Nk) for L <= Nk.
#ifndef ATTN_DECODE_TARGET_WGS
#define ATTN_DECODE_TARGET_WGS 768
#endif
static void decode_plan(int BH, int L, int d, int* n_split, int* split_len) {
    const int unit = 4 * (4096 / d);                   // four waves x one chunk
    const long long want = (ATTN_DECODE_TARGET_WGS + BH - 1) / BH;
    const long long max_split = (L + 4LL * unit - 1) / (4LL * unit);
    long long s = want < max_split ? want : max_split;
    if (s < 1) s = 1;
    long long len = (L + s - 1) / s;
    len = (len + unit - 1) / unit * unit;
    *split_len = (int)len;
    *n_split = (int)((L + len - 1) / len);
}

int attn_decode_max_splits(int BH, int Nk, int d) {
    const int unit = 4 * (4096 / d);
    const long long want = (ATTN_DECODE_TARGET_WGS + BH - 1) / BH;
    const long long max_split = (Nk + 4LL * unit - 1) / (4LL * unit);
    long long s = want < max_split ? want : max_split;
    return s < 1 ? 1 : (int)s;
}

int attn_launch_decode_bf16(const AttnLaunch& a, int Nk, int lo, int hi, float* part_o, float* part_lse,
                            int* n_split_used) {
    using namespace attn_decode;
    const int BH = a.B * a.H;
    DecodeArgs da;
    da.lo = lo;
    da.hi = hi;
    decode_plan(BH, hi - lo + 1, a.d, &da.n_split, &da.split_len);
    da.part_o = part_o;
    da.part_lse = part_lse;
    *n_split_used = da.n_split;
    const unsigned grid = (unsigned)(da.n_split * BH);
    hipStream_t st = (hipStream_t)a.stream;
    if (a.d == 128)
        hipLaunchKernelGGL((decode_kernel<128>), dim3(grid), dim3(256), 0, st, (const __bf16*)a.q, (const __bf16*)a.k,
                           (const __bf16*)a.v, (__bf16*)a.out, a.lse, BH, Nk, a.c_log2, a.negate_q, da);
    else
        hipLaunchKernelGGL((decode_kernel<64>), dim3(grid), dim3(256), 0, st, (const __bf16*)a.q, (const __bf16*)a.k,
                           (const __bf16*)a.v, (__bf16*)a.out, a.lse, BH, Nk, a.c_log2, a.negate_q, da);
    return 0;
}
