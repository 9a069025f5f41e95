// Exact blockwise attention forward for fp32 inputs (the small-shape path).
//
// Same result as the bf16 matrix-core path (softmax(scale Q K^T) V with masked
// keys excluded, plus the row log-sum-exp), on the vector ALUs.  Nothing is
// rounded below fp32: scores and the running maximum are carried in fp64, so the
// exponent arguments of the weights that matter (those near the maximum) are
// exact to fp32 even for large scores; probabilities and the V accumulation are
// fp32.
//
// A workgroup is eight waves, one per key group; all of them hold the same 8 query
// rows, each row spread over 8 neighbouring lanes with d / 8 of its dimensions,
// whose partial dot products meet in a lane butterfly (every lane of the row ends
// with the same bits).  Key group g takes every eighth key tile of the workgroup's
// range (tiles of TK keys, staged by the group's own wave in LDS with K widened to
// fp64 once, so the lanes read fp64 operands; no barrier between rounds), keeping
// its own running maximum and sum per row.  At the end
// the groups' partial results are combined exactly (each rescaled to the common
// maximum) and normalised once ("Blockwise Parallel Transformer in PyTorch", the
// blockwise_attention example and its numerical-stability pitfall; Mosaic
// long-sequence attention page, §3.2 and §5.1).  8 lanes per row and 8 rows per
// workgroup keep the serial chain of a lane short and the grid wide: the small
// shapes this path serves are latency-bound.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn_f32 {

constexpr int KS = 8;      // key groups, one wave each

template <int MASK>
__device__ __forceinline__ bool key_allowed(int qi, int kj, int N, int window) {
    if (kj >= N) return false;
    if (MASK == ATTN_MASK_CAUSAL) return kj <= qi;
    if (MASK == ATTN_MASK_WINDOW) return (qi - kj <= window) && (kj - qi <= window);
    if (MASK == ATTN_MASK_CAUSAL_WINDOW) return kj <= qi && qi - kj <= window;
    return true;
}

constexpr int NTHREADS = 64 * KS;

template <int D>
struct F32Cfg {
    static constexpr int DL = D / 8;                 // dimensions per lane
    static constexpr int SPLIT = D / DL;             // lanes per row
    static constexpr int ROWS = 64 / SPLIT;          // query rows per workgroup
    static constexpr int TK = D == 64 ? 8 : 4;       // keys per LDS tile
    static constexpr int KPITCH = DL + 2;            // fp64 words per (key, lane part) in LDS (padded: no bank conflicts)
    static constexpr int VPITCH = DL + 4;            // fp32 words per (key, lane part)
    static constexpr int KWORDS = TK * SPLIT * KPITCH;
    static constexpr int VWORDS = TK * SPLIT * VPITCH;
};

template <int D, int MASK>
__global__ __launch_bounds__(NTHREADS)
void fwd_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                float* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqt,
                float c_log2, int negate_q, int window) {
    using C = F32Cfg<D>;
    constexpr int DL = C::DL, SPLIT = C::SPLIT, ROWS = C::ROWS, TK = C::TK;
    // per group a K tile (fp64) and a V tile (fp32); the K area is reused at the end
    // for the groups' partial results
    __shared__ __attribute__((aligned(16))) double ksm[KS * C::KWORDS];
    __shared__ __attribute__((aligned(16))) float vsm[KS * C::VWORDS];
    static_assert((KS - 1) * 64 * (DL + 4) * 4 <= KS * C::KWORDS * 8, "merge area fits the K tiles");

    const int tid = threadIdx.x;
    const int grp = tid >> 6;                 // key group (wave)
    const int lane = tid & 63;
    const int part = lane % SPLIT;            // which DL dimensions
    const int row = lane / SPLIT;
    double* Ks = ksm + grp * C::KWORDS;
    float* Vs = vsm + grp * C::VWORDS;
    const int id = blockIdx.x;
    const int rank = id / BH;
    const int bh = id - rank * BH;
    const int qt = (MASK == ATTN_MASK_CAUSAL) ? (nqt - 1 - rank) : rank;
    const int q0 = qt * ROWS;
    const int my_q = q0 + row;
    const int qrow = min(my_q, N - 1);
    const size_t head = (size_t)bh * N * D;
    const int dof = part * DL;

    double q[DL];
    float acc[DL];
    const float sgn = negate_q ? -1.f : 1.f;
#pragma unroll
    for (int c = 0; c < DL; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(Q + head + (size_t)qrow * D + dof + c);
        q[c] = (double)(sgn * x.x); q[c + 1] = (double)(sgn * x.y);
        q[c + 2] = (double)(sgn * x.z); q[c + 3] = (double)(sgn * x.w);
        acc[c] = acc[c + 1] = acc[c + 2] = acc[c + 3] = 0.f;
    }
    double m = -INFINITY;      // running max of c_log2 * s (log2 domain)
    float l = 0.f;

    const int r1 = min(q0 + ROWS, N) - 1;
    const int last = (N - 1) / TK;
    int lo = 0, hi = last;
    if (MASK == ATTN_MASK_CAUSAL) hi = min(last, r1 / TK);
    if (MASK == ATTN_MASK_WINDOW) { lo = max(0, q0 - window) / TK; hi = min(N - 1, r1 + window) / TK; }
    if (MASK == ATTN_MASK_CAUSAL_WINDOW) { lo = max(0, q0 - window) / TK; hi = min(last, r1 / TK); }
    const double c = (double)c_log2;

    // Group g takes tiles lo + g, lo + g + KS, ...  A group stages and reads only its
    // own tiles, so its rounds need no barrier (LDS operations of one wave complete
    // in order); the next tile is fetched into registers before the current one is
    // used, so its load latency hides behind the arithmetic.
    constexpr int NLD = TK * D / (64 * 4);    // float4 loads per lane per tile and tensor
    float4 kreg[NLD], vreg[NLD];
    auto fetch = [&](int t) __attribute__((always_inline)) {
        const int key0 = t * TK;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int e = (i * 64 + lane) * 4;
            const int kr = e / D, col = e % D;
            kreg[i] = vreg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (key0 + kr < N) {
                kreg[i] = *reinterpret_cast<const float4*>(K + head + (size_t)(key0 + kr) * D + col);
                vreg[i] = *reinterpret_cast<const float4*>(V + head + (size_t)(key0 + kr) * D + col);
            }
        }
    };
    if (lo + grp <= hi) fetch(lo + grp);
    for (int t = lo + grp; t <= hi; t += KS) {
        // stage: element e = (key kr, column col) -> (kr, part col / DL, col % DL)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int e = (i * 64 + lane) * 4;
            const int kr = e / D, col = e % D;
            const int slot = kr * SPLIT + col / DL, cc = col % DL;
            double* kd = Ks + slot * C::KPITCH + cc;
            kd[0] = (double)kreg[i].x; kd[1] = (double)kreg[i].y; kd[2] = (double)kreg[i].z; kd[3] = (double)kreg[i].w;
            *reinterpret_cast<float4*>(Vs + slot * C::VPITCH + cc) = vreg[i];
        }
        if (t + KS <= hi) fetch(t + KS);
        const int key0 = t * TK;
        double s[TK];
        double mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            const double* kr = Ks + (j * SPLIT + part) * C::KPITCH;
            double dot = 0.0;
#pragma unroll
            for (int cc = 0; cc < DL; ++cc) dot = __builtin_fma(q[cc], kr[cc], dot);
#pragma unroll
            for (int o = 1; o < SPLIT; o <<= 1) dot += __shfl_xor(dot, o);
            s[j] = key_allowed<MASK>(my_q, key0 + j, N, window) ? dot * c : -INFINITY;
            mt = fmax(mt, s[j]);
        }
        const double m_new = fmax(m, mt);
        const double base = (m_new == -INFINITY) ? 0.0 : m_new;
        const float alpha = __builtin_amdgcn_exp2f((float)(m - base));
        l *= alpha;
#pragma unroll
        for (int cc = 0; cc < DL; ++cc) acc[cc] *= alpha;
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            const float p = __builtin_amdgcn_exp2f((float)(s[j] - base));
            l += p;
            const float* vr = Vs + (j * SPLIT + part) * C::VPITCH;
#pragma unroll
            for (int cc = 0; cc < DL; ++cc) acc[cc] = __builtin_fmaf(p, vr[cc], acc[cc]);
        }
        m = m_new;
    }
    __syncthreads();     // every group is done with its tiles before the merge reuses the K area

    // combine the groups: groups 1.. park (acc, l, m) in LDS, group 0 rescales and sums
    float* const park = reinterpret_cast<float*>(ksm);
    if (grp > 0) {
        float* const slot = park + ((grp - 1) * 64 + lane) * (DL + 4);
#pragma unroll
        for (int cc = 0; cc < DL; cc += 4)
            *reinterpret_cast<float4*>(slot + cc) = make_float4(acc[cc], acc[cc + 1], acc[cc + 2], acc[cc + 3]);
        slot[DL] = l;
        *reinterpret_cast<double*>(slot + DL + 2) = m;
    }
    __syncthreads();
    if (grp == 0) {
        double M = m;
#pragma unroll
        for (int g = 1; g < KS; ++g) M = fmax(M, *reinterpret_cast<const double*>(park + ((g - 1) * 64 + lane) * (DL + 4) + DL + 2));
        const float w0 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((float)(m - M));
        l *= w0;
#pragma unroll
        for (int cc = 0; cc < DL; ++cc) acc[cc] *= w0;
#pragma unroll
        for (int g = 1; g < KS; ++g) {
            const float* sg = park + ((g - 1) * 64 + lane) * (DL + 4);
            const double mg = *reinterpret_cast<const double*>(sg + DL + 2);
            const float wg = (mg == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((float)(mg - M));
            l = __builtin_fmaf(wg, sg[DL], l);
#pragma unroll
            for (int cc = 0; cc < DL; ++cc) acc[cc] = __builtin_fmaf(wg, sg[cc], acc[cc]);
        }
        m = M;
        if (my_q < N) {
            const float inv = 1.0f / l;
#pragma unroll
            for (int cc = 0; cc < DL; cc += 4) {
                float4 y = {acc[cc] * inv, acc[cc + 1] * inv, acc[cc + 2] * inv, acc[cc + 3] * inv};
                *reinterpret_cast<float4*>(O + head + (size_t)my_q * D + dof + cc) = y;
            }
            if (part == 0)
                LSE[(size_t)bh * N + my_q] =
                    (float)((m + (double)__builtin_amdgcn_logf(l)) * 0.69314718055994530942);
        }
    }
}

template <int D, int MASK>
static int launch(const AttnLaunch& a) {
    const int nqt = (a.N + F32Cfg<D>::ROWS - 1) / F32Cfg<D>::ROWS;
    const long long grid = (long long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd_kernel<D, MASK>), dim3((unsigned)grid), dim3(NTHREADS), 0,
                       (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (float*)a.out, a.lse, a.B * a.H, a.N, nqt, a.c_log2, a.negate_q, a.window);
    return 0;
}

template <int D>
static int by_mask(const AttnLaunch& a) {
    switch (a.mask_kind) {
        case ATTN_MASK_CAUSAL: return launch<D, ATTN_MASK_CAUSAL>(a);
        case ATTN_MASK_WINDOW: return launch<D, ATTN_MASK_WINDOW>(a);
        case ATTN_MASK_CAUSAL_WINDOW: return launch<D, ATTN_MASK_CAUSAL_WINDOW>(a);
        default: return launch<D, ATTN_MASK_NONE>(a);
    }
}

}  // namespace attn_f32

int attn_launch_f32(const AttnLaunch& a) {
    if (a.d == 128) return attn_f32::by_mask<128>(a);
    return attn_f32::by_mask<64>(a);
}
