// Exact blockwise attention forward for fp32 inputs (the small-shape path).
//
// Same result as the bf16 matrix-core path (softmax(scale Q K^T) V with masked
// keys excluded, plus the row log-sum-exp), on the vector ALUs.  Nothing is
// rounded below fp32: scores and the running maximum are carried in fp64, so the
// exponent arguments of the weights that matter (those near the maximum) are
// exact to fp32 even for large scores; probabilities and the V accumulation are
// fp32.
//
// A workgroup owns 64 query rows; each row is owned by D/64 neighbouring lanes
// holding 64 of its dimensions, whose partial dot products are combined with a
// lane shuffle.  The 256 threads form KS = 256 / (64 D/64) groups of such lanes,
// and group g takes every KS-th key tile of the workgroup's range, so the serial
// chain of a row is 1/KS of its keys.  K/V tiles of 32 keys are staged in LDS, one
// pair per group (lanes of one half read the same key row: an LDS broadcast), and
// each group keeps a running maximum and sum per row.  At the end the groups'
// partial results are combined exactly (each rescaled to the common maximum) and
// normalised once ("Blockwise Parallel Transformer in PyTorch", the
// blockwise_attention example and its numerical-stability pitfall; Mosaic
// long-sequence attention page, §3.2 and §5.1).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn_f32 {

constexpr int ROWS = 64;   // query rows per workgroup
constexpr int TK = 32;     // keys per LDS tile
constexpr int DD = 64;     // dimensions per lane

template <int MASK>
__device__ __forceinline__ bool key_allowed(int qi, int kj, int N, int window) {
    if (kj >= N) return false;
    if (MASK == ATTN_MASK_CAUSAL) return kj <= qi;
    if (MASK == ATTN_MASK_WINDOW) return (qi - kj <= window) && (kj - qi <= window);
    if (MASK == ATTN_MASK_CAUSAL_WINDOW) return kj <= qi && qi - kj <= window;
    return true;
}

constexpr int NTHREADS = 256;

template <int D, int MASK>
__global__ __launch_bounds__(NTHREADS)
void fwd_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                float* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqt,
                float c_log2, int negate_q, int window) {
    constexpr int SPLIT = D / DD;             // lanes per row
    constexpr int GT = ROWS * SPLIT;          // threads of one key group
    constexpr int KS = NTHREADS / GT;         // key groups
    constexpr int TILE = TK * D;              // floats of one K or V tile
    // per group a K and a V tile; reused at the end for the groups' partial results
    __shared__ __attribute__((aligned(16))) float smem[2 * KS * TILE];
    static_assert((KS - 1) * GT * (DD + 4) <= 2 * KS * TILE, "merge area fits the tile buffers");

    const int tid = threadIdx.x;
    const int grp = tid / GT;                 // which key group
    const int lt = tid - grp * GT;
    const int part = lt % SPLIT;              // which 64 dimensions
    const int row = lt / SPLIT;
    float* Ks = smem + grp * 2 * TILE;
    float* Vs = Ks + TILE;
    const int id = blockIdx.x;
    const int rank = id / BH;
    const int bh = id - rank * BH;
    const int qt = (MASK == ATTN_MASK_CAUSAL) ? (nqt - 1 - rank) : rank;
    const int q0 = qt * ROWS;
    const int my_q = q0 + row;
    const int qrow = min(my_q, N - 1);
    const size_t head = (size_t)bh * N * D;
    const int dof = part * DD;

    float q[DD], acc[DD];
    const float sgn = negate_q ? -1.f : 1.f;
#pragma unroll
    for (int c = 0; c < DD; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(Q + head + (size_t)qrow * D + dof + c);
        q[c] = sgn * x.x; q[c + 1] = sgn * x.y; q[c + 2] = sgn * x.z; q[c + 3] = sgn * x.w;
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

    // rounds: group g takes tile t0 + g; every group passes the same barriers
    for (int t0 = lo; t0 <= hi; t0 += KS) {
        const int t = t0 + grp;
        const bool mine = t <= hi;
        const int key0 = t * TK;
        if (mine) {
            for (int e = lt * 4; e < TILE; e += GT * 4) {
                const int kr = e / D, col = e % D;
                float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
                if (key0 + kr < N) {
                    kv = *reinterpret_cast<const float4*>(K + head + (size_t)(key0 + kr) * D + col);
                    vv = *reinterpret_cast<const float4*>(V + head + (size_t)(key0 + kr) * D + col);
                }
                *reinterpret_cast<float4*>(Ks + e) = kv;
                *reinterpret_cast<float4*>(Vs + e) = vv;
            }
        }
        __syncthreads();
        if (mine) {
            double s[TK];
            double mt = -INFINITY;
#pragma unroll
            for (int j = 0; j < TK; ++j) {
                double dot = 0.0;
#pragma unroll
                for (int cc = 0; cc < DD; ++cc) dot = __builtin_fma((double)q[cc], (double)Ks[j * D + dof + cc], dot);
                if (SPLIT == 2) dot += __shfl_xor(dot, 1);
                s[j] = key_allowed<MASK>(my_q, key0 + j, N, window) ? dot * c : -INFINITY;
                mt = fmax(mt, s[j]);
            }
            const double m_new = fmax(m, mt);
            const double base = (m_new == -INFINITY) ? 0.0 : m_new;
            const float alpha = __builtin_amdgcn_exp2f((float)(m - base));
            l *= alpha;
#pragma unroll
            for (int cc = 0; cc < DD; ++cc) acc[cc] *= alpha;
#pragma unroll
            for (int j = 0; j < TK; ++j) {
                const float p = __builtin_amdgcn_exp2f((float)(s[j] - base));
                l += p;
#pragma unroll
                for (int cc = 0; cc < DD; ++cc) acc[cc] = __builtin_fmaf(p, Vs[j * D + dof + cc], acc[cc]);
            }
            m = m_new;
        }
        __syncthreads();
    }

    // combine the groups: groups 1.. park (acc, l, m) in LDS, group 0 rescales and sums
    if (KS > 1) {
        float* slot = smem + ((grp - 1) * GT + lt) * (DD + 4);
        if (grp > 0) {
#pragma unroll
            for (int cc = 0; cc < DD; cc += 4)
                *reinterpret_cast<float4*>(slot + cc) = make_float4(acc[cc], acc[cc + 1], acc[cc + 2], acc[cc + 3]);
            slot[DD] = l;
            *reinterpret_cast<double*>(slot + DD + 2) = m;
        }
        __syncthreads();
        if (grp == 0) {
            double M = m;
#pragma unroll
            for (int g = 1; g < KS; ++g) M = fmax(M, *reinterpret_cast<const double*>(smem + ((g - 1) * GT + lt) * (DD + 4) + DD + 2));
            const float w0 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((float)(m - M));
            l *= w0;
#pragma unroll
            for (int cc = 0; cc < DD; ++cc) acc[cc] *= w0;
#pragma unroll
            for (int g = 1; g < KS; ++g) {
                const float* sg = smem + ((g - 1) * GT + lt) * (DD + 4);
                const double mg = *reinterpret_cast<const double*>(sg + DD + 2);
                const float wg = (mg == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((float)(mg - M));
                l = __builtin_fmaf(wg, sg[DD], l);
#pragma unroll
                for (int cc = 0; cc < DD; ++cc) acc[cc] = __builtin_fmaf(wg, sg[cc], acc[cc]);
            }
            m = M;
        }
    }

    if (grp == 0 && my_q < N) {
        const float inv = 1.0f / l;
#pragma unroll
        for (int cc = 0; cc < DD; cc += 4) {
            float4 y = {acc[cc] * inv, acc[cc + 1] * inv, acc[cc + 2] * inv, acc[cc + 3] * inv};
            *reinterpret_cast<float4*>(O + head + (size_t)my_q * D + dof + cc) = y;
        }
        if (part == 0)
            LSE[(size_t)bh * N + my_q] =
                (float)((m + (double)__builtin_amdgcn_logf(l)) * 0.69314718055994530942);
    }
}

template <int D, int MASK>
static int launch(const AttnLaunch& a) {
    const int nqt = (a.N + ROWS - 1) / ROWS;
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
