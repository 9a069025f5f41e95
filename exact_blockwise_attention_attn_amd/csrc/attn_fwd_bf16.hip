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
// Work decomposition.  One workgroup of four waves (one per SIMD) per (batch*head,
// block of BR = 128 QB query rows); each wave owns QB 32-row blocks: QB = 2 (one
// workgroup per CU) or QB = 1 (two per CU, two waves per SIMD), chosen by shape.
// Workgroups run in groups of heads whose K and V fit in the Infinity Cache
// (grouped_order).  The workgroup walks the key tiles (BC = 32 keys) that hold an
// allowed key for one of its rows; tiles wholly outside the mask are never visited
// and element masking runs only on tiles that straddle the mask or the sequence end.
// A grid too small for the device (no mask or causal) splits the keys as well: the
// four waves form 4 / KG sets of query rows times KG key groups, group j takes tiles
// t_lo + KG u + j, and the groups' softmax states are merged through LDS at the end
// with weights 2^(m_j - max m), the exact combination of softmax pieces over disjoint
// key sets (the Mosaic page's merge of local attention results, §2.1, of the blocks
// of its §2.2).  KG = 2 or 4 doubles or quadruples the workgroups of a shape.
//
// K/V staging.  Each K and V tile goes HBM -> LDS directly (buffer_load_dwordx4 ... lds,
// no VGPR round trip), row-major with the 16-byte chunks of a row XOR-swizzled by
// the row index.  K and V each rotate through two buffers; one barrier per tile.
// The four buffers are distinct LDS arrays and the tile loop is unrolled by two,
// so every LDS read names its buffer statically and the compiler can see it never
// aliases a load in flight into another one.
//
// One tile as a fixed schedule.  A tile's work is three independent streams: the
// matrix cores compute the scores of the next tile and the V product of the
// previous one, the vector ALUs the softmax of this one, and the LDS reads fetch
// the matrix operands a few instructions ahead.  They are laid out by hand, one
// matrix instruction per slot with a share of the softmax behind it, and the
// compiler's scheduler is fenced between slots, so the two kinds of work of a wave
// overlap (at QB = 1 a second wave on the SIMD adds its own).
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 64-wide wavefront).  Each wave
// computes the transposed score block S^T = K_tile Q_w^T (keys x queries), so a
// lane holds scores of ONE query (column n = lane % 32) for 16 of the 32 keys: row
// max and sums are in-lane plus one exchange with lane ^ 32 (v_permlane32_swap).
// The probabilities never leave registers: the C layout of S^T, packed to bf16, is
// the B operand of O^T += V^T P^T, where the 8 keys a lane holds per 16-key slab
// are {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); the A operand V^T is read from the
// row-major V tile with the transposing LDS read ds_read_b64_tr_b16 in exactly
// that key order (a contraction index may be permuted, as long as both operands
// agree).  Q sits in AGPRs for the whole kernel, read once; so does O.
//
// Softmax bookkeeping (log2 domain, c = |scale| log2 e).  Each row's probabilities
// are taken against a reference m (lazily raised running maximum): a wave vote on
// the lanes' tile maxima raises it only when some row's scores exceed m + TAU (and
// on a row's first allowed tile), and only then are O and the sums rescaled.  Two
// sums are kept: the fp32 sum of the probabilities (for LSE) and the sum of the
// same probabilities rounded to bf16, which normalises O: O is then an exact convex
// combination of V rows with the rounded weights, and the bf16 rounding of P
// perturbs relative weights only.
//
// Data in HBM: q, k, v, out are contiguous [B, H, N, d] bf16, lse is [B, H, N] fp32.
// Q is read once into registers, K and V once per query block (mostly L2/MALL
// hits), O and LSE written once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "attn_launch.h"
#include "attn_tile.h"

namespace attn_bf16 {

using namespace attn_tile;

constexpr float TAU = 8.0f;         // lazy rescale threshold (log2 domain)

// Tile shape: a wave owns QB blocks of 32 query rows; a key tile is KB blocks of
// 32 keys.  Each K or V operand read from LDS feeds QB matrix instructions.
// KG key groups: the waves of a workgroup form NW / KG row groups (distinct query
// rows) times KG key groups; at step u key group g takes tile t_lo + KG u + g, and
// the groups' softmax states are merged at the end (exact, as for disjoint key sets).
template <int D, int QB, int KB, int KG = 1>
struct Cfg {
    static constexpr int NW = 4;                    // waves per workgroup, one per SIMD
    static constexpr int RG = NW / KG;              // row groups
    static constexpr int RW = 32 * QB;              // query rows per wave
    static constexpr int BC = 32 * KB;              // keys per tile
    static constexpr int NT = 64 * NW;              // threads per workgroup
    static constexpr int BR = RW * RG;              // query rows per workgroup
    static constexpr int TILE_BYTES = BC * D * 2;   // one K or V tile
    static constexpr int LDS_BYTES = 4 * KG * TILE_BYTES;        // K and V, two buffers each, per key group
    static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / RG;  // a key group's waves load its tile, 1 KB per instruction
    static constexpr int RB = BC / 16;              // 16-row blocks of a tile (one 1 KB load each per chunk group)
    static_assert(KG == 1 || KG == 2 || KG == 4, "key groups");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 workgroup");
    static_assert(TILE_BYTES % (1024 * RG) == 0, "tile must split evenly over the waves");
    static_assert(D == 64 || D == 128, "head dim");
};

// Inclusive key-tile range (tiles of BC keys) holding an allowed key for some row of [r0, r1].
template <int MASK, int BC>
__device__ __forceinline__ void tile_range(int r0, int r1, int N, int window, int& lo, int& hi) {
    const int last = (N - 1) / BC;
    if (MASK == ATTN_MASK_CAUSAL) {
        lo = 0;
        hi = min(last, r1 / BC);
    } else if (MASK == ATTN_MASK_WINDOW) {
        lo = max(0, r0 - window) / BC;
        hi = min(N - 1, r1 + window) / BC;
    } else if (MASK == ATTN_MASK_CAUSAL_WINDOW) {
        lo = max(0, r0 - window) / BC;
        hi = min(last, r1 / BC);
    } else {
        lo = 0;
        hi = last;
    }
}

// Score MFMAs with the read-only Q operands pinned to the AGPR file
// (v_mfma_f32_32x32x16_bf16, acc += A B, accumulator in VGPRs).  At 64 query
// rows per wave, O (VGPRs, compiler-issued MFMAs), S, P and the temporaries fill
// the VGPR file; Q alone goes to the AGPRs.  The compiler cannot see into these
// asm statements, so the hazards it would pad are handled here: the chain
// accumulates back to back into the same registers (interlocked by hardware);
// settle_v() puts >= 18 wait states before any vector-ALU read of S, tied to S
// as an operand so nothing is scheduled across it; the A operand comes straight
// from an LDS load and Q is pinned (and padded) once at kernel start.
__device__ __forceinline__ void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& q) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma_s(f32x16& acc, const bf16x8& a, const bf16x8& q) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(q));
}
__device__ __forceinline__ void settle_qa(bf16x8& x) {     // pin an operand into AGPRs, padded
    asm volatile("s_nop 4" : "+a"(x));
}
__device__ __forceinline__ void settle_v(f32x16& x) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}

// Split-KV mode (queries fewer than keys, e.g. decode against a key/value cache):
// the keys of a (batch, head) are cut into n_split ranges of split_len keys, one
// workgroup per (query block, range); query row i sits at position q_off + i; each
// workgroup writes its range's normalised partial O (fp32) and log-sum-exp to a
// workspace, merged by merge_kernel.  With one range the workgroup writes O and LSE
// itself (every row then sees its own position, so its sum is positive).
struct SplitArgs {
    int Nk;            // keys per head
    int q_off;         // position of query row 0 among the keys
    int n_split;       // key ranges per head
    int split_len;     // keys per range (a multiple of the tile)
    float* part_o;     // [BH, n_split, N, D] fp32
    float* part_lse;   // [BH, n_split, N] fp32 (-inf for a range with no allowed key)
};

// Two workgroups per CU (two waves per SIMD, <= 256 registers each) at 32 rows per
// wave, d = 128: left alone the compiler takes 260-270 registers for several of these
// instantiations and runs one wave per SIMD; two waves per SIMD let one wave's
// softmax overlap the other's matrix instructions (+23% on causal cases, +35% on the
// narrow window).  The 64-row shapes need the whole register file; at d = 64 the
// 32-row kernels fit two waves anyway and the cap measured slower.  Key-group
// kernels: the d = 64 32-row ones keep two waves per SIMD (the cap costs them no
// spill); at d = 128 they run without the cap (under it the merge spills).
// Block-sparse layouts (internal mask kinds of the kernel; the C ABI has its own
// entry point): the allowed keys of a 128-row query block are the 128-key blocks
// its layout row marks, intersected with j <= i for the causal variant.
constexpr int MASK_BLOCK = 16;
constexpr int MASK_BLOCK_CAUSAL = 17;
constexpr int BLOCK_TOKENS = 128;      // layout block: one 32-rows-per-wave workgroup, four key tiles
constexpr int LEAD_BLOCKS = 2;         // query blocks of every head scheduled before the head groups
constexpr int MAX_LAYOUT_BLOCKS = 8192;

struct BlockArgs {
    const uint8_t* layout;   // [H, nb, nb], nonzero = allowed
    int H;
    int nb;                  // ceil(N / BLOCK_TOKENS)
};

template <int D, int QB, int MASK, bool SPLIT, int KG>
constexpr int min_waves_per_simd() {
    return ((D == 128 && QB == 1 && KG == 1) || (D == 64 && QB == 1 && KG > 1)) ? 2 : 1;
}

// WQ: the workgroup order goes through the work queue (wq_take); kernels launched
// without it compile no trace of it (its code and live values cost the register-
// capped 32-row kernels spills).
template <int D, int QB, int KB, int MASK, bool SPLIT = false, int KG = 1, bool WQ = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(min_waves_per_simd<D, QB, MASK, SPLIT, KG>(), 8)))
void fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                int BH, int N, int nqt, float c_log2, int negate_q, int window, SplitArgs sa = SplitArgs{},
                BlockArgs ba = BlockArgs{}, int hg = 0, unsigned* wq = nullptr, int wq_static = 0, int wq_dyn = 0) {
    using C = Cfg<D, QB, KB, KG>;
    constexpr int BC = C::BC;
    constexpr int NS = D / 16;       // 16-dim slabs of the contraction over d
    constexpr int ND = D / 32;       // 32-row blocks of O^T
    constexpr int NKS = BC / 16;     // 16-key slabs of the V product
    // K and V tiles rotate through two buffers each; four distinct arrays, each with
    // one tile per key group
    __shared__ __attribute__((aligned(1024))) char kbuf0[KG * C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kbuf1[KG * C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vbuf0[KG * C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vbuf1[KG * C::TILE_BYTES];
    constexpr bool BLK = (MASK == MASK_BLOCK || MASK == MASK_BLOCK_CAUSAL);
    constexpr bool CAUS = (MASK == ATTN_MASK_CAUSAL || MASK == MASK_BLOCK_CAUSAL);
    static_assert(!BLK || (QB == 1 && KB == 1 && !SPLIT), "block layouts use 128-row query blocks of 32-key tiles");
    static_assert(KG == 1 || (!BLK && !SPLIT), "key groups: dense masks of the full forward");
    // merge of the key groups: per-lane scalars (running max, both sums) of groups 1..KG-1
    __shared__ float mstate[KG > 1 ? (KG - 1) * C::RG * QB * 3 * 64 : 1];
    __shared__ uint16_t blist[BLK ? MAX_LAYOUT_BLOCKS : 1];   // allowed key blocks of this query block
    __shared__ int bcount;
    __shared__ int wq_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;        // lane half
    const int ln = lane & 31;
    const int kg = KG == 1 ? 0 : wave / C::RG;    // key group
    const int rg = KG == 1 ? wave : wave % C::RG; // row group
    // this key group's tile in each buffer
    char* const kb0 = kbuf0 + kg * C::TILE_BYTES;
    char* const kb1 = kbuf1 + kg * C::TILE_BYTES;
    char* const vb0 = vbuf0 + kg * C::TILE_BYTES;
    char* const vb1 = vbuf1 + kg * C::TILE_BYTES;

    // Workgroup order: heads in groups of hg (grouped_order), inside a group the
    // heaviest query blocks first for the causal mask.
    // With a work queue, workgroups from wq_static on claim their item (wq_take).
    static_assert(!WQ || (!SPLIT && !BLK), "the work queue serves the dense forward");
    int id = blockIdx.x;
    if constexpr (WQ) {
        if (id >= wq_static) {
            if (tid == 0) wq_item = wq_take(wq, BH * nqt, wq_static, wq_dyn);
            __syncthreads();
            id = __builtin_amdgcn_readfirstlane(wq_item);
            if (id < 0) return;                           // every item is taken (the whole workgroup)
        }
    }
    int rank, bh, split = 0;
    if constexpr (SPLIT) {
        rank = id / (BH * sa.n_split);
        const int rem = id - rank * (BH * sa.n_split);
        split = rem / BH;
        bh = rem - split * BH;
    } else if (BLK && hg > 0) {
        // block layouts: the first LEAD_BLOCKS query blocks of every head go first (the
        // global tokens of BigBird- and Longformer-style layouts sit there, and those rows
        // see every key block), then the rest in head groups
        const int P = min(LEAD_BLOCKS, nqt);
        if (id < P * BH) {
            rank = id / BH;
            bh = id - rank * BH;
        } else {
            grouped_order(id - P * BH, BH, nqt - P, hg, rank, bh);
            rank += P;
        }
    } else {
        grouped_order(id, BH, nqt, hg, rank, bh);
    }
    const int qt = CAUS ? (nqt - 1 - rank) : rank;
    const int q0 = qt * C::BR;
    // keys: Nk per head, this workgroup's range [kb, ke); query positions offset by qoff
    const int Nk = SPLIT ? sa.Nk : N;
    const int qoff = SPLIT ? sa.q_off : 0;
    const int kb = SPLIT ? split * sa.split_len : 0;
    const int ke = SPLIT ? min(Nk, kb + sa.split_len) : N;

    const size_t head = (size_t)bh * N * D;
    const size_t khead = (size_t)bh * Nk * D;
    const __bf16* Qh = Q + head;
    const __bf16* Kh = K + khead;
    const __bf16* Vh = V + khead;

    const int qw0 = q0 + rg * C::RW;             // first row of this wave
    int my_q[QB];                                // the query of this lane's column in each 32-row block
#pragma unroll
    for (int b = 0; b < QB; ++b) my_q[b] = qw0 + 32 * b + ln;

    // Q operands (B of S^T = K Q^T): lane holds Q[my_q[b]][16 s + 8 hl .. +8].
    bf16x8 qreg[QB][NS];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)min(my_q[b], N - 1) * D + s * 16 + hl * 8);
            if (negate_q) raw ^= 0x80008000u;    // exact sign flip: scale < 0 runs as -q with |scale|
            qreg[b][s] = __builtin_bit_cast(bf16x8, raw);
        }
    // ---- per-lane LDS and load addresses (byte offsets within a tile)
    // loader: wave instruction i fills 1 KB block b = rg * LPW + i, i.e. rows
    // 16 (b % RB) .. +15 of chunk group b / RB; lane -> (row, chunk)
    uint32_t ld_off[C::LOADS_PER_WAVE];          // byte offset of the lane's 16 bytes in the HBM tile
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
        const int b = rg * C::LOADS_PER_WAVE + i;
        const int row = 16 * (b % C::RB) + (lane >> 2);
        const int c = 4 * (b / C::RB) + ((lane & 3) ^ ((row >> 2) & 3));
        ld_off[i] = (uint32_t)(row * D + c * 8) * 2u;
    }
    // K operand: row 32 kb + ln, chunk 2 s + hl = group s / 2, in-group 2 (s % 2) + hl
    const int sw = (ln >> 2) & 3;
    const int kaddr_e = (4 * ln + (hl ^ sw)) * 16;          // s even
    const int kaddr_o = (4 * ln + ((2 + hl) ^ sw)) * 16;    // s odd
    // V operand (transposing reads), read r: supplier lane (g, s16) names key row
    // 8 r + 4 hl + s16 / 4 of the slab and 8 bytes of chunk 4 j + 2 (g % 2) + (s16 % 4) / 2
    int vaddr[2];
    {
        const int g = lane >> 4, s16 = lane & 15;
        const int k = 2 * (g & 1) + ((s16 & 3) >> 1);
#pragma unroll
        for (int r = 0; r < 2; ++r)
            vaddr[r] = ((8 * r + 4 * hl + (s16 >> 2)) * 4 + (k ^ (2 * r + hl))) * 16 + (s16 & 1) * 8;
    }

    int t_lo = 0, t_hi = -1;
    if constexpr (BLK) {
        // this query block's allowed key blocks, in order, compacted by wave 0 (ballots)
        if (wave == 0) {
            const uint8_t* lrow = ba.layout + ((size_t)(bh % ba.H) * ba.nb + qt) * ba.nb;
            const int kmax = CAUS ? min(ba.nb, qt + 1) : ba.nb;   // causal: no key block past the diagonal
            int cnt = 0;
            for (int base = 0; base < kmax; base += 256) {
                uint8_t byte[4];                 // four loads in flight per lane (clamped, then tested)
#pragma unroll
                for (int k = 0; k < 4; ++k) byte[k] = lrow[min(base + 64 * k + lane, kmax - 1)];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int blk = base + 64 * k + lane;
                    const bool on = blk < kmax && byte[k] != 0;
                    const unsigned long long m = __ballot(on);
                    if (on) blist[cnt + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)blk;
                    cnt += __popcll(m);
                }
            }
            if (lane == 0) bcount = cnt;
        }
        __syncthreads();
        t_hi = 4 * bcount - 1;                  // tiles u = 0 .. 4 count - 1 (t_lo unused)
        if (t_hi < 0) {
            // no allowed key for any row of the block: O = 0, LSE = -inf
            if (my_q[0] < N) {
                __bf16* Orow = O + (size_t)bh * N * D + (size_t)my_q[0] * D;
#pragma unroll
                for (int j = 0; j < D / 32; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) *reinterpret_cast<bf16x4*>(Orow + j * 32 + 8 * g + 4 * hl) = (bf16x4){};
                if (hl == 0) LSE[(size_t)bh * N + my_q[0]] = -INFINITY;
            }
            return;
        }
    } else {
        tile_range<MASK, BC>(q0 + qoff, min(q0 + C::BR, N) - 1 + qoff, Nk, window, t_lo, t_hi);
    }
    if constexpr (SPLIT) {
        t_lo = max(t_lo, kb / BC);
        t_hi = min(t_hi, (ke - 1) / BC);
        if (t_hi < t_lo) {
            // no allowed key for any row of this block in this range: empty partials
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                if (my_q[b] < N) {
                    const size_t pr_row = ((size_t)bh * sa.n_split + split) * N + my_q[b];
                    float* po = sa.part_o + pr_row * D;
#pragma unroll
                    for (int j = 0; j < D / 32; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            *reinterpret_cast<float4*>(po + j * 32 + 8 * g + 4 * hl) = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (hl == 0) sa.part_lse[pr_row] = -INFINITY;
                }
            }
            return;
        }
    }
    const int n_tiles = t_hi - t_lo + 1;
    const int n_steps = KG == 1 ? n_tiles : (n_tiles + KG - 1) / KG;
    // key tile of step u: the range's u-th tile (tile KG u + kg with key groups), or
    // the u-th tile of the allowed blocks (a block's tiles past the sequence end load
    // the last key row and are masked).  A key group's tile past t_hi (the last step
    // of a range that does not split evenly) holds no allowed key of the workgroup's
    // rows: it is masked out whole, and the last tile of the range is loaded for it.
    auto tile_of = [&](int u) __attribute__((always_inline)) -> int {
        if constexpr (BLK) return __builtin_amdgcn_readfirstlane(4 * (int)blist[u >> 2] + (u & 3));
        else return t_lo + KG * u + kg;
    };
    auto tile_ld = [&](int u) __attribute__((always_inline)) -> int {
        if constexpr (KG > 1) return min(tile_of(u), t_hi);
        else return tile_of(u);
    };
    // This wave's own steps wu_lo .. wu_hi: the tiles that hold an allowed key for one
    // of its rows (the workgroup's range is the union over its waves, so at a band's
    // ends or past a causal diagonal a wave's range is shorter).  Outside them the
    // wave only loads its share of the tiles and meets the barriers; the step before
    // its first computes that step's scores, the step after its last that step's V
    // product.  Key groups and block layouts keep the whole range.
    int wu_lo = 0, wu_hi = n_steps - 1;
    if constexpr (KG == 1 && !BLK) {
        if (qw0 >= N) {
            wu_lo = n_steps;                              // every row past the end: no step
        } else {
            int wlo, whi;
            tile_range<MASK, BC>(qw0 + qoff, min(qw0 + C::RW, N) - 1 + qoff, Nk, window, wlo, whi);
            wu_lo = __builtin_amdgcn_readfirstlane(max(wlo, t_lo) - t_lo);
            wu_hi = __builtin_amdgcn_readfirstlane(min(whi, t_hi) - t_lo);
        }
    }

    // direct HBM -> LDS load of tile t of one tensor into `dst` (this wave's share):
    // per-lane offsets fixed for the kernel, the tile's offset a scalar
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kh, (uint32_t)Nk * (uint32_t)(D * 2));
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(Vh, (uint32_t)Nk * (uint32_t)(D * 2));
    auto dma = [&](__amdgpu_buffer_rsrc_t rs, int t, char* dst) __attribute__((always_inline)) {
        const int key0 = t * BC;
        if (key0 + BC <= Nk) {
            const uint32_t soff = (uint32_t)key0 * (uint32_t)(D * 2);
#pragma unroll
            for (int i = 0; i < C::LOADS_PER_WAVE; ++i)
                dma16(rs, (lds_void*)(dst + (rg * C::LOADS_PER_WAVE + i) * 1024), ld_off[i], soff);
        } else {
            // last tile: rows past the end load the last key row (any valid row; masked
            // later).  A tile wholly past the end (the last block of a block layout)
            // has rows_left < 0 and loads that row for every row.
            int kb0 = key0;                                                  // first row read
            if constexpr (BLK) kb0 = min(key0, Nk - 1);     // only block layouts reach past the end
            const uint32_t soff = (uint32_t)kb0 * (uint32_t)(D * 2);
            const int rows_left = Nk - 1 - kb0;                              // >= 0
#pragma unroll
            for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
                const int row = (int)(ld_off[i] / (2 * D));
                const uint32_t off = ld_off[i] - (uint32_t)(row - min(row, rows_left)) * (2 * D);
                dma16(rs, (lds_void*)(dst + (rg * C::LOADS_PER_WAVE + i) * 1024), off, soff);
            }
        }
    };

    f32x16 o[QB][ND];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int j = 0; j < ND; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][j][r] = 0.f;
    float m_run[QB], l_exp[QB], l_rnd[QB];     // running max (log2 domain, lazily raised), sum p, sum bf16(p)
#pragma unroll
    for (int b = 0; b < QB; ++b) { m_run[b] = -INFINITY; l_exp[b] = 0.f; l_rnd[b] = 0.f; }
    // The sum of the bf16-rounded probabilities runs on the matrix cores: one
    // v_mfma_f32_16x16x32_bf16 per 16-key slab takes the P^T operand of the V product
    // as its B operand, read as 16 columns x 4 lane groups of 8 keys.  Lane group g
    // holds query (lane mod 32) = column n + 16 (g mod 2), keys of half g / 2; the
    // 0/1 A operand sums groups {0, 2} into output rows 0 and 8 and groups {1, 3} into
    // rows 4 and 12, which are exactly the rows a lane's register 0 holds: each lane
    // accumulates its own query's row sum in a 4-register accumulator.  It replaces 2
    // vector instructions per score (a quarter of the 32x32x16 cost the same sum took
    // before): causal B2 H32 N8192 +3.7%, H32 N131072 +4.2%, d = 64 +4.7%.  The
    // split-KV kernels at 32 rows per wave and d = 128 keep the vector sum: there the
    // accumulator overflows the two-waves-per-SIMD register cap.
    constexpr bool RSM = (D == 64) || (QB == 2) || !SPLIT;
    f32x4 lr_acc[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) lr_acc[b][r] = 0.f;
    bf16x8 sel8;                               // the 0/1 A operand of the row-sum instruction
    {
        const int m = lane & 15, g = lane >> 4;
        const bool on = ((m == 0 || m == 8) && (g == 0 || g == 2)) || ((m == 4 || m == 12) && (g == 1 || g == 3));
        const __bf16 x = on ? (__bf16)1.0f : (__bf16)0.0f;
        sel8 = (bf16x8){x, x, x, x, x, x, x, x};
    }
    f32x16 sc[2][QB][KB];                      // S^T of two tiles (alternating): [query block][32-key block]
    bf16x8 pr[2][QB][NKS];                     // P^T of two tiles (alternating), [query block][16-key slab]

    // S^T = K_tile Q^T into sc[X]; each K operand read feeds QB matrix instructions
    auto scores = [&](auto xc, const char* kb) __attribute__((always_inline)) {
        constexpr int X = decltype(xc)::value;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const char* kp = kb + (s >> 1) * (4 * BC * 16) + k * (32 * 4 * 16) + ((s & 1) ? kaddr_o : kaddr_e);
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp);
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    if (s == 0) mfma_s_first(sc[X][b][k], ka, qreg[b][s]);
                    else mfma_s(sc[X][b][k], ka, qreg[b][s]);
                }
            }
        }
    };
    // >= 18 wait states before the vector ALUs read sc[X]
    auto settle_scores = [&](auto xc) __attribute__((always_inline)) {
        constexpr int X = decltype(xc)::value;
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int k = 0; k < KB; ++k) settle_v(sc[X][b][k]);
    };

    // allowed keys of each row form one interval [key_lo, key_hi] (the mask and the
    // sequence end together); element masking is one unsigned range test per score
    int key_lo[QB], key_span[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int qi = min(my_q[b], N - 1) + qoff;        // position among the keys
        int lo = 0, hi = Nk - 1;
        if (CAUS) hi = qi;
        if (MASK == ATTN_MASK_WINDOW) { lo = max(0, qi - window); hi = min(Nk - 1, qi + window); }
        if (MASK == ATTN_MASK_CAUSAL_WINDOW) { lo = max(0, qi - window); hi = qi; }
        if constexpr (SPLIT) {
            lo = max(lo, kb);
            hi = min(hi, ke - 1);
            if (hi < lo) { lo = 1 << 29; hi = lo; }       // no key of the range: nothing passes the test
        }
        key_lo[b] = lo;
        key_span[b] = hi - lo;
    }

    // element mask of tile t, only where the tile straddles the mask or the end (a
    // tile with no allowed key for a row leaves it all -inf, so its p = 0)
    auto mask_tile = [&](auto xc, int t) __attribute__((always_inline)) {
        constexpr int X = decltype(xc)::value;
        const int key0 = t * BC;
        const int pw0 = qw0 + qoff;                       // position of the wave's first row
        bool need = key0 + BC > Nk;
        if (CAUS) need |= key0 + BC - 1 > pw0;
        if (MASK == ATTN_MASK_WINDOW) need |= (key0 < pw0 + C::RW - 1 - window) || (key0 + BC - 1 > pw0 + window);
        if (MASK == ATTN_MASK_CAUSAL_WINDOW) need |= (key0 < pw0 + C::RW - 1 - window) || (key0 + BC - 1 > pw0);
        if constexpr (SPLIT) need |= (key0 < kb) || (key0 + BC > ke);
        if (need) {
            asm volatile("" ::: "memory");   // a side effect: keeps this a branch, not selects on every tile
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int rel = key0 + 4 * hl - key_lo[b];       // key of element r is rel + offset(r) past key_lo
#pragma unroll
                for (int k = 0; k < KB; ++k)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 32 * k + 8 * (r >> 2) + (r & 3);
                        if ((unsigned)(rel + off) > (unsigned)key_span[b]) sc[X][b][k][r] = -INFINITY;
                    }
            }
        }
    };

    // O^T += V^T P^T with pr[X]; each V operand read feeds QB matrix instructions
    auto pv = [&](auto xc, const char* vb) __attribute__((always_inline)) {
        constexpr int X = decltype(xc)::value;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int j = 0; j < ND; ++j) {
                const bf16x4 lo = lds_read_tr(vb, j * (4 * BC * 16) + ks * (16 * 4 * 16) + vaddr[0]);
                const bf16x4 hi = lds_read_tr(vb, j * (4 * BC * 16) + ks * (16 * 4 * 16) + vaddr[1]);
                const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int b = 0; b < QB; ++b)
                    o[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pr[X][b][ks], o[b][j], 0, 0, 0);
            }
            if constexpr (RSM) {
#pragma unroll
                for (int b = 0; b < QB; ++b)
                    lr_acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel8, pr[X][b][ks], lr_acc[b], 0, 0, 0);
            }
        }
    };

    // ---- one key tile as a fixed instruction schedule
    // The work of a tile is three independent streams:
    //     matrix cores : S(t+1) = K(t+1) Q^T  (NSM instructions), then O += V(t-1)^T P(t-1)  (NPM)
    //     vector ALUs  : softmax of S(t) -> P(t)  (NTASK tasks: row maxima, then one task per score)
    //     LDS reads    : the K and V operands, a few matrix instructions ahead of their use
    // They are laid out by hand, one matrix instruction per slot with a share of the
    // softmax behind it, and the compiler's scheduler is fenced between slots, so the
    // vector work runs while the matrix cores are busy instead of after them.
    constexpr int NSM = NS * QB;                 // score instructions per tile
    constexpr int NPC = NKS * ND;                // V operands per tile
    constexpr int GPV = ND * QB + (RSM ? QB : 0);   // per 16-key slab: V products, then the row sums
    constexpr int NPM = NKS * GPV;               // V-product (and row-sum) instructions per tile
    constexpr int NSLOT = NSM + NPM;
    constexpr int NEL = 16 * QB;                 // scores per lane per tile (KB = 1)
    // The reference is checked after the probabilities (a vote on their sums) at 32 rows
    // per wave, before them (a vote on the lane maxima) at 64: there the sums' vote
    // keeps the scores of S(t) live to the end of the tile, which the full register
    // file cannot afford (causal B2 H32 N8192 -7%); at 32 rows per wave it saves the
    // maxima (causal d = 64 H16 N8192 +7%, window +3%).  The block-layout kernels keep
    // the maxima vote (under their two-waves-per-SIMD cap the sums' vote spills).
    constexpr bool SUMVOTE = (QB == 1) && !BLK;
    constexpr int P0 = SUMVOTE ? 0 : QB + 1;     // first probability task
    constexpr int NTASK = P0 + NEL + 2 + 1;      // [maxima, vote,] scores (three stages), [vote,] sums
    constexpr int KPRE = 3;                      // K operands read before the first slot
    constexpr int VLEAD = 4;                     // slots between a V read and its first use
    static_assert(KB == 1, "the schedule assumes 32-key tiles");

    auto read_k = [&](const char* kb, int s) __attribute__((always_inline)) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(kb + (s >> 1) * (4 * BC * 16) + ((s & 1) ? kaddr_o : kaddr_e));
    };
    auto read_v = [&](const char* vb, int c) __attribute__((always_inline)) -> bf16x8 {
        const int ks = c / ND, j = c % ND;
        const bf16x4 lo = lds_read_tr(vb, j * (4 * BC * 16) + ks * (16 * 4 * 16) + vaddr[0]);
        const bf16x4 hi = lds_read_tr(vb, j * (4 * BC * 16) + ks * (16 * 4 * 16) + vaddr[1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // reference state per query block: m_run (log2 domain, -inf before any allowed
    // key) and the exponent offset base_run (m_run, or 0 while m_run = -inf).  ready:
    // every row of the wave has a reference (wave-uniform; once true, it stays true).
    // thr_raw (maxima vote) = (m_run + TAU) / c, the raw score above which the reference is raised.
    float base_run[QB], thr_raw[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) { base_run[b] = 0.f; thr_raw[b] = -INFINITY; }
    const float inv_c = 1.0f / c_log2;
    bool ready = false;
    const float PMAX = __builtin_amdgcn_exp2f(TAU);     // the largest probability against the reference

    // softmax task k of S(t) in sc[X].
    // Maxima vote: the lane maxima of the tile, then a wave vote on whether any row's
    // scores pass its threshold; if so (rare), every row takes its exact running
    // maximum as reference before the probabilities are taken.
    // Sums vote: the probabilities are taken against the current reference without
    // looking at the tile's maximum first; the last task votes on their sums.  A lane
    // whose probabilities sum to at most 2^TAU holds none above it, so the reference
    // stands (the common case); otherwise, or when a row meets its first allowed key,
    // every row takes its exact running maximum and the tile's probabilities are
    // computed again (rare).
    auto task = [&](auto xc, auto kc, float* mx, float* alpha, float* se, float* sr, float (*ev)[16],
                    bool& raise_any, int key0) __attribute__((always_inline)) {
        constexpr int X = decltype(xc)::value;
        constexpr int k = decltype(kc)::value;
        // pack the bf16 pair (r - 1, r) of block b into P^T: keys 8 (r/4) + 4 hl + r % 4,
        // slab r / 8, position r % 8; the rounded pair's sum when it stays on the VALU
        auto pack = [&](int b, auto rc, float e0, float e1) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            bf16x2 pa;
            pa[0] = (__bf16)e0;
            pa[1] = (__bf16)e1;
            const uint32_t pb = __builtin_bit_cast(uint32_t, pa);
            if constexpr (!RSM) {
                const float lo = __uint_as_float(pb << 16), hi = __uint_as_float(pb & 0xffff0000u);
                sr[b] = (r == 1) ? lo + hi : sr[b] + lo + hi;
            }
            pr[X][b][r >> 3][(r & 7) - 1] = pa[0];
            pr[X][b][r >> 3][r & 7] = pa[1];
        };
        if constexpr (k < P0 && k < QB) {                     // lane maximum of block k (v_max3 chain)
            constexpr int b = k;
            float m = fmaxf(fmaxf(sc[X][b][0][0], sc[X][b][0][1]), sc[X][b][0][2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, sc[X][b][0][r]), sc[X][b][0][r + 1]);
            mx[b] = fmaxf(m, sc[X][b][0][15]);
        } else if constexpr (k < P0) {                       // maxima vote
            bool over = false;
#pragma unroll
            for (int b = 0; b < QB; ++b) { over |= mx[b] > thr_raw[b]; alpha[b] = 1.f; }
            raise_any = __any(over);
            if (raise_any) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    const float m_new = fmaxf(m_run[b], swap32_max(mx[b]) * c_log2);
                    const float base = (m_new == -INFINITY) ? 0.f : m_new;
                    alpha[b] = __builtin_amdgcn_exp2f(m_run[b] - base);   // 0 while m_run = -inf
                    m_run[b] = m_new;
                    base_run[b] = base;
                    thr_raw[b] = (m_new + TAU) * inv_c;
                }
            }
        } else if constexpr (k < P0 + NEL + 2) {
            // The probabilities in three stages, each a step behind the previous one:
            // task P0 + h takes the exponent argument of score h, the exponential of score
            // h - 1 and the sums and packing of score h - 2.  One task runs per matrix
            // instruction, so the three operations of a task are independent and each
            // waits on a result from an earlier slot, not on its own neighbour.
            constexpr int hc = k - P0 - 2;                   // sums and packing
            if constexpr (hc >= 0 && hc < NEL) {
                constexpr int b = hc / 16, r = hc % 16;
                const float e = ev[b][r];
                se[b] = (r == 0) ? e : se[b] + e;
                if constexpr (r & 1) pack(b, IntC<r>{}, ev[b][r - 1], e);
            }
            constexpr int hb = k - P0 - 1;                   // exponential
            if constexpr (hb >= 0 && hb < NEL) {
                constexpr int b = hb / 16, r = hb % 16;
                ev[b][r] = __builtin_amdgcn_exp2f(ev[b][r]);
            }
            constexpr int ha = k - P0;                       // exponent argument
            if constexpr (ha < NEL) {
                constexpr int b = ha / 16, r = ha % 16;
                ev[b][r] = __builtin_fmaf(sc[X][b][0][r], c_log2, -base_run[b]);
            }
        } else if constexpr (SUMVOTE) {                      // sums vote, then the running sums
            bool over = false;
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                over |= !(se[b] <= PMAX);
                alpha[b] = 1.f;
            }
            if (!ready) {
                // a row without a reference whose allowed keys meet this tile
#pragma unroll
                for (int b = 0; b < QB; ++b)
                    over |= m_run[b] == -INFINITY &&
                            (unsigned)(key0 + BC - 1 - key_lo[b]) <= (unsigned)(key_span[b] + BC - 1);
            }
            raise_any = __any(over);
            if (raise_any) {
                // rare: every row of the wave takes its exact running maximum as reference
                asm volatile("" ::: "memory");
                bool have = true;
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    float m = fmaxf(fmaxf(sc[X][b][0][0], sc[X][b][0][1]), sc[X][b][0][2]);
#pragma unroll
                    for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, sc[X][b][0][r]), sc[X][b][0][r + 1]);
                    m = fmaxf(m, sc[X][b][0][15]);
                    const float m_new = fmaxf(m_run[b], swap32_max(m) * c_log2);
                    const float base = (m_new == -INFINITY) ? 0.f : m_new;
                    alpha[b] = __builtin_amdgcn_exp2f(m_run[b] - base);   // 0 while m_run = -inf
                    m_run[b] = m_new;
                    base_run[b] = base;
                    have &= m_new != -INFINITY;
                    // this tile's probabilities again, against the new reference
                    static_for<0, 16>([&](auto rc) {
                        constexpr int r = decltype(rc)::value;
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[X][b][0][r], c_log2, -base));
                        se[b] = (r == 0) ? e : se[b] + e;
                        ev[b][r] = e;
                        if constexpr (r & 1) pack(b, rc, ev[b][r - 1], e);
                    });
                }
                ready = !__any(!have);
            }
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                l_exp[b] = __builtin_fmaf(alpha[b], l_exp[b], se[b]);
                if constexpr (!RSM) l_rnd[b] = __builtin_fmaf(alpha[b], l_rnd[b], sr[b]);
            }
        } else {                                             // running sums
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                l_exp[b] = __builtin_fmaf(alpha[b], l_exp[b], se[b]);
                if constexpr (!RSM) l_rnd[b] = __builtin_fmaf(alpha[b], l_rnd[b], sr[b]);
            }
        }
    };

    // rare (the maximum grows by > TAU); kept as a real branch (the empty asm is a
    // side effect the compiler may not speculate), so O is not touched on other tiles
    auto rescale_o = [&](const float* alpha) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int j = 0; j < ND; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][j][r] *= alpha[b];
        if constexpr (RSM) {
#pragma unroll
            for (int b = 0; b < QB; ++b) lr_acc[b][0] *= alpha[b];    // the register the row sum is read from
        }
    };

    // Tiles u = 0 .. n_tiles - 1 (t = t_lo + u).  K(t) lives in kbuf[u % 2], V(t) in
    // vbuf[u % 2], S(t) in sc[u % 2], P(t) in pr[u % 2].  Tile u streams K(t+2) and
    // V(t) into LDS, masks S(t) where the tile straddles the mask, then runs the
    // fixed schedule and one barrier.  Every wave runs every tile of the workgroup's
    // range (a tile outside its rows' mask comes out with p = 0); the last tile's
    // score stream reads a stale buffer and its result is never used.  P starts at
    // zero and vbuf1 is zero-filled, so the first V product adds 0.
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int k = 0; k < NKS; ++k) { pr[0][b][k] = (bf16x8){}; pr[1][b][k] = (bf16x8){}; }
    for (int i = tid * 16; i < KG * C::TILE_BYTES; i += C::NT * 16)
        *reinterpret_cast<u32x4*>(vbuf1 + i) = (u32x4){0u, 0u, 0u, 0u};
    dma(krs, tile_ld(0), kb0);
    if (n_steps > 1) dma(krs, tile_ld(1), kb1);
    // Q was requested at kernel start and is waited for only here (the wait orders
    // the pinning below after the tile requests), so the Q loads and the first K
    // tiles are in flight together.  From here on Q sits in AGPRs, written (and
    // padded) well before any MFMA reads it.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int s = 0; s < NS; ++s) settle_qa(qreg[b][s]);
    __syncthreads();
    if (wu_lo == 0) {
        scores(IntC<0>{}, kb0);
        settle_scores(IntC<0>{});
    }
    __syncthreads();     // every wave is done with K(t_lo) before tile 0 refills its buffer

    auto iter = [&](auto parity, int u) __attribute__((always_inline)) {
        constexpr int B = decltype(parity)::value;        // u % 2
        constexpr int X = 1 - B;
        const int t = tile_of(u);
        char* k_own = B ? kb1 : kb0;                      // held K(t) (consumed); receives K of step u+2
        const char* k_next = B ? kb0 : kb1;               // K of step u+1
        char* v_own = B ? vb1 : vb0;                      // held V of step u-2 (consumed); receives V(t)
        const char* v_prev = B ? vb0 : vb1;               // V of step u-1
        if (u + 2 < n_steps) dma(krs, tile_ld(u + 2), k_own);
        dma(vrs, KG > 1 ? tile_ld(u) : t, v_own);
        mask_tile(IntC<B>{}, t);

        float mx[QB], alpha[QB], se[QB], sr[QB];
        float ev[QB][16];
        bool raise_any = false;
        bf16x8 ka[NS], va[NPC];
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, KPRE>([&](auto sc_) { ka[decltype(sc_)::value] = read_k(k_next, decltype(sc_)::value); });
        task(IntC<B>{}, IntC<0>{}, mx, alpha, se, sr, ev, raise_any, t * BC);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, NSLOT>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            // matrix instruction of slot i
            if constexpr (i < NSM) {
                constexpr int s = i / QB, b = i % QB;
                if constexpr (s == 0) mfma_s_first(sc[X][b][0], ka[s], qreg[b][s]);
                else mfma_s(sc[X][b][0], ka[s], qreg[b][s]);
            } else {
                constexpr int ks = (i - NSM) / GPV, w = (i - NSM) % GPV;
                if constexpr (w < ND * QB) {
                    constexpr int j = w / QB, b = w % QB;
                    o[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks * ND + j], pr[X][b][ks], o[b][j], 0, 0, 0);
                } else {
                    constexpr int b = w - ND * QB;
                    lr_acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel8, pr[X][b][ks], lr_acc[b], 0, 0, 0);
                }
            }
            // LDS reads for later slots
            if constexpr (i < NSM && i % QB == 0 && i / QB + KPRE < NS) ka[i / QB + KPRE] = read_k(k_next, i / QB + KPRE);
            static_for<0, NPC>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                constexpr int first_use = NSM + (c / ND) * GPV + (c % ND) * QB;
                if constexpr (first_use - VLEAD == i || (i == 0 && first_use - VLEAD < 0)) va[c] = read_v(v_prev, c);
            });
            // softmax tasks of slot i: task k (>= 1) runs in slot (k - 1) NSLOT / (NTASK - 1)
            static_for<1, NTASK>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr ((k - 1) * NSLOT / (NTASK - 1) == i) task(IntC<B>{}, kc, mx, alpha, se, sr, ev, raise_any, t * BC);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        // the softmax results are consumed here (an empty asm), so they cannot sink below the branch
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            asm volatile("" ::"v"(l_exp[b]), "v"(l_rnd[b]));
#pragma unroll
            for (int k = 0; k < NKS; ++k) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pr[B][b][k])));
            // S(t+1) stays allocated at least until here, NPM matrix instructions after its
            // last score instruction (in order, so long complete).  On the last tile its
            // value is unused: without this the compiler could hand its registers to other
            // values while the asm score instructions, which it cannot see into, still
            // write them.
            asm volatile("" : "+v"(sc[X][b][0]));
        }
        if (raise_any) rescale_o(alpha);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    // a step outside the wave's own range: its loads, the wait and the barrier only
    auto idle = [&](int u) __attribute__((always_inline)) {
        if (u + 2 < n_steps) dma(krs, tile_ld(u + 2), (u & 1) ? kb1 : kb0);
        dma(vrs, tile_ld(u), (u & 1) ? vb1 : vb0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    // the step before the wave's first (its scores) or after its last (its V product)
    auto edge = [&](auto parity, int u, bool first) __attribute__((always_inline)) {
        constexpr int B = decltype(parity)::value;
        constexpr int X = 1 - B;
        if (u + 2 < n_steps) dma(krs, tile_ld(u + 2), B ? kb1 : kb0);
        dma(vrs, tile_ld(u), B ? vb1 : vb0);
        if (first) {
            scores(IntC<X>{}, B ? kb0 : kb1);
            settle_scores(IntC<X>{});
        } else {
            pv(IntC<X>{}, B ? vb0 : vb1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    int u = 0;
    for (; u < wu_lo - 1; ++u) idle(u);
    if (u == wu_lo - 1) {
        if (u & 1) edge(IntC<1>{}, u, true); else edge(IntC<0>{}, u, true);
        ++u;
    }
    if (u <= wu_hi && (u & 1)) iter(IntC<1>{}, u++);
    for (; u + 1 <= wu_hi; u += 2) {
        iter(IntC<0>{}, u);
        iter(IntC<1>{}, u + 1);
    }
    if (u <= wu_hi) iter(IntC<0>{}, u++);
    if (u == wu_hi + 1 && u < n_steps) {
        if (u & 1) edge(IntC<1>{}, u, false); else edge(IntC<0>{}, u, false);
        ++u;
    }
    for (; u < n_steps; ++u) idle(u);
    // closing step: the V product of the last step (its V in vbuf[(n_steps - 1) % 2]),
    // for a wave whose own steps reach it
    if (wu_hi == n_steps - 1) {
        if (u & 1) pv(IntC<0>{}, vb0); else pv(IntC<1>{}, vb1);
    }

    // ---- key groups: merge the softmax states of groups 1 .. KG-1 into group 0.  With
    // M = max over groups of the running maximum m_g and weight a_g = 2^(m_g - M) (0
    // for a group that met no allowed key of the row), O = sum a_g O_g, and both sums
    // likewise: the combination of softmax pieces over disjoint key sets.  Group g's
    // accumulators go through the (idle) tile buffers, lane by lane in the layout
    // both waves share.
    if constexpr (KG > 1) {
        // one piece per (group g >= 1, row group, 32-row block b): ND x 4 x 64 lanes x 16 bytes,
        // KG / 2 pieces per buffer
        constexpr int PIECE = ND * 4 * 64 * 16;
        constexpr int PPB = KG / 2;
        static_assert(PPB * PIECE <= KG * C::TILE_BYTES, "pieces fit a buffer");
        static_assert((KG - 1) * C::RG * QB <= 4 * PPB, "merge fits the tile buffers");
        __syncthreads();                 // every wave is done with the tile buffers
        auto o_slot = [&](int g, int b, int j, int q) __attribute__((always_inline)) -> float4* {
            // quarter q of 32-row block j of O^T; lanes contiguous
            const int piece = ((g - 1) * C::RG + rg) * QB + b;
            const int k = piece / PPB;
            char* const buf = k == 0 ? kbuf0 : k == 1 ? kbuf1 : k == 2 ? vbuf0 : vbuf1;
            return reinterpret_cast<float4*>(buf + (piece % PPB) * PIECE) + (j * 4 + q) * 64 + lane;
        };
        auto s_slot = [&](int g, int b, int k) __attribute__((always_inline)) -> float* {
            return mstate + ((((g - 1) * C::RG + rg) * QB + b) * 3 + k) * 64 + lane;
        };
        if (kg > 0) {
#pragma unroll
            for (int b = 0; b < QB; ++b) {
#pragma unroll
                for (int j = 0; j < ND; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *o_slot(kg, b, j, q) = make_float4(o[b][j][4 * q], o[b][j][4 * q + 1], o[b][j][4 * q + 2], o[b][j][4 * q + 3]);
                *s_slot(kg, b, 0) = m_run[b];
                *s_slot(kg, b, 1) = l_exp[b];
                *s_slot(kg, b, 2) = RSM ? lr_acc[b][0] : l_rnd[b];
            }
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                float mg[KG];
                mg[0] = m_run[b];
#pragma unroll
                for (int g = 1; g < KG; ++g) mg[g] = *s_slot(g, b, 0);
                float M = mg[0];
#pragma unroll
                for (int g = 1; g < KG; ++g) M = fmaxf(M, mg[g]);
                float a[KG];
#pragma unroll
                for (int g = 0; g < KG; ++g) a[g] = mg[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg[g] - M);
                float le = a[0] * l_exp[b], lr = a[0] * (RSM ? lr_acc[b][0] : l_rnd[b]);
#pragma unroll
                for (int g = 1; g < KG; ++g) {
                    le = __builtin_fmaf(a[g], *s_slot(g, b, 1), le);
                    lr = __builtin_fmaf(a[g], *s_slot(g, b, 2), lr);
                }
#pragma unroll
                for (int j = 0; j < ND; ++j) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[b][j][r] *= a[0];
#pragma unroll
                    for (int g = 1; g < KG; ++g)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 x = *o_slot(g, b, j, q);
                            o[b][j][4 * q] = __builtin_fmaf(a[g], x.x, o[b][j][4 * q]);
                            o[b][j][4 * q + 1] = __builtin_fmaf(a[g], x.y, o[b][j][4 * q + 1]);
                            o[b][j][4 * q + 2] = __builtin_fmaf(a[g], x.z, o[b][j][4 * q + 2]);
                            o[b][j][4 * q + 3] = __builtin_fmaf(a[g], x.w, o[b][j][4 * q + 3]);
                        }
                }
                m_run[b] = M;
                l_exp[b] = le;
                if constexpr (RSM) lr_acc[b][0] = lr;
                else l_rnd[b] = lr;
            }
        }
        __syncthreads();                 // the merge reads are done before the staging writes
        if (kg > 0) return;              // no barrier follows
    }

    // ---- epilogue: O = acc / sum bf16(p) (bf16, nearest even), LSE = (m + log2 sum p) ln 2
    // A lane holds 16 values of one O row, so direct stores would write 16-byte
    // pieces of 32 rows per instruction.  Instead each wave stages a 32-row block in
    // one of the (now idle) tile buffers, row-major with the 16-byte chunks rotated
    // by the row (no bank conflicts), and writes whole rows: 1 KB per instruction.
    const bool partials = SPLIT && sa.n_split > 1;
    if (!partials && KG == 1) __syncthreads();      // every wave is done with the tile buffers
    char* const stage = wave == 0 ? kbuf0 : wave == 1 ? kbuf1 : wave == 2 ? vbuf0 : vbuf1;
    constexpr int ROWB = 2 * D;          // bytes of one bf16 O row
    constexpr int NCH = D / 8;           // 16-byte chunks per row
    static_assert(32 * ROWB <= C::TILE_BYTES, "a 32-row block of O fits one tile buffer");
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float le = swap32_add(l_exp[b]);
        const float lr = RSM ? lr_acc[b][0] : swap32_add(l_rnd[b]);
        if (SPLIT && sa.n_split > 1) {
            if (my_q[b] < N) {
                // this range's partial: O normalised within the range (fp32), its LSE;
                // a row without an allowed key here gets O = 0 and LSE = -inf
                const size_t pr_row = ((size_t)bh * sa.n_split + split) * N + my_q[b];
                float* po = sa.part_o + pr_row * D;
                const float inv = lr > 0.f ? 1.0f / lr : 0.f;
#pragma unroll
                for (int j = 0; j < ND; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<float4*>(po + j * 32 + 8 * g + 4 * hl) =
                            make_float4(o[b][j][4 * g] * inv, o[b][j][4 * g + 1] * inv, o[b][j][4 * g + 2] * inv,
                                        o[b][j][4 * g + 3] * inv);
                if (hl == 0)
                    sa.part_lse[pr_row] = le > 0.f ? (m_run[b] + __builtin_amdgcn_logf(le)) * 0.69314718055994531f
                                                   : -INFINITY;
            }
            continue;
        }
        // stage: row ln, elements j 32 + 8 g + 4 hl .. +3 = half hl of chunk 4 j + g
        // (rows past the sequence end are staged too, never stored)
        const float inv = 1.0f / lr;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[b][j][4 * g + e] * inv);
                const int c = 4 * j + g;
                *reinterpret_cast<bf16x4*>(stage + ln * ROWB + ((c ^ (ln & (NCH - 1))) * 16) + 8 * hl) = val;
            }
        }
        __builtin_amdgcn_wave_barrier();     // the wave's LDS writes precede its reads (in order per wave)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 32 * ROWB / 1024; ++i) {
            const int f = i * 1024 + lane * 16;
            const int row = f / ROWB, c = (f % ROWB) / 16;
            const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * ROWB + ((c ^ (row & (NCH - 1))) * 16));
            const int qrow = qw0 + 32 * b + row;
            if (qrow < N) *reinterpret_cast<u32x4*>(O + head + (size_t)qrow * D + c * 8) = val;
        }
        asm volatile("" ::: "memory");       // the next block's staging writes follow these reads
        if (hl == 0 && my_q[b] < N)
            LSE[(size_t)bh * N + my_q[b]] = (m_run[b] + __builtin_amdgcn_logf(le)) * 0.69314718055994531f;
    }
}

// Grid and queue of a dense forward launch of `total` items.  With the queue, the
// first three quarters of every XCD's list stay fixed (workgroup i computes item i,
// no claim on the way) and the rest, plus half as many extra workgroups per XCD,
// claim the tail.  The library's own choice uses it for unmasked and causal grids of
// at least 8192 workgroups (A/B on one box: causal H32 N131072 +1.7%; causal B2 H32
// N8192, 2048 workgroups, -1.3%; window w = 512 H32 N32768, 8192 workgroups, -6%,
// where each head's short blocks lose their L2 sharing when claimed elsewhere).
struct WorkPlan {
    long long grid;
    unsigned* wq;
    int n_static, n_dyn;
};
static WorkPlan work_plan(long long total, bool eligible, bool band, hipStream_t stream) {
    WorkPlan p{total, nullptr, 0, 0};
    const int mode = attn_sched_work_queue();
    if (!eligible || mode == 0 || (mode < 0 && (band || total < 8192)) || total > (1LL << 30)) return p;
    // a launch captured into a graph keeps its slot for every replay, and replays of
    // one graph may overlap: captured launches run without the queue
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return p;
    }
    unsigned* wq = attn_wq_slot();
    if (!wq) return p;
    const long long n_min = total / WQ_XCD;                // items of the shortest list
    const long long fixed = n_min * 3 / 4;                 // per list
    const long long extra = std::max(4LL, (n_min - fixed) / 2);
    p.wq = wq;
    p.n_static = (int)(fixed * WQ_XCD);
    p.grid = total + extra * WQ_XCD;
    p.n_dyn = (int)(p.grid - p.n_static);
    return p;
}

template <int D, int QB, int KB, int MASK, int KG = 1>
static int launch(const AttnLaunch& a) {
    using C = Cfg<D, QB, KB, KG>;
    const int nqt = (a.N + C::BR - 1) / C::BR;
    const long long total = (long long)nqt * a.B * a.H;
    int hg = attn_sched_head_group();
    if (hg < 0) hg = head_group(a.N, a.d);      // K and V of a head: causal B4 H32 N16384 d128 +12%
    // the queue serves the 64-row kernels of the unmasked and causal forward
    constexpr bool ELIG = QB == 2 && KG == 1 && (MASK == ATTN_MASK_NONE || MASK == ATTN_MASK_CAUSAL);
    const WorkPlan wp = work_plan(total, ELIG, MASK == ATTN_MASK_WINDOW || MASK == ATTN_MASK_CAUSAL_WINDOW,
                                  (hipStream_t)a.stream);
    if constexpr (ELIG) {
        if (wp.wq) {
            hipLaunchKernelGGL((fwd_kernel<D, QB, KB, MASK, false, KG, true>), dim3((unsigned)wp.grid), dim3(C::NT),
                               0, (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                               (__bf16*)a.out, a.lse, a.B * a.H, a.N, nqt, a.c_log2, a.negate_q, a.window,
                               SplitArgs{}, BlockArgs{}, hg, wp.wq, wp.n_static, wp.n_dyn);
            return 0;
        }
    }
    hipLaunchKernelGGL((fwd_kernel<D, QB, KB, MASK, false, KG>), dim3((unsigned)total), dim3(C::NT), 0,
                       (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (__bf16*)a.out, a.lse, a.B * a.H, a.N, nqt, a.c_log2, a.negate_q, a.window, SplitArgs{},
                       BlockArgs{}, hg);
    return 0;
}

// ---- split-KV: merge the ranges' partials of every row by their log-sum-exp:
// LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the exact combination of
// softmax pieces over disjoint key sets).  One wave per row.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                    __bf16* __restrict__ O, float* __restrict__ LSE, long long rows,
                                                    int N, int n_split) {
    constexpr int PL = D / 64;                         // dims per lane
    constexpr int G = 8;                               // partial rows loaded together
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const long long bh = row / N, r = row - bh * N;
    const float* pl = part_lse + bh * n_split * (long long)N + r;
    float m = -INFINITY;
    for (int s = lane; s < n_split; s += 64) m = fmaxf(m, pl[(long long)s * N]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
    float l = 0.f;
    for (int s = lane; s < n_split; s += 64) l += __expf(pl[(long long)s * N] - m);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) l += __shfl_xor(l, k);
    const float lse = m == -INFINITY ? -INFINITY : m + __logf(l);   // no allowed key anywhere
    float acc[PL];
#pragma unroll
    for (int c = 0; c < PL; ++c) acc[c] = 0.f;
    const float* po0 = part_o + (bh * n_split * (long long)N + r) * D + lane * PL;
    const long long stride = (long long)N * D;         // between the ranges' partial rows
    for (int c0 = 0; c0 < n_split; c0 += 64) {
        // lane s holds the weight of range c0 + s (an empty range has O = 0 and weight 0)
        const int sl = c0 + lane;
        const float w_l = (sl < n_split && lse != -INFINITY) ? __expf(pl[(long long)sl * N] - lse) : 0.f;
        const int cn = min(64, n_split - c0);
        for (int g0 = 0; g0 < cn; g0 += G) {
            float v[G][PL];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int c = 0; c < PL; ++c) v[g][c] = (g0 + g < cn) ? po0[(c0 + g0 + g) * stride + c] : 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float w = __shfl(w_l, g0 + g);
#pragma unroll
                for (int c = 0; c < PL; ++c) acc[c] = __builtin_fmaf(w, v[g][c], acc[c]);
            }
        }
    }
    __bf16* orow = O + row * D + lane * PL;
#pragma unroll
    for (int c = 0; c < PL; ++c) orow[c] = (__bf16)acc[c];
    if (lane == 0) LSE[row] = lse;
}

template <int D, int MASK>
static int launch_split(const AttnLaunch& a, const SplitArgs& sa) {
    using C = Cfg<D, 1, 1>;
    const int nqt = (a.N + C::BR - 1) / C::BR;
    const long long grid = (long long)nqt * a.B * a.H * sa.n_split;
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL((fwd_kernel<D, 1, 1, MASK, true>), dim3((unsigned)grid), dim3(C::NT), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.out, a.lse,
                       a.B * a.H, a.N, nqt, a.c_log2, a.negate_q, a.window, sa);
    if (sa.n_split == 1) return 0;
    const long long rows = (long long)a.B * a.H * a.N;
    hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       sa.part_o, sa.part_lse, (__bf16*)a.out, a.lse, rows, a.N, sa.n_split);
    return 0;
}

template <int D>
static int by_mask_split(const AttnLaunch& a, const SplitArgs& sa) {
    switch (a.mask_kind) {
        case ATTN_MASK_CAUSAL: return launch_split<D, ATTN_MASK_CAUSAL>(a, sa);
        case ATTN_MASK_WINDOW: return launch_split<D, ATTN_MASK_WINDOW>(a, sa);
        case ATTN_MASK_CAUSAL_WINDOW: return launch_split<D, ATTN_MASK_CAUSAL_WINDOW>(a, sa);
        default: return launch_split<D, ATTN_MASK_NONE>(a, sa);
    }
}

template <int D, int QB, int KB, int KG = 1>
static int by_mask(const AttnLaunch& a) {
    switch (a.mask_kind) {
        case ATTN_MASK_CAUSAL: return launch<D, QB, KB, ATTN_MASK_CAUSAL, KG>(a);
        case ATTN_MASK_WINDOW: return launch<D, QB, KB, ATTN_MASK_WINDOW, KG>(a);
        case ATTN_MASK_CAUSAL_WINDOW: return launch<D, QB, KB, ATTN_MASK_CAUSAL_WINDOW, KG>(a);
        default: return launch<D, QB, KB, ATTN_MASK_NONE, KG>(a);
    }
}

// key groups: the dense masks only (no mask, causal)
template <int D, int QB, int KG>
static int by_mask_kg(const AttnLaunch& a) {
    switch (a.mask_kind) {
        case ATTN_MASK_CAUSAL: return launch<D, QB, 1, ATTN_MASK_CAUSAL, KG>(a);
        case ATTN_MASK_NONE: return launch<D, QB, 1, ATTN_MASK_NONE, KG>(a);
        default: return ATTN_ERR_BAD_MASK;      // never chosen for the band masks
    }
}

// the kernel of one tile shape: 32 or 64 query rows per wave, 1, 2 or 4 key groups
template <int D>
static int by_shape(const AttnLaunch& a, bool rows32, int key_groups) {
    switch (key_groups) {
        case 2: return rows32 ? by_mask_kg<D, 1, 2>(a) : by_mask_kg<D, 2, 2>(a);
        case 4: return rows32 ? by_mask_kg<D, 1, 4>(a) : by_mask_kg<D, 2, 4>(a);
        default: return rows32 ? by_mask<D, 1, 1>(a) : by_mask<D, 2, 1>(a);
    }
}

}  // namespace attn_bf16

#ifdef ATTN_FWD_D64_TU
// The dense d = 64 kernels, compiled in a translation unit of their own
// (attn_fwd_bf16_d64.hip) with matrix-instruction accumulators in VGPRs.
int attn_launch_bf16_d64(const AttnLaunch& a, bool rows32, int key_groups) {
    using namespace attn_bf16;
    return by_shape<64>(a, rows32, key_groups);
}
#else

// Compute units of the current device (cached per device; the value never changes).
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Rows per wave: 64 (two 32-row blocks: each K/V operand read feeds two matrix
// instructions) unless that leaves the grid short of two workgroups per compute
// unit, the mask is a narrow band (a window w < 2048, or a causal window w < 4096),
// or the mask is causal over fewer than 8192 keys (16384 at d = 64).  There 32 rows
// per wave win: half the key tiles a workgroup spans outside its band or past the
// diagonal, twice the workgroups, and a register budget that fits two waves per SIMD
// (interleaved A/B timing on one MI355X: causal N4096-6144 +4-10%, causal d = 64
// N8192 +3%; H32 N32768 window w512 755 against 677 TFLOP/s, w1024 871 against 858,
// causal window w1024 +13%, w2048 +2%; at N8192 causal d = 128, 64 rows per wave
// lead by 0.5-2%).  Wider bands go to 64 rows per wave, since each wave computes
// only its own rows' tiles: window w2048 +4.5%, w3072 +7%, w4096 +8% (d = 64: w2048
// +3%, w4096 +5%), causal window w4096 +5%, w8192 +7%.
int attn_launch_bf16(const AttnLaunch& a) {
    using namespace attn_bf16;
    const long long grid64 = (long long)((a.N + 255) / 256) * a.B * a.H;
    const bool band = (a.mask_kind == ATTN_MASK_WINDOW && a.window < 2048 && a.window < a.N - 1) ||
                      (a.mask_kind == ATTN_MASK_CAUSAL_WINDOW && a.window < 4096 && a.window < a.N - 1);
    const bool short_causal = (a.mask_kind == ATTN_MASK_CAUSAL ||
                               (a.mask_kind == ATTN_MASK_CAUSAL_WINDOW && a.window >= a.N - 1)) &&
                              a.N < (a.d == 64 ? 16384 : 8192);
    bool rows32 = band || short_causal || grid64 < 2LL * device_cus();

    // Key groups (no mask or causal) where the query blocks alone leave the device
    // short of work; g32 = workgroups of 128 query rows, c = compute units.  From A/B
    // timing of every shape on one MI355X (TFLOP/s, one key group -> the choice):
    //   d = 128: g32 <= c, or causal g32 <= 2c: 64 rows x 2 groups (H8 N4096 898 -> 962,
    //            causal H8 N8192 802 -> 948, causal H4 N16384 821 -> 1002);
    //   d = 64:  g32 <= c / 2, or causal g32 <= c: 64 rows x 4 groups (H4 N4096 319 -> 564,
    //            causal H4 N8192 328 -> 552); g32 <= c, or causal g32 <= 2c: 32 rows x
    //            2 groups (H8 N4096 584 -> 694, causal H8 N8192 605 -> 769).
    // Above that one group wins (H16 N4096 d64 840 against 757).
    const bool dense = a.mask_kind == ATTN_MASK_NONE || a.mask_kind == ATTN_MASK_CAUSAL;
    bool plan_rows32 = false;
    int plan_kg = 1;
    if (dense) {
        const bool causal = a.mask_kind == ATTN_MASK_CAUSAL;
        const long long c = device_cus();
        const long long g32 = (long long)((a.N + 127) / 128) * a.B * a.H;
        if (a.d == 128) {
            if (g32 <= (causal ? 2 * c : c)) plan_kg = 2;
        } else if (g32 <= (causal ? c : c / 2)) {
            plan_kg = 4;
        } else if (g32 <= (causal ? 2 * c : c)) {
            plan_kg = 2;
            plan_rows32 = true;
        }
    }
    // explicit choices (every choice computes the same attention; tests run each)
    const int forced_rows = attn_sched_rows_per_wave();
    const int forced_kg = attn_sched_key_groups();
    int kg = 1;
    if (forced_kg > 0) {
        kg = dense ? forced_kg : 1;
        if (forced_rows) rows32 = forced_rows == 32;
        else if (kg > 1) rows32 = a.d == 64 && kg == 2;
    } else if (plan_kg > 1 && (!forced_rows || (forced_rows == 32) == plan_rows32)) {
        kg = plan_kg;
        rows32 = plan_rows32;
    } else if (forced_rows) {
        rows32 = forced_rows == 32;
    }
    if (a.d == 128) return by_shape<128>(a, rows32, kg);
    return attn_launch_bf16_d64(a, rows32, kg);
}

// Key ranges for the split-KV path: enough workgroups to fill the 256 CUs twice, at
// least 256 keys per range, ranges a multiple of the 32-key tile.  A function of the
// shape alone (no device query), so the workspace size is known before any launch.
void attn_kv_split_plan(int B, int H, int Nq, int Nk, int* n_split, int* split_len) {
    const long long blocks = (long long)((Nq + 127) / 128) * B * H;
    const long long want = (512LL + blocks - 1) / blocks;
    const long long max_split = (Nk + 255) / 256;
    long long s = want < 1 ? 1 : want;
    if (s > max_split) s = max_split;
    if (s < 1) s = 1;
    long long len = (Nk + s - 1) / s;
    len = (len + 31) / 32 * 32;
    *split_len = (int)len;
    *n_split = (int)((Nk + len - 1) / len);
}

int attn_launch_block_bf16(const AttnLaunch& a, const uint8_t* layout, int causal) {
    using namespace attn_bf16;
    BlockArgs ba;
    ba.layout = layout;
    ba.H = a.H;
    ba.nb = (a.N + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
    const int BH = a.B * a.H;
    const unsigned grid = (unsigned)((long long)ba.nb * BH);
    // head groups after the leading blocks: BigBird H32 N32768 +2%, a uniform random
    // layout (10% of blocks) B2 H32 N16384 +12%
    int hg = attn_sched_head_group();
    if (hg < 0) hg = head_group(a.N, a.d);
    hipStream_t st = (hipStream_t)a.stream;
    const __bf16 *q = (const __bf16*)a.q, *k = (const __bf16*)a.k, *v = (const __bf16*)a.v;
    __bf16* o = (__bf16*)a.out;
    constexpr int NT = Cfg<128, 1, 1>::NT;
    if (a.d == 128) {
        if (causal)
            hipLaunchKernelGGL((fwd_kernel<128, 1, 1, MASK_BLOCK_CAUSAL>), dim3(grid), dim3(NT), 0, st, q, k, v, o, a.lse,
                               BH, a.N, ba.nb, a.c_log2, a.negate_q, 0, SplitArgs{}, ba, hg);
        else
            hipLaunchKernelGGL((fwd_kernel<128, 1, 1, MASK_BLOCK>), dim3(grid), dim3(NT), 0, st, q, k, v, o, a.lse, BH,
                               a.N, ba.nb, a.c_log2, a.negate_q, 0, SplitArgs{}, ba, hg);
    } else {
        if (causal)
            hipLaunchKernelGGL((fwd_kernel<64, 1, 1, MASK_BLOCK_CAUSAL>), dim3(grid), dim3(NT), 0, st, q, k, v, o, a.lse,
                               BH, a.N, ba.nb, a.c_log2, a.negate_q, 0, SplitArgs{}, ba, hg);
        else
            hipLaunchKernelGGL((fwd_kernel<64, 1, 1, MASK_BLOCK>), dim3(grid), dim3(NT), 0, st, q, k, v, o, a.lse, BH,
                               a.N, ba.nb, a.c_log2, a.negate_q, 0, SplitArgs{}, ba, hg);
    }
    return 0;
}

int attn_kv_max_splits(int B, int H, int Nq, int Nk, int d) {
    if (Nq == 1) return attn_decode_max_splits(B * H, Nk, d);
    int n_split, split_len;
    attn_kv_split_plan(B, H, Nq, Nk, &n_split, &split_len);
    return n_split;
}

int attn_launch_kv_bf16(const AttnLaunch& a, int Nk, int q_offset, float* part_o, float* part_lse) {
    using namespace attn_bf16;
    if (a.N == 1) {
        // decode: the query's allowed keys are one interval
        const int p = q_offset;
        int lo = 0, hi = Nk - 1;
        if (a.mask_kind == ATTN_MASK_CAUSAL) hi = p;
        if (a.mask_kind == ATTN_MASK_WINDOW) { lo = max(0, p - a.window); hi = min(Nk - 1, p + a.window); }
        if (a.mask_kind == ATTN_MASK_CAUSAL_WINDOW) { lo = max(0, p - a.window); hi = p; }
        int n_split = 1;
        attn_launch_decode_bf16(a, Nk, lo, hi, part_o, part_lse, &n_split);
        if (n_split > 1) {
            const long long rows = (long long)a.B * a.H;
            hipStream_t st = (hipStream_t)a.stream;
            if (a.d == 128)
                hipLaunchKernelGGL((merge_kernel<128>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, part_o,
                                   part_lse, (__bf16*)a.out, a.lse, rows, 1, n_split);
            else
                hipLaunchKernelGGL((merge_kernel<64>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, part_o,
                                   part_lse, (__bf16*)a.out, a.lse, rows, 1, n_split);
        }
        return 0;
    }
    SplitArgs sa;
    attn_kv_split_plan(a.B, a.H, a.N, Nk, &sa.n_split, &sa.split_len);
    sa.Nk = Nk;
    sa.q_off = q_offset;
    sa.part_o = part_o;
    sa.part_lse = part_lse;
    if (a.d == 128) return by_mask_split<128>(a, sa);
    return by_mask_split<64>(a, sa);
}

#endif  // ATTN_FWD_D64_TU
