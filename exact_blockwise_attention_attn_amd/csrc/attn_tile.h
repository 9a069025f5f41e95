// Shared pieces of the bf16 attention kernels (forward and backward): vector
// types, compile-time loops, the LDS layout of a 32-row operand tile and the LDS
// and cross-lane primitives the matrix-core mappings rely on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn_tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int V>
struct IntC { static constexpr int value = V; };

// Workgroup order over (block rank, head) pairs: the BH (batch, head) pairs in
// groups of hg (all of them when hg is 0), every rank of a group before the next
// group, the head varying fastest inside a group.  With hg a multiple of 8 every
// block of a head lands on the same XCD (workgroups are dealt to the 8 XCDs round
// robin) and shares its L2, and a group's K and V (or Q and dO) stay resident in
// the Infinity Cache while the group runs.
__device__ __forceinline__ void grouped_order(int id, int BH, int n_rank, int hg, int& rank, int& bh) {
    const int G = (hg > 0 && hg < BH) ? hg : BH;    // heads per group
    const int full = BH / G;                         // full groups; a last one holds BH - full G
    const int g = id / (G * n_rank);
    const int gsz = g < full ? G : BH - full * G;
    const int r = id - g * (G * n_rank);
    rank = r / gsz;
    bh = g * G + (r - rank * gsz);
}

// Work queue of one launch (an optional kernel argument).  The launch's items keep
// the order above: item i belongs to XCD i % 8, where the dispatcher deals workgroup
// i round robin, so all blocks of a head still share one L2.  Instead of owning item
// blockIdx.x, a workgroup takes the next unclaimed item of its own XCD's list, and
// once that list is empty, the next one of another XCD's.  The grid carries a few
// extra workgroups per XCD: on an XCD that runs ahead they take over the tail of a
// slower one's list, which a fixed item per workgroup cannot (each XCD would get
// exactly its share of the grid, however fast it runs).  Which workgroup computes an
// item never changes the item's result.
// The slot layout is in attn_launch.h (WQ_*).

// One lane per workgroup whose index is at least n_static (items below n_static
// belong to the workgroup of the same index): the item this workgroup computes, or
// -1 when every list is exhausted.  Item i of list x = i % 8 is claimed in list
// order from n_static / 8 on (n_static a multiple of 8); total = items of the
// launch, n_dyn = workgroups of the launch that claim.
__device__ __forceinline__ int wq_take(unsigned* wq, int total, int n_static, int n_dyn) {
    const int home = (int)(blockIdx.x % WQ_XCD);
    const int j0 = n_static / WQ_XCD;
    int item = -1;
    for (int k = 0; k < WQ_XCD; ++k) {
        const int x = (home + k) % WQ_XCD;
        const int n_x = (total - x + WQ_XCD - 1) / WQ_XCD - j0;   // unclaimed-at-launch items of list x
        if (n_x <= 0) continue;
        const unsigned c = atomicAdd(wq + x * WQ_STRIDE, 1u);
        if (c < (unsigned)n_x) {
            item = (j0 + (int)c) * WQ_XCD + x;
            break;
        }
    }
    __threadfence();                                   // the claims precede the count below
    const unsigned done = atomicAdd(wq + WQ_XCD * WQ_STRIDE, 1u);
    if (done == (unsigned)(n_dyn - 1)) {
        // every claiming workgroup is past its claims: the slot is clean for its next launch
        __threadfence();
        for (int x = 0; x <= WQ_XCD; ++x) atomicExch(wq + x * WQ_STRIDE, 0u);
    }
    return item;
}

// Heads per group for a kernel that streams two [N, d] bf16 tensors of a head: the
// largest multiple of 8 whose two tensors fit in 128 MB (half the 256 MB Infinity
// Cache), at least 8 (one head per XCD).
inline int head_group(int N, int d) {
    const long long per_head = 2LL * N * d * 2;
    const long long fit = (128LL << 20) / (8 * per_head);
    return 8 * (int)(fit < 1 ? 1 : (fit > (1 << 20) ? (1 << 20) : fit));
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0; offsets range-checked
// against `bytes`; word 3 is the gfx9 raw-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct HBM -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds): the
// bytes at byte offset voff + soff of the buffer land at dst + 16 * lane.  The
// MUBUF form matters: while a FLAT-encoded direct load (global_load_lds) is in
// flight the compiler cannot count LDS reads in order and waits for all of them
// (lgkmcnt(0)) before every use of one; with buffer loads its waits are exact.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds_void* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (int)voff, (int)soff, 0, 0);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<I + 1, N>(f);
    }
}

// LDS layout of a tile of BC rows x D/8 16-byte chunks (K, V, Q or dO rows).
// Chunks are grouped four at a time (64 bytes of a row); group J holds the chunks
// 4J..4J+3 of every row contiguously, row after row, and inside a row the four
// chunks are XOR-ed with (row / 4) mod 4:
//     slot(row, c) = (c / 4) * 4 BC + 4 row + ((c mod 4) ^ ((row / 4) mod 4))
// One 1 KB load instruction fills 16 rows of one group (64 contiguous bytes of
// each row: coalesced).  Both LDS read patterns are conflict-free on 64 banks:
// 16 consecutive rows at one chunk (row operand, 16-byte reads) and 4 consecutive
// rows x 4 chunks of a group (transposed operand, transposing 8-byte reads), and
// every read address is a per-lane base plus compile-time offsets.
template <int BC>
__device__ __forceinline__ int slot_of(int row, int c) {
    return (c >> 2) * (4 * BC) + 4 * row + ((c & 3) ^ ((row >> 2) & 3));
}

__device__ __forceinline__ float swap32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap32_add(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds_base, int byte_off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_base + byte_off));
    return __builtin_bit_cast(bf16x4, r);
}

// Per-lane byte offsets of the two LDS read patterns of a 32-row tile (BC = 32)
// in the layout above, for v_mfma_f32_32x32x16_bf16 operands:
//   row operand, slab s (16 columns): lane reads row lane % 32, columns
//     16 s + 8 (lane / 32) .. +8  at  (s / 2) * 4 BC * 16 + (s odd ? odd : even)
//   transposed operand (A of a product over the rows), 32-column block j and
//     16-row slab ks: two 8-byte transposing reads at
//     j * 4 BC * 16 + ks * 16 * 4 * 16 + tr[0] and + tr[1]; the 8 rows a lane
//     gets per slab are {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32), the order in
//     which the C layout of a 32 x 32 product holds its rows.
struct TileOffsets {
    int row_even, row_odd, tr[2];
    __device__ __forceinline__ explicit TileOffsets(int lane) {
        const int hl = lane >> 5, ln = lane & 31;
        const int sw = (ln >> 2) & 3;
        row_even = (4 * ln + (hl ^ sw)) * 16;
        row_odd = (4 * ln + ((2 + hl) ^ sw)) * 16;
        const int g = lane >> 4, s16 = lane & 15;
        const int k = 2 * (g & 1) + ((s16 & 3) >> 1);
#pragma unroll
        for (int r = 0; r < 2; ++r)
            tr[r] = ((8 * r + 4 * hl + (s16 >> 2)) * 4 + (k ^ (2 * r + hl))) * 16 + (s16 & 1) * 8;
    }
};

}  // namespace attn_tile
