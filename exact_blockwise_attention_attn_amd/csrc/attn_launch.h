// Internal launch descriptor shared by the host entry point and the kernel files.
#pragma once

#include <stdint.h>

#include "../../include/attn.h"

struct AttnLaunch {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int B, H, N, d;
    float c_log2;      // |scale| * log2(e), floored at 1e-30 so masked scores stay -inf
    int negate_q;      // scale < 0: the kernels negate q (exact for bf16/fp32) and use |scale|
    int mask_kind;
    int window;        // clamped to [0, N-1]
    void* stream;
};

struct AttnBwdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    int B, H, N, d;
    float c_log2;      // |scale| * log2(e), floored at 1e-30
    int negate_q;      // scale < 0: the kernels negate the register-resident q or k and use |scale|
    float scale;       // the signed scale, applied to dq and dk at the end
    int mask_kind;
    int window;        // clamped to [0, N-1]
    void* stream;
};

// Schedule overrides set through attn_set_schedule and attn_set_key_groups (0 / -1:
// the library's choice).
int attn_sched_rows_per_wave();   // 0, 32 or 64
int attn_sched_head_group();      // -1, 0 (one group) or n >= 1
int attn_sched_key_groups();      // -1, 1, 2 or 4
int attn_sched_work_queue();      // -1 (the library's choice), 0 (off) or 1 (on)

// Work-queue slot of a forward launch (wq_take in attn_tile.h), in unsigned words,
// each counter on its own 128-byte line: the claimed count of XCD x's item list at
// WQ_STRIDE x for x < WQ_XCD, then the count of workgroups that have finished
// claiming.  The last of those resets the slot to zero for the next launch that
// uses it.
constexpr int WQ_XCD = 8;
constexpr int WQ_STRIDE = 32;
constexpr int WQ_SLOT_WORDS = (WQ_XCD + 1) * WQ_STRIDE;
constexpr int WQ_SLOTS = 64;

// A slot of the current device's work-queue pool (wq_take in attn_tile.h), or
// nullptr when the pool's address cannot be had (the launch then runs without it).
unsigned* attn_wq_slot();

int attn_launch_bf16(const AttnLaunch& a);
int attn_launch_bf16_d64(const AttnLaunch& a, bool rows32, int key_groups);   // dense d = 64 (attn_fwd_bf16_d64.hip)
int attn_launch_bwd_bf16(const AttnBwdLaunch& a);
int attn_launch_f32(const AttnLaunch& a);

// split-KV forward (a.N = query rows): key ranges, then the merge of the partials.
// attn_kv_max_splits bounds the ranges any launch of the shape uses (it sizes the
// workspace: fp32 partial O [B*H, splits, Nq, d], then partial LSE [B*H, splits, Nq]).
void attn_kv_split_plan(int B, int H, int Nq, int Nk, int* n_split, int* split_len);
int attn_kv_max_splits(int B, int H, int Nq, int Nk, int d);
int attn_launch_kv_bf16(const AttnLaunch& a, int Nk, int q_offset, float* part_o, float* part_lse);

// block-sparse forward: layout [H, ceil(N/128), ceil(N/128)] bytes, nonzero = allowed
int attn_launch_block_bf16(const AttnLaunch& a, const uint8_t* layout, int causal);

// decode (one query per head): the key interval [lo, hi] in ranges, one workgroup each
int attn_decode_max_splits(int BH, int Nk, int d);
int attn_launch_decode_bf16(const AttnLaunch& a, int Nk, int lo, int hi, float* part_o, float* part_lse,
                            int* n_split_used);
