// Internal launch interface between the C-ABI layer (dit_api.cpp) and the
// kernel translation units. Every launcher assumes its arguments were validated
// by the C-ABI layer and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

struct ModulateArgs {
    void* y; const void* x; const float* gamma; const float* beta;
    int64_t tokens; int d_model; int64_t tokens_per_row; float eps;
};
hipError_t launch_adaln_modulate(const ModulateArgs& a, bool bf16, hipStream_t s);

struct RopeArgs {
    void* q; void* k; int64_t tokens; int heads; int head_dim;
    int grid_t, grid_h, grid_w;
    const int32_t* cu_seqlens; int num_seqs;
    int d_t, d_h, d_w; double log2_base;
    int32_t* pos_out;
};
hipError_t launch_rope3d(const RopeArgs& a, bool bf16, hipStream_t s);

struct AttnArgs {
    void* o; const void* q; const void* k; const void* v;
    int64_t tokens; int heads; int head_dim;   // tokens: query rows (q, o)
    const int32_t* cu_seqlens;   // query offsets; NULL => dense
    int num_seqs; int max_seqlen;   // dense: max_seqlen = tokens / num_seqs
    float scale_log2;            // log2(e) / sqrt(head_dim)
    float scale;                 // 1 / sqrt(head_dim)
    // keys / values of sequence s: rows cu_seqlens_k[s] .. cu_seqlens_k[s+1] of k, v
    // (dense: max_seqlen_k rows per sequence). For self-attention these are the
    // query-side values.
    const int32_t* cu_seqlens_k; int max_seqlen_k;
    float* lse;                  // NULL, or [tokens, heads]: ln sum_keys exp(q.k / sqrt(d))
};
hipError_t launch_attn3d_bf16(const AttnArgs& a, hipStream_t s);
// the same arithmetic; persistent launches use the file's static scratch slot
// (no launch tracking, no split tail)
hipError_t launch_attn3d_bf16_noalloc(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn3d_f32(const AttnArgs& a, hipStream_t s);

// (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_b, lse_b)); o_acc fp32.
struct MergeArgs {
    float* o_acc; float* lse_acc; const void* o_b; const float* lse_b;
    int64_t rows;   // tokens * heads
    int head_dim;
};
hipError_t launch_attn_merge(const MergeArgs& a, bool bf16, hipStream_t s);

struct EulerArgs {
    void* z_out; const void* z; const void* u; const float* dt_rows;
    int64_t tokens; int channels; int64_t tokens_per_row;
    float dt_scale = 1.0f;   // 0.5: the midpoint rule's half step
};
struct ResidualArgs {
    void* x_out; const void* x; const void* branch; const float* alpha;
    int64_t tokens; int d_model; int64_t tokens_per_row;
};
// residual may have tokens == 0 (Euler only); euler may be NULL.
hipError_t launch_epilogue(const ResidualArgs* r, const EulerArgs* e, bool bf16, hipStream_t s);

// x_t = (1 - t[row]) x0 + t[row] x1
struct InterpArgs {
    void* xt; const void* x0; const void* x1; const float* t_rows;
    int64_t tokens; int channels; int64_t tokens_per_row;
};
hipError_t launch_interpolant(const InterpArgs& a, bool bf16, hipStream_t s);

// loss_tok[tok] = sum_c (u - (x1 - x0))^2; loss_rows (nullable) = per-row sums
struct CfmArgs {
    float* loss_tok; float* loss_rows; const void* u; const void* x0; const void* x1;
    int64_t tokens; int channels; int64_t tokens_per_row;
};
hipError_t launch_cfm_loss(const CfmArgs& a, bool bf16, hipStream_t s);

// Flowception frame insertion (frames of tokens_per_frame token rows)
struct InsertArgs {
    void* z_out; float* t_out; int32_t* cu_out; int32_t* src_out;
    const void* z; const float* t_frames; const int32_t* cu_seqlens; int num_seqs;
    const int32_t* counts; const void* noise;
    int64_t frames, frames_out; int tokens_per_frame; int channels;
};
hipError_t launch_insert_frames(const InsertArgs& a, bool bf16, hipStream_t s);
hipError_t launch_frame_schedule(float* dt_out, float* t, int64_t frames, float dt_max, hipStream_t s);

// FP8 (OCP E4M3) attention, head_dim 128: quantisation of bf16 q, k, v and the
// attention on the codes (layouts in k_quant_fp8.hip)
struct QuantFp8Args {
    void* q8; void* k8; void* v8t; float* amax;   // amax [3][heads]: q, k, v
    const void* q; const void* k; const void* v;
    int64_t tokens; int heads;
    const int32_t* cu_seqlens; int num_seqs; int max_seqlen;
    int64_t ldv;   // bytes per v8t row
};
hipError_t launch_quant_fp8(const QuantFp8Args& a, hipStream_t s);

struct AttnFp8Args {
    void* o; const void* q8; const void* k8; const void* v8t; const float* amax;
    int64_t tokens; int heads;
    const int32_t* cu_seqlens; int num_seqs; int max_seqlen;
    int64_t ldv;
};
hipError_t launch_attn3d_fp8(const AttnFp8Args& a, hipStream_t s);

}  // namespace dit
