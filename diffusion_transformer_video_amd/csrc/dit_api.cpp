// C-ABI entry points (include/dit.h): argument validation, device check and
// dispatch to the gfx950 kernels. Validation is plain host code and runs before
// any HIP call, so a rejected call launches nothing and writes nothing, even on
// a machine without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "dit.h"
#include "dit_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DIT_OK;
}

int elem_size(int32_t dtype) { return dtype == DIT_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges)
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int check_dtype(int32_t dtype, const char* fn) {
    if (dtype != DIT_F32 && dtype != DIT_BF16)
        return fail(DIT_E_UNSUPPORTED, "%s: unknown dtype %d (expected DIT_F32=0 or DIT_BF16=1)", fn, dtype);
    return DIT_OK;
}

// Device check, cached per device: the kernels are built for gfx950 only.
std::atomic<int> g_dev_state[64];   // 0 unknown, 1 gfx950, 2 other

int check_device(const char* fn) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DIT_E_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(DIT_E_UNSUPPORTED, "%s: device ordinal %d out of range", fn, dev);
    int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(DIT_E_HIP, "%s: hipGetDeviceProperties: %s", fn, hipGetErrorString(e));
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_relaxed);
        if (st == 2)
            return fail(DIT_E_UNSUPPORTED, "%s: device %d is %s; this library is built for gfx950 only",
                        fn, dev, prop.gcnArchName);
    }
    if (st == 2) return fail(DIT_E_UNSUPPORTED, "%s: device %d is not gfx950", fn, dev);
    return DIT_OK;
}

int launched(hipError_t e, const char* fn) {
    if (e != hipSuccess) return fail(DIT_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int validate_rows(const char* fn, int64_t tokens, int64_t tokens_per_row) {
    if (tokens <= 0) return fail(DIT_E_INVAL, "%s: tokens must be > 0 (got %lld)", fn, (long long)tokens);
    if (tokens_per_row <= 0 || tokens % tokens_per_row != 0)
        return fail(DIT_E_INVAL, "%s: tokens (%lld) must be a positive multiple of tokens_per_row (%lld)",
                    fn, (long long)tokens, (long long)tokens_per_row);
    return DIT_OK;
}

int validate_euler(const char* fn, void* z_out, const void* z, const void* u, const float* dt_rows,
                   int64_t tokens, int32_t channels, int64_t tokens_per_row, int32_t dtype) {
    if (!z_out || !z || !u || !dt_rows) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    int rc = validate_rows(fn, tokens, tokens_per_row);
    if (rc) return rc;
    if (channels <= 0) return fail(DIT_E_INVAL, "%s: channels must be > 0", fn);
    if (channels % 8 != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: channels (%d) must be a multiple of 8", fn, channels);
    if (!aligned16(z_out) || !aligned16(z) || !aligned16(u) || !aligned16(dt_rows))
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned", fn);
    const int64_t bytes = tokens * channels * elem_size(dtype);
    if (z_out != z && overlaps(z_out, bytes, z, bytes))
        return fail(DIT_E_INVAL, "%s: z_out partially overlaps z", fn);
    if (overlaps(z_out, bytes, u, bytes)) return fail(DIT_E_INVAL, "%s: z_out overlaps u", fn);
    return DIT_OK;
}

}  // namespace

extern "C" {

const char* dit_last_error(void) { return g_err.c_str(); }

int dit_version(void) { return 10000; }

int dit_adaln_modulate(void* y, const void* x, const float* gamma, const float* beta,
                       int64_t tokens, int32_t d_model, int64_t tokens_per_row,
                       float eps, int32_t dtype, void* stream) {
    const char* fn = "dit_adaln_modulate";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!y || !x || !gamma || !beta) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (int rc = validate_rows(fn, tokens, tokens_per_row)) return rc;
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(DIT_E_INVAL, "%s: eps must be finite and > 0", fn);
    if (d_model <= 0) return fail(DIT_E_INVAL, "%s: d_model must be > 0", fn);
    if (d_model % 8 != 0 || d_model > 8192)
        return fail(DIT_E_UNSUPPORTED, "%s: d_model (%d) must be a multiple of 8 and <= 8192", fn, d_model);
    if (!aligned16(y) || !aligned16(x) || !aligned16(gamma) || !aligned16(beta))
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned", fn);
    const int64_t bytes = tokens * d_model * elem_size(dtype);
    if (y != x && overlaps(y, bytes, x, bytes)) return fail(DIT_E_INVAL, "%s: y partially overlaps x", fn);
    if (int rc = check_device(fn)) return rc;
    dit::ModulateArgs a{y, x, gamma, beta, tokens, d_model, tokens_per_row, eps};
    return launched(dit::launch_adaln_modulate(a, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int dit_rope3d(void* q, void* k, int64_t tokens, int32_t heads, int32_t head_dim,
               int32_t grid_t, int32_t grid_h, int32_t grid_w,
               const int32_t* cu_seqlens, int32_t num_seqs,
               int32_t d_t, int32_t d_h, int32_t d_w, float base,
               int32_t* pos_out, int32_t dtype, void* stream) {
    const char* fn = "dit_rope3d";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!q) return fail(DIT_E_INVAL, "%s: q is NULL", fn);
    if (tokens <= 0) return fail(DIT_E_INVAL, "%s: tokens must be > 0", fn);
    if (heads <= 0 || head_dim <= 0) return fail(DIT_E_INVAL, "%s: heads and head_dim must be > 0", fn);
    if (d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1)
        return fail(DIT_E_INVAL, "%s: d_t, d_h, d_w must be even and >= 0 (got %d/%d/%d)", fn, d_t, d_h, d_w);
    if (d_t + d_h + d_w != head_dim)
        return fail(DIT_E_INVAL, "%s: d_t + d_h + d_w (%d) must equal head_dim (%d)", fn, d_t + d_h + d_w, head_dim);
    if (!(base > 1.f) || !std::isfinite(base)) return fail(DIT_E_INVAL, "%s: base must be finite and > 1", fn);
    if (grid_h <= 0 || grid_w <= 0) return fail(DIT_E_INVAL, "%s: grid_h and grid_w must be > 0", fn);
    if (num_seqs <= 0) return fail(DIT_E_INVAL, "%s: num_seqs must be > 0", fn);
    if (cu_seqlens == nullptr) {
        if (grid_t <= 0) return fail(DIT_E_INVAL, "%s: grid_t must be > 0 in dense mode", fn);
        const int64_t L = (int64_t)grid_t * grid_h * grid_w;
        if (tokens != (int64_t)num_seqs * L)
            return fail(DIT_E_INVAL, "%s: dense tokens (%lld) != num_seqs * grid_t * grid_h * grid_w (%lld)",
                        fn, (long long)tokens, (long long)num_seqs * L);
    }
    if (head_dim % 8 != 0 || head_dim > 256 || (64 % (head_dim / 8)) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: head_dim (%d) must be one of 8, 16, 32, 64, 128, 256", fn, head_dim);
    if (!aligned16(q) || (k && !aligned16(k)))
        return fail(DIT_E_UNSUPPORTED, "%s: q and k must be 16-byte aligned", fn);
    const int64_t bytes = tokens * heads * head_dim * elem_size(dtype);
    if (k && overlaps(q, bytes, k, bytes)) return fail(DIT_E_INVAL, "%s: q and k overlap", fn);
    if (int rc = check_device(fn)) return rc;
    dit::RopeArgs a{q, k, tokens, heads, head_dim, grid_t, grid_h, grid_w, cu_seqlens, num_seqs,
                    d_t, d_h, d_w, std::log2((double)base), pos_out};
    return launched(dit::launch_rope3d(a, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

namespace {

// Shared validation and launch of dit_attn3d / dit_attn3d_lse.
int attn_common(const char* fn, void* o, float* lse, const void* q, const void* k, const void* v,
                int64_t tokens_q, int64_t tokens_k, int32_t heads, int32_t head_dim,
                const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs,
                int32_t max_q, int32_t max_k, int32_t dtype, void* stream, bool noalloc = false) {
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!o || !q || !k || !v) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (tokens_q <= 0 || tokens_k <= 0) return fail(DIT_E_INVAL, "%s: token counts must be > 0", fn);
    if (heads <= 0) return fail(DIT_E_INVAL, "%s: heads must be > 0", fn);
    if (num_seqs <= 0) return fail(DIT_E_INVAL, "%s: num_seqs must be > 0", fn);
    if ((cu_q == nullptr) != (cu_k == nullptr))
        return fail(DIT_E_INVAL, "%s: query and key offsets must both be given or both be NULL", fn);
    int32_t seq_q = max_q, seq_k = max_k;
    if (cu_q == nullptr) {
        if (tokens_q % num_seqs != 0 || tokens_k % num_seqs != 0)
            return fail(DIT_E_INVAL, "%s: dense token counts (%lld, %lld) must be multiples of num_seqs (%d)",
                        fn, (long long)tokens_q, (long long)tokens_k, num_seqs);
        if (tokens_q / num_seqs > 0x7fffffff || tokens_k / num_seqs > 0x7fffffff)
            return fail(DIT_E_UNSUPPORTED, "%s: sequence too long", fn);
        seq_q = (int32_t)(tokens_q / num_seqs);
        seq_k = (int32_t)(tokens_k / num_seqs);
    } else {
        if (max_q <= 0 || max_q > tokens_q)
            return fail(DIT_E_INVAL, "%s: packed mode needs 0 < max_seqlen <= tokens (got %d)", fn, max_q);
        if (max_k < 0 || max_k > tokens_k)
            return fail(DIT_E_INVAL, "%s: packed mode needs 0 <= max key count <= key tokens (got %d)", fn, max_k);
    }
    if (head_dim != 64 && head_dim != 128)
        return fail(DIT_E_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
    if (!aligned16(o) || !aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned", fn);
    if (lse != nullptr && ((uintptr_t)lse % 4) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: lse must be 4-byte aligned", fn);
    // the bf16 kernel addresses one sequence of one head with 32-bit byte offsets
    const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
    if ((int64_t)seq_q * row_bytes > INT32_MAX || (int64_t)seq_k * row_bytes > INT32_MAX)
        return fail(DIT_E_UNSUPPORTED, "%s: sequence length x heads x head_dim too large (%lld bytes per sequence)",
                    fn, (long long)(seq_q > seq_k ? seq_q : seq_k) * row_bytes);
    const int64_t qbytes = tokens_q * row_bytes, kbytes = tokens_k * row_bytes;
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
        return fail(DIT_E_INVAL, "%s: o must not overlap q, k or v", fn);
    if (lse != nullptr) {
        const int64_t lbytes = tokens_q * heads * 4;
        if (overlaps(lse, lbytes, o, qbytes) || overlaps(lse, lbytes, q, qbytes) ||
            overlaps(lse, lbytes, k, kbytes) || overlaps(lse, lbytes, v, kbytes))
            return fail(DIT_E_INVAL, "%s: lse must not overlap o, q, k or v", fn);
    }
    if (int rc = check_device(fn)) return rc;
    dit::AttnArgs a{o, q, k, v, tokens_q, heads, head_dim, cu_q, num_seqs, seq_q,
                    (float)(1.4426950408889634 / std::sqrt((double)head_dim)),
                    (float)(1.0 / std::sqrt((double)head_dim)), cu_k, seq_k, lse};
    hipError_t e = dtype != DIT_BF16 ? dit::launch_attn3d_f32(a, (hipStream_t)stream)
                   : noalloc         ? dit::launch_attn3d_bf16_noalloc(a, (hipStream_t)stream)
                                     : dit::launch_attn3d_bf16(a, (hipStream_t)stream);
    return launched(e, fn);
}

}  // namespace

int dit_attn3d(void* o, const void* q, const void* k, const void* v,
               int64_t tokens, int32_t heads, int32_t head_dim,
               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
               int32_t dtype, void* stream) {
    return attn_common("dit_attn3d", o, nullptr, q, k, v, tokens, tokens, heads, head_dim, cu_seqlens,
                       cu_seqlens, num_seqs, max_seqlen, max_seqlen, dtype, stream);
}

int dit_attn3d_noalloc(void* o, const void* q, const void* k, const void* v,
                       int64_t tokens, int32_t heads, int32_t head_dim,
                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                       int32_t dtype, void* stream) {
    return attn_common("dit_attn3d_noalloc", o, nullptr, q, k, v, tokens, tokens, heads, head_dim, cu_seqlens,
                       cu_seqlens, num_seqs, max_seqlen, max_seqlen, dtype, stream, true);
}

int dit_attn3d_lse(void* o, float* lse, const void* q, const void* k, const void* v,
                   int64_t tokens_q, int64_t tokens_k, int32_t heads, int32_t head_dim,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                   int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t dtype, void* stream) {
    if (!lse) return fail(DIT_E_INVAL, "dit_attn3d_lse: NULL pointer argument");
    return attn_common("dit_attn3d_lse", o, lse, q, k, v, tokens_q, tokens_k, heads, head_dim, cu_seqlens_q,
                       cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, dtype, stream);
}

int dit_attn_merge(float* o_acc, float* lse_acc, const void* o_b, const float* lse_b,
                   int64_t tokens, int32_t heads, int32_t head_dim, int32_t dtype, void* stream) {
    const char* fn = "dit_attn_merge";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!o_acc || !lse_acc || !o_b || !lse_b) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (tokens <= 0) return fail(DIT_E_INVAL, "%s: tokens must be > 0", fn);
    if (heads <= 0) return fail(DIT_E_INVAL, "%s: heads must be > 0", fn);
    if (head_dim != 64 && head_dim != 128)
        return fail(DIT_E_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
    if (!aligned16(o_acc) || !aligned16(o_b) || ((uintptr_t)lse_acc % 4) != 0 || ((uintptr_t)lse_b % 4) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: o arrays must be 16-byte and lse arrays 4-byte aligned", fn);
    const int64_t rows = tokens * heads;
    const int64_t abytes = rows * head_dim * 4, bbytes = rows * head_dim * elem_size(dtype), lbytes = rows * 4;
    if (overlaps(o_acc, abytes, o_b, bbytes) || overlaps(o_acc, abytes, lse_acc, lbytes) ||
        overlaps(o_acc, abytes, lse_b, lbytes) || overlaps(lse_acc, lbytes, o_b, bbytes) ||
        overlaps(lse_acc, lbytes, lse_b, lbytes) || overlaps(o_b, bbytes, lse_b, lbytes))
        return fail(DIT_E_INVAL, "%s: the four arrays must not overlap", fn);
    if (int rc = check_device(fn)) return rc;
    dit::MergeArgs a{o_acc, lse_acc, o_b, lse_b, rows, head_dim};
    return launched(dit::launch_attn_merge(a, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int dit_gated_residual(void* x_out, const void* x, const void* branch, const float* alpha,
                       int64_t tokens, int32_t d_model, int64_t tokens_per_row,
                       const dit_euler_args* euler, int32_t dtype, void* stream) {
    const char* fn = "dit_gated_residual";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!x_out || !x || !branch || !alpha) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (int rc = validate_rows(fn, tokens, tokens_per_row)) return rc;
    if (d_model <= 0) return fail(DIT_E_INVAL, "%s: d_model must be > 0", fn);
    if (d_model % 8 != 0) return fail(DIT_E_UNSUPPORTED, "%s: d_model (%d) must be a multiple of 8", fn, d_model);
    if (!aligned16(x_out) || !aligned16(x) || !aligned16(branch) || !aligned16(alpha))
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned", fn);
    const int64_t bytes = tokens * d_model * elem_size(dtype);
    if (x_out != x && overlaps(x_out, bytes, x, bytes))
        return fail(DIT_E_INVAL, "%s: x_out partially overlaps x", fn);
    if (overlaps(x_out, bytes, branch, bytes)) return fail(DIT_E_INVAL, "%s: x_out overlaps branch", fn);
    dit::EulerArgs ea{};
    if (euler) {
        if (int rc = validate_euler("dit_gated_residual(euler)", euler->z_out, euler->z, euler->u,
                                    euler->dt_rows, euler->tokens, euler->channels,
                                    euler->tokens_per_row, dtype))
            return rc;
        const int64_t zb = euler->tokens * euler->channels * elem_size(dtype);
        if (overlaps(euler->z_out, zb, x_out, bytes) || overlaps(euler->z_out, zb, x, bytes) ||
            overlaps(euler->z_out, zb, branch, bytes) || overlaps(x_out, bytes, euler->z, zb) ||
            overlaps(x_out, bytes, euler->u, zb))
            return fail(DIT_E_INVAL, "%s: Euler tensors overlap the residual tensors", fn);
        ea = dit::EulerArgs{euler->z_out, euler->z, euler->u, euler->dt_rows, euler->tokens,
                            euler->channels, euler->tokens_per_row};
    }
    if (int rc = check_device(fn)) return rc;
    dit::ResidualArgs ra{x_out, x, branch, alpha, tokens, d_model, tokens_per_row};
    return launched(dit::launch_epilogue(&ra, euler ? &ea : nullptr, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int rf_euler_step(void* z_out, const void* z, const void* u, const float* dt_rows,
                  int64_t tokens, int32_t channels, int64_t tokens_per_row,
                  int32_t dtype, void* stream) {
    const char* fn = "rf_euler_step";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (int rc = validate_euler(fn, z_out, z, u, dt_rows, tokens, channels, tokens_per_row, dtype)) return rc;
    if (int rc = check_device(fn)) return rc;
    dit::EulerArgs ea{z_out, z, u, dt_rows, tokens, channels, tokens_per_row};
    return launched(dit::launch_epilogue(nullptr, &ea, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int rf_midpoint_half(void* z_mid, const void* z, const void* u, const float* dt_rows,
                     int64_t tokens, int32_t channels, int64_t tokens_per_row,
                     int32_t dtype, void* stream) {
    const char* fn = "rf_midpoint_half";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (int rc = validate_euler(fn, z_mid, z, u, dt_rows, tokens, channels, tokens_per_row, dtype)) return rc;
    if (int rc = check_device(fn)) return rc;
    dit::EulerArgs ea{z_mid, z, u, dt_rows, tokens, channels, tokens_per_row, 0.5f};
    return launched(dit::launch_epilogue(nullptr, &ea, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int rf_interpolant(void* x_t, const void* x0, const void* x1, const float* t_rows,
                   int64_t tokens, int32_t channels, int64_t tokens_per_row,
                   int32_t dtype, void* stream) {
    const char* fn = "rf_interpolant";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!x_t || !x0 || !x1 || !t_rows) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (int rc = validate_rows(fn, tokens, tokens_per_row)) return rc;
    if (channels <= 0) return fail(DIT_E_INVAL, "%s: channels must be > 0", fn);
    if (channels % 8 != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: channels (%d) must be a multiple of 8", fn, channels);
    if (!aligned16(x_t) || !aligned16(x0) || !aligned16(x1) || ((uintptr_t)t_rows % 4) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned (t_rows 4-byte)", fn);
    const int64_t bytes = tokens * channels * elem_size(dtype);
    if ((x_t != x0 && overlaps(x_t, bytes, x0, bytes)) || (x_t != x1 && overlaps(x_t, bytes, x1, bytes)))
        return fail(DIT_E_INVAL, "%s: x_t partially overlaps x0 or x1", fn);
    if (int rc = check_device(fn)) return rc;
    dit::InterpArgs a{x_t, x0, x1, t_rows, tokens, channels, tokens_per_row};
    return launched(dit::launch_interpolant(a, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int rf_cfm_loss(float* loss_tokens, float* loss_rows, const void* u, const void* x0, const void* x1,
                int64_t tokens, int32_t channels, int64_t tokens_per_row, int32_t dtype, void* stream) {
    const char* fn = "rf_cfm_loss";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!loss_tokens || !u || !x0 || !x1) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (int rc = validate_rows(fn, tokens, tokens_per_row)) return rc;
    if (channels <= 0) return fail(DIT_E_INVAL, "%s: channels must be > 0", fn);
    if (channels % 8 != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: channels (%d) must be a multiple of 8", fn, channels);
    if (!aligned16(u) || !aligned16(x0) || !aligned16(x1) || ((uintptr_t)loss_tokens % 4) != 0 ||
        ((uintptr_t)loss_rows % 4) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: inputs must be 16-byte aligned, losses 4-byte", fn);
    const int64_t bytes = tokens * channels * elem_size(dtype), lb = tokens * 4;
    const int64_t rb = (tokens / tokens_per_row) * 4;
    if (overlaps(loss_tokens, lb, u, bytes) || overlaps(loss_tokens, lb, x0, bytes) ||
        overlaps(loss_tokens, lb, x1, bytes) ||
        (loss_rows && (overlaps(loss_rows, rb, loss_tokens, lb) || overlaps(loss_rows, rb, u, bytes) ||
                       overlaps(loss_rows, rb, x0, bytes) || overlaps(loss_rows, rb, x1, bytes))))
        return fail(DIT_E_INVAL, "%s: outputs must not overlap the inputs or each other", fn);
    if (int rc = check_device(fn)) return rc;
    dit::CfmArgs a{loss_tokens, loss_rows, u, x0, x1, tokens, channels, tokens_per_row};
    return launched(dit::launch_cfm_loss(a, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int flow_insert_frames(void* z_out, float* t_out, int32_t* cu_out, int32_t* src_out,
                       const void* z, const float* t_frames, const int32_t* cu_seqlens, int32_t num_seqs,
                       const int32_t* counts, const void* noise, int64_t frames, int64_t frames_out,
                       int32_t tokens_per_frame, int32_t channels, int32_t dtype, void* stream) {
    const char* fn = "flow_insert_frames";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (!z_out || !t_out || !cu_out || !src_out || !z || !t_frames || !cu_seqlens || !counts)
        return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (frames <= 0 || frames_out < frames)
        return fail(DIT_E_INVAL, "%s: need frames > 0 and frames_out >= frames (got %lld, %lld)", fn,
                    (long long)frames, (long long)frames_out);
    if (frames_out > frames && !noise) return fail(DIT_E_INVAL, "%s: noise is NULL but frames are inserted", fn);
    if (num_seqs <= 0) return fail(DIT_E_INVAL, "%s: num_seqs must be > 0", fn);
    if (tokens_per_frame <= 0 || channels <= 0) return fail(DIT_E_INVAL, "%s: sizes must be > 0", fn);
    if (channels % 8 != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: channels (%d) must be a multiple of 8", fn, channels);
    if (frames_out * tokens_per_frame > INT32_MAX)
        return fail(DIT_E_UNSUPPORTED, "%s: output token count exceeds int32 offsets", fn);
    if (!aligned16(z_out) || !aligned16(z) || (noise && !aligned16(noise)))
        return fail(DIT_E_UNSUPPORTED, "%s: latents must be 16-byte aligned", fn);
    if (((uintptr_t)t_out | (uintptr_t)cu_out | (uintptr_t)src_out | (uintptr_t)t_frames |
         (uintptr_t)cu_seqlens | (uintptr_t)counts) % 4 != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: index and time arrays must be 4-byte aligned", fn);
    const int64_t row = (int64_t)channels * elem_size(dtype);
    const int64_t zb = frames * tokens_per_frame * row, ob = frames_out * tokens_per_frame * row;
    const int64_t nb = (frames_out - frames) * tokens_per_frame * row;
    if (overlaps(z_out, ob, z, zb) || (noise && overlaps(z_out, ob, noise, nb)) ||
        overlaps(t_out, frames_out * 4, t_frames, frames * 4) || overlaps(t_out, frames_out * 4, src_out, frames_out * 4) ||
        overlaps(src_out, frames_out * 4, counts, frames * 4) || overlaps(cu_out, (num_seqs + 1) * 4, cu_seqlens, (num_seqs + 1) * 4) ||
        overlaps(cu_out, (num_seqs + 1) * 4, src_out, frames_out * 4) || overlaps(cu_out, (num_seqs + 1) * 4, t_out, frames_out * 4))
        return fail(DIT_E_INVAL, "%s: outputs must not overlap the inputs or each other", fn);
    if (int rc = check_device(fn)) return rc;
    dit::InsertArgs a{z_out, t_out, cu_out, src_out, z, t_frames, cu_seqlens, num_seqs, counts, noise,
                      frames, frames_out, tokens_per_frame, channels};
    return launched(dit::launch_insert_frames(a, dtype == DIT_BF16, (hipStream_t)stream), fn);
}

int flow_frame_schedule(float* dt_out, float* t_frames, int64_t frames, float dt_max, void* stream) {
    const char* fn = "flow_frame_schedule";
    if (!dt_out || !t_frames) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    if (frames <= 0) return fail(DIT_E_INVAL, "%s: frames must be > 0", fn);
    if (!(dt_max > 0.f) || !std::isfinite(dt_max)) return fail(DIT_E_INVAL, "%s: dt_max must be finite and > 0", fn);
    if (((uintptr_t)dt_out | (uintptr_t)t_frames) % 4 != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: arrays must be 4-byte aligned", fn);
    if (overlaps(dt_out, frames * 4, t_frames, frames * 4))
        return fail(DIT_E_INVAL, "%s: dt_out must not overlap t_frames", fn);
    if (int rc = check_device(fn)) return rc;
    return launched(dit::launch_frame_schedule(dt_out, t_frames, frames, dt_max, (hipStream_t)stream), fn);
}

int64_t dit_fp8_v_stride(int64_t tokens, int32_t num_seqs) {
    if (tokens <= 0 || num_seqs <= 0) return 0;
    return (tokens + 64 * (int64_t)num_seqs + 63) / 64 * 64;
}

namespace {

int fp8_common(const char* fn, int64_t tokens, int32_t heads, int32_t head_dim, const int32_t* cu_seqlens,
               int32_t num_seqs, int32_t max_seqlen, int64_t v_stride, int32_t* seqlen_out) {
    if (tokens <= 0) return fail(DIT_E_INVAL, "%s: tokens must be > 0", fn);
    if (heads <= 0) return fail(DIT_E_INVAL, "%s: heads must be > 0", fn);
    if (num_seqs <= 0) return fail(DIT_E_INVAL, "%s: num_seqs must be > 0", fn);
    if (head_dim != 128) return fail(DIT_E_UNSUPPORTED, "%s: head_dim must be 128 (got %d)", fn, head_dim);
    int32_t seqlen = max_seqlen;
    if (cu_seqlens == nullptr) {
        if (tokens % num_seqs != 0)
            return fail(DIT_E_INVAL, "%s: dense tokens (%lld) must be a multiple of num_seqs (%d)", fn,
                        (long long)tokens, num_seqs);
        if (tokens / num_seqs > 0x7fffffff) return fail(DIT_E_UNSUPPORTED, "%s: sequence too long", fn);
        seqlen = (int32_t)(tokens / num_seqs);
    } else if (max_seqlen <= 0 || max_seqlen > tokens) {
        return fail(DIT_E_INVAL, "%s: packed mode needs 0 < max_seqlen <= tokens (got %d)", fn, max_seqlen);
    }
    if (v_stride < dit_fp8_v_stride(tokens, num_seqs) || v_stride % 64 != 0)
        return fail(DIT_E_INVAL, "%s: v_stride (%lld) must be a multiple of 64 and >= %lld", fn, (long long)v_stride,
                    (long long)dit_fp8_v_stride(tokens, num_seqs));
    if ((int64_t)seqlen * heads * head_dim > INT32_MAX || (int64_t)head_dim * v_stride > INT32_MAX)
        return fail(DIT_E_UNSUPPORTED, "%s: sizes exceed 32-bit offsets", fn);
    *seqlen_out = seqlen;
    return DIT_OK;
}

}  // namespace

int dit_quant_fp8(void* q8, void* k8, void* v8t, float* amax, const void* q, const void* k, const void* v,
                  int64_t tokens, int32_t heads, int32_t head_dim, const int32_t* cu_seqlens, int32_t num_seqs,
                  int32_t max_seqlen, int64_t v_stride, int32_t dtype, void* stream) {
    const char* fn = "dit_quant_fp8";
    if (int rc = check_dtype(dtype, fn)) return rc;
    if (dtype != DIT_BF16) return fail(DIT_E_UNSUPPORTED, "%s: inputs must be bf16", fn);
    if (!q8 || !k8 || !v8t || !amax || !q || !k || !v) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    int32_t seqlen = 0;
    if (int rc = fp8_common(fn, tokens, heads, head_dim, cu_seqlens, num_seqs, max_seqlen, v_stride, &seqlen))
        return rc;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        ((uintptr_t)amax % 4) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned (amax 4-byte)", fn);
    const int64_t nb = tokens * heads * head_dim, ib = nb * 2, vb = (int64_t)heads * head_dim * v_stride;
    const int64_t ab = 3 * (int64_t)heads * 4;
    const void* ins[3] = {q, k, v};
    void* outs[4] = {q8, k8, v8t, amax};
    const int64_t osz[4] = {nb, nb, vb, ab};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 3; ++j)
            if (overlaps(outs[i], osz[i], ins[j], ib)) return fail(DIT_E_INVAL, "%s: outputs must not overlap the inputs", fn);
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], osz[i], outs[j], osz[j])) return fail(DIT_E_INVAL, "%s: outputs must not overlap", fn);
    }
    if (int rc = check_device(fn)) return rc;
    dit::QuantFp8Args a{q8, k8, v8t, amax, q, k, v, tokens, heads, cu_seqlens, num_seqs, seqlen, v_stride};
    return launched(dit::launch_quant_fp8(a, (hipStream_t)stream), fn);
}

int dit_attn3d_fp8(void* o, const void* q8, const void* k8, const void* v8t, const float* amax, int64_t tokens,
                   int32_t heads, int32_t head_dim, const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                   int64_t v_stride, void* stream) {
    const char* fn = "dit_attn3d_fp8";
    if (!o || !q8 || !k8 || !v8t || !amax) return fail(DIT_E_INVAL, "%s: NULL pointer argument", fn);
    int32_t seqlen = 0;
    if (int rc = fp8_common(fn, tokens, heads, head_dim, cu_seqlens, num_seqs, max_seqlen, v_stride, &seqlen))
        return rc;
    if (!aligned16(o) || !aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || ((uintptr_t)amax % 4) != 0)
        return fail(DIT_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned (amax 4-byte)", fn);
    const int64_t nb = tokens * heads * head_dim, vb = (int64_t)heads * head_dim * v_stride;
    if (overlaps(o, nb * 2, q8, nb) || overlaps(o, nb * 2, k8, nb) || overlaps(o, nb * 2, v8t, vb) ||
        overlaps(o, nb * 2, amax, 3 * (int64_t)heads * 4))
        return fail(DIT_E_INVAL, "%s: o must not overlap the inputs", fn);
    if (int rc = check_device(fn)) return rc;
    dit::AttnFp8Args a{o, q8, k8, v8t, amax, tokens, heads, cu_seqlens, num_seqs, seqlen, v_stride};
    return launched(dit::launch_attn3d_fp8(a, (hipStream_t)stream), fn);
}

}  // extern "C"
