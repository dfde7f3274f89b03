/*
 * dit.h -- C-ABI of the DiT attention-block hot path for AMD Instinct MI355X (gfx950).
 *
 * One DiT block's attention half plus the sampler update:
 *   dit_adaln_modulate   y  = gamma * LayerNorm(x) + beta            (adaLN-Zero)
 *   dit_rope3d           q, k <- R_3D(t', h', w') q, k               (3D-RoPE)
 *   dit_attn3d           o  = softmax(q k^T / sqrt(d_head)) v        (full 3D attention)
 *   dit_attn3d_lse       o, lse over a separate key block per sequence (ring step)
 *   dit_attn_merge       fold a partial (o, lse) into a float32 accumulator
 *   dit_gated_residual   x' = x + alpha * o   [+ fused Euler pass]   (gated residual)
 *   rf_euler_step        z' = z + dt * u                             (rectified-flow Euler)
 *   rf_midpoint_half     z_mid = z + (dt/2) * u                      (midpoint sampler, stage 1)
 *   rf_interpolant       x_t = (1 - t) x0 + t x1                     (straight-path input)
 *   rf_cfm_loss          |u - (x1 - x0)|^2 per token and per row     (flow-matching loss)
 *   dit_quant_fp8        q, k, v -> E4M3 codes + per-head amax       (8-bit attention inputs)
 *   dit_attn3d_fp8       attention on the E4M3 codes                 (8-bit attention)
 *   flow_insert_frames   new noise frames after existing ones        (Flowception insertion)
 *   flow_frame_schedule  dt_f = min(dt_max, 1 - t_f), t_f += dt_f    (per-frame local times)
 *
 * Definitions come from the pages "DiT, Flow Matching e 3D Attention: A Engenharia
 * de Video com IA" (sections "A ruptura da U-Net", "Flow Matching e Rectified Flow",
 * "3D-RoPE e atencao espaco-temporal", "Engenharia de inferencia e paralelismo de
 * contexto: Ulysses, Ring Attention e FP8") and "Por que e absurdamente dificil
 * gerar um filme inteiro usando IA" (section "Matematica por tras"), and the summary
 * of "Flowception: Temporally Expansive Flow Matching for Video Generation"
 * (section 2, "Metodologia: Flowception").
 *
 * Layout (every activation tensor is token-major and contiguous):
 *   hidden x, y, branch      [tokens][d_model]
 *   q, k, v, o               [tokens][heads][head_dim]   (== [tokens][d_model])
 *   latent z, u              [tokens][channels]          (channels = C*p_t*p_h*p_w)
 *   gamma, beta, alpha       [rows][d_model] float32, row = token / tokens_per_row
 *   dt_rows                  [rows] float32
 *   cu_seqlens               [num_seqs + 1] int32, offsets of packed sequences
 * Tokens of one sequence are ordered time-major, w' fastest:
 *   t' = n / (H'W'), h' = (n / W') % H', w' = n % W'   (n local to its sequence).
 *
 * Conventions shared by every entry point:
 *   - Pointers to tensors are DEVICE pointers owned by the caller. The library
 *     allocates no device memory at call time. Its only device state is loaded
 *     with the library, per device: 64 slots of work-queue counters and one
 *     array of split-item partials (512 x 130 KiB = 65 MiB, with its counters)
 *     that large bf16 attention launches use and leave cleared (see dit_attn3d).
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue work
 *     on it and never synchronise; results are visible after the stream is
 *     synchronised. Faults inside a running kernel surface at that sync.
 *   - `dtype` selects the activation storage: DIT_F32 or DIT_BF16. Parameters
 *     (gamma, beta, alpha, dt_rows) are float32 in both cases. All arithmetic is
 *     float32; each bf16 output is rounded once (round to nearest even).
 *   - Return DIT_OK on success. On error nothing is launched, nothing is
 *     written, and dit_last_error() describes the problem:
 *       DIT_E_INVAL        bad argument (NULL pointer, size, split, overlap ...)
 *       DIT_E_UNSUPPORTED  valid but unsupported (head_dim, alignment, device)
 *       DIT_E_HIP          a HIP call failed (message from hipGetErrorString)
 *     Arguments are validated before the device is queried, so argument errors
 *     are reported even on a machine without a GPU.
 *   - Device data is not inspected on the host: cu_seqlens must start at 0,
 *     be non-decreasing and end at `tokens` (unchecked precondition).
 */
#ifndef DIT_H_
#define DIT_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DIT_F32 = 0, DIT_BF16 = 1 } dit_dtype;

enum { DIT_OK = 0, DIT_E_INVAL = 1, DIT_E_UNSUPPORTED = 2, DIT_E_HIP = 3 };

/* Text of the last error on the calling thread ("" if none). Library-owned,
 * valid until the next dit_* / rf_* call on this thread. */
const char* dit_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int dit_version(void);

/*
 * adaLN-Zero modulation, "DiT, Flow Matching e 3D Attention", section "A ruptura
 * da U-Net" (block equations: gamma_1 * LayerNorm(x_l) + beta_1 feeds attention):
 *   y[tok][c] = gamma[row][c] * (x[tok][c] - mu) / sqrt(var + eps) + beta[row][c]
 * with mu, var the mean and biased variance of x[tok][:], row = tok / tokens_per_row.
 *
 *   y, x            [tokens][d_model] activations (dtype); y == x is allowed
 *   gamma, beta     [tokens/tokens_per_row][d_model] float32
 *   tokens > 0, tokens % tokens_per_row == 0, eps > 0
 *   d_model % 8 == 0 and 8 <= d_model <= 8192 (else DIT_E_UNSUPPORTED)
 */
int dit_adaln_modulate(void* y, const void* x, const float* gamma, const float* beta,
                       int64_t tokens, int32_t d_model, int64_t tokens_per_row,
                       float eps, int32_t dtype, void* stream);

/*
 * 3D rotary position embedding in place on q and k, "DiT, Flow Matching e 3D
 * Attention", section "3D-RoPE e atencao espaco-temporal": d_head = d_t + d_h + d_w
 * and q_rot = R_3D(t, y, x) q, k_rot = R_3D(t, y, x) k. Slices are laid out
 * [t | h | w]; pair j of the slice for axis a (width d_a, offset o_a) covers dims
 * (o_a + 2j, o_a + 2j + 1) and turns by phi = pos_a * base^(-2j / d_a):
 *   (x0, x1) <- (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi).
 * Every head of a token uses the same rotation. v is not rotated.
 *
 *   q, k         [tokens][heads][head_dim] (dtype), rotated in place; k may be NULL
 *   grid_h, grid_w   patched H', W' of every sequence
 *   dense mode  (cu_seqlens == NULL): num_seqs sequences of grid_t*grid_h*grid_w
 *                tokens each; tokens must equal num_seqs * grid_t * grid_h * grid_w
 *   packed mode (cu_seqlens != NULL): device int32 [num_seqs+1]; grid_t is
 *                ignored; each sequence length must be a multiple of grid_h*grid_w
 *                (unchecked precondition). Positions restart at 0 per sequence.
 *   d_t, d_h, d_w    even, >= 0, summing to head_dim; base > 1
 *   pos_out      nullable device int32 [tokens][3]: receives (t', h', w')
 *   head_dim % 8 == 0 and head_dim <= 256, heads >= 1
 * Accuracy: base^(-2j/d_a) / (2 pi) is computed in float64 and rounded to
 * float32; phi / (2 pi) = pos_a * that value is formed in float32 and its
 * fraction fed to the hardware sine/cosine of turns (error ~1.3e-7), so the
 * angle carries two float32 roundings, at most ~2^-23 relative: ~1.2e-5 rad at
 * phi = 100 rad.
 */
int dit_rope3d(void* q, void* k, int64_t tokens, int32_t heads, int32_t head_dim,
               int32_t grid_t, int32_t grid_h, int32_t grid_w,
               const int32_t* cu_seqlens, int32_t num_seqs,
               int32_t d_t, int32_t d_h, int32_t d_w, float base,
               int32_t* pos_out, int32_t dtype, void* stream);

/*
 * Full spatio-temporal attention, "Por que e absurdamente dificil gerar um filme
 * inteiro usando IA", section "Matematica por tras", with the scale of "DiT, Flow
 * Matching e 3D Attention", section "3D-RoPE e atencao espaco-temporal":
 *   o[i][h] = sum_j softmax_j(q[i][h] . k[j][h] / sqrt(head_dim)) v[j][h]
 * over every key j of the query's own sequence (bidirectional, no mask; packed
 * sequences never attend to each other).
 *
 *   o, q, k, v   [tokens][heads][head_dim] (dtype); o must not overlap q, k or v
 *   dense mode  (cu_seqlens == NULL): num_seqs sequences of tokens/num_seqs tokens
 *   packed mode (cu_seqlens != NULL): device int32 [num_seqs+1]; max_seqlen must
 *                be >= every sequence length (unchecked precondition)
 *   head_dim in {64, 128} (else DIT_E_UNSUPPORTED)
 * bf16 runs on MFMA with float32 accumulation; probabilities enter the second
 * product rounded to bf16. float32 runs on the vector ALUs in full float32.
 * Launch forms. Let G be the number of query tiles (256 queries, 128 at
 * head_dim 64) times heads times sequences, and R the blocks the device holds at
 * once (one per compute unit; two at head_dim 64). On the whole chip (256
 * compute units in 8 XCDs; a partitioned device always takes one block per
 * tile), with G >= 4R, or G >= 2R and a
 * last round of one-block-per-tile under 90% full, R persistent blocks draw
 * tiles from per-XCD queues (counters in library-owned device memory; a block
 * takes tiles of its own XCD first, then steals). At head_dim 128 the tiles of
 * each queue's last round are also cut along their keys into 2..16 pieces whose
 * partial results (unnormalised o, running max, row sum) go to the library's
 * split array; the last piece of a tile to finish merges them. Otherwise, and
 * always under stream capture, one block per tile.
 * Concurrency: each persistent launch takes one of 64 counter slots and, if no
 * unfinished launch on another stream holds it, the split array. Slots and the
 * split array are tracked with events, so concurrent launches on several streams
 * are safe; with all 64 slots held by unfinished launches on other streams a
 * launch runs one block per tile, and without the split array it runs unsplit.
 * Results: unsplit tiles are bitwise identical in every form; a split tile sums
 * its key blocks in another order (same float32 arithmetic, agreement within
 * rounding). For a given shape and device, repeated launches give identical bits
 * unless a concurrent launch on another stream holds the split array.
 */
int dit_attn3d(void* o, const void* q, const void* k, const void* v,
               int64_t tokens, int32_t heads, int32_t head_dim,
               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
               int32_t dtype, void* stream);

/*
 * dit_attn3d for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * validation, arithmetic and results as dit_attn3d; it calls no hipMalloc,
 * hipFree, event or other allocating routine. Its persistent launches (same
 * rule as dit_attn3d) take their queue counters from one fixed slot of a
 * library-owned device array of 576 bytes per device (resolved with
 * hipGetSymbolAddress on the first call on each device, kept until the process
 * ends, cleared by a kernel before every launch) and never cut tiles along their
 * keys, so no input needs more scratch than that; every tile's result is bitwise
 * that of an unsplit dit_attn3d tile. All calls on one device share the slot:
 * calls that overlap on one device (several streams, concurrent replays of
 * graphs that captured it) race and may skip or repeat tiles. Serialise them.
 */
int dit_attn3d_noalloc(void* o, const void* q, const void* k, const void* v,
                       int64_t tokens, int32_t heads, int32_t head_dim,
                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                       int32_t dtype, void* stream);

/*
 * One ring-attention step ("DiT, Flow Matching e 3D Attention", section
 * "Engenharia de inferencia e paralelismo de contexto: Ulysses, Ring Attention e
 * FP8"): each sequence's queries attend to that sequence's key/value block, and
 * the row log-sum-exp is returned so that blocks can be merged
 * (dit_attn_merge). For query i of sequence s and head h, over the keys j of
 * the sequence's block, with s_j = q[i][h] . k[j][h] / sqrt(head_dim):
 *   lse[i][h] = ln sum_j exp(s_j)           (natural log, float32)
 *   o[i][h]   = sum_j exp(s_j - lse[i][h]) v[j][h]
 * A sequence whose block has no keys gives o = 0 and lse = -inf.
 *
 *   o, q          [tokens_q][heads][head_dim] (dtype); o must not overlap q, k, v
 *   k, v          [tokens_k][heads][head_dim] (dtype)
 *   lse           [tokens_q][heads] float32; must not overlap o, q, k or v
 *   dense mode  (cu_seqlens_q == cu_seqlens_k == NULL): num_seqs sequences of
 *                tokens_q/num_seqs queries and tokens_k/num_seqs keys
 *   packed mode (both non-NULL): device int32 [num_seqs+1] each; sequence s has
 *                queries cu_seqlens_q[s]..cu_seqlens_q[s+1] and keys
 *                cu_seqlens_k[s]..cu_seqlens_k[s+1]; max_seqlen_q / max_seqlen_k
 *                must be >= every query / key count (unchecked precondition);
 *                key counts may be 0
 *   head_dim in {64, 128} (else DIT_E_UNSUPPORTED); tokens_q, tokens_k >= 1
 * Arithmetic and launch forms as dit_attn3d, which is the case k, v = the
 * queries' own tokens.
 */
int dit_attn3d_lse(void* o, float* lse, const void* q, const void* k, const void* v,
                   int64_t tokens_q, int64_t tokens_k, int32_t heads, int32_t head_dim,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                   int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t dtype, void* stream);

/*
 * Fold a partial attention over one key block into a running accumulator over
 * the blocks seen so far (same section as dit_attn3d_lse): for every
 * (token, head) row,
 *   lse_acc' = ln(exp(lse_acc) + exp(lse_b))
 *   o_acc'   = exp(lse_acc - lse_acc') o_acc + exp(lse_b - lse_acc') o_b
 * in place. An empty accumulator is o_acc = 0, lse_acc = -inf (merging into it
 * copies the partial); rows with lse_acc = lse_b = -inf stay o = 0, lse = -inf.
 *
 *   o_acc         [tokens][heads][head_dim] float32, read and written
 *   lse_acc       [tokens][heads] float32, read and written
 *   o_b           [tokens][heads][head_dim] (dtype: the partial's storage)
 *   lse_b         [tokens][heads] float32
 *   head_dim in {64, 128}; no two of the four arrays may overlap
 */
int dit_attn_merge(float* o_acc, float* lse_acc, const void* o_b, const float* lse_b,
                   int64_t tokens, int32_t heads, int32_t head_dim, int32_t dtype, void* stream);

/* Optional Euler pass fused into dit_gated_residual (same launch, same dtype). */
typedef struct {
    void* z_out;            /* [tokens][channels]; may equal z */
    const void* z;          /* [tokens][channels] */
    const void* u;          /* [tokens][channels] velocity */
    const float* dt_rows;   /* [tokens/tokens_per_row] float32 */
    int64_t tokens;
    int32_t channels;
    int64_t tokens_per_row;
} dit_euler_args;

/*
 * Gated residual, "DiT, Flow Matching e 3D Attention", section "A ruptura da
 * U-Net" (x'_l = x_l + alpha_1 * SelfAttention(...); alpha = 0 gives the identity):
 *   x_out[tok][c] = x[tok][c] + alpha[row][c] * branch[tok][c],  row = tok / tokens_per_row
 * branch is the attention output with heads merged (c = h * head_dim + i).
 *
 *   x_out, x, branch   [tokens][d_model] (dtype); x_out == x allowed
 *   alpha              [tokens/tokens_per_row][d_model] float32
 *   euler              nullable: also run rf_euler_step's update in the same launch
 *   d_model % 8 == 0
 */
int dit_gated_residual(void* x_out, const void* x, const void* branch, const float* alpha,
                       int64_t tokens, int32_t d_model, int64_t tokens_per_row,
                       const dit_euler_args* euler, int32_t dtype, void* stream);

/*
 * Rectified-flow Euler step, "DiT, Flow Matching e 3D Attention", section "Flow
 * Matching e Rectified Flow": along x_t = (1-t) x_0 + t x_1 (noise at t = 0, data at
 * t = 1) the velocity is x_1 - x_0 and an Euler sampler advances
 *   z_out[tok][c] = z[tok][c] + dt_rows[row] * u[tok][c],   row = tok / tokens_per_row
 * (one dt per sample, or per frame for per-frame local times).
 *
 *   z_out, z, u   [tokens][channels] (dtype); z_out == z allowed
 *   dt_rows       [tokens/tokens_per_row] float32
 *   channels % 8 == 0
 */
int rf_euler_step(void* z_out, const void* z, const void* u, const float* dt_rows,
                  int64_t tokens, int32_t channels, int64_t tokens_per_row,
                  int32_t dtype, void* stream);

/*
 * First stage of the explicit midpoint sampler, the second ODE sampler "DiT,
 * Flow Matching e 3D Attention", section "Flow Matching e Rectified Flow", names
 * beside Euler:
 *   z_mid = z + (dt_rows[row] / 2) * u,   u = velocity at (z, t)
 * The step finishes with rf_euler_step(z_out, z, u_mid, dt_rows, ...), u_mid the
 * velocity at (z_mid, t + dt/2). Arguments as rf_euler_step (z_mid == z allowed).
 */
int rf_midpoint_half(void* z_mid, const void* z, const void* u, const float* dt_rows,
                     int64_t tokens, int32_t channels, int64_t tokens_per_row,
                     int32_t dtype, void* stream);

/*
 * Straight-path training input (same section): x_t = (1 - t) x0 + t x1, with
 * x0 the noise, x1 the data and one flow time per row (sample or frame). t = 0
 * and t = 1 return x0 and x1 exactly.
 *   x_t, x0, x1   [tokens][channels] (dtype); x_t may be x0 or x1
 *   t_rows        [tokens/tokens_per_row] float32
 *   channels % 8 == 0
 */
int rf_interpolant(void* x_t, const void* x0, const void* x1, const float* t_rows,
                   int64_t tokens, int32_t channels, int64_t tokens_per_row,
                   int32_t dtype, void* stream);

/*
 * Conditional flow-matching loss (same section): the squared distance between
 * the predicted velocity u and the path's velocity x1 - x0,
 *   loss_tokens[tok] = sum_c (u[tok][c] - (x1[tok][c] - x0[tok][c]))^2
 *   loss_rows[r]     = sum of loss_tokens over row r's tokens (the sample's or
 *                      frame's squared norm; the loss estimate is their mean)
 * float32 arithmetic; deterministic (fixed reduction order).
 *   u, x0, x1     [tokens][channels] (dtype)
 *   loss_tokens   [tokens] float32 (output)
 *   loss_rows     nullable, [tokens/tokens_per_row] float32 (output)
 *   channels % 8 == 0; outputs must not overlap the inputs or each other
 */
int rf_cfm_loss(float* loss_tokens, float* loss_rows, const void* u, const void* x0, const void* x1,
                int64_t tokens, int32_t channels, int64_t tokens_per_row, int32_t dtype, void* stream);

/*
 * 8-bit floating point attention ("DiT, Flow Matching e 3D Attention", section
 * "Engenharia de inferencia e paralelismo de contexto: Ulysses, Ring Attention
 * e FP8", which pairs FlashAttention-3 with 8-bit quantisation). Format: OCP
 * E4M3 (bias 7, 3 mantissa bits, max 448, round to nearest even). One scale
 * per (tensor, head), amax[t][h] = max |x_t[:, h, :]|. k and v: codes =
 * E4M3(clamp(x * (448 / amax), +-448)) in float32 (below amax = 2^-100 formed
 * as (x * 2^64) * (448 / (amax * 2^64)): the same value wherever the plain form
 * is finite), dequantised value = code * amax / 448.
 * q: its scale s_q makes the score scale s_q * s_k * log2(e) / sqrt(128) an
 * exact power of two 2^n, n the smallest integer with
 * 2^n >= amax_q * amax_k * log2(e) / (448^2 * sqrt(128)) (decided in float64,
 * kept at most 127); codes = E4M3(clamp(q * g, +-448)) with the float32
 * multiplier g = (float)(amax_k * log2(e) / (448 * sqrt(128)) * 2^-n), so the
 * largest |q| maps into (224, 448], and s_q = 2^n * sqrt(128) / (s_k * log2(e)).
 * An all-zero head has codes 0, and so has q's head when k's is all zero (its
 * scores are 0 whatever q holds) or when n would lie below -127 (every score
 * under 1e-31: uniform weights to float32 precision); n is then 0.
 *
 * dit_quant_fp8 writes
 *   q8, k8     [tokens][heads][128] uint8 codes (row-major like q, k)
 *   v8t        [heads][128][v_stride] uint8: V transposed for the attention
 *              kernel -- each sequence padded with zero codes to a multiple of
 *              64 keys, sequences one after another, and inside each tile of 64
 *              keys key 32b + 8q + 4h + i at column 32h + 16b + 4q + i
 *   amax       [3][heads] float32 (q, k, v)
 * from bf16 q, k, v [tokens][heads][128]. v_stride (bytes per v8t row) must be
 * a multiple of 64 and >= dit_fp8_v_stride(tokens, num_seqs).
 *
 * dit_attn3d_fp8: o (bf16 [tokens][heads][128]) = softmax(q k^T / sqrt(128)) v
 * over the dequantised values, both products on E4M3 matrix cores with float32
 * accumulation (the score product scaled by 2^n, derived from amax as above);
 * the probabilities enter the second product rounded to E4M3, as
 * 2^(s - m + 6) with s the base-2 score and m an integer running maximum.
 * Sequences as dit_attn3d (dense: cu_seqlens NULL; packed: device offsets and
 * max_seqlen). head_dim must be 128. Outputs must not overlap inputs.
 */
int64_t dit_fp8_v_stride(int64_t tokens, int32_t num_seqs);
int dit_quant_fp8(void* q8, void* k8, void* v8t, float* amax, const void* q, const void* k, const void* v,
                  int64_t tokens, int32_t heads, int32_t head_dim, const int32_t* cu_seqlens, int32_t num_seqs,
                  int32_t max_seqlen, int64_t v_stride, int32_t dtype, void* stream);
int dit_attn3d_fp8(void* o, const void* q8, const void* k8, const void* v8t, const float* amax, int64_t tokens,
                   int32_t heads, int32_t head_dim, const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                   int64_t v_stride, void* stream);

/*
 * Flowception frame insertion ("Flowception: Temporally Expansive Flow Matching
 * for Video Generation", technical summary, section 2): during sampling, new
 * frames are inserted between existing ones, each starting as unit Gaussian
 * noise with its local time reset to 0. counts[f] new frames go right after
 * existing frame f (the draw from the predicted insertion rates is the
 * caller's; passive frames carry 0), taking the noise frames in order.
 *
 *   z             [frames * tokens_per_frame][channels] (dtype): the packed batch
 *   t_frames      [frames] float32 local times
 *   cu_seqlens    device int32 [num_seqs+1] token offsets of the sequences
 *                 (multiples of tokens_per_frame, from 0 to frames*tokens_per_frame)
 *   counts        device int32 [frames], >= 0, summing to frames_out - frames
 *   noise         [(frames_out - frames) * tokens_per_frame][channels] (dtype);
 *                 may be NULL when frames_out == frames
 *   z_out         [frames_out * tokens_per_frame][channels] (dtype)
 *   t_out         [frames_out] float32: source frames keep their time, new ones 0
 *   cu_out        device int32 [num_seqs+1]: the new token offsets
 *   src_out       device int32 [frames_out]: existing frame index, or -1 - n for
 *                 the n-th noise frame
 * The device-side arrays (cu_seqlens, counts) are preconditions the host cannot
 * check; if the counts do not sum to frames_out - frames the call still stays in
 * bounds (uncovered output frames are zero with src_out = INT32_MIN). No output
 * may overlap an input or another output; channels % 8 == 0.
 */
int flow_insert_frames(void* z_out, float* t_out, int32_t* cu_out, int32_t* src_out,
                       const void* z, const float* t_frames, const int32_t* cu_seqlens, int32_t num_seqs,
                       const int32_t* counts, const void* noise, int64_t frames, int64_t frames_out,
                       int32_t tokens_per_frame, int32_t channels, int32_t dtype, void* stream);

/*
 * Per-frame schedule of local times (same section): every frame advances from
 * its own local time, dt_out[f] = min(dt_max, 1 - t_frames[f]) and
 * t_frames[f] += dt_out[f] in place, so no frame passes t = 1 and a clipped
 * step lands on exactly 1. dt_out feeds rf_euler_step / rf_midpoint_half with
 * tokens_per_row = tokens_per_frame.
 *   dt_out, t_frames  [frames] float32, not overlapping; dt_max > 0
 */
int flow_frame_schedule(float* dt_out, float* t_frames, int64_t frames, float dt_max, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H_ */
