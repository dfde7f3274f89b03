"""Plain, slow, float64 CPU oracle of the DiT attention-block hot path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import this package. The product path (the HIP
library and its Python binding) never imports, calls or falls back to it.

It shares no code with the GPU path: no kernels, headers, helpers, tables or
constant generators. Inputs are the stored activation values (bf16 or fp32)
converted losslessly to float64; outputs stay unrounded float64.

What it follows (pages are cited by title and section):
  * grid      -- token <-> (t', h', w') patch-grid coordinates: "DiT, Flow Matching
                 e 3D Attention", section "A ruptura da U-Net" (patchify diagram,
                 N = (T/p_t)(H/p_h)(W/p_w)).
  * modulate  -- adaLN-Zero gamma * LayerNorm(x) + beta: same page and section,
                 the block equations for x'_l and x_(l+1).
  * rope      -- 3D-RoPE, d_head = d_t + d_h + d_w, q_rot = R_3D(t, y, x) q:
                 same page, section "3D-RoPE e atenção espaço-temporal".
  * attention -- softmax(q_rot k_rot^T / sqrt(d_head)) V: same section, and
                 "Por que é absurdamente difícil gerar um filme inteiro usando
                 IA", section "Matemática por trás"; the row log-sum-exp and
                 the merge of partials over key blocks for ring attention:
                 first page, section "Engenharia de inferência e paralelismo
                 de contexto: Ulysses, Ring Attention e FP8".
  * epilogue  -- gated residual x + alpha * out (block equations) and the
                 rectified-flow Euler update along u, section "Flow Matching e
                 Rectified Flow" (x_t = (1 - t) x_0 + t x_1, v = x_1 - x_0),
                 with the interpolant, the flow-matching loss and the midpoint
                 sampler's half step from the same section.
  * fp8       -- OCP E4M3 encode/decode and per-head quantisation of q, k, v
                 for FP8 attention: "DiT, Flow Matching e 3D Attention",
                 section "Engenharia de inferência e paralelismo de contexto:
                 Ulysses, Ring Attention e FP8" (the attention itself is the
                 attention oracle on the dequantised values).
  * flowception -- frame insertion with local-time reset and the per-frame
                 schedule: "Flowception: Temporally Expansive Flow Matching for
                 Video Generation", technical summary, section 2.

Every function is pinned by tests in tests/test_oracle_*.py against closed
forms, invariants, library special cases or brute force; none is "parity
unpinned".
"""
from . import attention, epilogue, flowception, fp8, grid, modulate, rope  # noqa: F401
