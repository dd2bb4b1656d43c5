"""CPU oracle for the GLQ E8RHTLinear forward — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, fp64 statement of what the GPU library computes.
It exists so that tests, the smoke check and the benchmark's CPU-baseline leg can
compare the HIP path against an independent implementation.  Nothing in the
product path (the C-ABI library and its Python binding) may import, call or link
anything in here, and nothing in here imports the product path.

Sources (the "glq" project pages):
  * glq 0.5.1 (PyPI project page), section "How it works", items 1, 2 and 4:
    a codebook of 2^16 innermost E8 points addressed by one 16-bit index per group
    of 8 weights, 8-bit (256-entry) or 16-bit residual stages, randomized
    Hadamard transform = random sign flips followed by a fast Walsh-Hadamard
    transform, matmul taken against the indices without forming W.
  * same page, table "Bit widths": bpw -> stages; one global scale per layer.
  * same page, section "Inference kernels": Y = X @ dequant(W)^T, N/8 codebook
    blocks per output row; the glq_dequant_matmul signature (Wscale, Qidxs2,
    codebook2, inv_resid_scale); the CPU path is dequantize-then-matmul.

Modules:
  e8        codebook enumeration (E8 shells, sort order, fp16 storage)
  hadamard  fast Walsh-Hadamard transform and the randomized Hadamard transform
  glq       dequantization (fp64 and the bit-exact fp32 rule) and the linear

Parity status of every function is stated in its docstring; functions whose
result no test pins to something outside the oracle say "parity unpinned".
"""

from . import e8, hadamard, glq  # noqa: F401
