"""CPU oracle for group-wise 4-bit weight quantization and dequant-matmul.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
statement of what the GPU library computes.  Only the test-suite, the smoke
check in ``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library (``weight_only_bit_unpack_amd``)
never imports, links or calls anything here, and nothing here imports the GPU
library: the two share no code.  The only module both sides use is the seeded
input generator in ``synthetic/``, which holds none of the method's
arithmetic.

Sources.  The pages this follows are cited by title and section:

* "MiniCPM5-1B 验证: 6× 压缩 ... 50ms Triton 推理" (the DyadicGumbel 4-bit
  page), sections 2.1 (dyadic codebook), 2.2 (block layout and
  reconstruction), 2.3 (argmin over the codebook) and 2.5 (nibble packing and
  storage accounting).
* "K-Means量化技术：突破LLM低比特部署瓶颈" (the k-means page), sections 1.2
  (per-block 1D k-means codebook, nearest-neighbour assignment) and 2.2
  (lookup-table decode).
* "int4-g32+warm 裸量化：原理与实验报告" (the int4-g32 page), sections 1.2
  (the transform families of the warm start), 1.3 (per-group pipeline:
  transform choice, nearest level, Lloyd refinement, sign + magnitude) and 2
  (storage format: 1 sign bit + 3-bit level index per weight, groups of 32).
* The survey page on GPTQ/AWQ/GGUF/BitNet, section on uniform affine
  quantization (INT4 range [-8, 7]), used only as a textbook pin.

Modules
-------
``bits``      bf16 / fp16 bit patterns and round-to-nearest-even from fp64.
``dyadic``    absmax scale, argmin over the 16 dyadic codes, dequant.
``packing``   two nibbles per byte, low nibble first.
``lut16``     per-group 16-entry LUT codec and its k-means fit.
``signmag8``  sign + 3-bit magnitude codec and its Lloyd fit.
``dyadic5``   dyadic codes of 3, 4 or 5 bits per group in one 5-bit index space.
``warmstart`` the SIGNMAG8 warm start: 112 parametric transforms per group,
              the best one's 8 levels, then Lloyd rounds.
``matmul``    fp64 GEMV/GEMM on dequantized weights and the error bound.
``native``    ctypes loader for ``liboracle.so`` (plain C, same definitions,
              used where the Python loops would take minutes).

Functions that have no independent pin say "parity unpinned" in their
docstring; every other function is pinned by ``tests/test_oracle_*.py``.
"""

from . import bits, packing, dyadic, dyadic5, lut16, signmag8, warmstart, matmul  # noqa: F401

__all__ = ["bits", "packing", "dyadic", "dyadic5", "lut16", "signmag8", "warmstart", "matmul"]
