"""CPU oracle for the CSA/HCA hybrid compressed attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import this
package; only the test suite, the smoke check and the CPU-baseline leg of the
benchmark call it.  It is a plain, slow, float64 NumPy restatement of what the
method computes, written from the public descriptions of DeepSeek-V4's
Compressed Sparse Attention (CSA) and Heavily Compressed Attention (HCA):

* "DeepSeek-V4" technical blog (haiqwa.github.io), sections on CSA / HCA,
  RMSNorm, Partial RoPE, the attention sink and FP4 indexer precision;
* the 硅星人 article on V4 (bjxrzxf.com mirror), paragraphs on the CSA data
  flow, the lightning indexer, HCA, the sliding window, the sink, the
  BF16/FP8 cache split and the state / classic caches;
* the QbitAI piece on batch invariance (juhe.plus mirror).

Number formats follow the OCP 8-bit floating point specification (E4M3) and
the OCP Microscaling (MX) v1.0 specification (E2M1 elements, E8M0 scales).

Modules:
  formats -- BF16 / FP8-E4M3 / E2M1 / E8M0 / MXFP4 / split-row encode+decode
  method  -- compressor, RMSNorm, partial RoPE, indexer, top-k, sink MQA,
             decode and prefill drivers

Every function is pinned by a CPU test in tests/test_oracle_*.py against
closed forms, library routines, brute force or invariants; see the header of
each module for the list.  Functions without such a pin would say
"parity unpinned" in their docstring; there are none at present except the
conventions the pages leave open, which are listed in method.READINGS.
"""

from . import formats, method  # noqa: F401
