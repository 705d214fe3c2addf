"""CPU oracle for Depth Exploration Decoding (DEX). TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never touches it and fails loudly
when its native extension is missing.

Everything here is plain and slow on purpose: NumPy float64, one obvious
implementation per quantity, written from "Depth Exploration for LLM Decoding"
(arXiv 2606.29223):

* ``model``  - the plain pre-RMSNorm SwiGLU RoPE decoder the method wraps,
               with the per-depth logits of the shared head (Section 3.4).
* ``depth``  - depth ceiling, resolution, exploration workload and speedups
               (Section 2.3, Definitions 4-5, Propositions 6-7, eqs. (6)-(14)).
* ``rule``   - the decoding rule with depth-coupled sampling (Algorithm 2,
               Section 3.3 and Appendix C.1).
* ``decode`` - plain autoregressive decoding, stable-EAD brute force
               (Definition 1, eqs. (1)-(3)) and the DEX lattice procedure
               (Algorithm 1, Section 3.2).

Parity status: the transformer forward is pinned against an independent
library implementation (Hugging Face ``LlamaForCausalLM`` in float64) and by
closed-form invariants; the depth arithmetic by the paper's worked example in
Appendix A.3; DEX by the paper's lossless invariant (DEX stream equals AR
stream) on real and scripted models. No function is left unpinned.
"""
