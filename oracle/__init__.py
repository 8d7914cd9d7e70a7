"""Reference oracle for the self-speculative rollout step (test infrastructure).

This package is a plain, slow CPU implementation of what the GPU path computes:
a pre-norm decoder transformer, the weight quantizers that turn the target into
its own drafter, the Philox4x32-10 counter-based generator, the speculative
sampler (draft, verify, accept/resample/bonus, rollback) and the roofline
controller that turns speculation on or off and chooses the draft length.

It exists only to check the GPU path.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does, and it shares no code with the HIP library.

Floating point runs in float64 unless a step is defined on a narrower type
(bf16/fp32 storage of weights, KV entries and linear-layer inputs, the quantizer
scales).  Every function cites the passage of the source pages it follows:

* p1 = "EfficientRollout: system-aware self-speculative decoding for RL
  rollouts" (ai-feeds summary of arXiv 2606.18967), sections "关键模块" (key
  modules) and "局限" (limitations).
* p2 = "Accelerating RL Post-Training Rollouts via System-Integrated
  Speculative Decoding" (chatpaper abstract).
* p3 = "TLT: reasoning RL long-tail rollout" reading notes, sections 1-3.
* p5 = "History Tree Dynamic RL 投机解码" (cann-recipes-train PR), sections
  2.2 and 4.

Parity status of each module is stated in its own header.
"""
