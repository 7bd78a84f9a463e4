"""CPU oracle for the ReplaySSM decode path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
(``hybrid_model_ssm_replay_amd``) never import it, and this package imports
nothing from them: the two sides share no code.  The only common module is
``synth`` (seeded inputs, no decode arithmetic).

Everything here is plain float64 NumPy, written for a reader to check by eye,
not for speed.

Pages cited (by title; sections as they appear on each page):

* [P1] "Hybrid-model decoding has a new bottleneck: stop writing the SSM state
  every step, and speculative throughput reaches 2.10x" -- Synopsis,
  Interpretation paragraphs 1-4, Perspective paragraphs 1-2.
* [P2] "NVIDIA and Dao AI Lab speed up hybrid-model decoding" -- lede and
  paragraphs 1-4.
* [P3] "SSM decoding stops writing state every step: caching recent inputs
  halves state traffic and matches vLLM speculation" -- Synopsis,
  Interpretation paragraphs 1-3, Perspective paragraphs 1-2.

The pages print no formulas.  The two recurrences are the published layer
definitions they name: Mamba-2 (Dao and Gu, "Transformers are SSMs", 2024,
single-token SSD decode) and Gated DeltaNet (Yang, Kautz and Hatamizadeh,
"Gated Delta Networks", 2024).  The replay identities in ``mamba2`` and
``gdn`` are unrolled forms of those recurrences, derived in their docstrings.

Modules:

* ``mamba2``, ``gdn``: the stepwise definition and the replay form (output
  from a checkpoint plus buffered records; fold of a window into a checkpoint).
* ``pointers``: the integer buffer-pointer machine (append, lazy flush,
  verify, commit, rollback).
* ``session``: the layer-level calls (init / step / flush / verify / commit)
  built twice: stepwise (the definition) and replay (the method).
"""
