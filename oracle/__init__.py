"""Plain CPU oracle of one draft -> confidence -> schedule -> verify cycle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never calls it, and nothing here is shared with the GPU code: the two are
written independently from the same description of the method.

Arithmetic is numpy float64 throughout; bf16 and fp32 inputs are read exactly.
Every function names the passage of the method it follows.  The pages are:

* "DSpark: semi-autoregressive generation and confidence-scheduled
  verification" (juhoplayground.github.io) -- the authority for the cycle;
  sections Overview, Background, Method (Semi-autoregressive generation;
  Confidence-scheduled verification), Results, Limitations.
* "[vLLM] MTP & DFlash" (blog.secrett2633.cloud) -- prior art for the parallel
  drafter whose outputs are synthesised here.

Readings taken where the pages are silent are listed per module.  Parity
status: every function is pinned by ``tests/test_oracle_*.py`` (known-answer
vectors, closed forms, exhaustive enumeration, chi-square sampling tests and
special cases); no function is parity-unpinned.
"""
from . import philox, sampling, draft, rnn, conf, sched, sts, verify, cycle  # noqa: F401
