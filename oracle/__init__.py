"""CPU oracle for the chunked Kimi Delta Attention (KDA) forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs anything in
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code, headers, tables or constants with the HIP
library; the two meet only through the seeded inputs of ``workloads.py``.

Contents
  recurrent.py    fp64 token-by-token recurrence: the definition of the forward.
  chunked.py      fp64 chunked (WY/UT) form as the pages lay it out, plus the two
                  unit-lower-triangular inverses (forward substitution and the Neumann
                  doubling product). Used only as an invariant (chunked == recurrent) and as
                  a diagnostic of the per-chunk intermediates.
  exact.py        the recurrence in exact rational arithmetic (fractions.Fraction) for tiny
                  inputs with rational decays.
  kda_oracle.c    the fp64 token recurrence in plain C, threaded over independent
                  (sequence, value head) units; the fast oracle for large workloads.
  prestage.py     fp64 pre-stage: q/k L2 normalisation, beta sigmoid and the two gate
                  activations (softplus and bounded sigmoid) that produce the recurrence's
                  q, k, g, beta from raw projections.
  backward.py     fp64 gradients of the forward (dq, dk, dv, dg, dbeta, dh0): the reverse-mode
                  token recurrence, derived by hand, plus torch.autograd on the fp64 forward
                  as an independent check; with the pre-stage's reverse mode (prestage.py),
                  the gradients with respect to raw inputs, A_log and dt_bias.
  backward_chunked.py  the same gradients by the chunked reverse sweep (chunk records, the
                  state and state-gradient chains, per-chunk local gradients): the algebra
                  the GPU backward follows, pinned against backward.py.
  kda_oracle_bwd.c  the fp64 reverse token recurrence of backward.py in plain C (states
                  rebuilt from checkpoints every 256 tokens), threaded over (sequence, q/k
                  head) tasks; the fast backward oracle for full-size workloads.
  native.py       ctypes loader for the C oracle.
  build.py        compiles kda_oracle.c and kda_oracle_bwd.c with gcc.

Sources (pages, by title): the KDA definition is read off the chunked listing in "手撕KDA"
("KDA by hand"), section 1 (the FLA naive_chunk_kda routine): a one-token chunk of that
listing reduces to the recurrence in recurrent.py, and section 5 of the same page names the
recurrent kernel (fused_recurrent_kda) as the cross-check of the chunked one. The
Neumann product follows "KDA源码剖析之FlashKDA（上）", part 12 (Neumann series inverse),
and the FlashKDA Neumann-inverse walkthrough page.

Every function here is pinned by tests/test_oracle.py against closed forms, special cases,
exact rational arithmetic, hand-worked fixtures (tests/golden/) and library routines.
"""
