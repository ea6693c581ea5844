"""CPU oracle for one speculative-decoding draft-tree step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link this
package: only the tests, the smoke check of ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` use it. The GPU library shares no code, header, table or helper
with it; both sides receive the same seeded arrays from ``workloads``.

What it is: a plain, slow, obviously correct float64 implementation of every stage of
the step, written from the four pages on the subject:

* ``rows``        - per-row max / argmax / log-sum-exp / top-K (the primitives that the
                    TALON formulas, greedy verification and the min(1, p/q) rule use);
* ``mask``        - depth and the ancestor-or-self mask of a draft tree;
* ``build``       - the TALON, GOOSE-spine and OPT-Tree tree builders and given trees;
* ``attention``   - tree-masked attention, each node over the prefix and its ancestors;
* ``verify``      - greedy longest-match and Leviathan accept/resample verification;
* ``compact``     - moving the accepted path's K/V rows behind the prefix;
* ``bookkeeping`` - E[A], draft efficiency eta = N_d / N_v and Speedup ~ E[A]/(1+gamma*eta);
* ``step``        - the four stages chained on one workload.

Readings of points the pages leave open are stated in the docstring of the function
that takes them. Parity status: every function is pinned by tests under ``tests/``
against closed forms, brute force, library routines or hand-derived fixtures, except
where its docstring says "parity unpinned".
"""
