"""CPU oracle (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The library under sparse_long_context_page_amd/ never imports
it, and it imports nothing from the library.

Modules: entmax_oracle.py (boxes, bounds, top-k selection, alpha-entmax,
sparse and full decode) and gauss_oracle.py (page moments and the
Gaussian-aware selection).

Parity pins: every function of both modules is pinned by a CPU test in
tests/test_oracle_*.py against something other than itself (a textbook
optimisation problem, a library routine, numerical integration, Monte Carlo,
brute force, a closed form or an invariant). No function here is "parity
unpinned".
"""
