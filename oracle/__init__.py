"""CPU oracle for the NVFP4 block-scaled batched GEMV.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import, call, link or run anything in this package; the
GPU library and its Python binding never do, and they share no code with it.

* ``reference``  - decode tables, the GEMV sums (plain C, fp64, sequential in
  k) and the fp32/fp16 epilogue;
* ``quantize``   - the BF16 -> NVFP4 quantisers: with a global scale from the
  tensor's amax (the Gaussian workload's bytes, the weight quantiser) or given
  by the caller (the graph-safe activation quantiser), under the three E2M1
  rounding rules the pages use or the library's readings of them; and the GEMV fed by a
  quantised activation;
* ``build``      - compiles ``nvfp4_ref.c`` with gcc.

Pinned by the not-gpu tests: the E2M1 table (the bridge page's constants), the
E4M3 decode (all 256 codes against torch's float8_e4m3fn), the sums (exact
rational brute force on tiny shapes, hand-derived single-block examples, an
independent float64 matmul), the fp16 rounding (ties and overflow), and
invariants (zero scales, sign flips, block and batch permutations, power-of-two
alpha), the quantisers (hand-derived one-block examples for every rounding
rule, the exact intervals where the half-step table departs from nearest
rounding, the E4M3 cast against the decode table, sign symmetry, power-of-two
scale invariance).  The pages print no quantised values of their own.
"""
