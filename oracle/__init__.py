"""CPU oracle for the NVFP4 block-scaled batched GEMV.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import, call, link or run anything in this package; the
GPU library and its Python binding never do, and they share no code with it.

* ``reference``  - decode tables, the GEMV sums (plain C, fp64, sequential in
  k) and the fp32/fp16 epilogue;
* ``quantize``   - the BF16 -> NVFP4 quantiser that turns the Gaussian
  workload's draws into bytes;
* ``build``      - compiles ``nvfp4_ref.c`` with gcc.

Pinned by the not-gpu tests: the E2M1 table (the bridge page's constants), the
E4M3 decode (all 256 codes against torch's float8_e4m3fn), the sums (exact
rational brute force on tiny shapes, hand-derived single-block examples, an
independent float64 matmul), the fp16 rounding (ties and overflow), and
invariants (zero scales, sign flips, block and batch permutations, power-of-two
alpha).  Parity unpinned: the quantiser's tie rule and output bytes (the pages
print no quantised values; only properties pin them).
"""
