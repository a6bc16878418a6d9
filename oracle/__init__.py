"""CPU oracle for one verify round of one-pass block drafting (TEST INFRASTRUCTURE).

This package is a plain, slow, float64 NumPy statement of what the verify path
computes.  It exists to check the HIP library and nothing else: only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import it.
The product path never calls it, and it shares no code with the HIP kernels,
their headers or their Python binding.

Sources ("the paper" = "Vision Is Not Overhead: One-Pass Block Drafting for
Lossless Speculative Decoding in Vision-Language Models", arXiv 2609.00355;
"the project page" = the GLANCE project page):

  draft.py  log-softmax of the offset-wise draft marginals   (paper §3.2, Assumption 1)
  tree.py   top-N prefix-closed candidate tree, layout, masks (paper §3.2 Def. 1, §4.2;
            project page "Verify pass")
  model.py  unpacked evaluation of every node's own sequence and the head's
            row statistics                                   (paper Def. 1; App. B.1 proof;
            §6 root entropy)
  walk.py   greedy continuation, accepted length A(S), the walk (paper Def. 1, App. B.1)
  round.py  one full round built from the above

Every function is "parity pinned" by tests under tests/ that check it against
brute force, closed forms, library routines or hand-built cases; none is
unpinned.
"""
