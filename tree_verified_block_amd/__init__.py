"""MI355X (gfx950) verify path of one-pass block drafting with tree-verified
acceptance: the HIP library libglance.so (include/glance.h) and its Python
binding.

    glance_build_tree   log-softmax + top-K of the draft marginals, top-N tree
    glance_tree_attn    one packed, ancestor-masked target layer over the rows
    glance_verify_head  LM head with argmax / top-2 gap / entropy epilogue
    glance_accept_walk  greedy accept walk: A(S), committed tokens, new root
"""
from ._lib import GLANCE_BF16, GLANCE_F32, GLANCE_MAX_L, GLANCE_MAX_ROWS, GlanceError, load  # noqa: F401
