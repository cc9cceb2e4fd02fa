"""CPU oracle for the fused attention forward and backward (TEST INFRASTRUCTURE ONLY).

Plain float64 implementations of what the AttnFuse pages' attention computes
("AttnFuse: A Composable DSL for Compiling Attentions to Fused GPU Kernels").
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
and imports nothing from it.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, a library routine (``torch.nn.functional.scaled_dot_product_attention``
in float64 on the CPU), a pure-Python brute force and, for the backward,
finite differences of the forward.  Parity unpinned: none.
"""
from .attention import allowed_mask, attention, rope_frequencies, rope_rotate  # noqa: F401
from .backward import attention_backward  # noqa: F401
from .brute import attention_brute  # noqa: F401
