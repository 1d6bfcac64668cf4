"""fp64 CPU oracle of one GPT-2 pre-training step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP path.
"""

from . import gpt2  # noqa: F401
