"""Plain fp64 CPU oracle for the routed 4-bit MoE expert layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``bit_quantized_moe_expert_amd``) never imports, calls or links it, and this
package imports nothing from the product path.
"""
from .nf4moe_oracle import *  # noqa: F401,F403
from .nf4moe_oracle import __all__  # noqa: F401
