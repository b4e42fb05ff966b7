"""KDA (Kimi Delta Attention) hot path for MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in
``include/kda.h`` (library ``libkda.so``). ``gated_delta_rule_109_amd.kda``
is the thin ctypes binding; ``gated_delta_rule_109_amd.workloads`` builds
seeded synthetic inputs.
"""
