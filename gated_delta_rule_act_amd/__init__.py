"""MI355X-native chunked Kimi Delta Attention (KDA) forward.

The compute path is the HIP library ``libkda.so`` behind the C ABI in
``include/kda.h``; ``gated_delta_rule_act_amd.kda.fwd`` is its thin binding
(it loads the library on first use and fails loudly if it is not built).
``workloads`` draws the seeded synthetic inputs.
"""
