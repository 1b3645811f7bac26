"""MI355X-native gated delta rule (KDA / Complex KDA / GDN): chunkwise forward
and recurrent decode behind a C ABI (include/kda.h, libkda.so).

* ``gated_delta_rule_46_amd.kda``    -- ctypes binding (chunk_fwd, decode_step)
* ``gated_delta_rule_46_amd.inputs`` -- seeded synthetic workloads
* ``gated_delta_rule_46_amd.build``  -- hipcc build of libkda.so for gfx950
"""
__version__ = "0.1.0"
