"""MI355X-native quantized Delta-rule decode step (GDN / KDA, packed 4/6/8-bit state).

The compute path is the HIP library ``libqdr.so`` behind the C ABI declared in
``include/qdr.h``; ``quantized_delta_rule_03_amd.qdr`` is its thin Python binding
(argument marshalling only). Importing the package does not load the library.
"""

__all__ = ["qdr", "workloads"]
