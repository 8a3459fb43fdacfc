"""MI355X-native MoE layer forward with MACS capacity routing and SERE re-routing.

The compute path is a HIP library (``csrc/``) behind a C ABI
(``include/moe_macs.h``); ``binding`` marshals torch tensors into it.
Importing this package loads nothing: ``from mixture_experts_layer_macs_amd
import binding`` loads the library and fails loudly when it is not built.
"""
