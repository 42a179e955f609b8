"""MI355X-native routed-expert MoE layer with a frozen int4 base and trained
low-rank adapters (TQP).  The compute path lives in the HIP library under
``csrc/`` behind the C ABI declared in ``include/moe_tqp.h``; ``binding``
marshals torch tensors into those calls."""
__all__ = ["configs", "inputs", "binding"]
