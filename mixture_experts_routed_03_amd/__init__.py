"""MI355X-native routed-expert MoE layer (dropless, all experts on one GPU).

The compute path is the C-ABI library ``libmoe.so`` built from ``csrc/``
(hand-written HIP for gfx950); ``binding`` marshals arguments to it.
``workloads`` holds the seeded synthetic input generators.

Nothing is imported eagerly: importing ``workloads`` must not load the GPU
library or initialise the GPU.
"""

__all__ = ["binding", "workloads"]
