"""HSTU pointwise aggregated attention and layer forward for AMD MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/hstu.h``); ``binding`` marshals PyTorch
device tensors into it.  ``synth`` generates seeded synthetic inputs.
"""
