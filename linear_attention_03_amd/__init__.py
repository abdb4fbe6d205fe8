"""libkda: Kimi Delta Attention (KDA) prefill, decode and target verify as
hand-written HIP kernels for MI355X (gfx950) behind a C-ABI.

``linear_attention_03_amd.kda`` is the Python binding (ctypes over
``libkda.so``); ``linear_attention_03_amd.workloads`` draws the seeded
synthetic inputs.  Importing the package loads neither.
"""

__all__ = ["kda", "workloads"]
