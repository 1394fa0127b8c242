"""LoRA / QLoRA adapted linear layer for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``liblq.so`` (hand-written HIP kernels,
declared in ``include/lq.h``); ``lq`` is its thin ctypes binding and
``workloads`` holds the seeded synthetic inputs.  Importing the package loads
nothing; the library is opened on the first call.
"""
