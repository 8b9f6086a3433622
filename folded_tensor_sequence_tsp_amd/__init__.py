"""MI355X-native TSP (Tensor + Sequence Parallelism) rank-share layer.

The compute path is the HIP library ``libtsp.so`` (C ABI, ``include/tsp.h``);
:mod:`folded_tensor_sequence_tsp_amd.tsp` is its thin ctypes binding and
:mod:`folded_tensor_sequence_tsp_amd.synth` draws seeded synthetic inputs.
"""
