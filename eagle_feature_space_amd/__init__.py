"""MI355X-native EAGLE draft-and-verify hot path.

The compute path is the HIP library ``libeagle.so`` behind the C-ABI declared
in ``include/eagle.h``; ``eagle_feature_space_amd.binding`` marshals torch
device tensors into it.  ``configs`` and ``synth`` hold workload shapes and
seeded synthetic inputs only.
"""
