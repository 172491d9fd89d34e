"""MI355X-native fused differential-attention forward (prefill + decode).

The compute lives in ``libdiffattn.so`` (HIP kernels for gfx950 behind a C
ABI declared in ``include/diffattn.h``); ``binding`` marshals torch tensors
into that ABI.  ``workloads`` draws the seeded synthetic inputs.
"""
