"""MI355X-native greedy speculative-decoding verify path.

``weight_bound_verify_amd.specverify`` binds the C-ABI library ``libspecverify.so`` (HIP
kernels for gfx950); ``weight_bound_verify_amd.synth`` makes seeded synthetic inputs.
Importing the package loads neither the library nor torch.
"""
