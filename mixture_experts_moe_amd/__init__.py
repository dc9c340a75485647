"""MI355X-native forward pass of one mixture-of-experts layer.

The compute path is the HIP library ``libmoe.so`` (C ABI: include/moe.h);
``mixture_experts_moe_amd.moe`` is its Python binding.  ``synth`` draws the
seeded synthetic inputs.  Importing the package loads nothing; the first call
into ``moe`` loads the library and raises if it is not built.
"""
