"""MI355X-native MoE FFN layer forward: HIP kernels behind a C ABI.

The compiled library (libmoe_mi355x.so, built by ``build.py``) is loaded on
first use by :mod:`.binding`; importing the package itself needs no GPU.
"""
