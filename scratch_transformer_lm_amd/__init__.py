"""MI355X-native GPT-2 fp32 training step: HIP kernels behind a C ABI.

The compiled library lives next to this file (libgpt2_mi355x.so); `gpt2` is the thin
ctypes binding and `synthetic` the seeded workload generators.
"""
