"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds shapes, seeds and counter-based random streams only; no attention or
merge arithmetic.  ``philox``/``configs`` are the CPU side; ``gpu`` fills
device tensors from the same streams with a small HIP kernel of its own.
"""
