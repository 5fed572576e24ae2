"""MI355X-native batched Online KL Shampoo / Shampoo preconditioner step.

The compute path is the HIP library under csrc/ (built to libokls.so) behind
the C ABI declared in include/okls.h; `okls` is its thin Python binding.
Importing the package does not load the library; the binding loads it on
first use and raises if it is missing.
"""
__all__ = ["okls", "workloads"]
