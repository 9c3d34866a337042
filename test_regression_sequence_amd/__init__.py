"""libmesa: the Mesa layer forward (chunked CG) and decode step on MI355X.

Heavy imports are lazy: ``test_regression_sequence_amd.inputs`` (synthetic
workloads) loads without torch's GPU runtime, and ``.mesa`` (the ctypes
binding of the HIP library) loads the shared library on first use.
"""

__all__ = ["mesa", "inputs", "build"]
