"""fp64 CPU oracle for the Multi-Token Attention forward layer.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the library never does. It shares no code
with the GPU library. ``oracle.forward`` wraps the C++ implementation in
``mta_oracle.cpp``; ``oracle.py_reference`` is a second, pure-Python transcription
used only to cross-check the C++ one on tiny inputs; ``oracle.backward`` gives the
exact gradients (plain PyTorch fp64 forward under autograd).
"""
from .oracle import build, forward, library_path, max_threads  # noqa: F401
