"""Seeded synthetic inputs for the lightning-indexer workloads.

This package is the only code shared between the fp64 oracle side (tests,
CPU baseline) and the GPU side.  It holds no indexer arithmetic: it draws
numbers from a counter-based generator, plants heavy keys, applies the
layer recurrence of the layer-reuse workload and quantises to the storage
formats (OCP e4m3fn with per-token fp32 scales, bf16).  ``synth.gen`` is the
numpy implementation; ``synth.gpu`` runs the same generator bit-for-bit on
the device for inputs too large to build on the host.
"""
from .gen import *  # noqa: F401,F403
