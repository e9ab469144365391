"""MI355X-native Muon hot path: Nesterov momentum and quintic Newton-Schulz
(NS5) orthogonalisation in bf16, as hand-written HIP kernels for gfx950 behind
the C-ABI library ``libmuon.so`` (declared in ``include/muon.h``).

``newton_schulz_09_amd.muon`` is the Python binding (argument marshalling
only; it raises if the HIP library is missing).  ``workloads`` holds the
seeded synthetic inputs.
"""
__all__ = ["muon", "workloads"]
