"""Plain, slow CPU oracle for the Muon hot path (Nesterov momentum + NS5).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the GPU library.  It
shares no code with ``newton_schulz_09_amd``.  Source: Synced (机器之心)
report on Modded-NanoGPT, section "Muon optimizer".

Every function is pinned by ``tests/test_oracle_*.py`` against facts fixed by
the page and by mathematics (closed forms, invariants, exact brute force).
"""
from .muon_oracle import (NS5_COEFFS, NS5_EPS, NS5_STEPS, apply_update, f32, momentum_nesterov,  # noqa: F401
                          muon_step, muon_step_apply, ns5, ns5_grouped, ns5_nominal_flops, polar_factor,
                          round_bf16, round_f32)
from .jacobi_svd import jacobi_svd  # noqa: F401
