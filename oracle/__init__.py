"""Float64 CPU oracle for the Muon / Dimuon optimizer step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never calls it, and it shares no code with the HIP library.
"""

from .muon_oracle import (  # noqa: F401
    NS5_COEFFS,
    DIMUON_EPS,
    round_to_dtype,
    momentum_update,
    nesterov_input,
    energies_f64,
    energies_f32_tree,
    pairwise_sum_f32,
    conditioning,
    newton_schulz,
    muon_step,
    dimuon_step,
    StepResult,
)
