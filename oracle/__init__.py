"""CPU oracle for the virtual-noise evolution-strategies linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the HIP path is checked against.  Only the test-suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of the bench
may import it; the product package never does, and it shares no code with the
HIP kernels (no common helpers, tables or constant generators).

Source of truth: the EvoX API documentation page
``evox.triton_kernels.kernels.virtual_noise`` (sections "RNG: fast
centered-uniform approximation", "Noise indexing scheme", the module
introduction with the model and gradient equations, and the API entries
``_splitmix64_step``, ``_cpu_normal_noise``, ``compute_offsets``,
``virtual_perturbed_linear``, ``virtual_weight_gradient``,
``virtual_bias_gradient`` and ``virtual_reduce_metric``).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (a published splitmix64 test vector, an
independently written big-integer sequential generator, the page's printed
``compute_offsets`` example, closed forms, statistical bounds and brute force
on tiny inputs).  The concrete bit patterns under readings A1-A3 (how seed and
index form the state, the finalizer multipliers, the u mapping) are fixed by
the documented readings, not by the page; see ``vn_oracle`` for each one.
"""

from .vn_oracle import (  # noqa: F401
    GAMMA,
    CANONICAL_M1,
    CANONICAL_M2,
    splitmix_finalize,
    canonical_seeds,
    initial_state,
    noise_bits_at,
    noise_u32_at,
    noise_u32,
    noise_at,
    noise,
    compute_offsets,
    perturbed_linear,
    perturbed_linear_at,
    weight_gradient,
    weight_gradient_at,
    bias_gradient,
    reduce_metric,
)
