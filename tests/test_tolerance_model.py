"""CPU: the backward tests' error model agrees with itself across its two
forms (the numpy one the small cases use, the float32 torch one the
full-size case uses)."""
import numpy as np

from bwd_tolerance import expert_sigmas, expert_sigmas_torch


def test_error_model_torch_form_equals_numpy_form():
    """The float32 torch form of the backward error model (used by the
    full-size GPU case) gives the numpy form's standard deviations."""
    rng = np.random.default_rng(53)
    x, dout = rng.standard_normal((37, 24)), rng.standard_normal((37, 24)) * 0.1
    w1, w2 = rng.standard_normal((40, 24)) * 0.3, rng.standard_normal((24, 40)) * 0.2
    a = expert_sigmas(x, dout, w1, w2)
    b = expert_sigmas_torch(x, dout, w1, w2)
    for key in ("z", "dz", "dx_perm", "dw1", "dw2"):
        np.testing.assert_allclose(b[key], a[key], rtol=2e-4, atol=1e-12, err_msg=key)
    c = expert_sigmas_torch(x, dout, w1, w2, weight_grads=False)
    assert "dw1" not in c and np.array_equal(c["dx_perm"], b["dx_perm"])
