"""Host checks of the parity tests' own helpers (no GPU needed): the half-ulp
bound used for rows with few live keys equals half the gap to the next
representable value of the output type, measured by stepping the type's
bit pattern."""
import numpy as np
import torch

from test_parity_gpu import _half_ulp


def _next_gap(x: np.ndarray, dtype: torch.dtype, int_view: torch.dtype) -> np.ndarray:
    """Gap from |x| rounded to `dtype` to the next larger value of `dtype`."""
    a = torch.from_numpy(np.abs(x)).to(dtype)
    nxt = (a.view(int_view) + 1).view(dtype)
    return (nxt.double() - a.double()).numpy()


def test_half_ulp_matches_the_types_spacing():
    rng = np.random.default_rng(3)
    # magnitudes from about 2^-13 to 2^13, each first rounded to the type
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-10, 11, size=4000))
    # (the smallest normal value: 2^-126 for bf16, 2^-14 for fp16)
    for name, dt, iv, tiny in (("bf16", torch.bfloat16, torch.int16, 2.0 ** -126),
                               ("f16", torch.float16, torch.int16, 2.0 ** -14)):
        xr = torch.from_numpy(x).to(dt).double().numpy()
        keep = np.abs(xr) >= tiny
        want = _next_gap(xr[keep], dt, iv) / 2
        got = _half_ulp(xr[keep], name)
        assert np.array_equal(got, want), name
    xr = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(_half_ulp(xr, "f32"), np.spacing(np.abs(xr).astype(np.float32)).astype(np.float64) / 2)
