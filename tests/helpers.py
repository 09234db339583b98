"""Shared test utilities: moving seeded inputs to the device and comparing
device results with the fp64 oracle."""

import numpy as np

from exact_attention_10_amd import inputs

# Tolerances of the parity gate (bf16 inputs, fp32 accumulation).
O_ATOL = 2e-2
LSE_TOL = 1e-3        # |dLSE| <= LSE_TOL * max(1, |LSE_ref|)
GRAD_ATOL = 5e-2


def to_device(arr, dtype, torch, device="cuda"):
    """Stored inputs (bf16 / fp16 bit patterns or fp32) -> torch tensor on `device`."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.float16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(w, name):
    return inputs.as_f64(w[name], w["dtype"])


def check_o(o_dev, o_ref, atol=O_ATOL, what="O"):
    o_dev = np.asarray(o_dev, dtype=np.float64)
    err = np.abs(o_dev - o_ref)
    assert np.all(np.isfinite(o_dev)), "%s has non-finite values" % what
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, "%s max-abs error %.3g > %.3g" % (what, worst, atol)
    return worst


def check_lse(l_dev, l_ref, tol=LSE_TOL):
    l_dev = np.asarray(l_dev, dtype=np.float64)
    inf_ref = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_dev), inf_ref), "LSE -inf pattern differs"
    fin = ~inf_ref
    if not fin.any():
        return 0.0
    err = np.abs(l_dev[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))
    worst = float(err.max())
    assert worst <= tol, "LSE error %.3g > %.3g" % (worst, tol)
    return worst
