"""Helpers for the GPU parity tests: device copies of the seeded inputs, the
parity metrics and the tolerance (max-abs <= 2e-2, relative Frobenius <= 5e-3,
on outputs and final states, for bf16 inputs with an fp32 state)."""
import numpy as np

TOL_MAX_ABS = 2e-2
TOL_REL_F = 5e-3


def dev_inputs(d, io="bf16", layout="bthd", device="cuda"):
    """Upload q, k, v (bf16-exact values, or fp32) and the fp32 gates.

    layout "bhtd" stores q/k/v/o as [B, H, T, D] and passes [B, T, H, D] views."""
    import torch
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v"):
        x = torch.from_numpy(np.ascontiguousarray(d[key], dtype=np.float32))
        if layout == "bhtd":
            x = x.permute(0, 2, 1, 3).contiguous().to(device=device, dtype=dt).permute(0, 2, 1, 3)
        else:
            x = x.to(device=device, dtype=dt)
        out[key] = x
    for key in ("a", "beta"):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key], dtype=np.float32)).to(device)
    return out


def empty_out(t):
    import torch
    v = t["v"]
    if v.stride(1) == v.shape[2] * v.shape[3]:
        return torch.empty_like(v)
    B, T, H, D = v.shape
    return torch.empty((B, H, T, D), dtype=v.dtype, device=v.device).permute(0, 2, 1, 3)


def metrics(gpu, ref):
    g = gpu.double().cpu().numpy() if hasattr(gpu, "cpu") else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "non-finite values in the GPU result"
    max_abs = float(np.abs(g - r).max()) if g.size else 0.0
    nr = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r)) / nr if nr > 0 else float(np.linalg.norm(g - r))
    return max_abs, rel


def assert_close(name, gpu, ref, max_abs=TOL_MAX_ABS, rel_f=TOL_REL_F):
    m, r = metrics(gpu, ref)
    print(f"  {name}: max_abs={m:.3e} rel_F={r:.3e}", flush=True)
    assert m <= max_abs and r <= rel_f, f"{name}: max_abs {m:.3e} (tol {max_abs}), rel_F {r:.3e} (tol {rel_f})"
    return m, r
