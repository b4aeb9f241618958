"""Shared test helpers: host <-> device marshalling and the parity bar."""
import numpy as np
import torch


def bf(a_u16, dev="cuda"):
    """numpy uint16 bf16 bits -> device bf16 tensor"""
    return torch.from_numpy(np.ascontiguousarray(a_u16).astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def words(a_u32, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a_u32).astype(np.uint32).view(np.int32)).to(dev)


def i32(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(dev)


def host_bf(t):
    """device bf16 tensor -> numpy uint16 bits"""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_i32(t):
    return t.detach().cpu().numpy().astype(np.int64)


def triple(m, dev="cuda"):
    return (words(m[0], dev), bf(m[1], dev), bf(m[2], dev))


def bf_to_f64(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_parity(got_u16, want_u16, tol=1e-2, name=""):
    """|gpu - oracle| <= tol * max|oracle| over the whole tensor (no floor)."""
    g = bf_to_f64(got_u16)
    w = bf_to_f64(want_u16)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite output"
    scale = np.abs(w).max() if w.size else 0.0
    err = np.abs(g - w).max() if w.size else 0.0
    assert err <= tol * scale, f"{name}: max err {err:.4g} > {tol} * {scale:.4g}"
    return err / scale if scale > 0 else 0.0
