"""Helpers for the GPU parity tests: run the library, compare with the oracle."""

import sys

import numpy as np

import oracle


def announce(msg: str) -> None:
    """Name the case on the real stderr before any GPU work, flushed."""
    print(f"[gpu-case] {msg}", file=sys.__stderr__, flush=True)


def dev_tensor(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def run_forward(h, x, mode, device="cuda"):
    """pi_ffn_forward on x [B][d]; returns (idx, count, y) on the host."""
    import torch
    n = h.desc.d_ffn
    xt = dev_tensor(x, device)
    y = torch.full_like(xt, float("nan"))
    idx = torch.full((n,), -7, dtype=torch.int32, device=device)
    count = torch.full((1,), -7, dtype=torch.int32, device=device)
    h.forward(xt, y, mode, idx, count)
    torch.cuda.synchronize()
    c = int(count.item())
    return idx[:max(c, 0)].cpu().numpy(), c, y.cpu().numpy()


def run_predict(h, x, device="cuda"):
    """pi_ffn_predict with logits; returns (idx, count, z)."""
    import torch
    n = h.desc.d_ffn
    xt = dev_tensor(x, device)
    idx = torch.full((n,), -7, dtype=torch.int32, device=device)
    count = torch.full((1,), -7, dtype=torch.int32, device=device)
    z = torch.full((x.shape[0], n), float("nan"), dtype=torch.float32, device=device)
    h.predict(xt, idx, count, z)
    torch.cuda.synchronize()
    c = int(count.item())
    return idx[:max(c, 0)].cpu().numpy(), c, z.cpu().numpy()


def run_masked(h, x, sel, device="cuda"):
    import torch
    xt = dev_tensor(x, device)
    y = torch.full_like(xt, float("nan"))
    idx = dev_tensor(np.asarray(sel, dtype=np.int32), device) if len(sel) else torch.zeros(1, dtype=torch.int32,
                                                                                              device=device)
    count = torch.tensor([len(sel)], dtype=torch.int32, device=device)
    h.forward_masked(xt, idx, count, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def rel_l2_rows(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    out = []
    for g, r in zip(got, ref):
        nr = np.linalg.norm(r)
        out.append(np.linalg.norm(g - r) / nr if nr > 0 else (0.0 if np.all(g == 0) else np.inf))
    return np.array(out)


def tol_for(act_dtype: str) -> float:
    return 1e-5 if act_dtype == "f32" else 1e-3


def check_idx_valid(idx, count, n):
    assert count >= 0 and count == len(idx)
    assert np.all(np.diff(idx) > 0), "index list not strictly ascending"
    assert count == 0 or (idx[0] >= 0 and idx[-1] < n)


def check_decisions(idx, n, values, band, threshold):
    """GPU selection agrees with the oracle wherever the oracle is certain; returns #ambiguous."""
    sel = np.zeros(n, dtype=bool)
    sel[idx] = True
    on, off = oracle.certain_union(values, band, threshold)
    missing = np.flatnonzero(on & ~sel)
    extra = np.flatnonzero(off & sel)
    assert missing.size == 0, f"certainly-selected neurons missing: {missing[:10]}"
    assert extra.size == 0, f"certainly-unselected neurons present: {extra[:10]}"
    return int(n - on.sum() - off.sum())
