"""Helpers shared by the GPU parity tests (tensor upload, tolerance checks)."""
from __future__ import annotations

import numpy as np
import torch

TOL = 1e-2  # max-abs error on unit-scale outputs (bf16 in, fp32 accumulate)


def dev(x: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """Upload host values (already bf16-representable for bf16) to cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def packed(c: np.ndarray, kr: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return dev(np.concatenate([c, kr], axis=-1), dtype)


def assert_close(got, ref, tol=TOL, what=""):
    """max|got-ref| <= tol and max|got-ref| / max|ref| <= tol."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 1.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol}"
    assert err <= tol * max(scale, 1e-30), f"{what}: error {err:.3e} vs output scale {scale:.3e}"
    return err, scale


def anchors_agree(gpu_anchor, ref_anchor, margin, min_margin=1e-3, min_sure_frac=0.5):
    """Anchors must match wherever the oracle's top-2 score margin exceeds
    min_margin. At least min_sure_frac of the groups must be that clear, so
    a margin that came out wrong (e.g. always tiny) cannot exempt them all."""
    gpu_anchor = np.asarray(gpu_anchor)
    ref_anchor = np.asarray(ref_anchor)
    sure = np.asarray(margin) > min_margin
    assert sure.shape == gpu_anchor.shape == ref_anchor.shape, "anchor arrays and margins must align"
    bad = np.flatnonzero((gpu_anchor != ref_anchor) & sure)
    assert bad.size == 0, f"{bad.size} anchors differ at margin > {min_margin}"
    n_sure = int(sure.sum())
    assert n_sure >= min_sure_frac * sure.size, \
        f"only {n_sure} of {sure.size} groups have a top-2 margin > {min_margin}"
    return n_sure


class AnchorTally:
    """Collects sampled groups one at a time and checks them together with
    anchors_agree (so the share of clear margins is judged over the sample)."""

    def __init__(self):
        self.got, self.ref, self.margin = [], [], []

    def add(self, gpu_anchor, ref_anchor, margin):
        self.got.append(np.ravel(gpu_anchor))
        self.ref.append(np.ravel(ref_anchor))
        self.margin.append(np.ravel(margin))

    def check(self, **kw):
        return anchors_agree(np.concatenate(self.got), np.concatenate(self.ref),
                             np.concatenate(self.margin), **kw)
