"""GPU parity of stage 2, the log-sum-exp merge, on its own against the
oracle's merge, on synthetic split partials that stage 1 would not produce
at these sizes: finite log-sum-exps in every slot up to 256 splits (the
kernel reads slot s from lane s % 64 of its register s / 64, and prefetches
the first 16 rows), the largest one past slot 64, empty splits (lse -inf,
zero rows, as stage 1 writes them), rows with every split empty, per-request
split counts, head dims 64 and 128, fp32 and bf16 outputs."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log


def _partials(B, qn, Hq, S, D, seed):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((B, qn, Hq, S, D)).astype(np.float32)
    lse = (rng.standard_normal((B, qn, Hq, S)) * 4).astype(np.float32)
    lse[rng.random(lse.shape) < 0.2] = -np.inf
    if S > 64:  # some rows peak in a late slot
        lse[:, :, ::3, S - 1 - (S % 7)] = 30.0
    lse[0, 0, 0, :] = -np.inf  # a row with every split empty
    o[np.isneginf(lse)] = 0.0
    return o, lse


def _check(out, lse, out_ref, lse_ref, label, tol=1e-5):
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{label}: -inf pattern"
    fin = ~np.isneginf(lse_ref)
    dl = float(np.max(np.abs(lse[fin] - lse_ref[fin]) / (1 + np.abs(lse_ref[fin])))) if fin.any() else 0.0
    do = float(np.max(np.abs(out - out_ref) / (1 + np.abs(out_ref))))
    log(f"  {label}: max rel |d out| = {do:.2e}, |d lse| = {dl:.2e}")
    assert do <= tol and dl <= tol, label


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 16, 17, 64, 65, 130, 256])
def test_merge_matches_oracle_fp32(gpu, S, D):
    o, lse = _partials(3, 2, 8, S, D, seed=1000 + S + D)
    out, l_out = gpu.decode_attn_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(),
                                       out_dtype=torch.float32, want_lse=True)
    out_ref, lse_ref = OA.merge(o.astype(np.float64), lse.astype(np.float64))
    _check(U.to_np(out), U.to_np(l_out), out_ref, lse_ref, f"merge S={S} D={D}")


@pytest.mark.parametrize("S", [40, 256])
def test_merge_split_counts(gpu, S):
    """Request b merges only its first counts[b] slots; the others may hold anything."""
    B = 5
    o, lse = _partials(B, 1, 8, S, 128, seed=77 + S)
    rng = np.random.default_rng(5 + S)
    counts = rng.integers(1, S + 1, size=B).astype(np.int32)
    counts[0], counts[1] = 1, S
    o_dev, l_dev = torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda()
    for b, c in enumerate(counts):  # unread slots: garbage
        o_dev[b, :, :, c:] = float("nan")
        l_dev[b, :, :, c:] = float("nan")
    out, l_out = gpu.decode_attn_merge(o_dev, l_dev, out_dtype=torch.float32, want_lse=True,
                                       split_counts=torch.from_numpy(counts).cuda())
    out_ref, lse_ref = OA.merge(o.astype(np.float64), lse.astype(np.float64), split_counts=counts)
    _check(U.to_np(out), U.to_np(l_out), out_ref, lse_ref, f"merge counts S={S} {counts.tolist()}")


def test_merge_bf16_output(gpu):
    o, lse = _partials(3, 2, 8, 200, 128, seed=3)
    out = gpu.decode_attn_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(),
                                out_dtype=torch.bfloat16)
    out_ref, _ = OA.merge(o.astype(np.float64), lse.astype(np.float64))
    U.check_bf16(U.to_np(out), out_ref, "merge S=200 bf16 out")
