"""The allocation-free cross-entropy forward (coda_linear_cross_entropy_fwd_noalloc)
against the workspace entry point it mirrors, through the C ABI: two calls in
a row, the second on a smaller input (the library's scratch keeps the first
call's contents), each compared with the workspace entry point on the same
inputs; and the refusal of a shape whose partials exceed the scratch."""
import numpy as np
import pytest

import coda_inputs as ci
from tests.helpers import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogue_fp8_amd as coda  # noqa: E402

DEV = "cuda"
BF = torch.bfloat16


def _outputs(M):
    f = lambda n: torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    i = lambda: torch.full((1,), -7, dtype=torch.int32, device=DEV)
    return dict(loss=f(1), lse=f(M), per_row=f(M), n_valid=i(), n_bad=i())


def _case(M, D, V, seed):
    rng = np.random.default_rng(seed)
    h = ci.to_bf16_values(rng.standard_normal((M, D)).astype(np.float32))
    W = ci.to_bf16_values((rng.standard_normal((D, V)) * D ** -0.5).astype(np.float32))
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[rng.choice(M, M // 20, replace=False)] = -100
    labels[[1, M - 2]] = [V, -5]                      # out of range: counted in n_bad
    return to_dev(h, BF), to_dev(W, BF), to_dev(labels)


def _run(fn, h, W, lab):
    o = _outputs(h.shape[0])
    fn(h, W, lab, o["loss"], o["lse"], o["n_valid"], per_row=o["per_row"], n_bad=o["n_bad"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def test_noalloc_matches_workspace_entry_point_twice():
    """Bitwise the workspace entry point's results (same kernels, same fixed
    reduction order), first on 1000 tokens x 2000 classes, then on 300 x 784:
    the second call reads none of the first call's leftovers."""
    for M, D, V, seed in ((1000, 256, 2000, 1), (300, 128, 784, 2)):
        h, W, lab = _case(M, D, V, seed)
        got = _run(coda.linear_cross_entropy_fwd_noalloc, h, W, lab)
        ref = _run(coda.linear_cross_entropy_fwd, h, W, lab)
        for k in ref:
            assert np.array_equal(got[k], ref[k], equal_nan=True), (M, k)
        assert got["n_bad"][0] == 2 and got["n_valid"][0] == M - M // 20 - 2
        assert np.isfinite(got["loss"][0])


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """2 ceil(V / 256) M + 3 M floats above the scratch size: CODA_ERR_WORKSPACE
    before any launch; the outputs stay untouched."""
    M, D, V = 16384, 8, 128256
    h = torch.zeros((M, D), dtype=BF, device=DEV)
    W = torch.zeros((D, V), dtype=BF, device=DEV)
    lab = torch.zeros(M, dtype=torch.int32, device=DEV)
    o = _outputs(M)
    with pytest.raises(coda.CodaError, match="CODA_ERR_WORKSPACE"):
        coda.linear_cross_entropy_fwd_noalloc(h, W, lab, o["loss"], o["lse"], o["n_valid"])
    torch.cuda.synchronize()
    assert np.isnan(o["loss"].item()) and o["n_valid"].item() == -7
