"""qg_kv_weighted_noalloc (the weighted sum over the library's fixed per-device workspace, for
callers that cannot allocate) against qg_kv_weighted_with_workspace, bit for bit, on two calls
in a row: the decode shape (32 heads, 8 KV heads, 4096 positions, head size 128), then a smaller
one (8 heads, 2 KV heads, 1000 positions, head size 64), whose result must not carry anything
of the first call's pieces.  Also the oracle on the smaller case ("Module numerics", Functions
weighted_int8), and the refusal of a shape whose pieces exceed the fixed workspace."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import block_format_gemv_amd as q
    oracle.set_threads(8)
    return q


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32).reshape(-1)


def cache(nkv, npos, hd, seed):
    vs, vc = oracle.kv_cache_rows(gen.kv_rows(nkv * npos, hd, seed))
    return vs.reshape(nkv, npos).copy(), vc.reshape(nkv, npos, hd)


def both(qg, nh, nkv, npos, hd, seed):
    vs, vc = cache(nkv, npos, hd, seed)
    probs = gen.attn_weights(nh, npos, seed + 1)
    args = (dev(probs), dev(vs.view(np.int16)), dev(vc))
    ws = torch.empty(qg.qg_kv_weighted_workspace(nh, npos, hd), dtype=torch.uint8, device=DEV)
    want = torch.full((nh, hd), 7.0, dtype=torch.float32, device=DEV)
    got = torch.full((nh, hd), 7.0, dtype=torch.float32, device=DEV)
    qg.qg_kv_weighted_with_workspace(nh, nkv, npos, hd, *args, want, ws)
    qg.qg_kv_weighted_noalloc(nh, nkv, npos, hd, *args, got)
    torch.cuda.synchronize()
    return probs, vs, vc, bits(got), bits(want)


def test_noalloc_matches_the_workspace_entry_on_two_calls(qg):
    say("noalloc call 1: nh=32 nkv=8 npos=4096 hd=128")
    _, _, _, got, want = both(qg, 32, 8, 4096, 128, 4100)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, f"call 1: {len(bad)} mismatches, first at {bad[0]}"
    say("noalloc call 2: nh=8 nkv=2 npos=1000 hd=64")
    probs, vs, vc, got, want = both(qg, 8, 2, 1000, 64, 4200)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, f"call 2: {len(bad)} mismatches, first at {bad[0]}"
    ref = oracle.kv_weighted(probs, vs, vc).view(np.uint32).reshape(-1)
    assert np.array_equal(got, ref), "call 2 against the oracle"


def test_noalloc_refuses_pieces_beyond_the_fixed_workspace(qg):
    nh, nkv, npos, hd = 64, 8, 8192, 128                  # 8 MiB of pieces
    assert qg.qg_kv_weighted_workspace(nh, npos, hd) > qg.KV_NOALLOC_BYTES
    out = torch.full((nh, hd), 7.0, dtype=torch.float32, device=DEV)
    probs = torch.zeros((nh, npos), dtype=torch.float32, device=DEV)
    vs = torch.zeros((nkv, npos), dtype=torch.int16, device=DEV)
    vc = torch.zeros((nkv, npos, hd), dtype=torch.int8, device=DEV)
    with pytest.raises(qg.QGError) as ei:
        qg.qg_kv_weighted_noalloc(nh, nkv, npos, hd, probs, vs, vc, out)
    assert ei.value.status == qg.E_SHAPE and "fixed workspace" in ei.value.reason
    torch.cuda.synchronize()
    assert (out == 7.0).all()
