"""The backward pass on its own: every stage fed the oracle's quantities.

fa_bwd normally receives O and lse from the GPU forward, so a forward error
and a backward error could mask or mimic each other.  Here the backward gets
the oracle's O (rounded to the working dtype, as a caller would store it) and
the oracle's lse, and the dK/dV and dQ stages get delta computed in fp64 from
the oracle's O, so each stage is compared with the oracle's gradients with
nothing of the GPU forward in its inputs; fa_bwd_dq_delta (dQ forming delta
itself) gets the oracle's O and lse.  delta_i = dO_i . O_i equals the
definition sum_j P_ij dP_ij because O_i = sum_j P_ij V_j (bornlex "Flash
Attention", "Standard Attention", with dP = dO V^T by the chain rule).
"""
import numpy as np
import pytest

from oracle import attention

from gpu_cases import compare_grad, host, say, to_dev
from test_parity import small_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


CASES = [
    # B, H, N, d, dtype, causal, kv, mask
    (1, 2, 128, 64, "f32", False, None, None),
    (1, 2, 200, 128, "f32", True, "rand", None),
    (2, 2, 63, 64, "bf16", True, None, None),
    (2, 2, 129, 128, "bf16", False, "rand", None),
    (1, 2, 300, 96, "bf16", True, None, "band"),
    (1, 2, 1000, 64, "bf16", True, "rand", None),
    (1, 1, 700, 256, "bf16", False, None, "bern"),
    (3, 1, 256, 160, "bf16", True, [0, 100, 256], None),
]


def _ids(c):
    return "B{}H{}N{}d{}{}{}{}{}".format(c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", "k" if c[6] else "",
                                         "m" if c[7] else "")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_from_oracle_forward(case):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, N, d, dt, causal, kv, mask = case
    inp = small_inputs(B, H, N, d, dt, causal, kv, mask, seed=31 + N + d)
    say(f"bwd isolation {case}")
    kw = dict(causal=causal, block_mask=inp["block_mask"], kv_len=inp["kv_len"])
    O, lse = attention.forward(inp["q"], inp["k"], inp["v"], inp["scale"], **kw)
    g_ref = attention.backward(inp["q"], inp["k"], inp["v"], inp["do"], inp["scale"], **kw)
    delta = (inp["do"].astype(np.float64) * O).sum(axis=-1)

    q, k, v, do, o = (to_dev(x, dt) for x in (inp["q"], inp["k"], inp["v"], inp["do"], O))
    tl = torch.from_numpy(lse.astype(np.float32)).cuda()
    td = torch.from_numpy(delta.astype(np.float32)).cuda()
    bm = None if inp["block_mask"] is None else torch.from_numpy(inp["block_mask"]).cuda()
    kl = None if inp["kv_len"] is None else torch.from_numpy(inp["kv_len"].astype(np.int32)).cuda()
    gkw = dict(scale=inp["scale"], causal=causal, block_mask=bm, kv_len=kl)
    zs = float(np.abs(inp["do"]).max() * np.abs(inp["v"]).max() * inp["scale"]
               * max(np.abs(inp["k"]).max(), np.abs(inp["q"]).max(), 1.0))

    # the whole backward on the oracle's O and lse
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, tl, **gkw)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        compare_grad(host(a), r, dt, f"fa_bwd {name}", zero_scale=zs)

    # the two matrix stages on the oracle's delta
    dk2, dv2 = fa.fa_bwd_dkdv(q, k, v, do, tl, td, **gkw)
    dq2 = fa.fa_bwd_dq(q, k, v, do, tl, td, **gkw)
    for name, a, r in zip(("dq", "dk", "dv"), (dq2, dk2, dv2), g_ref):
        compare_grad(host(a), r, dt, f"stage {name}", zero_scale=zs)

    # the preprocess: delta = rowsum(dO * O) of the tensors it was given, in
    # fp32 accumulation (error within d * 2^-24 * sum |dO O| per row)
    got = fa.fa_bwd_preprocess(o, do).cpu().numpy().astype(np.float64)
    do_h, o_h = host(do), host(o)
    want = (do_h * o_h).sum(axis=-1)
    bound = d * 2.0 ** -24 * np.abs(do_h * o_h).sum(axis=-1) + 1e-30
    err = np.abs(got - want)
    say(f"  delta max err {err.max():.3e} (max bound {bound.max():.3e})")
    assert np.all(err <= bound)

    # dQ forming delta itself from the oracle's O: the same bound on delta,
    # and dQ against the oracle's gradient
    dq3, delta3 = fa.fa_bwd_dq_delta(q, k, v, o, do, tl, **gkw)
    compare_grad(host(dq3), g_ref[0], dt, "dq_delta dq", zero_scale=zs)
    err = np.abs(delta3.cpu().numpy().astype(np.float64) - want)
    say(f"  dq_delta delta max err {err.max():.3e}")
    assert np.all(err <= bound)
