"""The no-allocation greedy entry point (tv_accept_greedy_noalloc) against
tv_accept_greedy: bit-identical outputs on calls in a row, the second with
a smaller input (the static scratch keeps the first call's contents). The
size limit of the scratch is checked on the host (tests/test_abi_host.py)."""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_config, make_custom

from gpu_util import check_greedy, upload
import tree_attention_draft_tv_amd as tv

pytestmark = pytest.mark.gpu


def _outputs(B, T):
    dev = torch.device("cuda:0")
    return (torch.full((B,), 7, dtype=torch.int32, device=dev),
            torch.full((B, T), 7, dtype=torch.int32, device=dev),
            torch.full((B,), 7, dtype=torch.int32, device=dev),
            torch.full((B, T), 7, dtype=torch.uint8, device=dev),
            torch.full((B,), 7, dtype=torch.int32, device=dev))


def _both(w):
    d = upload(w)
    ref = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"])
    got = tv.accept_greedy_noalloc(d["logits"], d["tokens"], d["parent"], d["n_nodes"],
                                   outputs=_outputs(w.B, w.T))
    torch.cuda.synchronize()
    ref = tuple(t.cpu().numpy() for t in ref)
    got = tuple(t.cpu().numpy() for t in got)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    check_greedy(got, oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes))
    return got


def test_noalloc_greedy_matches_workspace_call_twice():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    # First the headline workload (8 sequences, V = 152064: 10 slices per
    # row), then a smaller one (3 sequences, V = 40000, one padded): the
    # second call reads only partials its own argmax wrote.
    first = _both(make_config("C3"))
    assert (first[0] >= 4).sum() == 6
    w2 = make_custom(905, 3, 2, 1, 64, 40000, "bf16", [4, 4, 4], 20, plant_depth=4,
                     padded_rows=[1])
    second = _both(w2)
    assert second[0].tolist()[0] == 4 and second[0].tolist()[1] == 0
    # And once more with the large workload after the small one.
    _both(make_config("C2"))
