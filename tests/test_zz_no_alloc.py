"""The allocation-free draft head (nanospec_draft_logits_topk_noalloc) against
nanospec_draft_logits_topk on the same inputs, through the C ABI: two calls
in a row, the second with a smaller input (fewer rows, fewer hidden rows,
smaller k, another d), each bit-identical to the workspace call (the same
kernels in the same order) and within the draft-head tolerance of the
oracle.  A request above the fixed scratch is refused with NS_ESCRATCH."""
import numpy as np
import pytest
import torch

import oracle.nanospec_oracle as O
from dynamic_vocab_draft_amd import workloads as WL
from tests.gpu_common import check_logits, check_topk, dev_elems, dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ns():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocab_draft_amd import nanospec
    return nanospec


def _case(ns, V, d, n_max, n, M, k, seed):
    rng = np.random.default_rng(seed)
    W = WL.f32_to_bf16_bits((rng.standard_normal((V, d)) * 0.02).astype(np.float32))
    h = WL.f32_to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32))
    I = np.sort(rng.choice(V, size=n, replace=False)).astype(np.int64)
    ids = torch.full((n_max,), -1, dtype=torch.int32, device="cuda")
    ids[:n] = dev_i32(I)
    n_dev = torch.tensor([n], dtype=torch.int32, device="cuda")
    return W, h, I, dev_elems(W, "bf16"), dev_elems(h, "bf16"), ids, n_dev


def _head(ns, c, inputs, noalloc):
    W, h, I, W_dev, h_dev, ids, n_dev = inputs
    M, k, n_max = c["M"], c["k"], c["n_max"]
    logits = torch.full((M, n_max), float("nan"), device="cuda")
    tids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    tvals = torch.empty((M, k), dtype=torch.float32, device="cuda")
    if noalloc:
        ns.nanospec_draft_logits_topk_noalloc(W_dev, ns.NS_INDEXED, ids, n_dev, n_max, c["V"], c["d"], ns.NS_BF16,
                                              h_dev, M, k, logits, tids, tvals)
    else:
        ws = ns.alloc_workspace(n_max, M, k, c["d"])
        ns.nanospec_draft_logits_topk(W_dev, ns.NS_INDEXED, ids, n_dev, n_max, c["V"], c["d"], ns.NS_BF16, h_dev,
                                      M, k, logits, tids, tvals, ws)
    return logits, tids, tvals


def test_noalloc_matches_workspace_call(ns):
    cases = [dict(V=128256, d=4096, n_max=3072, n=1000, M=8, k=8, seed=71),
             dict(V=20000, d=1024, n_max=1024, n=300, M=4, k=4, seed=72)]
    inputs = [_case(ns, **c) for c in cases]
    # two allocation-free calls in a row (the second smaller, on the scratch
    # the first one left), then the workspace calls on the same inputs
    say("no-alloc draft head: two calls in a row")
    got = [_head(ns, c, x, True) for c, x in zip(cases, inputs)]
    want = [_head(ns, c, x, False) for c, x in zip(cases, inputs)]
    torch.cuda.synchronize()
    for c, x, (la, ia, va), (lb, ib, vb) in zip(cases, inputs, got, want):
        say(f"no-alloc draft head: {c}")
        W, h, I = x[0], x[1], x[2]
        n, k = c["n"], c["k"]
        la, ia, va = la.cpu().numpy(), ia.cpu().numpy(), va.cpu().numpy()
        lb, ib, vb = lb.cpu().numpy(), ib.cpu().numpy(), vb.cpu().numpy()
        assert np.array_equal(ia, ib) and np.array_equal(va.view(np.uint32), vb.view(np.uint32))
        assert np.array_equal(la[:, :n].view(np.uint32), lb[:, :n].view(np.uint32))
        assert np.isnan(la[:, n:]).all()
        ref, o_ids, o_vals = O.draft_head(h, W, I, k, "bf16")
        check_logits(la[:, :n], ref, "no-alloc")
        check_topk(ia, va, ref, I, o_ids, o_vals, k, "no-alloc")


def test_noalloc_refuses_oversize(ns):
    fake = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(ns.NanoSpecError) as e:
        ns.nanospec_draft_logits_topk_noalloc(fake, ns.NS_INDEXED, fake, fake, 16384, 151936, 4096, ns.NS_BF16,
                                              fake, 64, 16, None, fake, fake)
    assert e.value.code == ns.NS_ESCRATCH
