"""The verifiers on the GPU, through the C ABI, against the oracle
(TensorRT Edge-LLM "DSpark kernels" page: `dsparkGreedyAccept`,
`dsparkProbabilisticAccept`).

Greedy acceptance is integer work and must match bit for bit. The
probabilistic verifier's accept decisions are exact (binary64 products);
its sampled token must match wherever the oracle's CDF margin exceeds what
a different summation order can move (every row here, in practice; the
count is reported).
"""

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import markov_draft_sampling_step_amd as m  # noqa: E402
from markov_draft_sampling_step_amd import workloads  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()
    return torch.device("cuda:0")


def run_greedy(w, dev, draft=None, ws=None):
    draft = w.draft_greedy if draft is None else draft
    lg = torch.from_numpy(w.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    acc = torch.full((w.B, w.P + 1), -7, dtype=torch.int64, device=dev)
    n = torch.zeros(w.B, dtype=torch.int32, device=dev)
    ws = m.new_verify_workspace(w.B, w.P, device=dev) if ws is None else ws
    m.greedy_accept(lg, torch.from_numpy(np.ascontiguousarray(draft)).to(dev),
                    torch.from_numpy(w.lengths).to(dev), acc, n, ws)
    torch.cuda.synchronize()
    assert not ws.cpu().numpy().any(), "workspace left dirty"
    return acc.cpu().numpy(), n.cpu().numpy()


def run_prob(w, dev, ws=None):
    t = torch.from_numpy(w.target).to(dev)
    q = torch.from_numpy(w.draftp).to(dev)
    acc = torch.full((w.B, w.P + 1), -7, dtype=torch.int64, device=dev)
    n = torch.zeros(w.B, dtype=torch.int32, device=dev)
    ws = m.new_verify_workspace(w.B, w.P, device=dev) if ws is None else ws
    m.prob_accept(t, q, torch.from_numpy(w.draft_sampled).to(dev), torch.from_numpy(w.lengths).to(dev),
                  torch.from_numpy(w.uniforms).to(dev), acc, n, ws)
    torch.cuda.synchronize()
    assert not ws.cpu().numpy().any(), "workspace left dirty"
    return acc.cpu().numpy(), n.cpu().numpy()


def check_greedy(w, dev):
    import oracle

    acc, n = run_greedy(w, dev)
    acc_o, n_o = oracle.greedy_accept(w.logits, w.draft_greedy, w.lengths)
    assert np.array_equal(n, n_o) and np.array_equal(acc, acc_o)
    say(f"  greedy {w.name}: accepted lengths {np.bincount(n, minlength=w.P + 2).tolist()}")


def check_prob(w, dev):
    import oracle

    acc, n = run_prob(w, dev)
    acc_o, n_o, margin, mass = oracle.prob_accept(w.target, w.draftp, w.draft_sampled, w.lengths,
                                                  w.uniforms)
    assert np.array_equal(n, n_o), np.argwhere(n != n_o)[:5]
    decided = margin > (w.V + 2) * 2.0 ** -52 * mass
    for b in range(w.B):
        k = n[b] - 1
        assert np.array_equal(acc[b, :k], acc_o[b, :k]) and (acc[b, k + 1:] == -1).all()
        if decided[b]:
            assert acc[b, k] == acc_o[b, k], (b, acc[b, k], acc_o[b, k])
        else:
            assert 0 <= acc[b, k] < w.V
    say(f"  prob {w.name}: lengths {np.bincount(n, minlength=w.P + 2).tolist()}, "
        f"decided {int(decided.sum())}/{w.B}")


# (the last case's probabilistic chunks hold more than 32 weights per thread,
# so its finisher walks its run from memory instead of from LDS)
@pytest.mark.parametrize("B,P,V,seed", [(16, 5, 4096, 81), (7, 3, 40960, 82), (33, 1, 16384, 83),
                                        (5, 0, 2048, 84), (4, 2, 300000, 87)])
def test_verifiers_small(dev, B, P, V, seed):
    w = workloads.make_verify(B=B, P=P, V=V, data_seed=seed, name=f"v{seed}")
    check_greedy(w, dev)
    check_prob(w, dev)


def test_verifiers_full_size(dev):
    """64 rows, 5 proposals, V = 163840 (the large drafting workload's shape)."""
    w = workloads.make_verify()
    check_greedy(w, dev)
    check_prob(w, dev)


def test_greedy_edge_cases(dev):
    """Ties (lowest id), NaN logits (first NaN), lengths 0 and above P,
    invalid draft ids, a draft stride above P, and a reused workspace."""
    import oracle

    w = workloads.make_verify(B=6, P=3, V=2048, data_seed=85, name="edges")
    w.logits[0, 0, [100, 50]] = workloads.to_bf16_bits(np.float32([40.0, 40.0]))
    w.logits[1, 1, [7, 9]] = workloads.BF16_NAN
    w.lengths[:] = [3, 3, 0, 9, -2, 3]
    wide = np.full((w.B, 5), -1, dtype=np.int64)
    wide[:, :3] = w.draft_greedy
    wide[0, 0] = 50
    wide[1, :2] = [int(np.argmax(workloads.bf16_bits_to_f32(w.logits[1, 0]))), 7]
    wide[5, 1] = 99999
    ws = m.new_verify_workspace(w.B, w.P, device=dev)
    for _ in range(2):
        acc, n = run_greedy(w, dev, draft=wide, ws=ws)
        acc_o, n_o = oracle.greedy_accept(w.logits, wide, w.lengths)
        assert np.array_equal(n, n_o) and np.array_equal(acc, acc_o)
    assert acc[0, 0] == 50


def test_prob_edge_cases(dev):
    """No residual mass (p == q and a p = 0 draft), an out-of-range draft id,
    zero uniforms and short proposals."""
    import oracle

    B, P, V = 4, 2, 64
    rng = np.random.default_rng(86)
    t = rng.dirichlet(np.ones(V), size=(B, P + 1)).astype(np.float32)
    t[:, :, 10] = 0.0
    q = t[:, :P].copy()
    q[2:] = rng.dirichlet(np.ones(V), size=(2, P)).astype(np.float32)
    draft = np.array([[10, 3], [-4, 3], [5, 6], [7, 8]], dtype=np.int64)
    u = rng.random((B, 2 * P + 1)).astype(np.float32)
    u[3] = 0.0
    lengths = np.array([2, 2, 1, 2], dtype=np.int32)
    w = workloads.VerifyWorkload(name="pedges", B=B, P=P, V=V, logits=None, target=t, draftp=q,
                                 draft_greedy=None, draft_sampled=draft, lengths=lengths, uniforms=u)
    check_prob(w, dev)
