"""Pins of the main-branch backward oracle against independent formulations: autograd of a
dense masked attention, torch's scaled_dot_product_attention in the dense special case, and
finite differences."""
import numpy as np
import pytest
import torch

from oracle import msa_backward as B
from oracle.msa_ref import _key_set, query_positions


def _masked_dense(q, k, v, sel, scale, causal):
    """Autograd reference: dense attention with every key outside the query's selected
    blocks masked out; GQA by repeating K / V over the group's heads."""
    n_q, hq, d = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    mask = np.zeros((hq, n_q, n_k), dtype=bool)
    for i in range(n_q):
        for g in range(hkv):
            keys = _key_set(sel[i, g], n_k, 128, int(pos[i]), causal)
            mask[g * grp:(g + 1) * grp, i, keys] = True
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kh = tk.repeat_interleave(grp, dim=1).permute(1, 0, 2)          # [Hq, Nk, D]
    vh = tv.repeat_interleave(grp, dim=1).permute(1, 0, 2)
    s = scale * torch.matmul(tq.permute(1, 0, 2), kh.transpose(1, 2))   # [Hq, N, Nk]
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vh).permute(1, 0, 2)
    return tq, tk, tv, o


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_autograd_of_masked_dense_attention(causal):
    rng = np.random.default_rng(1 + causal)
    n_q, n_k, hq, hkv, d, kk = 300, 700 if not causal else 300, 8, 2, 16, 4
    q = rng.standard_normal((n_q, hq, d))
    k = rng.standard_normal((n_k, hkv, d))
    v = rng.standard_normal((n_k, hkv, d))
    do = rng.standard_normal((n_q, hq, d))
    nb = -(-n_k // 128)
    pos = query_positions(n_q, n_k)
    sel = rng.integers(0, nb, size=(n_q, hkv, kk))
    sel[:, :, 0] = np.minimum(pos // 128, nb - 1)[:, None]     # every row sees a key
    sel[::7, :, 2] = sel[::7, :, 1]                            # repeated
    sel[::5, :, 3] = -1                                        # empty slot
    sel[::11, 0, 1] = 10_000                                   # out of range
    scale = 0.3
    dq, dk, dv, o, lse = B.sparse_attention_backward(q, k, v, sel, do, scale, 128, causal)
    tq, tk, tv, to = _masked_dense(q, k, v, sel, scale, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-10, atol=1e-12)
    (to * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_dense_case_matches_sdpa():
    """Every block selected, non-causal: the gradients of torch's scaled_dot_product_attention."""
    rng = np.random.default_rng(7)
    n_q, n_k, hq, hkv, d = 200, 384, 4, 1, 32
    q = rng.standard_normal((n_q, hq, d))
    k = rng.standard_normal((n_k, hkv, d))
    v = rng.standard_normal((n_k, hkv, d))
    do = rng.standard_normal((n_q, hq, d))
    sel = np.tile(np.arange(3), (n_q, hkv, 1))
    dq, dk, dv, _, _ = B.sparse_attention_backward(q, k, v, sel, do, 1 / np.sqrt(d), 128, False)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2)[None], tk.repeat_interleave(hq, 1).permute(1, 0, 2)[None],
        tv.repeat_interleave(hq, 1).permute(1, 0, 2)[None])
    (o[0].permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_finite_differences():
    """Central differences of L = sum(O * dO) along random directions of Q, K and V."""
    rng = np.random.default_rng(3)
    n_q, n_k, hq, hkv, d = 140, 260, 4, 2, 8
    q, do = rng.standard_normal((n_q, hq, d)), rng.standard_normal((n_q, hq, d))
    k, v = rng.standard_normal((n_k, hkv, d)), rng.standard_normal((n_k, hkv, d))
    nb = -(-n_k // 128)
    sel = rng.integers(0, nb, size=(n_q, hkv, 2))
    sel[:, :, 0] = (query_positions(n_q, n_k) // 128)[:, None]
    dq, dk, dv, _, _ = B.sparse_attention_backward(q, k, v, sel, do, 0.5, 128, True)

    def loss(qq, kk_, vv):
        o = B.sparse_attention_backward(qq, kk_, vv, sel, do, 0.5, 128, True)[3]
        return float(np.sum(o * do))
    eps = 1e-6
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        e = rng.standard_normal(grad.shape)
        args = {"q": q, "k": k, "v": v}
        plus = dict(args); plus[which] = args[which] + eps * e
        minus = dict(args); minus[which] = args[which] - eps * e
        fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * eps)
        assert abs(fd - float(np.sum(grad * e))) <= 1e-6 * max(1.0, abs(fd))


def test_row_gradient_matches_the_whole_sequence_backward():
    """dQ of sampled rows alone (used at full size) equals the whole-sequence backward's."""
    from oracle import msa_case
    from oracle.msa_backward import query_rows_gradient, sparse_attention_backward
    from synth import msa_inputs as mi
    from synth.msa_inputs import widen
    cfg = mi.custom("rows", n_q=(300,), n_k=(700,), hq=8, hkv=2, topk=4)
    case = mi.make_case(cfg, seed=3)
    do = widen(mi.grad_output(case))
    q, k, v = widen(case.q), widen(case.k), widen(case.v)
    lists = msa_case.run(case, want_output=False).topk_idx
    dq = sparse_attention_backward(q, k, v, lists, do, case.softmax_scale, 128, True)[0]
    rows = np.array([0, 5, 150, 299])
    got = query_rows_gradient(q, k, v, lists[rows], do[rows], rows, case.softmax_scale, 128, True)
    assert np.array_equal(got, dq[rows])


def test_key_block_gradient_matches_the_whole_sequence_backward():
    """dK, dV of one (group, block) column alone (used at full size) equal the whole-sequence
    backward's rows for those keys: every column of a ragged causal case, G = 4."""
    from oracle import msa_case
    from oracle.msa_backward import key_block_gradient, sparse_attention_backward
    from synth import msa_inputs as mi
    from synth.msa_inputs import widen
    cfg = mi.custom("cols", n_q=(300,), n_k=(700,), hq=8, hkv=2, topk=3)
    case = mi.make_case(cfg, seed=5)
    do = widen(mi.grad_output(case))
    q, k, v = widen(case.q), widen(case.k), widen(case.v)
    lists = msa_case.run(case, want_output=False).topk_idx
    _, dk, dv, _, _ = sparse_attention_backward(q, k, v, lists, do, case.softmax_scale, 128, True)
    for g in range(2):
        for b in range(6):
            gk, gv = key_block_gradient(q, k, v, lists, do, g, b, case.softmax_scale, 128, True)
            lo, hi = 128 * b, min(128 * b + 128, 700)
            np.testing.assert_allclose(gk, dk[lo:hi, g], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(gv, dv[lo:hi, g], rtol=1e-12, atol=1e-14)
    # the compared values are far from zero, so the comparison is not vacuous
    assert np.abs(dv[:128, 0]).max() > 1e-3
