"""Pins of the proxy-backward oracle: autograd of the KL objective written densely with masks
(torch, float64), finite differences of the oracle's own loss, and the special case where the
proxy distribution equals the main one (zero gradient, zero loss)."""
import numpy as np
import pytest
import torch

from oracle import msa_proxy_backward as PB
from oracle.msa_ref import _key_set, query_positions


def _lists(rng, n_q, n_k, hkv, kk, causal):
    pos = query_positions(n_q, n_k)
    nb = -(-n_k // 128)
    sel = np.full((n_q, hkv, kk), -1, dtype=np.int32)
    for i in range(n_q):
        top = int(pos[i]) // 128 if causal else nb - 1
        for g in range(hkv):
            c = rng.permutation(top + 1)[:kk]
            sel[i, g, :c.size] = c
    return sel


def _dense_kl(q, k, qi, ki, sel, scale, pscale, causal):
    n_q, hq, _ = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    mask = np.zeros((hkv, n_q, n_k), dtype=bool)
    for i in range(n_q):
        for g in range(hkv):
            mask[g, i, _key_set(sel[i, g], n_k, 128, int(pos[i]), causal)] = True
    m = torch.from_numpy(mask)
    tq, tk = torch.tensor(q), torch.tensor(k)
    tqi = torch.tensor(qi, requires_grad=True)
    tki = torch.tensor(ki, requires_grad=True)
    kh = tk.repeat_interleave(grp, dim=1).permute(1, 0, 2)
    s = scale * torch.matmul(tq.permute(1, 0, 2), kh.transpose(1, 2))        # [Hq, N, Nk]
    s = s.masked_fill(~m.repeat_interleave(grp, dim=0), float("-inf"))
    t = torch.softmax(s, dim=-1).reshape(hkv, grp, n_q, n_k).mean(dim=1)     # [Hkv, N, Nk]
    z = pscale * torch.matmul(tqi.permute(1, 0, 2), tki.permute(1, 2, 0))     # [Hkv, N, Nk]
    logp = torch.log_softmax(z.masked_fill(~m, float("-inf")), dim=-1)
    kl = torch.where(m & (t > 0), t * (torch.log(t.clamp_min(1e-300)) - logp),
                     torch.zeros_like(t)).sum()
    kl.backward()
    return tqi.grad.numpy(), tki.grad.numpy(), float(kl.detach())


@pytest.mark.parametrize("causal", [True, False])
def test_proxy_gradients_match_autograd_of_the_kl_objective(causal):
    rng = np.random.default_rng(7 + causal)
    n_q, n_k, hq, hkv, d, dp, kk = 200, 200 if causal else 520, 8, 2, 16, 8, 3
    q = rng.standard_normal((n_q, hq, d))
    k = rng.standard_normal((n_k, hkv, d))
    qi = rng.standard_normal((n_q, hkv, dp))
    ki = rng.standard_normal((n_k, hkv, dp))
    sel = _lists(rng, n_q, n_k, hkv, kk, causal)
    dq, dk, loss, _ = PB.proxy_backward(q, k, qi, ki, sel, 0.25, 0.35, 128, causal)
    wq, wk, wl = _dense_kl(q, k, qi, ki, sel, 0.25, 0.35, causal)
    assert abs(loss - wl) <= 1e-10 * max(1.0, abs(wl))
    np.testing.assert_allclose(dq, wq, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dk, wk, rtol=1e-9, atol=1e-12)


def test_proxy_gradients_match_finite_differences():
    rng = np.random.default_rng(3)
    n_q, n_k, hq, hkv, d, dp = 6, 300, 4, 1, 8, 4
    q, k = rng.standard_normal((n_q, hq, d)), rng.standard_normal((n_k, hkv, d))
    qi, ki = rng.standard_normal((n_q, hkv, dp)), rng.standard_normal((n_k, hkv, dp))
    sel = _lists(rng, n_q, n_k, hkv, 2, True)
    dq, dk, _, _ = PB.proxy_backward(q, k, qi, ki, sel, 0.3, 0.5, 128, True)
    h = 1e-6
    for (i, g, c) in [(0, 0, 1), (5, 0, 3)]:
        a, b = qi.copy(), qi.copy()
        a[i, g, c] += h
        b[i, g, c] -= h
        num = (PB.proxy_backward(q, k, a, ki, sel, 0.3, 0.5, 128, True)[2]
               - PB.proxy_backward(q, k, b, ki, sel, 0.3, 0.5, 128, True)[2]) / (2 * h)
        assert abs(num - dq[i, g, c]) <= 1e-6 * max(1.0, abs(num))
    u = int(np.argmax(np.abs(dk[:, 0, 0])))
    a, b = ki.copy(), ki.copy()
    a[u, 0, 0] += h
    b[u, 0, 0] -= h
    num = (PB.proxy_backward(q, k, qi, a, sel, 0.3, 0.5, 128, True)[2]
           - PB.proxy_backward(q, k, qi, b, sel, 0.3, 0.5, 128, True)[2]) / (2 * h)
    assert abs(num - dk[u, 0, 0]) <= 1e-6 * max(1.0, abs(num))


def test_proxy_equal_to_the_main_attention_has_zero_loss_and_gradient():
    """G = 1 and proxies equal to Q, K with the same scale: the proxy softmax is the main one."""
    rng = np.random.default_rng(5)
    n_q, n_k, h, d = 40, 300, 2, 8
    q, k = rng.standard_normal((n_q, h, d)), rng.standard_normal((n_k, h, d))
    sel = _lists(rng, n_q, n_k, h, 2, True)
    dq, dk, loss, lsep = PB.proxy_backward(q, k, q, k, sel, 0.4, 0.4, 128, True)
    assert abs(loss) < 1e-12
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.all(np.isfinite(lsep))


def test_row_and_column_gradients_match_the_whole_sequence_proxy_backward():
    """dq_idx and LSEp of sampled rows alone, and dk_idx of one (group, block) column alone
    (used at full size), equal the whole-sequence proxy backward's values."""
    from oracle import msa_case
    from synth import msa_inputs as mi
    from synth.msa_inputs import widen
    cfg = mi.custom("pcols", n_q=(300,), n_k=(600,), hq=8, hkv=2, topk=3, dp=32)
    case = mi.make_case(cfg, seed=6)
    q, k = widen(case.q), widen(case.k)
    qi, ki = widen(case.q_idx), widen(case.k_idx)
    lists = msa_case.run(case, want_output=False).topk_idx
    ps = 1.0 / np.sqrt(32)
    dqi, dki, _, lsep = PB.proxy_backward(q, k, qi, ki, lists, case.softmax_scale, ps, 128, True)
    rows = np.array([0, 7, 128, 299])
    gq, gl = PB.proxy_rows_gradient(q, k, qi, ki, lists[rows], rows, case.softmax_scale, ps,
                                    128, True)
    np.testing.assert_allclose(gq, dqi[rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gl, lsep[rows], rtol=1e-13)
    for g in range(2):
        for b in range(5):
            got = PB.proxy_key_block_gradient(q, k, qi, ki, lists, g, b, case.softmax_scale, ps,
                                              128, True)
            lo, hi = 128 * b, min(128 * b + 128, 600)
            np.testing.assert_allclose(got, dki[lo:hi, g], rtol=1e-12, atol=1e-14)
