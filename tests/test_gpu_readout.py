"""Screened readout over the nibble-split planes of an 8-bit weight (the
LLaDA2.2-mini card's lm_head kept at 8 bits and split into high / low nibble
planes for a screened readout) on the GPU, through the C ABI:
  * the coarse logits of every row (high nibbles as a 4-bit weight) against
    the oracle's, within the linear layers' tolerance;
  * the survivors: the selection is decided on the GPU's fp16 coarse logits,
    so it is checked as a selection of those values (larger first, ties to
    the lower row, nothing left out that beats the last survivor), and against
    the oracle's fp64 coarse logits within twice the coarse error seen;
  * the survivors' exact logits against the oracle's 8-bit readout;
  * the 8-bit argmax survives a screen of eight or more rows on these seeded
    inputs."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


def make_readout(L, w, k, n, workload, item):
    s = synth.signs(k, workload=workload, item=item)
    planes, meta = L.pack(w, 8, s)
    r = L.PackedReadout.from_host(planes, meta, s, k, n)
    return s, planes, meta, r


def check_selection(coarse, ids, cand):
    """ids [M][cand] must be the cand largest coarse values of each row, larger
    first, ties to the lower row (plain numpy, independent of the library)."""
    m, n = coarse.shape
    for t in range(m):
        c = coarse[t].astype(np.float64)
        sel = ids[t]
        k = min(cand, n)
        assert np.all(sel[k:] == -1)
        sel = sel[:k]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < n
        v = c[sel]
        # sorted: value descending, row ascending among equal values
        for a in range(k - 1):
            assert v[a] > v[a + 1] or (v[a] == v[a + 1] and sel[a] < sel[a + 1]), (t, a)
        rest = np.setdiff1d(np.arange(n), sel)
        if len(rest):
            last_v, last_r = v[-1], sel[-1]
            assert np.all((c[rest] < last_v) | ((c[rest] == last_v) & (rest > last_r))), t


def run_case(L, dev, w, k, n, m, cand, workload, item, label, argmax=True):
    s, planes, meta, r = make_readout(L, w, k, n, workload, item)
    x = synth.activations(m, k, workload=workload, item=item + 1)
    coarse, ids, logits = L.readout_screened(r, to_dev(x, dev), cand)
    coarse = coarse.cpu().numpy().astype(np.float64)
    ids = ids.cpu().numpy()
    logits = logits.cpu().numpy().astype(np.float64)
    pl8, m8 = planes.view(np.uint32).reshape(n, -1, 8, 4), meta.view(np.uint16).reshape(n, -1, 2)
    lo, hi = O.split_nibbles(pl8)
    want_coarse = O.linear_rtn(x, hi, O.nibble_hi_meta(m8), s, 4, n, k)
    full = O.linear_rtn(x, pl8, m8, s, 8, n, k)
    e_c = O.rel_l2(coarse, want_coarse)
    check_selection(coarse, ids, cand)
    kk = min(cand, n)
    e_x = O.rel_l2(logits[:, :kk], np.take_along_axis(full, ids[:, :kk].astype(np.int64), axis=1))
    err = np.abs(coarse - want_coarse).max()
    for t in range(m):
        thr = np.sort(want_coarse[t])[::-1][kk - 1]
        assert np.all(want_coarse[t, ids[t, :kk]] >= thr - 2 * err - 1e-12), t
        if argmax and cand >= 8:   # a screen of one row need not hold the exact argmax
            assert int(np.argmax(full[t])) in ids[t].tolist(), t
    say(f"{label}: coarse rel_l2 {e_c:.3e}  exact rel_l2 {e_x:.3e}")
    assert e_c < TOL and e_x < TOL


@pytest.mark.parametrize("n,k", [(300, 256), (1000, 2048), (20000, 512), (40000, 1024)])
@pytest.mark.parametrize("m,cand", [(1, 1), (1, 64), (3, 8), (8, 32)])
def test_readout_against_oracle(L, dev, n, k, m, cand):
    w = synth.weights(n, k, workload=70, item=n + k)
    run_case(L, dev, w, k, n, m, cand, 70, n + k, f"readout n={n} k={k} m={m} cand={cand}")


def test_readout_ties_go_to_the_lower_row(L, dev):
    """64 distinct rows repeated over 18000 rows (two select chunks): every
    coarse logit appears many times, so the survivors are decided by the
    row-order tie rule, also across chunks."""
    k, n = 512, 18000
    base = synth.weights(64, k, workload=71, item=1)
    w = np.ascontiguousarray(np.tile(base, (n // 64 + 1, 1))[:n])
    # (every survivor is then a copy of one row: the exact argmax may be another)
    run_case(L, dev, w, k, n, 2, 48, 71, 1, "readout ties", argmax=False)


def test_readout_fewer_rows_than_survivors(L, dev):
    k, n = 256, 20
    w = synth.weights(n, k, workload=72, item=1)
    s, planes, meta, r = make_readout(L, w, k, n, 72, 1)
    x = synth.activations(2, k, workload=72, item=2)
    coarse, ids, logits = L.readout_screened(r, to_dev(x, dev), 32)
    ids = ids.cpu().numpy()
    logits = logits.cpu().numpy()
    check_selection(coarse.cpu().numpy(), ids, 32)
    assert np.all(logits[:, n:] == 0)
    full = O.linear_rtn(x, planes.view(np.uint32), meta.view(np.uint16), s, 8, n, k)
    assert O.rel_l2(logits[:, :n], np.take_along_axis(full, ids[:, :n].astype(np.int64), axis=1)) < TOL


def test_readout_zero_tokens_and_repeat(L, dev):
    import torch

    k, n = 512, 5000
    w = synth.weights(n, k, workload=73, item=1)
    s, planes, meta, r = make_readout(L, w, k, n, 73, 1)
    x = to_dev(synth.activations(3, k, workload=73, item=2), dev)
    a = L.readout_screened(r, x, 16)
    b = L.readout_screened(r, x, 16)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    c, i, lg = L.readout_screened(r, x[:0], 16)
    assert c.numel() == 0 and i.numel() == 0


def test_readout_vocabulary_size_sampled(L, dev):
    """A vocabulary-sized readout, 131072 rows x 2048 inputs (eight select
    chunks, two select stages), one and four tokens: the selection checked on
    the GPU's coarse logits, the coarse logits on sampled rows and on every
    survivor, the exact logits of every survivor against the oracle."""
    k, n = 2048, 131072
    w = synth.weights(n, k, workload=74, item=1)
    s, planes, meta, r = make_readout(L, w, k, n, 74, 1)
    pl8, m8 = planes.view(np.uint32).reshape(n, -1), meta.view(np.uint16).reshape(n, -1, 2)
    for m in (1, 4):
        x = synth.activations(m, k, workload=74, item=m)
        coarse, ids, logits = L.readout_screened(r, to_dev(x, dev), 64)
        coarse = coarse.cpu().numpy().astype(np.float64)
        ids = ids.cpu().numpy()
        logits = logits.cpu().numpy().astype(np.float64)
        check_selection(coarse, ids, 64)
        rows = np.unique(np.concatenate([np.random.default_rng(m).choice(n, 256, replace=False), ids.reshape(-1)]))
        sub_pl, sub_m = pl8[rows], m8[rows]
        lo, hi = O.split_nibbles(sub_pl)
        want_c = O.linear_rtn(x, hi, O.nibble_hi_meta(sub_m), s, 4, len(rows), k)
        e_c = O.rel_l2(coarse[:, rows], want_c)
        full = O.linear_rtn(x, sub_pl, sub_m, s, 8, len(rows), k)
        pos = np.searchsorted(rows, ids)
        e_x = O.rel_l2(logits, np.take_along_axis(full, pos, axis=1))
        say(f"readout vocabulary m={m}: coarse rel_l2 {e_c:.3e} (sampled)  exact rel_l2 {e_x:.3e}")
        assert e_c < TOL and e_x < TOL
