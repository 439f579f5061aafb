"""GPU parity of the routed-expert MoE block through the C ABI: router
outputs (integers bit-exact), and the block output against the oracle."""
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


def _check_route(L, dev, lg, top_k):
    ids, wts, counts, offsets, perm = [t.cpu().numpy() for t in L.moe_route(to_dev(lg, dev), top_k)]
    oid, ow = O.route(lg, top_k)
    assert np.array_equal(ids, oid)
    np.testing.assert_allclose(wts, ow, rtol=2e-6, atol=1e-7)
    m, e = lg.shape
    want_counts = np.bincount(oid.ravel(), minlength=e)
    assert np.array_equal(counts, want_counts)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(want_counts)]))
    flat = oid.ravel()
    want_perm = np.concatenate([np.nonzero(flat == x)[0] for x in range(e)]).astype(np.int32)
    assert np.array_equal(perm, want_perm)


@pytest.mark.parametrize("m,e,k", [(32, 256, 8), (1, 8, 1), (5, 16, 16), (100, 64, 4), (1024, 256, 8), (7, 1000, 32)])
def test_route_matches_oracle(L, dev, m, e, k):
    say(f"route m={m} e={e} k={k}")
    _check_route(L, dev, synth.logits(m, e, workload=synth.W_MOE, item=m + e), k)


def test_route_ties_go_to_lower_id(L, dev):
    lg = np.zeros((3, 64), np.float32)
    lg[1, [5, 9, 40]] = 2.0
    lg[2] = np.repeat(np.arange(8, dtype=np.float32), 8)[::-1]
    _check_route(L, dev, lg, 6)


def _block(L, E, hidden, ffn, top_k, bits, workload):
    sh = synth.signs(hidden, workload=workload, item=1)
    sf = synth.signs(ffn, workload=workload, item=2)
    w_gu = lambda e: synth.weights(2 * ffn, hidden, workload=workload, item=1000 + e)   # noqa: E731
    w_dn = lambda e: synth.weights(hidden, ffn, workload=workload, item=5000 + e)       # noqa: E731
    packed = L.pack_moe_host(w_gu, w_dn, bits, sh, sf)
    dev_moe = L.moe_from_host(packed, bits, sh, sf, hidden, ffn, top_k)
    return sh, sf, w_gu, w_dn, dev_moe


def _oracle_expert(w_gu, w_dn, bits, sh, sf, hidden, ffn):
    cache = {}

    def get(e):
        if e not in cache:
            b = int(bits[e])
            pg, mg, _ = O.pack_rtn(w_gu(e), b, sh)
            pd, md, _ = O.pack_rtn(w_dn(e), b, sf)
            cache[e] = (O.dequant_weight_rtn(pg, mg, sh, b, 2 * ffn, hidden),
                        O.dequant_weight_rtn(pd, md, sf, b, hidden, ffn))
        return cache[e]
    return get


# hidden and ffn multiples of 512 (with 16-byte aligned signs) run the
# matrix-core expert kernels; the others the VALU expert kernels
@pytest.mark.parametrize("m,E,hidden,ffn,top_k", [(5, 8, 256, 128, 2), (1, 4, 384, 256, 4), (19, 16, 512, 256, 3),
                                                  (3, 8, 512, 512, 2), (13, 16, 1024, 512, 4), (1, 8, 2048, 1024, 8)])
def test_moe_small_blocks(L, dev, m, E, hidden, ffn, top_k):
    say(f"moe small m={m} E={E} hidden={hidden} ffn={ffn} k={top_k}")
    bits = synth.expert_bits(E, workload=17, item=E)
    sh, sf, w_gu, w_dn, moe = _block(L, E, hidden, ffn, top_k, bits, 17)
    x = synth.activations(m, hidden, workload=17, item=m)
    lg = synth.logits(m, E, workload=17, item=m)
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev)).cpu().numpy().astype(np.float64)
    want = O.moe_forward(x, lg, top_k, _oracle_expert(w_gu, w_dn, bits, sh, sf, hidden, ffn))
    e = O.rel_l2(y, want)
    say(f"  rel_l2={e:.3e}")
    assert e < TOL


@pytest.mark.parametrize("hidden,ffn", [(256, 128), (512, 512)], ids=["valu", "matrix_core"])
def test_moe_every_width_and_crowded_expert(L, dev, hidden, ffn):
    """All tokens pick the same experts (more than one token chunk per expert:
    8 on the VALU kernels, 4 on the matrix cores) and each width appears."""
    E, top_k, m = 6, 3, 21
    bits = np.array([2, 3, 4, 2, 3, 4], np.uint8)
    sh, sf, w_gu, w_dn, moe = _block(L, E, hidden, ffn, top_k, bits, 18)
    x = synth.activations(m, hidden, workload=18)
    lg = np.tile(np.array([[3.0, 2.0, 1.0, 0.0, -1.0, -2.0]], np.float32), (m, 1))
    lg[::4] = lg[::4][:, ::-1]
    # 63 assignments over 6 experts would take the grouped GEMMs; the expert
    # GEMV kernels are the ones under test here
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev), path=L.PATH_GEMV).cpu().numpy().astype(np.float64)
    want = O.moe_forward(x, lg, top_k, _oracle_expert(w_gu, w_dn, bits, sh, sf, hidden, ffn))
    assert O.rel_l2(y, want) < TOL


def test_moe_repeat_calls_bit_identical(L, dev):
    E, hidden, ffn, top_k, m = 16, 512, 512, 4, 13
    bits = synth.expert_bits(E, workload=19, item=E)
    sh, sf, w_gu, w_dn, moe = _block(L, E, hidden, ffn, top_k, bits, 19)
    x = to_dev(synth.activations(m, hidden, workload=19), dev)
    lg = to_dev(synth.logits(m, E, workload=19), dev)
    a = L.moe_forward(moe, x, lg).cpu().numpy()
    b = L.moe_forward(moe, x, lg).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_moe_block_full_size_sampled_tokens(L, dev):
    """256 experts, hidden 2048, ffn 1024, top-8, 32 tokens, widths drawn
    2/3/4 with p = 0.7/0.2/0.1; the oracle checks 4 of the tokens."""
    cfg = synth.MOE_BLOCK
    E, hidden, ffn, top_k, m = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["top_k"], cfg["M"]
    say("moe full block")
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    sh, sf, w_gu, w_dn, moe = _block(L, E, hidden, ffn, top_k, bits, synth.W_MOE)
    x = synth.activations(m, hidden, workload=synth.W_MOE)
    lg = synth.logits(m, E, workload=synth.W_MOE)
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev)).cpu().numpy().astype(np.float64)
    y2 = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, y2)
    toks = np.array([0, 9, 22, 31])
    want = O.moe_forward(x[toks], lg[toks], top_k, _oracle_expert(w_gu, w_dn, bits, sh, sf, hidden, ffn))
    e = O.rel_l2(y[toks], want)
    say(f"  rel_l2={e:.3e}")
    assert e < TOL
