"""GPU parity of the routed-expert block on the grouped MFMA GEMM path (many
tokens per expert: the expert linears as grouped dequant-GEMMs over the
expert-sorted assignment list, codes decoded in the mainloop), against the
oracle's MoE block on the same seeded inputs."""
import numpy as np
import pytest

import synth
from oracle import lbq_oracle as O
from _helpers import TOL, cuda, say, to_dev
import _oracle_pool as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda()


@pytest.fixture(scope="module")
def L():
    from bit_weight_only_amd import lbq
    lbq.lib()
    return lbq


def _block(L, E, hidden, ffn, top_k, bits, workload):
    sh = synth.signs(hidden, workload=workload, item=1)
    sf = synth.signs(ffn, workload=workload, item=2)
    w_gu = lambda e: synth.weights(2 * ffn, hidden, workload=workload, item=1000 + e)   # noqa: E731
    w_dn = lambda e: synth.weights(hidden, ffn, workload=workload, item=5000 + e)       # noqa: E731
    packed = L.pack_moe_host(w_gu, w_dn, bits, sh, sf)
    return L.moe_from_host(packed, bits, sh, sf, hidden, ffn, top_k)


# hidden / ffn from 256 to 2048; 2 to 150 list entries per expert (token tiles
# of 16, 32 and 64 entries, several tiles per expert, ragged last tiles)
@pytest.mark.parametrize("m,E,hidden,ffn,top_k", [(5, 8, 256, 128, 2), (64, 16, 512, 256, 4), (100, 8, 1024, 512, 3),
                                                  (300, 16, 2048, 1024, 8), (130, 4, 512, 1024, 2)])
def test_grouped_gemm_path_every_token(L, dev, m, E, hidden, ffn, top_k):
    wl = 50
    say(f"moe grouped m={m} E={E} hidden={hidden} ffn={ffn} k={top_k}")
    bits = synth.expert_bits(E, workload=wl, item=E)
    bits[: min(E, 3)] = [2, 3, 4][: min(E, 3)]          # every width present
    moe = _block(L, E, hidden, ffn, top_k, bits, wl)
    x = synth.activations(m, hidden, workload=wl, item=m)
    lg = synth.logits(m, E, workload=wl, item=m)
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev), path=L.PATH_GEMM).cpu().numpy().astype(np.float64)
    want = P.moe_all_tokens(x, lg, top_k, bits, hidden, ffn, wl)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL
    for t in range(m):
        assert O.rel_l2(y[t], want[t]) < TOL, t


def test_grouped_gemm_crowded_experts_and_repeat(L, dev):
    """Every token picks the same experts (one expert's list spans several
    64-entry tiles); repeat calls are bit-identical; the expert GEMV path gives
    the same block within the tolerance."""
    E, hidden, ffn, top_k, m = 6, 512, 512, 3, 150
    bits = np.array([2, 3, 4, 2, 3, 4], np.uint8)
    moe = _block(L, E, hidden, ffn, top_k, bits, 51)
    x = synth.activations(m, hidden, workload=51)
    lg = np.tile(np.array([[3.0, 2.0, 1.0, 0.0, -1.0, -2.0]], np.float32), (m, 1))
    lg[::5] = lg[::5][:, ::-1]
    xd, ld = to_dev(x, dev), to_dev(lg, dev)
    a = L.moe_forward(moe, xd, ld, path=L.PATH_GEMM).cpu().numpy()
    b = L.moe_forward(moe, xd, ld, path=L.PATH_GEMM).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    c = L.moe_forward(moe, xd, ld, path=L.PATH_GEMV).cpu().numpy()
    want = P.moe_all_tokens(x, lg, top_k, bits, hidden, ffn, 51)
    assert O.rel_l2(a.astype(np.float64), want) < TOL
    assert O.rel_l2(c.astype(np.float64), want) < TOL
    assert O.rel_l2(a.astype(np.float64), c.astype(np.float64)) < 1e-3


def test_moe_block_prefill_256_tokens_every_token(L, dev):
    """The MoE block (256 experts, hidden 2048, ffn 1024, top-8, widths drawn
    2/3/4) at 256 tokens: AUTO takes the grouped GEMMs; every token."""
    cfg = synth.MOE_BLOCK
    E, hidden, ffn, top_k, m = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["top_k"], 256
    say("moe prefill 256 tokens")
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    moe = _block(L, E, hidden, ffn, top_k, bits, synth.W_MOE)
    x = synth.activations(m, hidden, workload=synth.W_MOE, item=256)
    lg = synth.logits(m, E, workload=synth.W_MOE, item=256)
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev)).cpu().numpy().astype(np.float64)
    want = P.moe_all_tokens(x, lg, top_k, bits, hidden, ffn, synth.W_MOE)
    e = O.rel_l2(y, want)
    say(f"  rel_l2 {e:.3e} over {m} tokens")
    assert e < TOL


def test_moe_block_prefill_2048_tokens_sampled(L, dev):
    """2048 tokens (16384 assignments, 64-entry token tiles): the block runs
    whole on the GPU; the oracle checks 24 sampled tokens (routing and the
    combine are per token)."""
    cfg = synth.MOE_BLOCK
    E, hidden, ffn, top_k, m = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["top_k"], 2048
    say("moe prefill 2048 tokens")
    bits = synth.expert_bits(E, workload=synth.W_MOE)
    moe = _block(L, E, hidden, ffn, top_k, bits, synth.W_MOE)
    x = synth.activations(m, hidden, workload=synth.W_MOE, item=2048)
    lg = synth.logits(m, E, workload=synth.W_MOE, item=2048)
    y = L.moe_forward(moe, to_dev(x, dev), to_dev(lg, dev)).cpu().numpy().astype(np.float64)
    toks = np.sort(np.random.default_rng(4).choice(m, 24, replace=False))
    toks[0], toks[-1] = 0, m - 1
    want = P.moe_all_tokens(x[toks], lg[toks], top_k, bits, hidden, ffn, synth.W_MOE)
    e = O.rel_l2(y[toks], want)
    say(f"  rel_l2 {e:.3e} over {len(toks)} sampled tokens")
    assert e < TOL
