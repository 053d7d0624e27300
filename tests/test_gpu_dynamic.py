"""GPU parity of the dynamic block-sparse path for dense layers (FlashPrefill
page: section 2.1 probe queries against pooled keys, 2.2 max-based
threshold, 2.3 index-driven tile walk): the pooled keys, the selected tile
lists and attention over those lists, each against oracle/dynamic.py.

The keep decision compares a score with alpha times the maximum score; the
GPU takes it in fp32 and the oracle in fp64 on the same bf16 pooled keys, so
tiles whose oracle score lies within AMBIG (relative to the maximum) of the
threshold may be decided either way.  Every other tile must agree; every GPU
list must be valid (ascending, causal range, diagonal tiles present, flags);
attention is compared on every row against the oracle over the list the GPU
walked, and on the rows whose lists agree also over the oracle's own list.
"""
import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
import synth
from oracle import dynamic as odyn
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

AMBIG = 1e-4


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


def peaky_inputs(seed, B, Hq, Hkv, N, d, qscale, dev):
    """Seeded bf16 Q/K/V with Q scaled by qscale (then rounded to bf16), so
    that tile scores spread out and the threshold drops tiles."""
    qb, kb, vb = synth.qkv_bf16_bits(seed, B, Hq, Hkv, N, d)
    if qscale != 1.0:
        qb = synth.f32_to_bf16_bits((gu.as_f64(qb) * qscale).astype(np.float32))
    bits = (qb, kb, vb)
    return bits, tuple(gu.bits_to_device(x, dev) for x in bits)


def gpu_plan(q, k, alpha):
    p = tsa.dyn_plan(q, k, alpha)
    torch.cuda.synchronize()
    rp = p.d_row_ptr.cpu().numpy().astype(np.int64)
    nnz = int(rp[-1])
    assert 0 < nnz <= p.max_nnz
    return p, rp, p.d_k_tile[:nnz].cpu().numpy(), p.d_flags[:nnz].cpu().numpy()


def check_row(got, flags, want, scores, t, N):
    """Validity of one GPU list, and agreement with the oracle's list away
    from the threshold.  Returns True when the two lists are identical."""
    nc = (min(N, (t + 1) * 128) - 1) // 64 + 1
    assert np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < nc
    diag = np.arange(nc)[np.arange(nc) * 64 + 63 > t * 128]
    assert set(diag.tolist()) <= set(got.tolist())
    assert np.array_equal(flags, np.where(got * 64 + 63 > t * 128, tsa.TRI_TILE_PARTIAL,
                                          tsa.TRI_TILE_FULL))
    s, thr = scores
    for kt in set(got.tolist()) ^ set(want.tolist()):
        assert abs(s[kt] - thr) <= AMBIG * s.max(), (t, kt, s[kt], thr)
    return np.array_equal(got, want)


CASES = [  # N, d, B, Hq, Hkv, alpha, qscale
    (1000, 128, 1, 4, 2, 0.5, 4.0),
    (777, 64, 1, 3, 1, 0.3, 8.0),
    (1, 128, 1, 2, 1, 0.5, 1.0),
    (2500, 128, 1, 2, 2, 0.9, 4.0),
    (700, 128, 1, 4, 1, 1.0, 6.0),
    (129, 64, 1, 2, 2, 0.2, 3.0),
    (900, 128, 2, 4, 2, 0.6, 5.0),   # batch 2: rows (b * Hq + h) * nq + t
    (600, 128, 2, 7, 1, 0.5, 4.0),   # seven query heads per KV head (the Qwen2.5-7B grouping)
]


@pytest.mark.parametrize("N,d,B,Hq,Hkv,alpha,qscale", CASES)
def test_pooled_keys_lists_and_attention(dev, N, d, B, Hq, Hkv, alpha, qscale):
    gu.note(f"dynamic N={N} d={d} B={B} Hq={Hq} Hkv={Hkv} alpha={alpha} qscale={qscale}")
    bits, (q, k, v) = peaky_inputs(100 + N, B, Hq, Hkv, N, d, qscale, dev)
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    p, rp, kt, fl = gpu_plan(q, k, alpha)

    # pooled keys (workspace offset 0, bf16 [B, Hkv, nkt, d]): bit-exact
    nkt = -(-N // 64)
    n = B * Hkv * nkt * d
    pooled = p.workspace[:2 * n].view(torch.int16).cpu().numpy().view(np.uint16).reshape(B, Hkv, nkt, d)
    ref_pooled = odyn.pooled_keys(kf, 64)
    assert np.array_equal(synth.bf16_bits_to_f64(pooled), ref_pooled)

    # lists
    rrp, rkt, _, scores = odyn.select_tiles(qf, kf, alpha, return_scores=True)
    nq = -(-N // 128)
    same = {}
    for r in range(B * Hq * nq):
        t = r % nq
        same[r] = check_row(kt[rp[r]:rp[r + 1]], fl[rp[r]:rp[r + 1]], rkt[rrp[r]:rrp[r + 1]],
                            scores[r], t, N)
    gu.note(f"  {sum(same.values())}/{len(same)} rows with identical lists, nnz {rp[-1]}"
            f" of {p.max_nnz}")
    assert sum(same.values()) >= 0.9 * len(same)

    # attention over the GPU lists: every row against the oracle over the GPU's
    # own list (a row whose list differs near the threshold is checked too),
    # and the rows whose lists agree also against the oracle's own list
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="lists", plan=p, o_dtype=torch.float32, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ref = odyn.attention_tiles(qf, kf, vf, rrp, rkt)
    own = odyn.attention_tiles(qf, kf, vf, rp, kt)
    for b in range(B):
        for h in range(Hq):
            ro, rl = ref[(b, h)]
            go, gl = own[(b, h)]
            for t in range(nq):
                rows = slice(t * 128, min(N, (t + 1) * 128))
                gu.check(o[b, h, rows], lse[b, h, rows], go[rows], gl[rows], f"b={b} h={h} t={t} (GPU list)")
                if same[(b * Hq + h) * nq + t]:
                    gu.check(o[b, h, rows], lse[b, h, rows], ro[rows], rl[rows], f"b={b} h={h} t={t}")


def test_alpha_zero_lists_are_causal_and_bit_identical_to_dense(dev):
    # alpha = 0 keeps every causal tile: the list walk must reproduce the
    # dense causal kernel bit for bit (same tiles, same ascending order)
    gu.note("dynamic alpha=0 vs dense causal kernel, N=1500")
    N = 1500
    bits, (q, k, v) = gu.make_inputs(31, 1, 4, 2, N, 128, dev)
    p, rp, kt, fl = gpu_plan(q, k, 0.0)
    nq = -(-N // 128)
    for r in range(4 * nq):
        t = r % nq
        nc = (min(N, (t + 1) * 128) - 1) // 64 + 1
        assert np.array_equal(kt[rp[r]:rp[r + 1]], np.arange(nc))
    oc, lc = gu.run(q, k, v, "causal", o_dtype=torch.bfloat16)
    o = torch.empty_like(oc)
    lse = torch.empty_like(lc)
    tsa.prefill(q, k, v, mode="lists", plan=p, o_dtype=torch.bfloat16, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)


def test_llama_128k_sampled(dev):
    # the dense 128K Llama-shaped layer at the benchmark's alpha: lists of
    # sampled query tiles of every head against the oracle, validity of every
    # list, attention on a few (head, tile) pairs
    N, Hq, Hkv, d, alpha = 131072, 32, 8, 128, 0.9
    gu.note("dynamic 128K: inputs")
    bits, (q, k, v) = gu.make_inputs(0, 1, Hq, Hkv, N, d, dev)
    gu.note("dynamic 128K: plan")
    p, rp, kt, fl = gpu_plan(q, k, alpha)
    nq = N // 128
    counts = np.diff(rp)
    assert np.all(counts >= 1)
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    tiles = [0, 1, 17, 300, nq // 2, nq - 2, nq - 1]
    same, wants = {}, {}
    for g in range(Hkv):
        kbar = odyn.pooled_keys(kf[:, g:g + 1], 64)[0, 0]
        for h in range(g * 4, g * 4 + 4):
            for t in tiles:
                rows = odyn.probe_rows(t, N)
                last = min(N, (t + 1) * 128) - 1
                s = odyn.tile_scores(qf[0, h, rows], kbar, rows, last, d ** -0.5)
                thr = alpha * s.max()
                kts = np.arange(s.size)
                want = kts[(s >= thr) | (kts * 64 + 63 > t * 128)]
                wants[(h, t)] = want
                r = h * nq + t
                same[(h, t)] = check_row(kt[rp[r]:rp[r + 1]], fl[rp[r]:rp[r + 1]], want, (s, thr), t, N)
    gu.note(f"  {sum(same.values())}/{len(same)} sampled lists identical; density "
            f"{rp[-1] / p.max_nnz:.3f}")
    assert sum(same.values()) >= 0.9 * len(same)
    o = torch.empty((1, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="lists", plan=p, o_dtype=torch.bfloat16, out=o, lse=lse)
    torch.cuda.synchronize()
    for (h, t) in [(0, 0), (5, 17), (31, nq - 1), (12, 300)]:
        # the oracle over the list the GPU walked (its own when the two agree),
        # as a one-head CSR
        r = h * nq + t
        lists = [kt[rp[r]:rp[r + 1]]] + ([wants[(h, t)]] if same[(h, t)] else [])
        for lst in lists:
            one_rp = np.concatenate([np.zeros(t + 1, np.int64), np.full(nq - t, lst.size)])
            ref = odyn.attention_tiles(qf[:, h:h + 1], kf[:, h // 4:h // 4 + 1], vf[:, h // 4:h // 4 + 1],
                                       one_rp, lst, qtiles=[t])
            ro, rl = ref[(0, 0)]
            rows = slice(t * 128, (t + 1) * 128)
            gu.check(o[0, h, rows], lse[0, h, rows], ro, rl, f"128K h={h} t={t}")
