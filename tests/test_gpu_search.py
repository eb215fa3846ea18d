"""GPU parity of the per-head pattern search (asa_pattern_search) against the float64 oracle
(oracle.pattern_search: the Sparse-vDiT search loss and selection formula).

The search is checked link by link:
  1. Reduction.  The GPU's MSE_i must equal the oracle's pattern_mse of the GPU's own fp32
     outputs (asa_attention_fwd on the oracle's masks: the same kernel the search runs) to
     1e-12 relative: the two sum the same float64 squares in different orders.  This also
     fixes which mask each candidate used, since any other mask changes the outputs.
  2. Sparsity.  L_i - MSE_i on the GPU must equal lambda * (1 - S_i) with the oracle's S_i.
  3. Decision.  choice must be the selection rule applied to the GPU's own L (float64 on
     both sides, so exact).
  4. End to end.  The GPU's outputs stay within the forward's parity bound of the oracle's
     float64 attention, so with e = (O_i - O_0)_gpu - (O_i - O_0)_oracle and
     R = sqrt(mean e^2):  |MSE_gpu - MSE_oracle| <= 2 sqrt(MSE_oracle) R + R^2
     (Cauchy-Schwarz on mean(2 (O_i - O_0) e + e^2)).  The choice must equal the oracle's
     wherever that tolerance cannot change the decision; other heads are logged as
     ambiguous, and each case may hold only a few.
"""
import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, csr_to_device, oracle_inputs, say, to_device

pytestmark = pytest.mark.gpu

# the page's default setting: the first row of its Table 3 (tests/golden/sparse_vdit_table3.json)
_T3 = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sparse_vdit_table3.json")))
LAM, EPS = _T3["rows"][0]["lambda"], _T3["rows"][0]["epsilon"]


def _cands(cfg):
    frame = cfg.Hs * cfg.Ws
    return [(gen.SKIP, 0), (gen.DIAG, 0), (gen.MULTIDIAG, frame), (gen.VSTRIPE, 2)]


def _cases():
    st = replace(gen.scaled(gen.STATIC, H=6, frames=2), name="search_lowrank_d64",
                 v_head_scale=[1.0, 0.3, 0.1, 0.01, 0.2, 0.05], q_head_scale=[1, 1, 1, 1, 0.3, 2.0])
    wan = replace(gen.scaled(gen.WAN, H=4, frames=2), name="search_smooth_d128",
                  v_head_scale=[1.0, 0.25, 0.03, 0.12])
    # ragged: 1000 tokens in blocks of 128 (last block 104), d=64
    rag = gen.Config(name="search_ragged_1000", seed=12, B=2, H=3, N=1000, d=64, blk=128, dtype="bf16",
                     frames=1, Hs=20, Ws=50, structure="smooth", kind="static",
                     v_head_scale=[1.0, 0.2, 0.02])
    # fp32 inputs, blk 64 with d 128
    f32 = gen.Config(name="search_f32_blk64", seed=13, B=1, H=3, N=1536, d=128, blk=64, dtype="f32",
                     frames=2, Hs=24, Ws=32, structure="lowrank", kind="static",
                     v_head_scale=[1.0, 0.2, 0.02])
    return [st, wan, rag, f32]


def _gpu_outputs(asa, xd, cfg, cands):
    """fp32 outputs of the full mask and of each candidate on the oracle's masks."""
    outs = []
    for pid, prm in [(gen.FULL, 0)] + list(cands):
        M = O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, [(pid, prm)] * cfg.H)
        rp, ci = csr_to_device(M)
        o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
        outs.append(o)
    torch.cuda.synchronize()
    return [o.cpu().numpy().astype(np.float64) for o in outs]


def _check_links_1_to_3(cfg, cands, choice, loss, mse, gouts):
    H, n = cfg.H, len(cands)
    g_mse = np.stack([O.pattern_mse(gouts[1 + i], gouts[0]) for i in range(n)], axis=1)
    rel = np.abs(mse - g_mse) / np.maximum(np.abs(g_mse), 1e-300)
    say(f"  [reduction] max rel diff vs oracle MSE of the GPU outputs {float(rel.max()) if rel.size else 0:.2e}")
    assert np.all((np.abs(mse - g_mse) <= 1e-12 * np.abs(g_mse)) | (mse == g_mse)), (mse, g_mse)
    S = np.array([O.pattern_sparsity(p, q, cfg.N, cfg.blk) for p, q in cands])
    pen = loss - mse
    assert np.all(np.abs(pen - LAM * (1.0 - S)[None, :]) <= 1e-15), (pen, S)
    assert np.array_equal(choice, O.select_patterns(loss, EPS)), (choice, loss)
    return S


def _robust_choice(L, t, eps, dup):
    """The oracle's choice if no perturbation of L within +-t can change it, else None.
    dup[k] is True when candidate k keeps exactly the tiles of an earlier candidate: both
    sides then compute identical outputs for the two, the losses tie exactly, and the tie
    goes to the earlier one, so k takes no part in the comparison."""
    idx = [k for k in range(L.size) if not dup[k]]
    if not idx:
        return 0
    if all(L[k] - t[k] > eps for k in idx):
        return 0
    j = min(idx, key=lambda k: (L[k], k))
    if L[j] + t[j] > eps:
        return None
    for k in idx:
        if k != j and not (L[j] + t[j] < L[k] - t[k]):
            return None
    return j + 1


@pytest.mark.parametrize("cfg", _cases(), ids=lambda c: c.name)
def test_search_scaled(asa_lib, cfg):
    asa = asa_lib
    cands = _cands(cfg)
    say(f"case {cfg.name}: pattern search B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} blk={cfg.blk} "
        f"candidates {cands}")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    choice_t, loss_t, mse_t = asa.asa_pattern_search(xd["q"], xd["k"], xd["v"], cfg.blk, cands, lam=LAM, eps=EPS)
    torch.cuda.synchronize()
    choice = choice_t.cpu().numpy().astype(np.int64)
    loss, mse = loss_t.cpu().numpy(), mse_t.cpu().numpy()
    gouts = _gpu_outputs(asa, xd, cfg, cands)
    _check_links_1_to_3(cfg, cands, choice, loss, mse, gouts)

    q64, k64, v64 = oracle_inputs(x)
    r_choice, r_L, r_mse, r_S = O.pattern_search(q64, k64, v64, cfg.blk, cands, LAM, EPS)
    r_outs = [O.dense_attention(q64, k64, v64)] + [
        O.attention(q64, k64, v64, O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, [c] * cfg.H), cfg.blk)
        for c in cands]
    fwd_max = F32_MAX_ABS if cfg.dtype == "f32" else BF16_MAX_ABS
    for g, r in zip(gouts, r_outs):
        err = np.abs(g - r)
        assert float(err.max()) <= fwd_max
        if cfg.dtype == "bf16":
            assert float(err.mean()) <= BF16_MEAN_ABS
    masks = [O.static_mask(1, 1, cfg.N, cfg.blk, [c]) for c in cands]
    dup = [any(np.array_equal(masks[k], masks[j]) for j in range(k)) for k in range(len(cands))]
    for k in range(len(cands)):
        if dup[k]:
            first = next(j for j in range(k) if np.array_equal(masks[k], masks[j]))
            assert np.array_equal(loss[:, k], loss[:, first]), "identical masks must tie exactly"
    amb = []
    for h in range(cfg.H):
        t = np.empty(len(cands))
        for i in range(len(cands)):
            e = (gouts[1 + i][:, h] - gouts[0][:, h]) - (r_outs[1 + i][:, h] - r_outs[0][:, h])
            R = float(np.sqrt(np.mean(e * e)))
            t[i] = 2.0 * np.sqrt(r_mse[h, i]) * R + R * R
            t[i] = t[i] * (1 + 1e-9) + 1e-15
        assert np.all(np.abs(mse[h] - r_mse[h]) <= t), (h, mse[h], r_mse[h], t)
        want = _robust_choice(r_L[h], t, EPS, dup)
        say(f"  head {h}: L gpu {np.array2string(loss[h], precision=5)} oracle "
            f"{np.array2string(r_L[h], precision=5)} tol {np.array2string(t, formatter={'float_kind': '{:.1e}'.format})} "
            f"choice gpu {choice[h]} oracle {r_choice[h]}{'' if want is not None else ' (ambiguous)'}")
        if want is None:
            amb.append(h)
            # an ambiguous head's choice is still one of the candidates the tolerance allows
            lo = r_L[h] - t
            hi = r_L[h] + t
            if choice[h] == 0:
                assert np.all(hi > EPS)
            else:
                j = choice[h] - 1
                assert lo[j] <= EPS and np.all(lo[j] <= hi)
        else:
            assert choice[h] == want, f"head {h}: GPU chose {choice[h]}, oracle {want}"
    assert len(amb) <= max(1, cfg.H // 3), f"too many ambiguous heads {amb}"
    # the cases reach more than one branch of the selection formula
    assert len(set(r_choice.tolist())) >= 2


def test_search_special_candidates(asa_lib):
    """A full-attention candidate scores MSE exactly 0 (same kernel, same mask); no
    candidates gives full attention everywhere; repeated calls are bit-identical."""
    asa = asa_lib
    cfg = replace(gen.scaled(gen.STATIC, H=2, frames=1), name="search_special")
    x = to_device(gen.make_inputs(cfg))
    c, L, m = asa.asa_pattern_search(x["q"], x["k"], x["v"], cfg.blk, [(gen.FULL, 0), (gen.SKIP, 0)])
    c2, L2, m2 = asa.asa_pattern_search(x["q"], x["k"], x["v"], cfg.blk, [(gen.FULL, 0), (gen.SKIP, 0)])
    c0, L0, m0 = asa.asa_pattern_search(x["q"], x["k"], x["v"], cfg.blk, [])
    torch.cuda.synchronize()
    assert torch.all(m[:, 0] == 0.0) and torch.all(L[:, 0] == LAM)
    assert torch.equal(L, L2) and torch.equal(m, m2) and torch.equal(c, c2)
    assert torch.all(c0 == 0) and L0.numel() == 0
    # FULL scores lam = 0.01 <= eps, SKIP scores mean(O_0^2) > eps here: FULL wins
    assert torch.all(c == 1)


def test_search_full_size_wan(asa_lib):
    """Wan-shaped layer at full size (B=1, H=12, N=32760, d=128) with the four page
    patterns: links 1-3 on the whole layer, and sampled outputs against the oracle."""
    asa = asa_lib
    cfg = gen.WAN
    cands = _cands(cfg)
    say(f"case {cfg.name}: full-size pattern search, candidates {cands}")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    choice_t, loss_t, mse_t = asa.asa_pattern_search(xd["q"], xd["k"], xd["v"], cfg.blk, cands, lam=LAM, eps=EPS)
    torch.cuda.synchronize()
    choice = choice_t.cpu().numpy().astype(np.int64)
    loss, mse = loss_t.cpu().numpy(), mse_t.cpu().numpy()
    say(f"  choice {choice.tolist()}")
    gouts = _gpu_outputs(asa, xd, cfg, cands)
    _check_links_1_to_3(cfg, cands, choice, loss, mse, gouts)
    q64, k64, v64 = oracle_inputs(x)
    rng = np.random.default_rng(707)
    rows = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, cfg.H, 6), rng.integers(0, cfg.N, 6))]
    rows.append((0, cfg.H - 1, cfg.N - 1))
    for n, (pid, prm) in enumerate([(gen.FULL, 0)] + cands):
        M = O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, [(pid, prm)] * cfg.H)
        want = O.attention_rows(q64, k64, v64, M, cfg.blk, rows)
        got = np.stack([gouts[n][b, h, i] for b, h, i in rows])
        assert float(np.abs(got - want).max()) <= BF16_MAX_ABS, (pid, prm)
