"""GPU parity on seeded random configurations: the mask builders (adaptive and static-only),
the forward (with lse), the split-row forward, the pattern search and the backward, against
the float64 oracle.

Each case draws B, H, N (ragged tails and single-block sequences included), d, blk, input
dtype and structure, top-k or tau (with and without a cap), text tokens, the diagonal, and
per-head static patterns (full, skip, diagonal, multi-diagonal, vertical stripe, frame
tiles, adaptive).  The bounds are the suite's own: CSR bit-exact outside ambiguous rows;
forward 2e-2 max / 2e-3 mean absolute (bf16 inputs), 1e-4 (fp32 inputs); lse within
2^-8 + 1e-4; gradients within 2e-2 of the largest and 5e-3 of the mean reference entry (bf16
inputs), and within 2^-12 of each element's product sums plus 2^-14 of the largest entry
(fp32 inputs).
The GPU attends the oracle's own mask, so no oracle input comes from the HIP path.
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import compare_masks, compare_outputs, csr_to_device, gpu_csr_rows, oracle_inputs, say, to_device

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 2.0 ** -8 + 1e-4
GRAD_MAX_REL, GRAD_MEAN_REL = 2e-2, 5e-3
N_CASES = 128


def _random_config(seed):
    rng = np.random.default_rng(7000 + seed)
    blk = int(rng.choice([64, 128]))
    d = int(rng.choice([64, 128]))
    Nb = int(rng.integers(1, 18))
    N = max(1, Nb * blk - int(rng.integers(0, blk)))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    n_text = int(rng.integers(1, min(N, 300))) if (N > 1 and rng.random() < 0.3) else 0
    structure = str(rng.choice(["none", "lowrank", "smooth"]))
    mode = gen.TOPK if rng.random() < 0.6 else gen.TAU
    k = int(rng.integers(0, Nb + 3))
    tau = float(rng.uniform(0.3, 1.0))
    k_cap = int(rng.integers(1, Nb + 1)) if rng.random() < 0.5 else 0
    patterns = None
    if rng.random() < 0.5:
        choices = [(gen.ADAPTIVE, 0), (gen.FULL, 0), (gen.SKIP, 0), (gen.DIAG, 0),
                   (gen.MULTIDIAG, int(rng.integers(1, 4 * blk))), (gen.VSTRIPE, int(rng.integers(0, 3))),
                   (gen.FRAME_TILE, int(rng.integers(1, max(2, N))))]
        patterns = [choices[int(rng.integers(0, len(choices)))] for _ in range(H)]
    cfg = gen.Config(name=f"random_{seed}", seed=9000 + seed, B=B, H=H, N=N, d=d, blk=blk,
                     dtype="bf16" if rng.random() < 0.75 else "f32", frames=1, Hs=1, Ws=N - n_text,
                     structure=structure, kind="adaptive", mode=mode, k=k, tau=tau, k_cap=k_cap,
                     n_text=n_text, keep_diag=int(rng.integers(0, 2)), patterns=patterns)
    return cfg


def _grad_close(got, want, label):
    g = got.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{label}: non-finite gradient"
    err = np.abs(g - want)
    smax, smean = float(np.abs(want).max()), float(np.abs(want).mean())
    say(f"  [{label}] max abs err {err.max():.3e} (ref max {smax:.3e})  mean {err.mean():.3e} (ref mean {smean:.3e})")
    assert err.max() <= GRAD_MAX_REL * smax + 1e-6, label
    assert err.mean() <= GRAD_MEAN_REL * smean + 1e-7, label


def _grad_close_f32(got, ref, terms, label):
    """fp32 inputs: 2^-12 of each element's product sums plus 2^-14 of the gradient's scale
    (the bound of test_gpu_backward_f32, derived there); exact zeros where nothing adds."""
    from test_gpu_backward_f32 import SCALE_REL, TERMS_REL
    a = got.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(a)), f"{label}: non-finite gradient"
    err = np.abs(a - ref)
    bound = TERMS_REL * terms + SCALE_REL * float(np.abs(ref).max())
    assert np.all(err <= bound), f"{label} (fp32): {int((err > bound).sum())} elements over the rounding bound"
    zero = ref == 0.0
    assert np.all(a[zero] == 0.0), f"{label} (fp32): nonzero gradient where no tile contributes"


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_config(asa_lib, seed):
    asa = asa_lib
    cfg = _random_config(seed)
    say(f"case {cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} blk={cfg.blk} {cfg.dtype} {cfg.structure} "
        f"mode={cfg.mode} k={cfg.k} tau={cfg.tau:.3f} cap={cfg.k_cap} text={cfg.n_text} diag={cfg.keep_diag} "
        f"patterns={cfg.patterns}")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M, det = O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap,
                          n_text=cfg.n_text, keep_diag=cfg.keep_diag, patterns=cfg.patterns,
                          return_details=True)
    rp_t, ci_t = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                                    k_cap=cfg.k_cap, n_text=cfg.n_text, keep_diag=cfg.keep_diag,
                                    patterns=cfg.patterns)
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    amb = O.ambiguous_rows(det["S"], det["P"], mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap)
    diff = compare_masks(rp, ci, M, det, amb, cfg.mode, cfg.k, cfg.tau, cfg.k_cap)
    say(f"  mask density {O.density(M):.4f}, ambiguous rows {int(amb.sum())}, differing rows {len(diff)}")

    # the static-only builder on the same patterns (an adaptive head takes the diagonal here:
    # static calls accept static patterns only), bit-exact
    if cfg.patterns is not None:
        spats = [(gen.DIAG, 0) if pid == gen.ADAPTIVE else (pid, prm) for pid, prm in cfg.patterns]
        srp_t, sci_t = asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, spats, "cuda:0")
        torch.cuda.synchronize()
        srp, sci = gpu_csr_rows(srp_t, sci_t)
        orp, oci = O.to_csr(O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, spats))
        assert np.array_equal(srp, orp) and np.array_equal(sci, oci), "static mask differs from the oracle"

    # forward (and lse) on the oracle's mask; skipped heads are all zeros
    Meff = M.copy()
    if cfg.patterns is not None:
        for h, (pid, _) in enumerate(cfg.patterns):
            if pid == O.SKIP:
                Meff[:, h] = False
    rp_o, ci_o = csr_to_device(M)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    out = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp_o, ci_o, cfg.blk, patterns=cfg.patterns, lse=lse)
    torch.cuda.synchronize()
    want = O.attention(q64, k64, v64, Meff, cfg.blk)
    compare_outputs(out.cpu().numpy(), want, cfg.dtype == "f32", cfg.name)
    # the split-row forward at a random chunk length T (rows of more than T blocks are cut)
    T = 1 + seed % max(1, cfg.Nb)
    o_split = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp_o, ci_o, cfg.blk, split_blocks=T,
                                          patterns=cfg.patterns)
    torch.cuda.synchronize()
    compare_outputs(o_split.cpu().numpy(), want, cfg.dtype == "f32", f"{cfg.name} split T={T}")
    L = O.attention_lse(q64, k64, Meff, cfg.blk)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(lg), ~fin), "lse: -inf pattern differs"
    if fin.any():
        assert float(np.abs(lg[fin] - L[fin]).max()) <= LSE_MAX_ABS

    # the per-head pattern search on random static candidates (even seeds): the loss carries
    # exactly lam * (1 - S_i) with the oracle's S_i, and the choice follows the selection
    # rule on the GPU's own losses
    if seed % 2 == 0:
        rng = np.random.default_rng(11000 + seed)
        pool = [(gen.SKIP, 0), (gen.DIAG, 0), (gen.FULL, 0), (gen.MULTIDIAG, int(rng.integers(1, 4 * cfg.blk))),
                (gen.VSTRIPE, int(rng.integers(0, 3))), (gen.FRAME_TILE, int(rng.integers(1, max(2, cfg.N))))]
        cands = [pool[int(i)] for i in rng.choice(len(pool), size=int(rng.integers(1, 5)), replace=False)]
        choice, loss, mse = asa.asa_pattern_search(xd["q"], xd["k"], xd["v"], cfg.blk, cands)
        torch.cuda.synchronize()
        S = np.array([O.pattern_sparsity(pid, prm, cfg.N, cfg.blk) for pid, prm in cands])
        L_np = loss.cpu().numpy()
        pen = L_np - mse.cpu().numpy()
        # L - MSE recovers the penalty up to the rounding of the subtraction (a few ulps of L)
        assert np.all(np.abs(pen - 0.01 * (1.0 - S)[None, :]) <= 1e-15 * (1.0 + np.abs(L_np))), "search penalty"
        assert np.array_equal(choice.cpu().numpy(), O.select_patterns(loss.cpu().numpy(), 0.1)), "search choice"
        say(f"  search over {cands}: choices {choice.cpu().numpy().tolist()}")

    if cfg.dtype == "bf16" and Meff.any():
        g = torch.from_numpy(np.random.default_rng(seed).standard_normal(tuple(x["q"].shape)).astype(np.float32))
        dout = g.to(torch.bfloat16)
        dq, dk, dv = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], out, dout.to("cuda:0"), lse, rp_o, ci_o,
                                           cfg.blk, patterns=cfg.patterns)
        torch.cuda.synchronize()
        rdq, rdk, rdv = O.attention_bwd(q64, k64, v64, dout.to(torch.float64).numpy(), Meff, cfg.blk)
        _grad_close(dq, rdq, "dQ")
        _grad_close(dk, rdk, "dK")
        _grad_close(dv, rdv, "dV")
    if cfg.dtype == "f32" and Meff.any():
        g = np.random.default_rng(seed).standard_normal(tuple(x["q"].shape)).astype(np.float32)
        grads = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], out, torch.from_numpy(g).to("cuda:0"), lse, rp_o,
                                      ci_o, cfg.blk, patterns=cfg.patterns)
        torch.cuda.synchronize()
        g64 = g.astype(np.float64)
        refs = O.attention_bwd(q64, k64, v64, g64, Meff, cfg.blk)
        terms = O.attention_bwd_terms(q64, k64, v64, g64, Meff, cfg.blk)
        for got, ref, t, label in zip(grads, refs, terms, ("dQ", "dK", "dV")):
            _grad_close_f32(got, ref, t, label)


# Launches of at least 768 query-block rows at d = 128, blk = 128 take the 32-key-step
# kernel; the family above stays below that, so a second family draws such launches.
N_LARGE_CASES = 12


def _random_large_config(seed):
    rng = np.random.default_rng(17000 + seed)
    Nb = int(rng.integers(48, 97))
    B = int(rng.integers(1, 3))
    H = max(int(rng.integers(4, 13)), -(-768 // (B * Nb)))
    N = Nb * 128 - int(rng.integers(0, 128))
    mode = gen.TOPK if rng.random() < 0.6 else gen.TAU
    patterns = None
    if rng.random() < 0.5:
        choices = [(gen.ADAPTIVE, 0), (gen.SKIP, 0), (gen.DIAG, 0), (gen.MULTIDIAG, int(rng.integers(1, 2048))),
                   (gen.VSTRIPE, int(rng.integers(0, 3))), (gen.FRAME_TILE, int(rng.integers(128, 4096)))]
        patterns = [choices[int(rng.integers(0, len(choices)))] for _ in range(H)]
    return gen.Config(name=f"random_large_{seed}", seed=19000 + seed, B=B, H=H, N=N, d=128, blk=128,
                      dtype="bf16" if rng.random() < 0.75 else "f32", frames=1, Hs=1, Ws=N,
                      structure=str(rng.choice(["none", "smooth"])), kind="adaptive", mode=mode,
                      k=int(rng.integers(1, 10)), tau=float(rng.uniform(0.3, 0.95)),
                      k_cap=int(rng.integers(4, 16)) if mode == gen.TAU else 0,
                      keep_diag=int(rng.integers(0, 2)), patterns=patterns)


@pytest.mark.parametrize("seed", range(N_LARGE_CASES))
def test_random_large_launch(asa_lib, seed):
    """Mask, forward (with lse) and split forward over whole outputs at >= 768 rows."""
    asa = asa_lib
    cfg = _random_large_config(seed)
    assert cfg.B * cfg.H * cfg.Nb >= 768
    say(f"case {cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N} rows={cfg.B * cfg.H * cfg.Nb} {cfg.dtype} "
        f"{cfg.structure} mode={cfg.mode} k={cfg.k} tau={cfg.tau:.3f} cap={cfg.k_cap} diag={cfg.keep_diag} "
        f"patterns={cfg.patterns}")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M, det = O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap,
                          keep_diag=cfg.keep_diag, patterns=cfg.patterns, return_details=True)
    rp_t, ci_t = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                                    k_cap=cfg.k_cap, keep_diag=cfg.keep_diag, patterns=cfg.patterns)
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    amb = O.ambiguous_rows(det["S"], det["P"], mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap)
    diff = compare_masks(rp, ci, M, det, amb, cfg.mode, cfg.k, cfg.tau, cfg.k_cap)
    say(f"  mask density {O.density(M):.4f}, ambiguous rows {int(amb.sum())}, differing rows {len(diff)}")
    Meff = M.copy()
    if cfg.patterns is not None:
        for h, (pid, _) in enumerate(cfg.patterns):
            if pid == O.SKIP:
                Meff[:, h] = False
    rp_o, ci_o = csr_to_device(M)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    out = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp_o, ci_o, cfg.blk, patterns=cfg.patterns, lse=lse)
    T = 2 + seed % 5
    o_split = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp_o, ci_o, cfg.blk, split_blocks=T,
                                          patterns=cfg.patterns)
    torch.cuda.synchronize()
    want = O.attention(q64, k64, v64, Meff, cfg.blk)
    compare_outputs(out.cpu().numpy(), want, cfg.dtype == "f32", cfg.name)
    compare_outputs(o_split.cpu().numpy(), want, cfg.dtype == "f32", f"{cfg.name} split T={T}")
    L = O.attention_lse(q64, k64, Meff, cfg.blk)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(lg), ~fin), "lse: -inf pattern differs"
    if fin.any():
        assert float(np.abs(lg[fin] - L[fin]).max()) <= LSE_MAX_ABS
