"""GPU block summaries on blocks that stress the eigensolver, against the oracle.

The decode tests feed the summary build random, spiked and needle blocks.  Here
each (b, K/V head) pair holds one kind of block the solver must also get right:

* few distinct tokens (covariance rank 1, 2 or 4: zero eigenvalues past the rank,
  whose factor rows must vanish);
* top eigenvalues that tie exactly (axis-aligned tokens, exact in bfloat16) or in
  a rotated frame (tied up to the keys' bfloat16 rounding): such rows are checked
  against their eigenspace, since any orthonormal basis of it is correct;
* constant blocks (every eigenvalue 0: every factor row exactly 0, nothing NaN);
* keys scaled by 1e-3 and by 1e3 (the reflections and the multisection are
  scale-free; the bound on a row's error scales with the block's lambda_1).

Factor rows follow ``check_factor_rows`` with the Davis-Kahan slack of
``eig_error`` (|dG| <= 1e-5 lambda_1), as in the decode tests; means to fp32
rounding of the keys' magnitude.  Both sides read the same bfloat16 keys.
"""

import numpy as np
import pytest

import oracle

from gpu_util import block_spectra, check_factor_rows, eig_error

pytestmark = pytest.mark.gpu

S = 64


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _block(kind, rng, d):
    """One block [S, d] of keys (float64, before the bfloat16 rounding)."""
    c = rng.normal(size=d)
    if kind.startswith("distinct"):  # m distinct tokens, m - 1 independent directions
        m = int(kind.split("_")[1])
        tokens = rng.normal(size=(m, d))
        return tokens[rng.integers(0, m, S)]
    if kind == "tied_axes":  # (±1, ±1) on dims 0, 1, ±0.5 on dim 2, ±0.25 on dim 3: lambda 1, 1, 1/4, 1/16
        X = np.zeros((S, d))
        t = np.arange(S)
        X[:, 0] = np.where(t & 1, 1.0, -1.0)
        X[:, 1] = np.where(t & 2, 1.0, -1.0)
        X[:, 2] = np.where(t & 4, 0.5, -0.5)
        X[:, 3] = np.where(t & 8, 0.25, -0.25)
        return X + np.round(c * 4) / 4  # an exact offset keeps every entry exact in bfloat16
    if kind == "tied_rotated":  # the same spectrum in a random frame (ties up to rounding)
        Qm, _ = np.linalg.qr(rng.normal(size=(d, 4)))
        t = np.arange(S)
        coef = np.stack([np.where(t & 1, 1.0, -1.0), np.where(t & 2, 1.0, -1.0),
                         np.where(t & 4, 0.5, -0.5), np.where(t & 8, 0.25, -0.25)], axis=1)
        return c + 3.0 * coef @ Qm.T
    if kind == "constant":
        return np.tile(c, (S, 1))
    if kind == "tiny":
        return 1e-3 * rng.normal(size=(S, d))
    if kind == "huge":
        return 1e3 * rng.normal(size=(S, d))
    raise ValueError(kind)


KINDS = ["distinct_2", "distinct_3", "distinct_5", "tied_axes", "tied_rotated", "constant", "tiny", "huge"]


@pytest.mark.parametrize("d,rank", [(128, 4), (64, 8)])
def test_summaries_on_edge_blocks_against_the_oracle(api, d, rank):
    import torch
    rng = np.random.default_rng(77 + d + rank)
    nb = 3  # blocks per pair, all of the pair's kind
    Hkv = len(KINDS)
    K64 = np.stack([np.concatenate([_block(k, rng, d) for _ in range(nb)]) for k in KINDS])[None]  # [1, Hkv, nb S, d]
    Kt = torch.from_numpy(K64.astype(np.float32)).to(torch.bfloat16)
    K = Kt.float().double().numpy()  # the bfloat16 keys both sides read
    print(f"[summaries edge] d={d} rank={rank} kinds={KINDS}", flush=True)
    shape = api.make_shape(1, Hkv, Hkv, d, nb * S)
    mean = torch.full((1, Hkv, nb, d), float("nan"), device="cuda")
    factor = torch.full((1, Hkv, nb, rank, d), float("nan"), device="cuda")
    api.bsattn_build_summaries(shape, Kt.cuda(), rank, 0, nb, nb, mean, factor)
    torch.cuda.synchronize()
    mean_g = mean.cpu().numpy().astype(np.float64)
    fac_g = factor.cpu().numpy().astype(np.float64)
    assert np.isfinite(mean_g).all() and np.isfinite(fac_g).all()
    for g, kind in enumerate(KINDS):
        m_ref, f_ref = oracle.block_summaries(K[0, g], S, rank)
        kmax = float(np.abs(K[0, g]).max())
        assert np.abs(mean_g[0, g] - m_ref).max() <= 1e-6 * kmax + 1e-30, f"mean of {kind}"
        lam, vec = block_spectra(K[0, g], nb, S)
        slack = eig_error(lam, rank) + 1e-6 * np.sqrt(lam[:, :1])
        n1, n2 = check_factor_rows(fac_g[0, g], f_ref, lam, vec, rank, slack)
        print(f"[summaries edge] {kind}: rows checked singly {n1}, as clusters {n2}", flush=True)
        if kind == "constant":
            assert np.all(fac_g[0, g] == 0.0), "a constant block's factor rows are not exactly zero"
        if kind.startswith("distinct"):
            m = int(kind.split("_")[1])
            # rows past the covariance's rank m - 1 carry only the rounding of the mean
            past = fac_g[0, g][:, m - 1:]
            assert np.all(np.linalg.norm(past, axis=2) <= 1e-5 * np.sqrt(lam[:, :1])), f"rows past the rank of {kind}"
