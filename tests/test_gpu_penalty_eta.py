"""GPU parity of ts_penalty_sample_eta against the float64 oracle.

z: |z_gpu - z_ref| <= 1e-5 |z_ref|. keep: bit-exact outside the band
|p_i / min(eta, max p) - 1| <= 1e-4 (the cutoff). probs: |q_gpu - q_ref| <=
1e-5 max(q_ref). token: a kept id whose oracle CDF interval contains u up
to 1e-5.
"""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from oracle import eta_sample
from synth import CONFIGS, penalty_inputs
from tests.gpu_util import banner

pytestmark = pytest.mark.gpu
F32 = np.float32


def _compare(x, penalty, temp, eps, alpha):
    logits = torch.from_numpy(x["logits"]).cuda()
    window = torch.from_numpy(np.ascontiguousarray(x["window"])).cuda()
    u = torch.from_numpy(x["u"]).cuda()
    z, keep, probs, tok = ts.penalty_sample_eta(logits, window, penalty, temp, eps, alpha, u=u)
    torch.cuda.synchronize()
    z, keep, probs, tok = z.cpu().numpy(), keep.cpu().numpy().astype(bool), probs.cpu().numpy(), tok.cpu().numpy()
    r = eta_sample(x["logits"], x["window"], float(F32(penalty)), float(F32(temp)), float(F32(eps)),
                   float(F32(alpha)), x["u"])
    assert np.all(np.abs(z - r.z) <= 1e-5 * np.abs(r.z))
    band = np.abs(r.ratio - 1.0) <= 1e-4
    mism = (keep != r.keep) & ~band
    assert not mism.any(), np.argwhere(mism)[:10]
    for i in range(r.z.shape[0]):
        if ((keep[i] != r.keep[i]) & band[i]).any():
            continue  # a band token changed the pool: normalisation differs
        assert np.max(np.abs(probs[i] - r.probs[i])) <= 1e-5 * r.probs[i].max()
        t = int(tok[i])
        assert keep[i, t]
        cdf = np.cumsum(r.probs[i])
        lo = cdf[t - 1] if t > 0 else 0.0
        assert lo - 1e-5 <= float(x["u"][i]) < cdf[t] + 1e-5
    return keep, r


@pytest.mark.parametrize("name", ["tiny", "1.5b", "7b", "8b", "14b"])
def test_vocab_sizes(name):
    c = CONFIGS[name]
    banner(f"eta {name} V={c['V']}")
    x = penalty_inputs(c["seed"] + 50, 2, c["V"], c["W"], sigma=c["sigma"])
    _compare(x, 1.2, 1.0, 3e-4, np.sqrt(3e-4))


@pytest.mark.parametrize("eps,alpha,sigma", [(3e-4, 0.0173, 2.0), (1e-3, 0.0316, 4.0), (0.02, 0.1, 1.0),
                                             (1.0, 1.0, 2.0), (0.5, 0.0, 2.0), (1.0, 1e6, 2.0), (1e-6, 1e-3, 0.5)])
def test_regimes_24_rows(eps, alpha, sigma):
    banner(f"eta regimes eps={eps} alpha={alpha} sigma={sigma}")
    x = penalty_inputs(60, 24, 128256, 1024, sigma=sigma)
    keep, r = _compare(x, 1.2, 1.0, eps, alpha)
    if alpha == 0.0:
        assert keep.all()
    if eps == 1.0 and alpha == 1e6:   # eta = 1 is above every probability: only the top token stays
        assert np.all(keep.sum(axis=1) == 1)


@pytest.mark.parametrize("temp,penalty", [(0.4, 1.2), (1.2, 1.5), (0.7, 1.0)])
def test_temperature_and_penalty(temp, penalty):
    x = penalty_inputs(61, 3, 32000, 1024)
    _compare(x, penalty, temp, 3e-4, 0.0173)


def test_ragged_vocab_and_shared_window():
    x = penalty_inputs(62, 5, 1001, 300, shared_window=True, dup_window=True)
    _compare(x, 1.2, 1.0, 0.01, 0.1)


def test_exact_logit_ties_at_the_top():
    x = penalty_inputs(63, 2, 50000, 0)
    x["logits"][:, 100:110] = 30.0     # ten tied maxima (above every N(0, 4) draw), all kept whatever eta is
    keep, _ = _compare(x, 1.0, 1.0, 1.0, 1e6)
    assert np.all(keep[:, 100:110])


@pytest.mark.parametrize("sigma", [1.0, 4.0])
def test_u_at_the_ends(sigma):
    """u = 0 takes the first kept id; u just below 1 the last kept one (the
    target can round up to the whole kept mass)."""
    x = penalty_inputs(64, 6, 128256, 1024, sigma=sigma)
    x["u"] = np.array([0.0, 1e-12, 0.5, 1.0 - 2.0 ** -24, 1.0 - 2.0 ** -20, 0.999], dtype=np.float32)
    keep, r = _compare(x, 1.2, 1.0, 3e-4, 0.0173)
    tok_first = np.argmax(keep[0])
    assert keep[0, tok_first]


def test_rows_of_a_128_node_tree():
    """The logit rows of a step with a 128-node tree (128 + 4 draft rows)."""
    banner("eta 132 rows")
    x = penalty_inputs(65, 132, 128256, 1024)
    _compare(x, 1.2, 1.0, 3e-4, 0.0173)


def test_largest_vocabulary():
    """V at the header's limit (262144 ids)."""
    banner("eta V=262144")
    x = penalty_inputs(66, 2, 262144, 1024)
    _compare(x, 1.2, 1.0, 3e-4, 0.0173)
