"""GPU parity of ts_penalty_sample against the float64 oracle.

z (penalised, tempered logits): |z_gpu - z_ref| <= 1e-5 |z_ref|.
keep: bit-exact outside the bands |E(i) - top_p| <= 1e-4 and
|p_i / p_max - min_p| <= 1e-4 (E(i) = mass before i in (p desc, id asc)).
probs: |q_gpu - q_ref| <= 1e-5 max(q_ref) (not in the stated bar; derived
from fp32 softmax error). token: a kept id whose oracle CDF interval
contains u up to 1e-5.
"""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from oracle import penalty_sample
from synth import CONFIGS, penalty_inputs
from tests.gpu_util import banner

pytestmark = pytest.mark.gpu
F32 = np.float32


def _run(x, penalty, temp, top_p, min_p, shared=False):
    logits = torch.from_numpy(x["logits"]).cuda()
    window = torch.from_numpy(np.ascontiguousarray(x["window"])).cuda()
    u = torch.from_numpy(x["u"]).cuda()
    z, keep, probs, tok = ts.penalty_sample(logits, window, penalty, temp, top_p, min_p, u=u)
    torch.cuda.synchronize()
    return z.cpu().numpy(), keep.cpu().numpy().astype(bool), probs.cpu().numpy(), tok.cpu().numpy()


def _compare(x, penalty, temp, top_p, min_p):
    z, keep, probs, tok = _run(x, penalty, temp, top_p, min_p)
    r = penalty_sample(x["logits"], x["window"], float(F32(penalty)), float(F32(temp)), float(F32(top_p)),
                       float(F32(min_p)), x["u"])
    assert np.all(np.abs(z - r.z) <= 1e-5 * np.abs(r.z))
    band = (np.abs(r.excl_mass - float(F32(top_p))) <= 1e-4) | (np.abs(r.ratio - float(F32(min_p))) <= 1e-4)
    mism = (keep != r.keep) & ~band
    assert not mism.any(), np.argwhere(mism)[:10]
    rows = r.z.shape[0]
    for i in range(rows):
        if ((keep[i] != r.keep[i]) & band[i]).any():
            continue  # a band token changed the kept set: normalisation differs
        assert np.max(np.abs(probs[i] - r.probs[i])) <= 1e-5 * r.probs[i].max()
        t = int(tok[i])
        assert keep[i, t]
        cdf = np.cumsum(r.probs[i])
        lo = cdf[t - 1] if t > 0 else 0.0
        assert lo - 1e-5 <= float(x["u"][i]) < cdf[t] + 1e-5
    return keep


def test_tiny_workload():
    c = CONFIGS["tiny"]
    banner("penalty tiny")
    x = penalty_inputs(c["seed"], 1, c["V"], c["W"], sigma=c["sigma"])
    _compare(x, 1.2, 1.0, 0.9, 0.05)


@pytest.mark.parametrize("name", ["1.5b", "7b", "8b", "14b"])
def test_vocab_sizes_table11(name):
    c = CONFIGS[name]
    banner(f"penalty {name} V={c['V']}")
    x = penalty_inputs(c["seed"], 2, c["V"], c["W"], sigma=c["sigma"])
    _compare(x, 1.2, 1.0, 0.9, 0.05)


@pytest.mark.parametrize("top_p,min_p,sigma", [(0.5, 0.0, 2.0), (0.9, 0.0, 2.0), (0.99, 0.0, 2.0), (1.0, 0.05, 2.0),
                                               (1.0, 0.5, 2.0), (0.9, 0.05, 1.4142), (0.0, 0.0, 2.0), (1.0, 1.0, 2.0),
                                               (1.0, 0.0, 2.0)])
def test_filter_regimes(top_p, min_p, sigma):
    banner(f"penalty regimes top_p={top_p} min_p={min_p}")
    x = penalty_inputs(21, 24, 128256, 1024, sigma=sigma)
    _compare(x, 1.2, 1.0, top_p, min_p)


@pytest.mark.parametrize("temp,penalty", [(0.4, 1.2), (1.2, 1.5), (0.7, 1.0)])
def test_temperature_and_penalty(temp, penalty):
    x = penalty_inputs(22, 3, 32000, 1024)
    _compare(x, penalty, temp, 0.9, 0.05)


def test_shared_window_duplicates_and_ragged_vocab():
    x = penalty_inputs(23, 3, 1001, 300, shared_window=True, dup_window=True)
    x["window"][:5] = [-1, 1001, 5000, -7, 3]
    _compare(x, 1.2, 1.0, 0.9, 0.05)


def test_exact_logit_ties():
    x = penalty_inputs(24, 2, 4096, 64, sigma=0.5)
    x["logits"][:, 100:140] = x["logits"][:, 7:8]    # 41 equal logits per row
    x["window"][:] = -1
    _compare(x, 1.2, 1.0, 0.3, 0.0)


def test_single_token_vocab_and_empty_window():
    x = penalty_inputs(25, 1, 1, 0)
    z, keep, probs, tok = _run(x, 1.2, 1.0, 0.9, 0.05)
    assert keep.tolist() == [[True]] and probs[0, 0] == 1.0 and tok[0] == 0


def test_top_p_cut_inside_min_p_set():
    """The min-p set carries almost all the mass, so top-p cuts inside it: the
    listed set is sorted and cut by prefix mass (several rows, ragged vocab)."""
    x = penalty_inputs(26, 4, 128251, 1024)
    rng = np.random.default_rng(26)
    x["logits"][:] = rng.normal(-6.0, 1.0, x["logits"].shape).astype(F32)
    for r in range(4):
        hot = rng.choice(128251, 300, replace=False)
        x["logits"][r, hot] = rng.normal(4.0, 1.0, 300).astype(F32)
    x["logits"][1, 5:9] = x["logits"][1, 4]   # ties inside the set
    for top_p in (0.5, 0.9, 0.0):
        _compare(x, 1.2, 1.0, top_p, 0.001)


def test_one_chunk_list_overflows():
    """Thousands of logits equal to the row maximum in one chunk overflow that
    chunk's candidate list: the whole-row radix select decides, ties ranked by id."""
    x = penalty_inputs(27, 3, 128256, 1024)
    top = x["logits"].max(axis=1)
    for r in range(3):
        x["logits"][r, 20000:23000] = top[r]
    x["window"][:] = -1
    _compare(x, 1.2, 1.0, 0.3, 0.05)
    _compare(x, 1.2, 1.0, 0.9, 0.05)


def test_min_p_set_larger_than_lds():
    """About 4500 min-p candidates spread so that no chunk list overflows but the
    row's set exceeds what one workgroup decides in LDS: radix-select path."""
    rows, V = 2, 128256
    x = penalty_inputs(28, rows, V, 1024)
    rng = np.random.default_rng(28)
    x["logits"][:] = np.float32(-20.0)
    for r in range(rows):
        hot = rng.choice(V, 4500, replace=False)
        x["logits"][r, hot] = rng.uniform(0.0, 1.0, 4500).astype(F32)
    x["window"][:] = -1
    _compare(x, 1.2, 1.0, 0.9, 0.05)


def test_rows_of_a_128_node_tree():
    """The logit rows of a step with a 128-node tree (128 + 4 draft rows)."""
    banner("penalty 132 rows")
    x = penalty_inputs(29, 132, 128256, 1024)
    _compare(x, 1.2, 1.0, 0.9, 0.05)


def test_largest_vocabulary():
    """V at the header's limit (262144 ids): the most chunks per row."""
    banner("penalty V=262144")
    x = penalty_inputs(30, 2, 262144, 1024)
    _compare(x, 1.2, 1.0, 0.9, 0.05)
    _compare(x, 1.2, 1.0, 0.5, 0.0)
