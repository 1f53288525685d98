"""GPU parity at the magnitudes where the decode's power-of-two normalisations matter.

The key scale folded into q, the value scale folded into the softmax weights and q itself
are each brought into the normal fp16 range by a power of two before they meet the matrix
cores.  These cases drive those exponents far from the N(0,1) workloads:

  * keys scaled by 2^-16 and 2^-24: fp16 key scales and zeros are subnormal (2^-24: a bit or
    two of precision), the scores are tiny and the softmax nearly uniform;
  * values scaled by 2^-16 and 2^-24: subnormal value scales and zeros;
  * keys scaled by 2^3, or q by 2^2: larger scores and a peaked softmax (kept where the
    binary32 rounding of a score stays well inside the bar);
  * q scaled by 2^-12: near-zero scores;
  * pages whose every key channel is constant over the page and values whose every
    32-channel group is constant: every scale is 0 and the zeros carry the values.

Powers of two keep the bf16 inputs exact.  Both sides quantize the scaled inputs and the
packed pages must be the same bytes (the pack's quotient by a subnormal fp16 scale
included).  Attention is linear in V: outputs of values scaled
by c are compared at the bar scaled by c.  That is the same relative accuracy the fp32 path
holds on unit-scale values, so a path that flushed a subnormal scale to zero or lost
an exponent would fail it.  The lse does not depend on V and keeps its own bar.
"""
import numpy as np
import pytest

from kvq_cases import ATOL, LSE_RTOL, Case, host_array, live_resid_equal, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def _scaled(t, f):
    import torch
    return (t.to(torch.float32) * f).to(t.dtype)


def _const_key_pages(k):
    """every key channel constant over each 32-token page (the page's first token)"""
    out = k.clone()
    T = k.shape[1]
    for g0 in range(0, T, 32):
        out[:, g0:g0 + 32] = k[:, g0:g0 + 1]
    return out


def _const_value_groups(v):
    """every 32-channel value group of every token constant (the group's first channel)"""
    out = v.clone()
    for j in range(4):
        out[..., 32 * j:32 * j + 32] = v[..., 32 * j:32 * j + 1]
    return out


def _run(kvq, orc, c, v_scale, what):
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages), f"{what}: packed pages differ"
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, c.lens), f"{what}: K residual differs"
    assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, c.lens), f"{what}: V residual differs"
    o_ref, l_ref = c.oracle_decode(orc)
    for pps in (0, 2):
        out, lse = c.device_decode(kvq, pages_per_split=pps)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"{what}: non-finite outputs"
        err = np.abs(out.astype(np.float64) - o_ref).max()
        assert err <= ATOL * v_scale, f"{what} pps={pps}: max abs err {err:.3e} > {ATOL * v_scale:.3e}"
        lerr = (np.abs(lse.astype(np.float64) - l_ref) / np.maximum(1.0, np.abs(l_ref))).max()
        assert lerr <= LSE_RTOL, f"{what} pps={pps}: lse rel err {lerr:.3e}"


CASES = [
    ("k*2^-16", 2.0 ** -16, 1.0, 1.0),
    ("k*2^-24", 2.0 ** -24, 1.0, 1.0),
    ("v*2^-16", 1.0, 2.0 ** -16, 1.0),
    ("v*2^-24", 1.0, 2.0 ** -24, 1.0),
    ("k*2^3", 2.0 ** 3, 1.0, 1.0),
    ("q*2^2", 1.0, 1.0, 2.0 ** 2),
    ("q*2^-12", 1.0, 1.0, 2.0 ** -12),
]


@pytest.mark.parametrize("kmode", [0, 1], ids=["keys-per-channel", "keys-per-token"])
@pytest.mark.parametrize("name,ks,vs,qs", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("kb,vb", [(4, 2), (2, 2), (4, 8), (8, 4)])
def test_scaled_inputs(kvq, orc, kb, vb, name, ks, vs, qs, kmode):
    log(f"magnitudes K{kb}V{vb} {name} kmode={kmode}")
    c = Case(kb, vb, H=2, G=4, lens=[200, 33, 517], seed=kb * 7 + vb + 31 * kmode, kmode=kmode)
    c.k, c.v, c.q = _scaled(c.k, ks), _scaled(c.v, vs), _scaled(c.q, qs)
    _run(kvq, orc, c, vs, f"K{kb}V{vb} {name} kmode={kmode}")


@pytest.mark.parametrize("kmode", [0, 1], ids=["keys-per-channel", "keys-per-token"])
@pytest.mark.parametrize("kb,vb,G", [(4, 2, 4), (8, 8, 7), (2, 4, 16)])
def test_constant_groups(kvq, orc, kb, vb, G, kmode):
    """All key scales 0 on every page and all value scales 0: codes are 0, values are the zeros."""
    log(f"constant groups K{kb}V{vb} G={G} kmode={kmode}")
    c = Case(kb, vb, H=2, G=G, lens=[96, 65, 300], seed=kb + vb + G + kmode, kmode=kmode)
    c.k = _const_key_pages(c.k) if kmode == 0 else _const_value_groups(c.k)
    c.v = _const_value_groups(c.v)
    _run(kvq, orc, c, 1.0, f"constant K{kb}V{vb} G={G} kmode={kmode}")
