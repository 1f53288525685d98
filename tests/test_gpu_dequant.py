"""GPU parity of kvq_dequant: every token of a packed cache decoded back to binary32 equals
the oracle's binary64 page decode (code * s + z exact, E4M3 value * scale, bf16) rounded
once to binary32 -- bit-exact -- for all nine integer pairs in both key modes, FP8 with
calibrated scales and BF16; residual tokens come back as their bf16 values and tokens past
seq_len are left untouched."""
import numpy as np
import pytest

from kvq_cases import Case, host_array, log

pytestmark = pytest.mark.gpu

PAIRS = [(kb, vb) for kb in (2, 4, 8) for vb in (2, 4, 8)]


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def expected(orc, c):
    """The oracle's decode of the case's cache, [B][T][H][128] binary32 (zeros past seq_len)."""
    out_k = np.zeros((c.B, c.T, c.H, 128), dtype=np.float32)
    out_v = np.zeros_like(out_k)
    for b, L in enumerate(c.lens):
        for g in range(int(L) // 32):
            for h in range(c.H):
                ks, vs = (1.0, 1.0) if c.scales is None else (float(c.scales[h, 0]), float(c.scales[h, 1]))
                k, v = orc.dequant_page(c.o_pages[c.bt[b, g], h], c.kb, c.vb, c.kmode, ks, vs)
                out_k[b, 32 * g:32 * g + 32, h] = k.astype(np.float32)
                out_v[b, 32 * g:32 * g + 32, h] = v.astype(np.float32)
        t0 = int(L) // 32 * 32
        n = int(L) - t0
        if n:
            out_k[b, t0:L] = _bf16_to_f32(c.o_rk[b, :, :n]).transpose(1, 0, 2)
            out_v[b, t0:L] = _bf16_to_f32(c.o_rv[b, :, :n]).transpose(1, 0, 2)
    return out_k, out_v


def _check(kvq, orc, c):
    import torch
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    k, v = kvq.kvq_dequant(c.model, 0, c.cache, c.lens_d, c.T)
    torch.cuda.synchronize()
    ek, ev = expected(orc, c)
    assert np.array_equal(k.cpu().numpy().view(np.uint32), ek.view(np.uint32)), "K differs"
    assert np.array_equal(v.cpu().numpy().view(np.uint32), ev.view(np.uint32)), "V differs"


@pytest.mark.parametrize("kmode", [0, 1], ids=["keys-per-channel", "keys-per-token"])
@pytest.mark.parametrize("kb,vb", PAIRS)
def test_dequant_integer_bit_exact(kvq, orc, kb, vb, kmode):
    log(f"dequant K{kb}V{vb} kmode={kmode}")
    _check(kvq, orc, Case(kb, vb, H=2, G=1, lens=[77, 64, 5, 0, 200], seed=kb * 10 + vb + 100 * kmode,
                          kmode=kmode))


def test_dequant_fp8_and_bf16_bit_exact(kvq, orc):
    c = Case(8, 8, H=2, G=1, lens=[70, 33, 128], seed=4, kmode=2, scales=[[0.02, 0.01], [0.5, 0.003]])
    log("dequant fp8")
    _check(kvq, orc, c)
    log("dequant bf16")
    _check(kvq, orc, Case(16, 16, H=2, G=1, lens=[70, 33, 128], seed=5, kmode=3, src="f32"))


def test_dequant_leaves_tokens_past_seq_len(kvq, orc):
    """Output rows past seq_len keep the caller's contents; shorter lengths read fewer pages."""
    import torch
    c = Case(4, 2, H=2, G=1, lens=[96, 40], seed=8)
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    shape = (c.B, c.T, c.H, 128)
    k0 = torch.full(shape, 7.0, dtype=torch.float32, device=c.dev)
    v0 = torch.full(shape, -3.0, dtype=torch.float32, device=c.dev)
    short = torch.tensor([64, 40], dtype=torch.int32, device=c.dev)
    k, v = kvq.kvq_dequant(c.model, 0, c.cache, short, c.T, k_out=k0, v_out=v0)
    torch.cuda.synchronize()
    ek, ev = expected(orc, c)
    kk, vv = k.cpu().numpy(), v.cpu().numpy()
    assert np.array_equal(kk[0, :64], ek[0, :64]) and np.array_equal(vv[0, :64], ev[0, :64])
    assert (kk[0, 64:] == 7.0).all() and (vv[0, 64:] == -3.0).all()
    assert np.array_equal(kk[1, :40], ek[1, :40]) and (kk[1, 40:] == 7.0).all()
