"""The benchmark's byte accounting (the roofline's algorithmic bytes) against the closed
forms of the workloads, computed here term by term: the full pages covering the attended
tokens at 512 * (kb + vb + 2) bytes per page and KV head, the live bf16 residual tokens
(K and V), q in bf16, out and lse in fp32; for the prefill pack the bf16 source plus the
pages.  The per-layer tables are checked against their equivalent bit widths."""
import pytest

import bench

B, H, HQ, D = 16, 8, 32, 128


def _page(kb, vb):
    return 512 * (kb + vb + 2)


def test_llama_table_is_the_3_25_bit_layout():
    pairs = bench.CONFIGS["llama"]["pairs"]
    assert len(pairs) == 32
    assert [i for i, p in enumerate(pairs) if p == (4, 8)] == [0, 1, 2, 31]
    assert sum(kb + vb for kb, vb in pairs) / (2 * len(pairs)) == 3.25
    assert sum(kb + vb for kb, vb in bench.CONFIGS["qwen"]["pairs"]) / (2 * 28) == 4.0


def test_llama_decode_step_bytes():
    """C = 4096 cached tokens + the appended one: 128 full pages and 1 residual token per
    (sequence, KV head)."""
    pairs = bench.CONFIGS["llama"]["pairs"]
    pages = sum(B * H * 128 * _page(kb, vb) for kb, vb in pairs)
    assert pages == 2_281_701_376
    resid = 32 * B * H * 1 * D * 2 * 2
    q = 32 * B * HQ * D * 2
    out = 32 * B * HQ * D * 4
    lse = 32 * B * HQ * 4
    assert (resid, q, out) == (2_097_152, 4_194_304, 8_388_608)
    total = pages + resid + q + out + lse
    per_layer = [bench.decode_alg_bytes(kb, vb, B, H, HQ, 4097) for kb, vb in pairs]
    assert sum(per_layer) == total == 2_296_446_976
    assert sum(per_layer) / 32 == 71_763_968      # the bench's mean bytes per launch
    # with the append (read of the new K, V; write into the residual slot) for every layer
    assert sum(per_layer) + 32 * bench.append_alg_bytes(B, H) == total + 32 * (2 * B * H * D * 2 * 2)


def test_ragged_bytes_follow_each_length():
    """A sequence of length L costs floor(L/32) pages and L mod 32 residual tokens."""
    lens = [1, 31, 32, 33, 64, 4097]
    kb, vb = 4, 2
    expect = 0
    for L in lens:
        expect += H * (L // 32) * _page(kb, vb) + H * (L % 32) * D * 2 * 2
    expect += len(lens) * HQ * D * (2 + 4) + len(lens) * HQ * 4
    assert bench.ragged_decode_alg_bytes(kb, vb, lens, H, HQ) == expect


def test_prefill_pack_bytes():
    """32,768 bf16 tokens per layer: the 4 GiB source and 1,140,850,688 bytes of pages over
    the 32 layers; 169,869,312 bytes per launch on average."""
    cfg = bench.CONFIGS["pack"]
    T = cfg["context"]
    assert (cfg["batch"], T) == (1, 32768)
    src = 32 * T * H * D * 2 * 2
    pages = sum(T // 32 * H * _page(kb, vb) for kb, vb in cfg["pairs"])
    assert (src, pages) == (4_294_967_296, 1_140_850_688)
    assert (src + pages) / 32 == pytest.approx(169_869_312)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """bench.py measures one GPU; asked for more (flag or launcher) it exits with status 2
    and says why, before touching torch or the GPU."""
    import os
    import subprocess
    import sys
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), *argv],
                       capture_output=True, text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""
