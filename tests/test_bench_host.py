"""Host-side logic of bench.py, checked without a GPU: the single-GPU
refusal, the algorithmic bytes per token against the library's own pool
layout, and the rule that counter-based HBM traffic is reported only while
the kernel's source is the one the counters were taken on."""
import os
import subprocess
import sys

import pytest

import attention_quantized_kv_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("codec", [0, kvq.KVQ_CODEC_INT2])
@pytest.mark.parametrize("n_kv,D", [(4, 256), (2, 128), (8, 256)])
def test_bytes_per_token_match_the_pool_layout(codec, n_kv, D):
    """bench's algorithmic bytes per token and layer equal the library's pool
    size per cached token (pages of 256 tokens, every KV head)."""
    n_pages, P = 10, 256
    L = kvq.Layout(n_kv, D, P, n_pages, codec)
    assert kvq.kvq_pool_bytes(L) == n_pages * P * bench.kv_bytes_per_token_layer(n_kv, D, codec)


def test_decode_workload_bytes():
    """Q8_0 K + Q4_0 V at 4 KV heads and head_dim 256: 416 B per KV head and
    token; 262,144 tokens make the 436,207,616 bytes per layer the decode
    line reports.  The 2-bit cache takes 144 B per KV head and token."""
    assert bench.kv_bytes_per_token_layer(4, 256, 0) == 4 * 416
    assert bench.kv_bytes_per_token_layer(4, 256, 0) * 262144 == 436207616
    assert bench.kv_bytes_per_token_layer(4, 256, 1) == 4 * 144


def test_traffic_only_for_the_profiled_source(monkeypatch):
    """A committed counter row is reported while the kernel's source digest
    matches it, and dropped (None) once the source differs."""
    for workload, kname in (("decode262k", "attn_mfma_stream"), ("int2decode262k", "attn_int2")):
        rows = [l.split() for l in open(os.path.join(ROOT, "profiles", "hbm_traffic.txt"))
                if l.startswith(workload + " ")]
        assert len(rows) == 1
        if rows[0][2] != bench.source_digest(kname):
            pytest.skip(f"{kname} changed since its counters were taken")
        t = bench.measured_traffic(workload, kname)
        assert t == pytest.approx(float(rows[0][-1]))
    monkeypatch.setattr(bench, "source_digest", lambda kname: "0" * 64)
    assert bench.measured_traffic("decode262k", "attn_mfma_stream") is None
    assert bench.measured_traffic("no_such_workload", "attn_mfma_stream") is None


def test_prefill_outliers_are_the_generators_channels():
    """The timed prefill inputs carry the workload's outlier channels: the
    same seeded 1% of the flattened (head, dim) channels the oracle-side
    generators pick, scaled x20, and no other value changed."""
    import numpy as np
    import torch
    import synth
    w = synth.WORKLOADS["prefill262k"]
    ck, cv, cq = bench.outlier_channels(w, 0, "cpu")
    assert np.array_equal(ck.numpy(), synth.outlier_channels((0, w.wid, 0, synth.K), w.n_kv * w.head_dim))
    assert np.array_equal(cv.numpy(), synth.outlier_channels((0, w.wid, 0, synth.V), w.n_kv * w.head_dim))
    assert np.array_equal(cq.numpy(), synth.outlier_channels((0, w.wid, 0, synth.Q), w.n_heads * w.head_dim))
    assert len(ck) == 10 and len(cq) == 61
    x = torch.randn(5, w.n_kv, w.head_dim)
    y = bench.with_outliers(x.clone(), ck)
    xf, yf = x.reshape(5, -1), y.reshape(5, -1)
    assert torch.equal(yf[:, ck], xf[:, ck] * 20.0)
    mask = torch.ones(w.n_kv * w.head_dim, dtype=torch.bool)
    mask[ck] = False
    assert torch.equal(yf[:, mask], xf[:, mask])
    assert bench.outlier_channels(synth.WORKLOADS["decode262k"], 0, "cpu") == (None, None, None)


def test_cpu_model_is_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model() != ""


def test_source_digest_covers_the_included_headers(tmp_path, monkeypatch):
    """The digest that gates the committed traffic covers the kernel file and
    every local header it includes, directly or through another: an edit to
    kvq_quant.h (included by the streaming and 2-bit kernels, not the tiled
    one) changes exactly the digests of the kernels that include it."""
    import shutil
    src = os.path.join(ROOT, "attention_quantized_kv_amd", "csrc")
    dst = tmp_path / "attention_quantized_kv_amd" / "csrc"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.o"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    names = {k: [os.path.basename(f) for f in bench.kernel_source_files(k)]
             for k in ("attn_mfma_stream", "attn_int2", "attn_mfma_tiled")}
    assert names["attn_mfma_stream"][0] == "attn_mfma_stream.hip"
    assert {"kvq_internal.h", "kvq_mfma.h", "kvq_quant.h", "kvq_waits.h"} <= set(names["attn_mfma_stream"])
    assert {"kvq_internal.h", "kvq_mfma.h", "kvq_quant.h"} <= set(names["attn_int2"])
    assert "kvq_quant.h" not in names["attn_mfma_tiled"]
    before = {k: bench.source_digest(k) for k in names}
    with open(dst / "kvq_quant.h", "a") as f:
        f.write("\n// edited\n")
    after = {k: bench.source_digest(k) for k in names}
    assert after["attn_mfma_stream"] != before["attn_mfma_stream"]
    assert after["attn_int2"] != before["attn_int2"]
    assert after["attn_mfma_tiled"] == before["attn_mfma_tiled"]
