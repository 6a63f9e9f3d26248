"""Host-side logic of bench.py (no GPU): the algorithmic byte and FLOP counts its
roofline fractions divide by, re-derived here from the model's dimensions (the
checkpoint layout in synth.py, the GPT-2 124M shape of the LeanExe GPT-2 README), the
position schedule of the timed steps, the traffic summary's source check, and the
one-GPU guard of --gpus."""
import os
import subprocess
import sys

import bench
import synth

D = synth.GPT2


def _block_matrix_weights(d=D):
    return sum(w for _, w, kind in synth.block_tensors(d) if kind == "matrix")


def _block_small_words(d=D):
    return sum(w for _, w, kind in synth.block_tensors(d) if kind != "matrix")


def test_fp32_step_bytes_follow_from_the_layout():
    mats = 4 * D.n_layer * _block_matrix_weights()
    head = 4 * D.vocab * D.d_model
    small = 4 * (D.n_layer * _block_small_words() + 2 * D.d_model)  # blocks + final LayerNorm
    emb = 4 * 2 * D.d_model  # one token row and one position row
    assert bench.F32_FIXED == mats + head + small + emb
    assert bench.KV_PER_POS == 4 * D.n_layer * 2 * D.d_model
    assert bench.LOGITS == 4 * D.vocab


def test_int8_and_binary16_step_bytes_follow_from_the_layout():
    # int8: one byte per weight; one binary32 scale per 64 inputs of every output row
    rows_k = [(3 * D.d_model, D.d_model), (D.d_model, D.d_model), (D.d_ff, D.d_model), (D.d_model, D.d_ff)]
    codes = D.n_layer * _block_matrix_weights() + D.vocab * D.d_model
    scales = 4 * (D.n_layer * sum(r * (k // 64) for r, k in rows_k) + D.vocab * (D.d_model // 64))
    small = 4 * (D.n_layer * _block_small_words() + 2 * D.d_model)
    assert bench.Q8_FIXED == codes + scales + small + 4 * 2 * D.d_model
    # binary16: two bytes per weight, binary32 embedding rows
    f16 = 2 * (D.n_layer * _block_matrix_weights() + D.vocab * D.d_model)
    assert bench.F16_FIXED == f16 + small + 4 * 2 * D.d_model


def test_prefill_and_batched_flop_counts():
    T = 128
    gemm = 2 * T * D.n_layer * _block_matrix_weights()
    # causal attention: q.k and the weighted sum, 2 FLOP per multiply-add, over keys 0..t
    attn = D.n_layer * D.n_head * 2 * 2 * D.head_dim * sum(t + 1 for t in range(T))
    assert bench.PREFILL_FLOP == gemm + attn
    assert bench.BATCH_FLOP == 2 * bench.BATCH * (D.n_layer * _block_matrix_weights() + D.vocab * D.d_model)
    # the vector FMA rate the batched fraction divides by: 256 CUs x 4 SIMDs x 16 lanes x 2 x 2.4 GHz
    assert abs(bench.FP32_VECTOR_PEAK_TF - 256 * 4 * 16 * 2 * 2.4e9 / 1e12) < 0.05


def test_step_bytes_grow_with_the_cache():
    assert bench.step_bytes(bench.F32_FIXED, 0) == bench.F32_FIXED + bench.KV_PER_POS + bench.LOGITS
    assert bench.step_bytes(bench.F32_FIXED, 127) - bench.step_bytes(bench.F32_FIXED, 0) == 127 * bench.KV_PER_POS


def test_timed_positions_span_the_session():
    assert sorted(bench.spread_positions(128)) == list(range(128))
    p20 = bench.spread_positions(20)
    assert len(set(p20)) == 20 and min(p20) == 0
    assert {p // 16 for p in p20} == set(range(8))  # 20 steps visit every 16-position range
    # any 128 consecutive steps visit every position once
    assert sorted(bench.spread_positions(128, start=57)) == list(range(128))


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(monkeypatch, tmp_path):
    summary = tmp_path / "traffic.md"
    summary.write_text("# t\n- sources_sha256: `abc`\n- traffic_bytes_per_launch: `123`\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "abc")
    assert bench.measured_traffic() == 123
    assert bench.measured_traffic("traffic_bytes_per_launch_q8") is None
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "def")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
