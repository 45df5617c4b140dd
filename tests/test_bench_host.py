"""bench.py's host-side contract, on the CPU: it runs on one GPU only, the
stored HBM counters are used only on the kernel source they were taken on, and
the CPU baseline record has the fields the result line reports."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_stored_traffic_is_used_only_on_its_kernel_source(monkeypatch):
    text = open(bench.COUNTERS_FILE).read()
    stored_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text).group(1)
    hbm = float(re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text).group(1))
    alg = float(re.search(r"alg_bytes_per_launch:\s*([0-9.eE+]+)", text).group(1))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: stored_hash)
    # scaled to this run's algorithmic bytes per launch
    assert bench.stored_traffic(alg) == round(hbm)
    assert bench.stored_traffic(alg / 2) == round(hbm / 2)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic(alg) is None


def test_kernel_source_hash_covers_the_decode_sources():
    names = sorted(os.path.basename(f) for f in bench.KERNEL_SRCS)
    assert names == ["pkv_decode_valu.h", "pkv_device.h", "pkv_internal.h", "pkv_kernels.hip"]
    assert re.fullmatch(r"[0-9a-f]{16}", bench.kernel_source_hash())


def test_cpu_baseline_record():
    """The record's fields, on a 4-sequence batch held in host tensors (the
    bench passes the last timed step's device tensors), and the max abs error
    between the given outputs and the oracle's: a planted error of 0.25 in one
    output element is what it reports."""
    import numpy as np
    import torch
    import pkv_workloads as W
    from oracle import pkv_oracle as O
    w = W.shaped_13b(seed=2, num_seqs=4)
    r = O.replay(w.ops, w.k_rows, w.v_rows, w.num_blocks, w.num_kv_heads, w.head_dim, w.initial_free_order)
    tables = [r.alloc.block_table(s) for s in w.decode_seqs]
    lens = np.array([r.alloc.num_tokens(s) for s in w.decode_seqs])
    ref = O.decode_attention(w.q, r.k_pool, r.v_pool, tables, lens, w.scale)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    out = torch.from_numpy(ref.astype(np.float32))
    out[1, 3, 7] += 0.25
    tensors = (bf16(w.q), bf16(r.k_pool), bf16(r.v_pool), out)
    rec = bench.cpu_baseline(lambda l: 2 if l is None else tensors, tables, lens, w.scale, 0.2, 2e-3)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s" and rec["cores"] == 1
    assert rec["value"] > 0 and "layers" in rec["sample"] and "best of 3" in rec["sample"]
    assert abs(rec["max_abs_err"] - 0.25) < 1e-6 and rec["tol"] == 2e-3
    assert rec["rows_checked"] in (4 * 40, 2 * 4 * 40)
    assert rec["all_cores"]["value"] > 0 and rec["all_cores"]["cores"] >= 1
