"""Host checks of bench.py's own arithmetic (no GPU): the algorithmic bytes
and flops its roofline fractions divide by, the counter file's source-digest
check, and the refusal of a multi-GPU run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gated_delta_rule_83_amd import inputs as gi  # noqa: E402


def test_prefill_algorithmic_bytes_by_hand():
    """The layer shape B8 T4096 H16 d128, bf16 q/k/v/o, fp32 gates: per token
    and head q, k, v, o at 256 bytes each, a and b at 512, w at 512; plus the
    fp32 final state of every head."""
    c = gi.config(1)
    by, fl = bench.prefill_algorithmic(c, 32)
    per_token_head = 4 * 128 * 2 + 2 * 128 * 4 + 128 * 4
    assert by == 8 * 4096 * 16 * per_token_head + 8 * 16 * 128 * 128 * 4 == 1350565888
    # flops per token and head at C = 32: 4C d_k + 4C d_v + 8 d_k d_v + C^2/3 + d_k d_v / C
    assert fl == pytest.approx((4 * 32 * 128 * 2 + 8 * 128 * 128 + 32 * 32 / 3 + 128 * 128 / 32) * 8 * 4096 * 16)
    # bf16 pre-activation gates: the gate bytes halve
    by2, _ = bench.prefill_algorithmic(c, 32, gate_bytes=2)
    assert by - by2 == 8 * 4096 * 16 * (2 * 128 * 2 + 128 * 2)


def test_decode_algorithmic_bytes_by_hand():
    """N256 H16 d128: the fp32 state read and written (128 KiB per head), bf16
    v, o, fp32 a, b, w per head, bf16 q, k per query/key head."""
    per_head = 128 * 128 * 4 * 2 + 128 * 2 * 2 + 128 * 4 * 2 + 128 * 4
    assert bench.decode_algorithmic(256, 16, 16, 128, 128) == 256 * 16 * per_head + 256 * 16 * 128 * 2 * 2
    assert bench.decode_algorithmic(256, 16, 16, 128, 128) == 547356672


def test_traffic_is_read_only_for_its_own_source(tmp_path):
    """A counter summary counts only when its digest is the kernel sources'."""
    digest = bench.source_digest(bench.PREFILL_KERNEL_SOURCES)
    f = tmp_path / "t.txt"
    f.write_text(f"# header: ignored\nkernel_source_digest: {digest}\nhbm_bytes_per_launch: 123\n")
    assert bench.read_traffic(str(f), digest) == 123.0
    f.write_text("kernel_source_digest: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    assert bench.read_traffic(str(f), digest) is None
    assert bench.read_traffic(str(tmp_path / "missing.txt"), digest) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
