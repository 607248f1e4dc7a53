"""CPU checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_counter_hash_covers_every_kernel_source():
    """The HBM counters in profiles/ are used only while the kernel sources
    hash to the value stored with them; every device source must be hashed."""
    import bench
    csrc = os.path.join(ROOT, "persistent_rnn_fwd_amd", "csrc")
    device_sources = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    assert device_sources == set(bench.KERNEL_SOURCES), device_sources ^ set(bench.KERNEL_SOURCES)
    assert len(bench.kernel_source_hash()) == 16
