"""bench.py's command-line contract on a machine without a GPU: more than one
GPU is refused with a message and exit status 2 before anything touches a
device, and the help text lists the workloads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("llama8b_32k", "qwen7b_32k", "llama8b_128k_loop", "mistral7b_step"):
        assert w in r.stdout


def test_algorithmic_bytes_of_the_32k_launch():
    """The roofline numerator at the Llama 32K shape, worked by hand: 8 kv heads
    x (25 bf16 windows x 128 tokens x 128 dims x 2 (K, V) x 2 bytes + 139 INT2
    entries x 128 x 128 x 3/4 bytes (2-bit codes plus fp16 scale and min per 32
    values)), plus the bf16 query and fp32 output of 32 heads x 128 dims, the
    fp32 masses of 32 heads x 256 windows and the 256 page-table entries."""
    sys.path.insert(0, ROOT)
    import bench
    from workload import CONFIGS
    kv = 8 * (25 * 128 * 128 * 2 * 2 + 139 * 128 * 128 * 3 // 4)
    io = 32 * 128 * 2 + 32 * 128 * 4 + 32 * 256 * 4 + 256 * 4
    assert kv + io == 26829824
    assert bench.attn_bytes(CONFIGS["llama8b_32k"], 25, 139, 256) == 26829824
