"""bench.py's command-line contract on a host without a GPU: several GPUs are
refused with a message before anything touches a device, and the algorithmic
work it reports follows the closed forms stated in its docstring."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_work_closed_forms():
    sys.path.insert(0, ROOT)
    import bench
    w = bench.algorithmic_work(4096, 4096, 262144)
    assert w["syrk"] == 4096 * 4097 * 262144            # d(d+1)n flops: one triangle
    assert w["prep"] == 2 * 4096 ** 3 / 3               # potrf, trtri
    assert bench.algorithmic_work(4096, 4096, 262144, three_step=True)["prep"] == \
        4 * 4096 ** 3 / 3                                # potrf, trtri, lauum, potrf
    nb = 4096 // 128
    assert w["lazy"] == 4096 * 128 * 128 * nb * (nb - 1)  # rows * B^2 * nb (nb - 1)


def test_three_step_has_no_act_order_variant():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--three-step",
                        "--act-order"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--three-step has no act-order variant" in r.stderr
    assert r.stdout.strip() == ""
