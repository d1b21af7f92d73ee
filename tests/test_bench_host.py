"""Host-side checks of bench.py (no GPU): it measures one GPU only and says so for
more."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr



def test_kernel_hash_ignores_comments_and_layout_only():
    import bench
    src = 'int f(int a) {\n    // twice\n    return a * 2; /* done */\n}\nconst char *s = "x  //y";\n'
    same = 'int f(int a)\n{\n  return a * 2;\n}\n\n// note\nconst char *s = "x  //y";'
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(src.replace("* 2", "* 3"))
    # text inside string literals is code
    assert bench._code_only(src) != bench._code_only(src.replace('"x  //y"', '"x //y"'))


def test_recorded_traffic_follows_the_kernel_sources():
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        sha = [l.split()[1] for l in f if l.startswith("kernel_sha ")]
    assert sha, "the traffic summary names the kernel sources it was taken on"
    assert (bench.recorded_traffic("gemv_nt4") is not None) == (sha[0] == bench.kernel_hash())
