"""Host-side checks of the benchmark's command line (no GPU needed)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""  # no JSON line for an unsupported run


def test_path_choices_match_the_binding():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    from sparse_attention_long_router_amd.binding import MogaForward
    path = bench.make_parser()._option_string_actions["--path"]
    assert tuple(path.choices) == MogaForward.PATHS
    assert path.default == MogaForward.PATHS[0]
