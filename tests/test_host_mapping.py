"""Host-side check of the prefill work mapping (kvc_device.h, compiled as plain
C++ against the HIP headers): the snake order of position blocks deals each
32-position block of a chunk to exactly one (item, slot), and the planner's
per-item key range (prefill_item_end) is the end of the item's last block.
Chunked prefill: news.myit.tw continuous-batching article, "Chunked prefill"."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_snake_block_mapping(tmp_path):
    exe = tmp_path / "prefill_map_check"
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'batching_kv_append_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "native", "prefill_map_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
