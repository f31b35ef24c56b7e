"""Host-side pieces of bench.py: the algorithmic byte and FLOP model that `achieved` and
the roofline fractions are built on, worked out by hand for small cases."""
from dataclasses import replace

import bench
import workloads as W


def test_algorithmic_model_by_hand():
    # one user, one head, D = 2, history N = 3, k = 2 candidates, bf16 (2 bytes)
    w = replace(W.WORKLOADS[1], B=1, H=1, D=2, k=2)
    pf, pb, df, db = bench.algorithmic(w, [3])
    # prefill: N(N+1)/2 = 6 allowed pairs, 4D = 8 FLOPs each; bytes 6 N D e = 6*3*2*2
    assert pf == 6 * 8 and pb == 72
    # decode: k(N+1) = 8 pairs; bytes (2N + 4k) D e = (6 + 8) * 2 * 2
    assert df == 8 * 8 and db == 56


def test_algorithmic_model_serving_shape():
    # the 12-layer serving shape, one layer: 64 users x 8 heads, N = 512, D = 64, k = 1000
    w = W.WORKLOADS[3]
    pf, pb, df, db = bench.algorithmic(w, [512] * 64)
    assert pb == 6 * 512 * 64 * 2 * 64 * 8 == 201_326_592
    assert db == (2 * 512 + 4 * 1000) * 64 * 2 * 64 * 8 == 329_252_864
    assert df == 4 * 64 * 1000 * 513 * 64 * 8
    assert pf == 4 * 64 * (512 * 513 // 2) * 64 * 8


def test_kernel_source_hash_covers_the_kernel_sources():
    import os
    names = {os.path.basename(p) for p in bench.KERNEL_SRC}
    assert {"attn_bf16.hip", "lds_dma.h", "e4m3.h", "attn_launch.h"} <= names
    assert len(bench.kernel_source_hash()) == 16


def test_more_than_one_gpu_is_refused():
    # the bench measures one GPU; asking for more ends with a message and status 2,
    # before any device is touched
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "--gpus must be 1" in line["error"]


def test_every_profile_summary_names_its_sources_and_command():
    # each committed rocprofv3 summary records the source set it was taken on, that
    # set's hash as of the run, and the command that made it
    import os
    import re
    status = bench.profile_status()
    assert status, "no profile summaries"
    for name, st in status.items():
        assert st["sources"] in bench.PROFILE_SOURCES, name
        fields = bench.summary_fields(os.path.join(bench.PROFILES, name))
        assert re.fullmatch(r"[0-9a-f]{16}", fields["kernel_source_sha256"]), name
        with open(os.path.join(bench.PROFILES, name)) as f:
            text = f.read()
        assert "# Commands" in text, name
        assert "_work" not in text, name
    for kind, files in bench.PROFILE_SOURCES.items():
        for f in files:
            assert os.path.isfile(os.path.join(bench.CSRC, f)), (kind, f)
