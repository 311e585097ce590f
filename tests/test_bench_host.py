"""Host logic of bench.py, on the CPU: the algorithmic byte counts that the
roofline divides by kernel times, the source hash that guards the counter
figures, and the one-GPU guard.  The library is loaded only for its
host-side size query."""
import os
import shutil
import subprocess
import sys

import bench
from bit_quantized_routed_router_amd import synthetic as S

# packed sizes from the formats' block sizes: CB2 66 bytes and Q2K 84 bytes per 256 weights
CB2_GATE = 2048 * 4096 // 256 * 66
Q2K_DOWN = 4096 * 2048 // 256 * 84
EXPERT = 2 * CB2_GATE + Q2K_DOWN


def test_decode1_bytes():
    cfg = S.CONFIGS["decode1"]
    b = bench.decode_bytes(cfg, 6, T=1)
    assert EXPERT == 7_077_888
    # router F16 + shared F16 (3 matrices) + 6 experts + bf16 x in + fp32 y out
    assert b["total"] == 256 * 4096 * 2 + 3 * 2048 * 4096 * 2 + 6 * EXPERT + 4096 * 2 + 4096 * 4 == 94_920_704
    # stage 2: routed gate/up, shared gate and up, x16 in, routed and shared h out
    assert b["k_dec_stage2"] == 6 * 2 * CB2_GATE + 2 * 2048 * 4096 * 2 + 4096 * 2 + 6 * 2048 * 2 + 2048 * 2
    assert b["k_dec_stage2"] == 59_543_552
    assert b["k_dec_stage1"] == 256 * 4096 * 2 + 4096 * 2


def test_decode_bytes_follow_distinct_experts():
    cfg = S.CONFIGS["decode1"]
    for T in (2, 8, 16):
        a, b = bench.decode_bytes(cfg, 6, T=T), bench.decode_bytes(cfg, 12, T=T)
        assert b["total"] - a["total"] == 6 * EXPERT
        assert b["k_dec_stage2"] - a["k_dec_stage2"] == 6 * 2 * CB2_GATE
        assert b["k_dec_stage3"] - a["k_dec_stage3"] == 6 * Q2K_DOWN


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    src = os.path.join(bench.ROOT, "bit_quantized_routed_router_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    h0 = bench.kernel_source_hash(str(dst))
    assert h0 == bench.kernel_source_hash()
    p = dst / "prefill.hip"
    p.write_text(p.read_text() + "\n// a comment\n/* another\n comment */\n\n   \n")
    assert bench.kernel_source_hash(str(dst)) == h0
    p.write_text(p.read_text() + "\nstatic int ds4_extra_symbol = 1;\n")
    assert bench.kernel_source_hash(str(dst)) != h0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profiles_and_traffic_figure_name_one_source_hash():
    """The rocprofv3 summaries under profiles/ and the HBM traffic figure in
    bench.py come from one set of kernel sources: every summary names the
    same source hash, and it is the hash the traffic figure was taken at."""
    import re
    pdir = os.path.join(bench.ROOT, "profiles")
    hashes = {}
    for name in sorted(os.listdir(pdir)):
        if name.endswith(".md"):
            m = re.search(r"Kernel source hash \(bit_quantized_routed_router_amd/csrc\): `([0-9a-f]{16})`",
                          open(os.path.join(pdir, name)).read())
            assert m, f"{name} names no kernel source hash"
            hashes[name] = m.group(1)
    assert hashes and len(set(hashes.values())) == 1, hashes
    assert set(hashes.values()) == {bench.TRAFFIC_SOURCE_HASH}
