"""Host-side logic of bench.py (no GPU): the one-GPU rule, the algorithmic
byte and flop counts the roofline divides by, and the code hash that ties
recorded counters to the kernel they were taken on."""
import subprocess
import sys

import numpy as np

import bench
import gen


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_bytes_per_written_token():
    # kv 1152 + cos/sin 256 + slot 8 read; ckv 1024 (bf16) or 512 + 4 (one
    # byte per code + float32 scale), k 128 written
    assert gen.kvrc_bytes_per_written_token(512, 64, "bf16") == 2568
    assert gen.kvrc_bytes_per_written_token(512, 64, "int8") == 2060
    assert gen.kvrc_bytes_per_written_token(512, 64, "fp8") == 2060


def test_paged_batch_bytes_count_skips_and_gamma():
    case = gen.make_config("decode_paged")
    total, tokens = bench.algorithmic_bytes(case)
    skipped = int((case["slot_mapping"] < 0).sum())
    assert tokens == case["B"] * case["S"]
    assert total == (tokens - skipped) * 2568 + skipped * 8 + 512 * 2


def test_selection_bytes_by_hand():
    case = gen.qsa_select_case(3, N=2, H=16, Di=32, Bcap=10, kbs=8, sel_ratio=2, cmp_ratio=1,
                               topk=4)
    kl = case["key_length"]
    want = sum(16 * 32 * 2 + (int(kl[n]) // 8) * 32 * 2 + 8 + case["Jcap"] * 4 + 4 * 4
               for n in range(2))
    assert bench.algorithmic_bytes(case) == (want, 2)


def test_mla_flops():
    case = gen.mla_kv_head_case(1, B=1, S=3, He=64, num_blocks=2, block_size=4)
    assert bench.algorithmic_flops(case) == 2 * 3 * 576 * 64


def test_code_hash_ignores_comments_not_code():
    src = "int f(int a)\n{\n    return a + 1;  // one more\n}\n"
    assert bench._code_only("k.hip", src) == bench._code_only(
        "k.hip", "/* a block\n comment */\n" + src.replace("// one more", "// other words"))
    assert bench._code_only("k.hip", src) != bench._code_only("k.hip", src.replace("+ 1", "+ 2"))
    py = "# note\nx = 1  # trailing\n"
    assert bench._code_only("b.py", py) == "x = 1  # trailing"


def test_committed_profiles_match_the_kernel_sources():
    """Every workload has a committed trace summary and traffic record, taken
    on the kernel code as it stands (the bench reports no traffic for a
    record of other code)."""
    import json
    import os
    for w in bench.WORKLOAD_TEXT:
        path = os.path.join(bench.ROOT, "profiles", f"traffic_{w}.json")
        assert os.path.exists(path), f"no traffic record for {w}"
        with open(path) as f:
            rec = json.load(f)
        assert rec["source_hash"] == bench.source_hash(w), f"{w}: profile taken on other code"
        # summaries are named <kernel>_<workload>.md
        names = os.listdir(os.path.join(bench.ROOT, "profiles"))
        assert any(name.endswith(f"_{w}.md") for name in names), f"no trace summary for {w}"
