"""Host-side logic of bench.py (CPU only): the one-GPU contract, the algorithmic work counts
the roofline figures divide by, the parsing of rocprofv3 output and of clock tables, and the rule that stored
counter traffic is reported only for the kernel sources it was taken on."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("C", [32, 64, 128, 256])
def test_causal_flop_count_matches_pair_count(C):
    """(C+1)(dk+dv) per token is 2 (dk + dv) flops for each (query, key) pair at or below
    the diagonal of a chunk, averaged over its C tokens: count the pairs directly."""
    dk, dv = 96, 192
    pairs = sum(i + 1 for i in range(C))
    assert 2 * pairs * (dk + dv) == C * (C + 1) * (dk + dv)
    assert bench.fwd_flops_per_token_head(C) * C == 2 * pairs * (dk + dv) + 4 * dk * dv * C


@pytest.mark.parametrize("C", [32, 64, 128])
def test_issued_flop_count_counts_the_triangle_blocks(C):
    """Score blocks: NIB (NIB + 1) / 2 blocks of 16 x 16 x dk; output strips: strip K of 32
    queries against K + 1 key pairs of 32 x dv; plus Q S and K^T V in full."""
    dk, dv = 96, 192
    nib = C // 16
    blocks = sum(1 for ib in range(nib) for jb in range(nib) if jb <= ib)
    pairs = sum(1 for K in range(C // 32) for p in range(C // 32) if p <= K)
    total = blocks * 16 * 16 * dk * 2 + pairs * 32 * 32 * dv * 2
    assert bench.fwd_issued_flops_per_token_head(C) == total // C + 4 * dk * dv
    assert bench.fwd_issued_flops_per_token_head(C) >= bench.fwd_flops_per_token_head(C)


def test_byte_counts():
    # q, k (96) and v, o (192) in bf16 per token-head
    assert bench.FWD_BYTES_PER_TOKEN_HEAD["bf16"] == 1152
    # forward 1152 + backward (q, k, v, do in; dq, dk, dv out) + two bf16 96 x 192
    # snapshots per chunk (start state, state gradient), each written once and read once
    for C, want in ((32, 7680), (64, 5376), (128, 4224), (256, 3648)):
        assert bench.train_bytes_per_token_head(C) == want
        assert want == 1152 + 2 * (96 + 96 + 192 + 192) + 2 * (96 + 96 + 192) + 2 * 2 * (96 * 192 * 2) // C
    # decode: the 96 x 192 fp32 page read and written, q, k, v, o in bf16
    assert bench.DEC_BYTES_PER_SEQ_HEAD == 2 * 73728 + 1152
    assert bench.DEC_EPI_BYTES_PER_SEQ_HEAD == bench.DEC_BYTES_PER_SEQ_HEAD + 384


def test_short_kernel_names():
    assert bench._short_kernel_name("void gla::(anonymous namespace)::fwd_out_kernel<128, 104, 2, false>"
                                    "(gla::FwdArgs, gla::EpilogueArgs)") == "fwd_out_kernel<128, 104, 2, false>"
    assert bench._short_kernel_name("gla::dlambda_reduce_kernel(float const*, int)") == "dlambda_reduce_kernel"


def test_counter_groups_split_at_marker_copies():
    k = lambda name: {"kernel": name}
    disp = {1: k("void gla::fwd_bf16_kernel<128>(x)"), 2: k("void gla::grad_fused_bf16<128>(x)"),
            3: k("__amd_rocclr_copyBuffer"), 4: k("void gla::fwd_chain_kernel<128>(x)"),
            5: k("void gla::fwd_out_kernel<128>(x)"), 6: k("__amd_rocclr_copyBuffer"),
            7: k("void gla::fwd_bf16_kernel<128>(x)"), 8: k("__amd_rocclr_copyBuffer"),
            9: k("void gla::decode_kernel<>(x)"), 10: k("__amd_rocclr_copyBuffer")}
    groups, marks = bench._group_dispatches(disp)
    assert groups == {"train": [1, 2], "fwd": [4, 5], "long": [7], "decode": [9]}
    assert marks == [3, 6, 8, 10]


def test_stored_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "gated_linear_attention_simple_amd", "csrc"),
                    root / "gated_linear_attention_simple_amd" / "csrc")
    (root / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(root))
    digest = bench.src_digest("grad")
    rec = {"kernels": {"grad": {"src_digest": digest, "hbm_bytes_per_launch": 123.0}}}
    (root / "profiles" / "counters.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("grad", 1.0) == 123.0
    assert bench.stored_traffic("decode", 1.0) is None          # no record
    # a change to a source of the group voids it; a change elsewhere does not
    (root / "gated_linear_attention_simple_amd" / "csrc" / "gla_conv.hip").write_text("// changed\n")
    assert bench.stored_traffic("grad", 1.0) == 123.0
    with open(root / "gated_linear_attention_simple_amd" / "csrc" / "gla_grad_bf16.hip", "a") as f:
        f.write("\n// changed\n")
    assert bench.stored_traffic("grad", 1.0) is None


def test_clock_level_parsing():
    """The active level of a pp_dpm_* table is the line marked '*'; none marked: None."""
    assert bench._dpm_current("0: 500Mhz\n1: 1800Mhz *\n2: 2400Mhz\n") == "1800Mhz"
    assert bench._dpm_current("0: 900Mhz\n1: 1300Mhz\n") is None
    assert bench._dpm_current(None) is None


def test_machine_info_without_a_device():
    """On a host with no GPU the record still has every field (unknown ones null)."""
    import torch

    info = bench.machine_info(torch)
    for key in ("rocm", "torch", "hip_runtime", "sclk", "mclk"):
        assert key in info
    json.dumps(info)
