"""Host-side checks of bench.py: the work it divides by (the roofline's numerator), the
one-GPU contract, and the rule that a stored traffic figure is reported only for its own
workload and kernel source. No GPU is used."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_saliency_amd import synth  # noqa: E402


def _random_routing(rng, B, Hkv, T, C, k):
    """k distinct ascending positions in every complete chunk, as the routing output holds them."""
    nCc = T // C
    sel = np.zeros((B, Hkv, nCc, k), dtype=np.int32)
    for b in range(B):
        for h in range(Hkv):
            for c in range(nCc):
                sel[b, h, c] = np.sort(rng.choice(C, size=k, replace=False)) + c * C
    return sel


def _pairs_by_partition(sel, T, C, w, G):
    """Softmax pairs counted one by one from the partition rule: key j <= i is a softmax key
    of query i when it lies in the window (j > i - w) or in an earlier chunk and selected."""
    B, Hkv = sel.shape[:2]
    n = 0
    for b in range(B):
        for h in range(Hkv):
            chosen = np.zeros(T, dtype=bool)
            chosen[sel[b, h].reshape(-1)] = True
            for i in range(T):
                j = np.arange(i + 1)
                sa = (j > i - w) | ((j // C < i // C) & chosen[j])
                n += int(sa.sum())
    return n * G


@pytest.mark.parametrize("w,k,T", [(64, 8, 300), (16, 4, 257), (0, 8, 200), (64, 64, 192), (1, 16, 130)])
def test_softmax_pair_count_matches_partition(w, k, T):
    rng = np.random.default_rng(w * 1000 + k * 10 + T)
    B, Hq, Hkv, C = 2, 4, 2, 64
    wl = synth.Workload("count", B, T, Hq, Hkv, 64, 64, w, C, k, "bf16", seed=0)
    sel = _random_routing(rng, B, Hkv, T, C, k)
    got = bench.algorithmic_work(wl, sel)["sa_pairs"]
    assert got == _pairs_by_partition(sel, T, C, w, Hq // Hkv)


def test_layer_flops_add_up():
    """The attention kernel's share plus the prep side's (saliency, key-side NP-Map and state
    update) is the layer total, and a softmax pair costs 4 D flops."""
    rng = np.random.default_rng(5)
    wl = synth.Workload("sum", 1, 256, 4, 1, 64, 64, 64, 64, 8, "bf16", seed=0)
    sel = _random_routing(rng, 1, 1, 256, 64, 8)
    r = bench.algorithmic_work(wl, sel)
    T, Hq, Hkv, D, F = 256, 4, 1, 64, 64
    win = np.minimum(np.arange(T) + 1, 64).sum()
    prep = 2.0 * D * win * Hq + (2.0 * F * D + 2.0 * F) * Hkv * T + 2.0 * D * F * Hkv * T
    assert r["flops"] == pytest.approx(r["attn_flops"] + prep, rel=1e-12)
    assert r["attn_flops"] - (2.0 * F * D + 2.0 * F + 2.0 * D * F) * Hq * T == pytest.approx(4.0 * D * r["sa_pairs"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout
    assert not r.stdout.strip().startswith("{")


def test_traffic_needs_the_same_workload_and_source(tmp_path):
    sha = bench.source_sha1(bench.ATTN_SRCS)
    p = tmp_path / "traffic.txt"
    p.write_text(f"# comment: ignored\nhbm_bytes_per_launch: 12345\nworkload: wl-a\nsource_sha1: {sha}\n")
    assert bench.measured_traffic("wl-a", str(p)) == 12345.0
    assert bench.measured_traffic("wl-b", str(p)) is None
    p.write_text("hbm_bytes_per_launch: 12345\nworkload: wl-a\nsource_sha1: 0000\n")
    assert bench.measured_traffic("wl-a", str(p)) is None
    assert bench.measured_traffic("wl-a", str(tmp_path / "missing.txt")) is None


def test_counter_summary_names_and_shares(tmp_path):
    from linear_attention_saliency_amd import profile_summary as PS

    assert PS._short_name("_ZN5still13bwd_dq_kernelIDF16bLi128ELi128ELi2EEEvNS_7BwdArgsE") == "bwd_dq_kernel<bf16,128,128,2>"
    assert PS._short_name("_ZN5still11scan_kernelIDF16bLi32EEEvPviiiPKfPfii") == "scan_kernel<bf16,32>"
    assert PS._short_name("_ZN5still11attn_kernelIfLi64ELi64ELi4EEEvNS_8AttnArgsE") == "attn_kernel<f32,64,64,4>"
    assert PS._short_name("still::bwd_dw_sum_kernel(float const*, float*, int, int)") == "bwd_dw_sum_kernel"
    # one kernel over two passes: 4 waves, 16 VALU and 8 MFMA instructions in all; 102400 MFMA
    # busy cycles summed over the SIMDs against 1024 SIMDs x 8000 / 8 active cycles is 10%
    k = "_ZN5still11attn_kernelIDF16bLi64ELi64ELi4EEEvNS_8AttnArgsE"
    hdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    (tmp_path / "p1").mkdir()
    (tmp_path / "p2").mkdir()
    (tmp_path / "p1" / "run_counter_collection.csv").write_text(
        hdr + f"1,{k},SQ_WAVES,4\n1,{k},SQ_VALU_MFMA_BUSY_CYCLES,102400\n1,{k},SQ_WAVE_CYCLES,1000\n1,{k},SQ_WAIT_ANY,250\n")
    (tmp_path / "p2" / "run_counter_collection.csv").write_text(
        hdr + f"1,{k},SQ_INSTS_VALU,16\n1,{k},SQ_INSTS_MFMA,8\n1,{k},GRBM_GUI_ACTIVE,8000\n")
    rows = PS.counters([str(tmp_path / "p1"), str(tmp_path / "p2")]).splitlines()
    assert len(rows) == 3
    cells = [c.strip() for c in rows[2].strip("|").split("|")]
    assert cells[0] == "attn_kernel<bf16,64,64,4>"
    assert cells[2].startswith("4 / 2 / ")  # per wave
    assert cells[3] == "2.0"                 # VALU per MFMA
    assert cells[4] == "10.0%"               # 102400 / (1024 SIMDs * 8000 / 8)
    assert cells[6] == "25% of wave time"


def test_attention_kernel_name_follows_the_launch_rule():
    """bench.py names the attention kernel the library launches: the fixed-frame kernel for
    bf16, head_dim = feat_dim (64 or 128), window = chunk and four query heads per routing
    head."""
    import bench
    from linear_attention_saliency_amd import synth
    assert bench.attention_kernel_name(synth.L1B_16K, "kv_head") == "attn_ff_kernel"
    assert bench.attention_kernel_name(synth.L8B_4K, "kv_head") == "attn_ff_kernel"
    assert bench.attention_kernel_name(synth.L8B_4K.replace(feat_dim=64), "kv_head") == "attn_kernel"
    assert bench.attention_kernel_name(synth.L1B_16K, "query_head") == "attn_kernel"
    assert bench.attention_kernel_name(synth.L1B_16K.replace(window=32), "kv_head") == "attn_kernel"
    assert bench.attention_kernel_name(synth.TINY_F32, "kv_head") == "attn_kernel"
