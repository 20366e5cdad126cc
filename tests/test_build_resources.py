"""CPU check of the compiled kernels' resources (the compiler's
kernel-resource-usage report written by the build): no kernel spills registers
to scratch memory, and the decode step's two grouped GEMMs (gate/up with SiLU*up,
and down) keep four waves per SIMD."""
import importlib
import os

import pytest


@pytest.fixture(scope="module")
def resources():
    import ffn_int4_g128_amd as q
    b = importlib.import_module("ffn_int4_g128_amd.build")
    if not os.path.exists(b.RESOURCES) or not os.path.exists(q.LIB_PATH):
        q.build()
    rows = []
    for line in open(b.RESOURCES):
        src, name, *kv = line.split()
        rows.append((src, name, {k: int(v) for k, v in (x.split("=") for x in kv)}))
    return rows


def test_every_kernel_reported(resources):
    names = " ".join(n for _, n, _ in resources)
    for k in ("qgemm_kernel", "prefill_big_kernel", "prefill_small_kernel", "route_sort_kernel",
              "quantize_act_kernel", "pack_codes8_kernel", "quantize_kernel"):
        assert k in names, k


def test_no_kernel_spills(resources):
    spills = [(s, n, r["scratch"]) for s, n, r in resources if r.get("scratch", 0) != 0]
    assert not spills, spills


@pytest.mark.parametrize("epi", [1, 0])
def test_grouped_decode_gemms_keep_four_waves(resources, epi):
    # qgemm_kernel<4 tiles, 1 M tile, fp16 rows with a row exponent, 2 stages,
    # SiLU*up (1) or none (0: down), 128-wide groups>
    tag = f"qgemm_kernelILi4ELi1ELi3ELi2ELi{epi}ELi1E"
    hot = [r for _, n, r in resources if tag in n]
    assert hot and all(r["occupancy"] >= 4 and r["vgprs"] <= 128 for r in hot), hot
