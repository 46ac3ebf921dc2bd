"""Host-side checks of the counter analysis (fine_grained_mixture_top_amd.hbm_traffic).

The kernel names are the ones rocprofv3 reports for one layer step; every
GEMM of the step must land in its own row, the weight-gradient kernel's two
launches per step alternating dW1 / dW2, and the calibration copy must scale
the counters to the copy's known size.
"""
import csv
import json

from fine_grained_mixture_top_amd import hbm_traffic as H

STEP = [  # one fg7b_bf16 layer step, in launch order, with the expected row
    ("void moe::grouped_gemm_kernel<unsigned short, 128, 128, false, 1, false, moe::EpiStore<unsigned short, "
     "float, 128, 128, 256>, 1>(moe::GemmShape, moe::Operand, moe::Operand, moe::EpiStore<unsigned short, "
     "float, 128, 128, 256>::Params)", "router_logits"),
    ("void moe::(anonymous namespace)::k_topk<4>(float const*, int, int, int, int, int*, float*, unsigned char*, "
     "int*)", None),
    ("void moe::g5::grouped_gemm5_kernel<true, true, moe::g4::G4SwiGLU>(moe::GemmShape, moe::Operand, "
     "moe::Operand, unsigned int, unsigned int, moe::g4::G4SwiGLU::Params)", "up"),
    ("void moe::g4::grouped_gemm4_kernel<false, true, false, moe::g4::G4Store>(moe::GemmShape, moe::Operand, "
     "moe::Operand, unsigned int, unsigned int, moe::g4::G4Store::Params)", "down"),
    ("void moe::(anonymous namespace)::k_aggregate_o<unsigned short, 3>(unsigned short const*, float const*, "
     "int const*, int const*, int, int, unsigned short*)", "agg_o"),
    ("void moe::g5::grouped_gemm5_kernel<false, false, moe::g5::G5DH>(moe::GemmShape, moe::Operand, "
     "moe::Operand, unsigned int, unsigned int, moe::g5::G5DH::Params)", "dh"),
    ("void moe::(anonymous namespace)::k_router_dz<unsigned short>(float const*, int, float const*, int const*, "
     "int const*, int const*, int, int, float*, float*, unsigned short*)", "router_grad"),
    ("void moe::g5::grouped_gemm5_kernel<false, false, moe::g4::G4StoreRouter>(moe::GemmShape, moe::Operand, "
     "moe::Operand, unsigned int, unsigned int, moe::g4::G4StoreRouter::Params)", "dxt"),
    ("void moe::(anonymous namespace)::k_aggregate_o<unsigned short, 3>(unsigned short const*, float const*, "
     "int const*, int const*, int, int, unsigned short*)", "agg_dx"),
    ("void moe::grouped_gemm_kernel<unsigned short, 128, 64, true, 1, false, moe::EpiStore<unsigned short, "
     "float, 128, 64, 256>, 1>(moe::GemmShape, moe::Operand, moe::Operand, moe::EpiStore<unsigned short, "
     "float, 128, 64, 256>::Params)", "dwr"),
    ("moe::(anonymous namespace)::k_wgt_plan(int const*, int, int, int, int, int*, HIP_vector_type<int, 4u>*, "
     "moe::PlanUnit*)", None),
    ("void moe::g4::grouped_gemm4_kernel<true, true, false, moe::g4::G4StoreW>(moe::GemmShape, moe::Operand, "
     "moe::Operand, unsigned int, unsigned int, moe::g4::G4StoreW::Params)", "dw1"),
    ("void moe::g4::grouped_gemm4_kernel<true, true, false, moe::g4::G4StoreW>(moe::GemmShape, moe::Operand, "
     "moe::Operand, unsigned int, unsigned int, moe::g4::G4StoreW::Params)", "dw2"),
]


def test_classify_one_step():
    seen = {"n": 0}
    for _ in range(2):  # two steps: the dW1 / dW2 alternation carries over
        got = [H.classify(name, seen) for name, _ in STEP]
        assert got == [want for _, want in STEP]


def test_every_step_gemm_has_its_own_row():
    seen = {"n": 0}
    rows = [H.classify(name, seen) for name, _ in STEP]
    gemms = [r for r in rows if r in ("up", "down", "dh", "dxt", "dw1", "dw2")]
    assert sorted(gemms) == sorted(set(gemms)) and len(gemms) == 6


def _write_csv(path, counter, dispatches):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for did, (name, kib) in enumerate(dispatches, 1):
            for part in (0.25, 0.75):  # a counter reported by several instances is summed
                w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": kib * part})


def test_main_calibrates_with_the_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    up, dh = STEP[2][0], STEP[5][0]
    gib = 1 << 30
    # the copy's fetch counter reads half its bytes, its write counter all of them
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, gib / 2048), (up, 1000.0), (dh, 300.0), (dh, 500.0)])
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, gib / 1024), (up, 10.0), (dh, 20.0), (dh, 40.0)])
    out = tmp_path / "t.json"
    H.main(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(gib), str(out))
    res = json.loads(out.read_text())
    assert abs(res["fetch_factor"] - 2.0) < 1e-12 and abs(res["write_factor"] - 1.0) < 1e-12
    k = res["kernels"]
    assert set(k) == {"up", "dh"}
    assert k["up"]["fetch_bytes"] == 2 * 1000.0 * 1024 and k["up"]["write_bytes"] == 10.0 * 1024
    assert k["dh"]["dispatches"] == 2
    assert k["dh"]["fetch_bytes"] == 2 * 400.0 * 1024 and k["dh"]["write_bytes"] == 30.0 * 1024
    assert res["source_hash"] == H.source_hash()
