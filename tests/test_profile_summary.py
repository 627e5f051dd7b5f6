"""Host logic of the profile summariser: stage names of the library's kernels, and the split of one
bench run's dispatches into phases (one per workload) so that the same kernel at the same grid in two
workloads is kept apart."""
import csv

from latent_width_expert_amd import profile_summary as ps

GATEUP = "void k3::panel_gemm_kernel<1, 0, 4, 1, true, 0, false, 1>(k3::GemmArgs)"
MID = "void k3::panel_rows_kernel<0, 3, 4, 2>(k3::GemmArgs)"
PACK = "k3::pack_kernel(k3::PackJob)"
STREAM = "k3::stream_read_kernel(unsigned int const*, unsigned long, unsigned int*)"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<int>>(int)"


def test_stage_names():
    assert ps.stage_of(GATEUP) == "gateup"
    assert ps.stage_of(MID) == "down"
    assert ps.stage_of("void k3::tiled_f8_kernel<8, 12, 2, 2, 1, 1>(k3::GemmArgs)") == "gateup"
    assert ps.stage_of("void k3::skinny_reduce_kernel<3>(k3::GemmArgs, int)") == "y_gemm (reduce)"
    assert ps.stage_of(PACK) == "pack"
    assert ps.stage_of(FILL) is None


def _write_trace(path, seq):
    """seq: (kernel, grid, duration ns) in dispatch order."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for name, grid, dur in seq:
            w.writerow({"Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
                        "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 10


def test_phases_split_workloads(tmp_path):
    # stream read, the decode weights packed in two runs split by a fill, two decode steps; then a
    # second workload packs its own weights (again split) and runs the same kernel at the same grid
    seq = [(STREAM, 1024, 50), (PACK, 64, 5), (FILL, 64, 1), (PACK, 64, 5),
           (GATEUP, 256, 100), (MID, 256, 30), (GATEUP, 256, 102),
           (PACK, 64, 5), (FILL, 64, 1), (PACK, 64, 5),
           (GATEUP, 256, 300), (GATEUP, 256, 304)]
    p = tmp_path / "kt_kernel_trace.csv"
    _write_trace(p, seq)
    per = ps.trace(str(p))
    assert per[(GATEUP, 256, 1)] == [100, 102]
    assert per[(GATEUP, 256, 2)] == [300, 304]
    assert per[(MID, 256, 1)] == [30]
    assert per[(STREAM, 1024, 0)] == [50]
    # the packing that precedes a workload's steps belongs to it
    assert len(per[(PACK, 64, 1)]) == 2 and len(per[(PACK, 64, 2)]) == 2
    assert (PACK, 64, 0) not in per


def test_counter_passes_use_the_same_phases(tmp_path):
    seq = [(STREAM, 1024), (PACK, 64), (GATEUP, 256), (PACK, 64), (GATEUP, 256)]
    p = tmp_path / "c_counter_collection.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, (name, grid) in enumerate(seq, start=1):
            for c, v in (("FETCH_SIZE", 10.0 * d), ("GRBM_GUI_ACTIVE", 1.0)):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": c,
                            "Counter_Value": v})
        w.writerow({"Dispatch_Id": 6, "Kernel_Name": "copyBuffer", "Grid_Size": 4096, "Counter_Name": "FETCH_SIZE",
                    "Counter_Value": 524288.0})
    per, calib = ps.counter_passes(str(p))
    assert per[(GATEUP, 256, 1)]["FETCH_SIZE"] == 30.0
    assert per[(GATEUP, 256, 2)]["FETCH_SIZE"] == 50.0
    assert calib["FETCH_SIZE"] == 524288.0
