"""Host-side checks of the rocprofv3 summary tool (no GPU, no profiler).

The traffic record feeds the benchmark's roofline: when one program runs
several instances of a kernel slot (the V-slice calls use other head dims
than the workload), the record must hold the workload's own instance.
"""
import csv
import json

from vision_transformer_attention_psa_amd import rocprof_summary as rs

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
CALIB = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, "
         "at::native::binary_internal::MulFunctor<float> > >")
# bwd_main instances: the workload's (dk = dv = 64) and a V-slice call's (dv = 32), in that order
MAIN64 = "_ZN3psa20psa_bwd_fused_kernelIDF16bLi64ELi64ELi2ELi64ELi3ELi64ELi4ELb1ELb1EEEvPKT_"
MAIN32 = "_ZN3psa20psa_bwd_fused_kernelIDF16bLi64ELi32ELi2ELi64ELi3ELi64ELi4ELb1ELb1EEEvPKT_"
PRE64 = "_ZN3psa18psa_bwd_pre_kernelIDF16bLi64ELb1EEEvPKT_S3_PKfPfii"
PRE32 = "_ZN3psa18psa_bwd_pre_kernelIDF16bLi32ELb1EEEvPKT_S3_PKfPfii"


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": val})


def test_traffic_keeps_the_workloads_instance(tmp_path):
    # calibration: 1 MiB moved reads 512 fetch units (2 KiB each) and 1024 write units (1 KiB each)
    fetch = [(CALIB, 512.0), (MAIN64, 1000.0), (MAIN64, 1000.0), (PRE64, 10.0), (MAIN32, 7.0), (PRE32, 3.0)]
    write = [(CALIB, 1024.0), (MAIN64, 100.0), (MAIN64, 100.0), (PRE64, 1.0), (MAIN32, 9.0), (PRE32, 5.0)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(fp, "FETCH_SIZE", fetch)
    _write(wp, "WRITE_SIZE", write)
    out_json, out_md = tmp_path / "t.json", tmp_path / "t.md"
    rs.traffic(str(fp), str(wp), "highres_n6400_bf16", 1, str(out_json), str(out_md), "cmd", "abc")
    rec = json.load(open(out_json))
    got = rec["workloads"]["highres_n6400_bf16"]
    assert rec["fingerprint"] == "abc"
    assert got["bwd_main"] == 1000.0 * 2048 + 100.0 * 1024
    assert got["bwd_pre"] == 10.0 * 2048 + 1.0 * 1024
    md = open(out_md).read()  # every instance is still listed
    assert "bwd_main<bf16,64,64," in md and "bwd_main<bf16,64,32," in md


def test_short_names():
    assert rs.short_name(MAIN64).startswith("bwd_main<bf16,64,64,2,64,3,64,4")
    assert rs.short_name(PRE32) == "bwd_pre<bf16,32>"
    demangled = "void psa::psa_fwd_kernel<float, 16, 16, 1, 4, 32, true, 0>(float const*, float*, float*, int)"
    assert rs.short_name(demangled) == "fwd<f32,16,16,1,4,32>"
