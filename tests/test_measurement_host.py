"""Host logic of the measurement tooling (no GPU): kernel naming in the rocprofv3
summaries, the traffic calibration arithmetic, and the staleness rule that turns
the committed HBM byte counts off once a measured kernel's sources change."""
import csv
import json
import os

import pytest

from kv_cache_vector_diag_amd import rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,short", [
    ("void tq::(anonymous namespace)::encode128_kernel<2, true, 1>(tq::(anonymous namespace)::Enc128Args)",
     "encode_keys"),
    ("void tq::(anonymous namespace)::encode128_kernel<4, false, 1>(tq::(anonymous namespace)::Enc128Args)",
     "encode_values"),
    ("void tq::(anonymous namespace)::encode_tiled_kernel<256, true>(tq::(anonymous namespace)::TiledArgs)",
     "tiled_keys"),
    ("void tq::(anonymous namespace)::split256_kernel<3, 4, false>(tq::(anonymous namespace)::SplitArgs)",
     "split256_values"),
    ("void tq::(anonymous namespace)::score128_kernel<2>(tq::(anonymous namespace)::Score128Args)", "score"),
    ("void tq::(anonymous namespace)::split256_prep_kernel(tq::(anonymous namespace)::PrepArgs)",
     "split256_prep"),
    ("void tq::(anonymous namespace)::attend_fused_kernel<1, 2>(tq::(anonymous namespace)::FusedArgs)",
     "attend_fused"),
    ("void tq::(anonymous namespace)::attend_qprep_kernel<1>(tq::(anonymous namespace)::QprepArgs)",
     "attend_qprep"),
    ("void tq::(anonymous namespace)::attend_merge_kernel(tq::(anonymous namespace)::MergeArgs)",
     "attend_merge"),
    ("void tq::(anonymous namespace)::gram_scores_fast_kernel<5, 32, 4>(tq::GramScoreArgs)", "gram_scores"),
    ("tq::(anonymous namespace)::gram_scores_generic_kernel(tq::GramScoreArgs, int, int, int, long)",
     "gram_scores_generic"),
    ("tq::(anonymous namespace)::gram_encode_kernel(tq::GramEncArgs)", "gram_encode"),
    ("void tq::(anonymous namespace)::encode128_pair_kernel<2, 3, 1>(tq::(anonymous namespace)::Enc128Args, "
     "tq::(anonymous namespace)::Enc128Args)", "encode_pair"),
    ("void tq::(anonymous namespace)::encode_wide_kernel<0, true>(tq::(anonymous namespace)::WideArgs)",
     "wide_keys"),
    ("void tq::(anonymous namespace)::encode_wide_kernel<2, false>(tq::(anonymous namespace)::WideArgs)",
     "wide_values"),
    ("void tq::(anonymous namespace)::decode_wh_kernel<128, false>(tq::(anonymous namespace)::DecodeWHArgs)",
     "decode_values"),
    ("__amd_rocclr_copyBuffer", "copy"),
])
def test_short_names(name, short):
    assert rs.short_name(name) == short


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_calibration_and_staleness(tmp_path, monkeypatch):
    enc = "void tq::(anonymous namespace)::encode128_kernel<2, true, 1>(x)"
    cp = "__amd_rocclr_copyBuffer"
    # the copy of 1 GiB reads back half its bytes in FETCH_SIZE and all in WRITE_SIZE
    _counter_csv(tmp_path / "f.csv", [(enc, "FETCH_SIZE", 1000.0), (enc, "FETCH_SIZE", 1002.0)])
    _counter_csv(tmp_path / "w.csv", [(enc, "WRITE_SIZE", 300.0)])
    _counter_csv(tmp_path / "cf.csv", [(cp, "FETCH_SIZE", 524288.0), (cp, "FETCH_SIZE", 10.0)])
    _counter_csv(tmp_path / "cw.csv", [(cp, "WRITE_SIZE", 1048576.0)])
    out = tmp_path / "traffic.json"
    rs.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
             "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
             "--map", "encode_keys=encode_c3", "--out", str(out)])
    ent = json.load(open(out))["encode_c3"]
    assert ent["fetch_factor"] == pytest.approx(2.0)
    assert ent["write_factor"] == pytest.approx(1.0)
    assert ent["read_bytes"] == pytest.approx(1001.0 * 1024 * 2)
    assert ent["write_bytes"] == pytest.approx(300.0 * 1024)
    assert ent["kernel"] == "encode_keys"
    assert ent["source_sha"] == rs.kernel_sources_sha(ROOT, "encode_keys")

    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench._traffic("encode_c3", 0.0) == pytest.approx(ent["hbm_bytes_per_launch"])
    assert bench._traffic("score_c3", 0.0) is None            # never measured
    ent["source_sha"] = "0" * 16                                # sources changed since
    json.dump({"encode_c3": ent}, open(out, "w"))
    assert bench._traffic("encode_c3", 0.0) is None


def test_kernel_source_sets_exist():
    for kern, files in rs.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.normpath(os.path.join(ROOT, "kv_cache_vector_diag_amd", "csrc", f))), f
        assert len(rs.kernel_sources_sha(ROOT, kern)) == 16


def test_traffic_of_a_step_of_kernels(tmp_path, monkeypatch):
    """A map entry a+b+c=key sums the kernels' per-dispatch means (one launch
    of each per step) and hashes the union of their sources."""
    qp = "void tq::(anonymous namespace)::attend_qprep_kernel<1>(x)"
    fu = "void tq::(anonymous namespace)::attend_fused_kernel<1, 2>(x)"
    mg = "tq::(anonymous namespace)::attend_merge_kernel(x)"
    cp = "__amd_rocclr_copyBuffer"
    _counter_csv(tmp_path / "f.csv", [(qp, "FETCH_SIZE", 10.0), (fu, "FETCH_SIZE", 1000.0), (fu, "FETCH_SIZE", 1004.0),
                                      (mg, "FETCH_SIZE", 40.0)])
    _counter_csv(tmp_path / "w.csv", [(qp, "WRITE_SIZE", 5.0), (fu, "WRITE_SIZE", 60.0), (mg, "WRITE_SIZE", 1.0)])
    _counter_csv(tmp_path / "cf.csv", [(cp, "FETCH_SIZE", 524288.0)])
    _counter_csv(tmp_path / "cw.csv", [(cp, "WRITE_SIZE", 1048576.0)])
    out = tmp_path / "traffic.json"
    step = "attend_qprep+attend_fused+attend_merge"
    rs.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
             "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
             "--map", f"{step}=attend_c4", "--out", str(out)])
    ent = json.load(open(out))["attend_c4"]
    assert ent["read_bytes"] == pytest.approx((10.0 + 1002.0 + 40.0) * 1024 * 2)
    assert ent["write_bytes"] == pytest.approx((5.0 + 60.0 + 1.0) * 1024)
    assert ent["source_sha"] == rs.kernel_sources_sha(ROOT, step)
    assert rs.kernel_sources_sha(ROOT, step) != rs.kernel_sources_sha(ROOT, "attend_merge")
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench._traffic("attend_c4", 0.0) == pytest.approx(ent["hbm_bytes_per_launch"])
