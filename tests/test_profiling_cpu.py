"""Host-side checks of the measurement plumbing: the rocprofv3 CSV readers
behind the committed traffic figures, and the profiling entry points' argument
handling (no GPU needed)."""

import ctypes
import os

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd import profiling as P


def test_short_name_strips_namespace_templates_and_arguments():
    n = "void msa::(anonymous namespace)::sparse_kv_outer<128, 3>(unsigned short const*, int)"
    assert P.short_name(n) == "sparse_kv_outer"
    assert P.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_counter_per_dispatch_averages_over_dispatches(tmp_path):
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True)
    rows = [
        # two dispatches of one kernel, counter split over two rows each (as per-XCD rows come)
        ("1", "void msa::(anonymous namespace)::k_a<1>(int)", "FETCH_SIZE", "10"),
        ("1", "void msa::(anonymous namespace)::k_a<1>(int)", "FETCH_SIZE", "5"),
        ("2", "void msa::(anonymous namespace)::k_a<1>(int)", "FETCH_SIZE", "20"),
        ("2", "void msa::(anonymous namespace)::k_a<1>(int)", "FETCH_SIZE", "25"),
        ("3", "__amd_rocclr_copyBuffer", "FETCH_SIZE", "7"),
        ("3", "__amd_rocclr_copyBuffer", "WRITE_SIZE", "9"),
    ]
    with open(d / "x_counter_collection.csv", "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for r in rows:
            fh.write(",".join(f'"{x}"' for x in r) + "\n")
    got = P.counter_per_dispatch(str(tmp_path / "run"), "FETCH_SIZE")
    assert got["k_a"] == (30.0, 2)
    assert got["__amd_rocclr_copyBuffer"] == (7.0, 1)
    assert P.counter_per_dispatch(str(tmp_path / "run"), "WRITE_SIZE") == {"__amd_rocclr_copyBuffer": (9.0, 1)}


def test_sources_hash_tracks_device_sources():
    h = P.kernel_sources_sha256("sparse_kv_outer")
    assert len(h) == 64 and h == P.kernel_sources_sha256("sparse_kv_outer")
    assert h != P.kernel_sources_sha256("index_scores_tiled")


def test_profile_end_rejects_null_count():
    lib = M.lib()
    assert lib.msa_profile_end(None, 0, None) == 1          # MSA_ERR_NULL
    n = ctypes.c_int32(-1)
    assert lib.msa_profile_end(None, 0, ctypes.byref(n)) == 0 and n.value == 0


def test_counters_table_lists_each_kernel_and_counter(tmp_path, capsys):
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True)
    rows = [
        ("1", "void msa::(anonymous namespace)::dense_prefill<128, 3>(int)", "SQ_INSTS_MFMA", "100"),
        ("1", "void msa::(anonymous namespace)::dense_prefill<128, 3>(int)", "SQ_INSTS_MFMA", "50"),
        ("1", "void msa::(anonymous namespace)::dense_prefill<128, 3>(int)", "SQ_INSTS_VALU", "600"),
        ("2", "void msa::(anonymous namespace)::dense_prefill<128, 3>(int)", "SQ_INSTS_MFMA", "250"),
        ("2", "void msa::(anonymous namespace)::dense_prefill<128, 3>(int)", "SQ_INSTS_VALU", "800"),
        ("3", "__amd_rocclr_copyBuffer", "SQ_INSTS_VALU", "4"),
    ]
    with open(d / "x_counter_collection.csv", "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for r in rows:
            fh.write(",".join(f'"{x}"' for x in r) + "\n")
    P.main(["counters", str(tmp_path / "run"), "--kernel", "dense_prefill"])
    out = capsys.readouterr().out.strip().splitlines()
    assert out[0] == "| kernel | dispatches | SQ_INSTS_MFMA | SQ_INSTS_VALU |"
    assert len(out) == 3                                  # header, rule, one kernel (the copy is filtered out)
    assert out[2] == "| `dense_prefill` | 2 | 200 | 700 |"
