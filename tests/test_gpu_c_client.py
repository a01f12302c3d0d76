"""The C ABI without Python in the loop: tests/c_abi/kvc_c_client (plain C11,
HIP runtime for memory and a stream) plans and compresses a ragged pool-16
batch written here from the seeded generator; its outputs are held to the
same bar as the Python-driven parity tests."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from kv_cache_compression_pool_amd import synth
from tests.c_abi.build_client import OUT as CLIENT
from tests.helpers import rel_err_rows
from tests.test_gpu_parity import VEC_TOL, check_codes, check_scales, note, reference_for

pytestmark = pytest.mark.gpu


def test_c_client_ragged_prefill_matches_oracle(tmp_path):
    assert os.path.exists(CLIENT), f"{CLIENT} is missing: run __graft_entry__.build()"
    d = synth.pool16_ragged(seed=9, num_seqs=7, max_len=900)
    d["seq_lens"].astype(np.int64).tofile(tmp_path / "seq_lens.i64")
    d["keys"].astype(np.uint16).tofile(tmp_path / "keys.u16")
    d["scores"].astype(np.uint16).tofile(tmp_path / "scores.u16")
    d["ape"].astype(np.float32).tofile(tmp_path / "ape.f32")
    note(f"C client: {d['seq_lens'].size} sequences, {d['keys'].shape[0]} rows")
    r = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"C client failed ({r.returncode}): {r.stderr}"
    note(r.stdout.strip())
    rows = np.fromfile(tmp_path / "rows.i32", np.int32)
    n = rows.size
    codes = np.fromfile(tmp_path / "codes.u8", np.uint8).reshape(n, 128)
    scales = np.fromfile(tmp_path / "scales.f32", np.float32)
    pooled = np.fromfile(tmp_path / "pooled.f32", np.float32).reshape(n, 128)
    assert np.array_equal(rows, oracle.pool_plan(d["seq_lens"]))
    assert n > 50
    rc, rs, rx = oracle.compress_prefill(d["keys"], d["scores"], d["ape"], rows, True)
    assert rel_err_rows(pooled, rx).max() <= VEC_TOL
    ref_c, ref_s, _ = reference_for(pooled, rx, rc, rs, True, "C client prefill")
    check_codes(codes, ref_c, "C client prefill")
    check_scales(scales, ref_s, True, "C client prefill")
