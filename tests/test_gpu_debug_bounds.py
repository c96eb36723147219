"""The PAKV_DEBUG_BOUNDS build (libpakv_bounds.so) counts the page-table
entries outside the pool that the kernels meet, and only for positions a call
uses: a bad entry behind a sliding window is not counted.  Run in a child
process (bounds_case.py) that loads that build through PAKV_LIBRARY.

Expected counts (sequences of 70, 40, 100 positions; page 1 of sequence 1 and
page 0 of sequence 2 bad):
  clean store, decode and extend      0, 0, 0
  chunk store: sequence 0 rows 0..9, sequence 1 rows 16..31, sequence 2
  rows 0..3                           20 rows dropped
  row store: one row per sequence, two on bad pages    22
  full-layer decode: one bad chunk in sequences 1 and 2   plans 2
  sliding decode (W 32): only sequence 1's bad page is visible   plans 3
  extend: sequences 1 (kv [0, 40)) and 2 (kv [0, 100)), one workgroup each
                                      extend 2
"""

import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import need_gpu

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_debug_bounds_build_counts_bad_page_ids():
    need_gpu()
    sys.path.insert(0, os.path.dirname(HERE))
    from full_attention_amd.build import library_path
    lib = library_path("bounds")
    if not os.path.exists(lib):
        pytest.skip("libpakv_bounds.so is not built (__graft_entry__.build() builds it)")
    env = dict(os.environ, PAKV_LIBRARY=lib)
    print("[bounds] child: tests/bounds_case.py with", lib, flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "bounds_case.py")], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print("[bounds]", res, flush=True)
    assert res["reset"] == [0, 0, 0]
    assert res["clean_store"] == [0, 0, 0]
    assert res["clean_attend"] == [0, 0, 0]
    assert res["bad_chunk_store"] == [0, 20, 0]
    assert res["bad_row_store"] == [0, 22, 0]
    assert res["bad_full_decode"] == [2, 22, 0]
    assert res["bad_sliding_decode"] == [3, 22, 0]
    assert res["bad_extend"] == [3, 22, 2]
