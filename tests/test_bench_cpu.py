"""Host-side checks of bench.py: the algorithmic byte counts that the roofline
fractions divide by, spelled out tensor by tensor for the 2.7B-layer workload,
and the single-GPU contract of its command line."""
import os
import subprocess
import sys

import bench
import ssd_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_bytes_of_the_headline_workload():
    w = si.WORKLOADS["m2p7_bf16"]
    assert (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype) == (4, 4096, 80, 64, 128, 1, "bf16")
    tokens = 4 * 4096
    x = tokens * 80 * 64 * 2            # bf16 input, read once
    y = tokens * 80 * 64 * 4            # fp32 output, written once
    dt = tokens * 80 * 4
    bc = 2 * tokens * 1 * 128 * 2       # B and C, one group, bf16
    per_head = 2 * 80 * 4               # A_log and D
    final = 4 * 80 * 64 * 128 * 4       # one fp32 final state per (row, head)
    assert bench.algorithmic_bytes(w, init_nonzero=False) == x + y + dt + bc + per_head + final == 527_434_368
    # a given initial state is read once more
    assert bench.algorithmic_bytes(w, init_nonzero=True) == 527_434_368 + final


def test_backward_bytes_of_the_headline_workload():
    w = si.WORKLOADS["m2p7_bf16"]
    tokens = 4 * 4096
    reads = (tokens * 80 * 64 * 2 + 2 * tokens * 128 * 2     # x, B, C
             + tokens * 80 * 4 + 2 * 80 * 4                  # dt, A_log, D
             + tokens * 80 * 64 * 4                          # dy
             + 4 * 80 * 64 * 128 * 4)                        # dfinal
    writes = (tokens * 80 * 64 * 4 + tokens * 80 * 4         # dx, ddt
              + 2 * tokens * 128 * 4                         # dB, dC (fp32)
              + 4 * 80 * 64 * 128 * 4                        # dinit
              + 3 * 80 * 4)                                  # dA_log, dD, ddt_bias
    assert bench.backward_algorithmic_bytes(w, init_nonzero=False) == reads + writes


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_metric_names_its_workload():
    assert bench.metric_name(si.WORKLOADS["m2p7_bf16"]) == \
        "SSD fwd tokens/sec (2.7B-layer shape, T=4096) and % of MFMA/HBM roofline"
    m = bench.metric_name(si.WORKLOADS["long_n256"])
    assert m.startswith("SSD fwd tokens/sec (long_n256: b=1, T=16384, H=32, P=64, N=256, bf16)")
