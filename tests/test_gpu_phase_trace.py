"""The tile-loop cycle accounting (bench.py --phase-trace, the diagnostic library) runs and
reports a consistent breakdown: every wave of the 216 workgroups of the Ulysses-2 share's launch
recorded its intervals, and a step takes at least the 64 MFMAs' 2048 cycles a SIMD issues in it.
The synthetic ping-pong beside it reports each variant, every interval with MFMAs again at least
the 32 MFMAs' 1024 cycles a SIMD issues per interval on average."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_phase_trace_reports_every_interval():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_attention_dits_amd.build import PHASE_TRACE_LIB
    if not os.path.exists(os.path.join(ROOT, "context_attention_dits_amd", PHASE_TRACE_LIB)):
        pytest.skip("diagnostic library not built")
    print("[case] bench.py --phase-trace (child process)", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--phase-trace"], capture_output=True,
                       text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads(r.stdout.strip().splitlines()[-1])["phase_trace"]
    assert rec["workload"] == "flux1024_ulysses2_bf16" and rec["workgroups"] == 216
    # 72 key tiles: 2 * 72 barriers per wave, the first three left out
    assert rec["intervals_per_wave"] == 2 * 72 - 3
    assert rec["cycles_per_step"] >= rec["mfma_cycles_per_simd_step"]
    for k in rec["intervals"]:
        for g in ("A", "B"):
            assert k[g]["work"] > 0 and k[g]["wait"] >= 0
            assert k[g]["work"] + k[g]["wait"] <= 1.5 * k["cycles"]
    mix = rec["synthetic_mix"]
    assert set(mix) == {"as_the_loop", "mfma_16x16x32", "fragments_in_registers", "groups_in_phase",
                        "fragment_reads_only", "fragment_reads_only_all_waves", "8_reads_one_half_early",
                        "16_reads_one_half_early"}
    for name, v in mix.items():
        assert v["ms"] > 0
        if "reads_only" not in name:
            assert v["cycles_per_interval"] >= 1024
    # the reads of all 8 waves take longer than those of 4
    assert mix["fragment_reads_only_all_waves"]["cycles_per_interval"] > mix["fragment_reads_only"]["cycles_per_interval"]
