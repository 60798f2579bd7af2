"""The bench's host-side contract, on the CPU: it imports, refuses more than one GPU with a
message, and its oracle timing leg reports what it measured."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_reports_threads_and_sample():
    sys.path.insert(0, ROOT)
    import bench
    from gated_deltanet_linear_decode_amd import configs, synth

    class Rot:
        pass

    rot = Rot()
    shape = configs.TINY.with_(num_state_slots=8)
    rot.w_cpu, rot.call_cpu = synth.make_weights(shape, 0), synth.make_call(shape, 2, 0)
    many = bench.cpu_baseline(shape, rot, 2, 0.2)
    one = bench.cpu_baseline(shape, rot, 2, 0.2, single_thread=True)
    for r in (many, one):
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
        assert "oracle decode calls" in r["sample"]
    assert one["cores"] == 1
