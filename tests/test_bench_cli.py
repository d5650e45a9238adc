"""The benchmark's command-line contract that needs no GPU: more than one GPU is refused with a
one-line JSON message and a non-zero status, before anything touches a device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_activation_model_hand_computed():
    """The pages' activation model 11bshd + 5bhs^2 + 2bshd (appendix A.4.2) at values worked by hand:
    b=1, s=1024, h=64, d=128: 11*8388608 + 5*64*1048576 + 2*8388608 = 92274688 + 335544320 + 16777216;
    s=49152: 13*49152*8192 + 320*49152^2 = 5234491392 + 773094113280 (about 725 GiB)."""
    import bench
    assert bench.activation_model_bytes(1, 1024, 64, 128) == 444_596_224
    assert bench.activation_model_bytes(1, 49152, 64, 128) == 778_328_604_672
    assert bench.activation_model_bytes(2, 1024, 64, 128) == 2 * 444_596_224  # linear in the batch


def test_scratch_remark_parser():
    """The build's scratch check reads the compiler's kernel resource-usage remarks."""
    from mask_aware_dense_amd import build
    txt = ("a.hip:1:1: remark: Function Name: _ZN3mad1kEv [-Rpass-analysis=kernel-resource-usage]\n"
           "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]\n"
           "a.hip:9:1: remark: Function Name: _ZN3mad1jEv [-Rpass-analysis=kernel-resource-usage]\n"
           "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build._scratch_sizes(txt) == {"_ZN3mad1kEv": 24, "_ZN3mad1jEv": 0}
