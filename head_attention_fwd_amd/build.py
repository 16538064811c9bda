"""Build libsdpa.so (HIP, gfx950) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libsdpa.so")
# calibration kernels for the measurements (bench.py --overlap-probe), not the attention path
CALIB_LIBRARY = os.path.join(HERE, "libsdpa_calib.so")
CALIB_SOURCES = ["sdpa_calib.hip"]
# the same sources with per-workgroup timestamps (SDPA_TIMELINE, csrc/sdpa_timeline.h),
# loaded only by bench.py --timeline
TIMELINE_LIBRARY = os.path.join(HERE, "libsdpa_timeline.so")
SOURCES = ["sdpa_api.hip", "sdpa_decode_row.hip", "sdpa_fwd_generic.hip", "sdpa_fwd_mfma.hip",
           "sdpa_fwd_mfma_wide.hip", "sdpa_proj_gemm.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    # no packed fp32 VALU instructions (v_pk_{add,mul,fma}_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the softmax reads every score, and
    # AGPR-resident accumulators would cost a v_accvgpr_read per score
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc(sources, target, verbose, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + list(extra) + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature flag
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building %s" % os.path.basename(target))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, target)
    return target


def build(verbose: bool = False) -> str:
    """Compile every HIP source of the attention path into head_attention_fwd_amd/libsdpa.so,
    the same sources with timestamps into libsdpa_timeline.so, and the calibration
    kernels into libsdpa_calib.so (three hipcc processes at once)."""
    jobs = [(SOURCES, LIBRARY, ()), (SOURCES, TIMELINE_LIBRARY, ("-DSDPA_TIMELINE",)),
            (CALIB_SOURCES, CALIB_LIBRARY, ())]
    with ThreadPoolExecutor(len(jobs)) as ex:
        done = [ex.submit(_hipcc, src, tgt, verbose, extra) for src, tgt, extra in jobs]
        return [f.result() for f in done][0]


if __name__ == "__main__":
    print(build(verbose=True))
