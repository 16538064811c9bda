"""Child process of test_abi_sanitizers.py: loads the sanitizer build of the
host layer given on the command line in place of libsdpa.so, runs the CPU ABI
battery (tests/test_abi_cpu.py) against it, then requires that no call reached
a kernel launcher stand-in.  With a second argument, instead calls the planted
overrun of that control library and expects never to return."""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)


def main():
    if len(sys.argv) == 3:
        ctl = ctypes.CDLL(sys.argv[2])
        ctl.planted_overrun.restype = ctypes.c_int
        ctl.planted_overrun.argtypes = [ctypes.c_int]
        print("planted overrun returned", ctl.planted_overrun(16), flush=True)
        return 0

    from head_attention_fwd_amd import _binding
    _binding.load_library(sys.argv[1])
    import pytest
    rc = pytest.main(["-q", "-s", "-p", "no:cacheprovider", os.path.join(HERE, "test_abi_cpu.py")])
    if rc != 0:
        return int(rc)
    lib = ctypes.CDLL(sys.argv[1])
    lib.sdpa_test_stub_launches.restype = ctypes.c_int
    launches = lib.sdpa_test_stub_launches()
    print("sanitized host layer: launcher calls %d" % launches, flush=True)
    return 0 if launches == 0 else 3


if __name__ == "__main__":
    sys.exit(main())
