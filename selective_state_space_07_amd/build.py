"""Build libmamba_scan.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree under selective_state_space_07_amd/lib/ so that
it travels with the source tree. Device code is compiled with packed-FP32
instruction generation switched off.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libmamba_scan.so")
SOURCES = ["mamba_scan_api.cpp", "scan_fwd.hip", "scan_fwd_quad.hip", "scan_fwd_row.hip", "scan_step.hip",
           "scan_bwd.hip", "ssd.hip", "scan_noalloc.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    # no v_pk_{add,mul,fma}_f32 from the compiler
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(out=LIB, verbose=False, defines=(), sources=SOURCES):
    """Compile `sources` (by default every scan-library source) into `out`;
    raise CalledProcessError on failure. `defines` are extra NAME=VALUE
    preprocessor definitions (tuning knobs)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *["-D" + d for d in defines], "-I", os.path.join(HERE, "..", "include"),
           "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd, output="\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


MIXER_SOURCES = ["mixer/mamba_mixer.cpp", "mixer/mixer_conv.hip"]
MIXER_LIB = os.path.join(LIB_DIR, "libmamba_mixer.so")


def build_mixer(out=MIXER_LIB, scan_lib=LIB, verbose=False):
    """Compile the mixer layer library (rocBLAS projections around the scan
    library, which it links by name from its own directory)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(HERE, "..", "include"), "-I", os.path.join(rocm, "include"),
           "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in MIXER_SOURCES]
    cmd += ["-L", os.path.dirname(scan_lib), "-l:" + os.path.basename(scan_lib), "-L", os.path.join(rocm, "lib"),
            "-lrocblas", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd, output="\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


PROBE_SOURCES = ["probe/valu_probe.hip"]
PROBE_LIB = os.path.join(LIB_DIR, "libmamba_probe.so")


def build_probe(out=PROBE_LIB, verbose=False):
    """Compile the VALU issue-rate probe (bench.py --valu-probe), the
    measurement behind the prefill's ALU roofline."""
    return build(out=out, verbose=verbose, sources=PROBE_SOURCES)


def device_asm(source="scan_fwd.hip", defines=()):
    """Return the gfx950 assembly of one source (for inspection)."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], *["-D" + d for d in defines],
           "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, source)]
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_mixer(verbose=True))
    print(build_probe(verbose=True))
