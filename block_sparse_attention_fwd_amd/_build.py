"""Build the gfx950 library libbsa.so in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsa.so")
UNITS_LIB = os.path.join(HERE, "libbsa_units.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are kept out of every device build.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _embed_lut():
    """Embed lut/gfx950.lut as the library's built-in lookup table."""
    src = os.path.join(HERE, "lut", "gfx950.lut")
    text = open(src).read()
    out = os.path.join(CSRC, "lut_default.inc")
    body = "".join('    "' + line.replace("\\", "\\\\").replace('"', '\\"') + '\\n"\n' for line in text.splitlines())
    content = "// generated from lut/gfx950.lut by _build.py -- do not edit\nstatic const char kDefaultLut[] =\n" + body + "    \"\";\n"
    if not os.path.exists(out) or open(out).read() != content:
        with open(out, "w") as f:
            f.write(content)


def build(verbose: bool = False) -> str:
    _embed_lut()
    objs = []
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include")]
    for name in ("api.cpp", "attn_fwd.hip", "attn_fwd_f32.hip", "plan_device.hip", "route_probe.hip"):
        src = os.path.join(CSRC, name)
        obj = os.path.join(CSRC, name + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC, *lang, *common, *DEVICE_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"], check=True)
    os.replace(tmp, LIB)
    # unit microbenchmarks (bench.py --units): a library of their own
    src = os.path.join(CSRC, "units.hip")
    cmd = [HIPCC, "-x", "hip", *common, *DEVICE_FLAGS, "-shared", src, "-o", UNITS_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(UNITS_LIB + ".tmp", UNITS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
