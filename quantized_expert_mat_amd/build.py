"""Build libqmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every source compiles to its own object in parallel (the decode kernels of each
code width are a separate file, the bulk of the build), then one link."""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmoe.so")
SOURCES = ["qmoe_api.hip", "qmoe_pack.hip", "qmoe_decode.hip", "qmoe_decode_k2.hip", "qmoe_decode_k3.hip",
           "qmoe_decode_k4.hip", "qmoe_prefill.hip"]
HEADERS = ["qmoe_internal.h", "qmoe_decode_dev.h"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _clean(text):
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip())


def build(verbose=False):
    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="qmoe_build_") as tmpd:
        procs, objs = [], []
        for s in SOURCES:
            o = os.path.join(tmpd, s + ".o")
            objs.append(o)
            cmd = [HIPCC] + FLAGS + inc + ["-c", os.path.join(CSRC, s), "-o", o]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        errors = []
        for s, p in procs:
            out = _clean(p.communicate()[0])
            if p.returncode != 0:
                errors.append(f"{s}:\n{out}")
            elif verbose and out:
                print(out)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = LIB + ".tmp"
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + _clean(r.stdout + r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))


def source_hash():
    """Hash of the kernel sources: ties a stored counter measurement to the code it measured."""
    import hashlib
    h = hashlib.sha256()
    for s in SOURCES + HEADERS:
        with open(os.path.join(CSRC, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]
