"""Build libnha.so (HIP, gfx950) in-tree with hipcc.

    python -m softmax_attention_nha_amd.build

Every .hip / .cpp file under csrc/ is compiled to an object in parallel and
linked into softmax_attention_nha_amd/libnha.so.  Packed-FP32 instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnha.so")
ARCH = os.environ.get("NHA_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = ["hipcc"] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _stale(src, headers_mtime):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    return os.path.getmtime(obj) < max(os.path.getmtime(src), headers_mtime)


def build(verbose=True, incremental=False):
    """Compile every source (incremental=True: only those whose object is older
    than the source or any header) and link libnha.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    headers = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    hm = max(os.path.getmtime(h) for h in headers)
    todo = [x for x in srcs if _stale(x, hm)] if incremental else srcs
    jobs = max(1, min(len(todo), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(OBJ, os.path.basename(x) + ".o") for x in srcs]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
