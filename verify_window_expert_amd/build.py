"""Build libstrata_window.so in-tree with hipcc for gfx950."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libstrata_window.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose=False, defines=(), out=None):
    """Compile every HIP source of the library into libstrata_window.so (always rebuilds):
    one hipcc per source, run side by side, then one link. defines: extra -D options (a
    tuning variant); out: the library's path (default: the package's)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmpdir = tempfile.mkdtemp(prefix="strata_build_")
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc] + [f for f in HIPCC_FLAGS if f != "-shared"] + ["-D" + d for d in defines] +
                    ["-c", src, "-o", obj])

    def run(cmd):
        return subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, min(8, os.cpu_count() or 1)))) as ex:
        results = list(ex.map(run, cmds))
    for cmd, res in zip(cmds, results):
        if res.returncode != 0:
            raise RuntimeError("hipcc failed: " + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    lib_path = out or LIB_PATH
    tmp = lib_path + ".tmp%d" % os.getpid()
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = run(link)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
    if verbose:
        print("\n".join(" ".join(c) for c in cmds + [link]))
    for o in objs:
        os.remove(o)
    os.rmdir(tmpdir)
    os.replace(tmp, lib_path)
    return lib_path
