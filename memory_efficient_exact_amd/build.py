"""Build libmea.so (the HIP kernels plus the C ABI) for gfx950, in-tree, and the
issue-cost probe program.

Usage: ``python -m memory_efficient_exact_amd.build [-v]``. Each source under
``csrc/`` is compiled to an object in ``_build/`` (in parallel), then linked
into ``memory_efficient_exact_amd/libmea.so`` atomically; ``probes/mea_probe.hip``
becomes the executable ``probes/mea_probe`` (run by ``bench.py --mode probe``).
The same sources built with ``MEA_SYNC_TIMERS=1`` give
``memory_efficient_exact_amd/libmea_synctimers.so``, the timing library that
counts the cycles of the tiled loops' end-of-tile waits (``bench.py --mode
sync``); nothing else loads it. Always recompiles.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libmea.so")
SYNC_LIB = os.path.join(PKG, "libmea_synctimers.so")
PROBE_SRC = os.path.join(PKG, "probes", "mea_probe.hip")
PROBE = os.path.join(PKG, "probes", "mea_probe")
ARCH = os.environ.get("MEA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit mul+add fusion: the kernels write every FMA they want
    # explicitly, and the softmax bookkeeping relies on rounded products
    # (fl(m*C)) staying rounded
    "-ffp-contract=off",
    # only the C ABI (marked MEA_API in include/mea.h) is exported
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; drop that warning
    err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln
                    and "is not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False):
    sync_dir = os.path.join(BUILD, "synctimers")
    os.makedirs(sync_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    sync_objs = [os.path.join(sync_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    probe_tmp = PROBE + ".tmp"
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(_run, [HIPCC, *FLAGS, "-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        futs += [ex.submit(_run, [HIPCC, *FLAGS, "-DMEA_SYNC_TIMERS=1", "-c", s, "-o", o], verbose)
                 for s, o in zip(srcs, sync_objs)]
        futs.append(ex.submit(_run, [HIPCC, *FLAGS, PROBE_SRC, "-o", probe_tmp], verbose))
        for f in futs:
            f.result()
    for out, parts in ((LIB, objs), (SYNC_LIB, sync_objs)):
        tmp = out + ".tmp"
        _run([HIPCC, *FLAGS, "-shared", "-o", tmp, *parts], verbose)
        os.replace(tmp, out)
    os.replace(probe_tmp, PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
