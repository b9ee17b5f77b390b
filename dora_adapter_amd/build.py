"""Compile libdora.so (HIP, gfx950) in-tree: dora_adapter_amd/libdora.so, and
the benchmark's stream-ceiling helper libstreamceil.so.

Every source is compiled with hipcc for gfx950 only.  Packed-fp32 VALU ops are
disabled for device code (they are left to scalar fp32 instructions).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdora.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

# (source, extra defines, object name): the pipelined GEMM's tile
# configurations are one source compiled once per configuration, so that they
# build in parallel.
SOURCES = [("gemm_bf16.hip", (), "gemm_bf16"), ("gemm_f32.hip", (), "gemm_f32"),
           ("elementwise.hip", (), "elementwise"), ("dora_api.cpp", (), "dora_api"),
           ("noalloc.hip", (), "noalloc")] + \
          [("gemm_dma_cfg.hip", (f"-DDORA_DMA_CFG={k}",), f"gemm_dma_cfg{k}") for k in range(8)]
# Measurement helper for bench.py (not part of the DoRA library): the HBM
# rate of a plain two-in / one-out stream.
STREAM_SOURCE = ("stream_ceiling.hip", (), "stream_ceiling")
STREAM_LIB = os.path.join(HERE, "libstreamceil.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(unit, extra=()):
    src, defines, name = unit
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *defines, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("'-packed-fp32-ops' is not a recognized feature for this target",)
    err = "\n".join(l for l in res.stderr.splitlines() if not any(q in l for q in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose=False, extra=()):
    """Build libdora.so and the benchmark's stream-ceiling helper."""
    os.makedirs(BUILD, exist_ok=True)
    units = SOURCES + [STREAM_SOURCE]
    with cf.ThreadPoolExecutor(max_workers=min(len(units), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), units))
    for (obj, err) in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    _link([o for o, _ in results[:len(SOURCES)]], LIB)
    _link([results[-1][0]], STREAM_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
