"""Compile the hardware fixtures of the tests and the benchmark for gfx950,
with the library's flags:
  libfp8mfma_probe.so  the fp8 matrix instruction on given codes (tests)
  libstream_read.so    a plain streaming read (the benchmark's read floor)
  libreciprocal_probe.so  the library's reciprocal_rn against division (tests)"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURES = {"fp8_mfma_probe.hip": "libfp8mfma_probe.so", "stream_read.hip": "libstream_read.so",
            "reciprocal_probe.hip": "libreciprocal_probe.so"}
CSRC = os.path.join(os.path.dirname(os.path.dirname(HERE)), "fp8_kv_cache_append_amd", "csrc")


def _one(src: str, lib: str) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    src, lib = os.path.join(HERE, src), os.path.join(HERE, lib)
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", CSRC, src,
           "-o", lib + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    os.replace(lib + ".tmp", lib)
    return lib


def build() -> list:
    return [_one(s, l) for s, l in FIXTURES.items()]


if __name__ == "__main__":
    print(build())
