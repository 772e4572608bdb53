"""Build the test instruments under tests/probes (gfx950 shared libraries).

They are measurement tools for the test suite, not part of the attention
library: fp8_mfma_probe evaluates dot products with the fp8 matrix
instruction so the tests can pin down how it accumulates.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = {"libfp8_mfma_probe.so": "fp8_mfma_probe.hip"}


def build() -> None:
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"
    for lib, src in PROBES.items():
        out = os.path.join(HERE, lib)
        cmd = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-o", out + ".tmp", os.path.join(HERE, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build()
