"""Builds the test-support probe libraries tests/hwprobe/libencoder_probe.so
and tests/hwprobe/libsmfmac_probe.so (gfx950) from encoder_probe.hip and
smfmac_probe.hip with the library's compiler flags.  Called by the
repository's build entry point; the GPU tests that use them fail when they
are missing."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ("encoder_probe", "smfmac_probe")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    for name in PROBES:
        out = os.path.join(HERE, f"lib{name}.so")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fvisibility=hidden",
               os.path.join(HERE, f"{name}.hip"), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}.hip:\n{r.stdout}\n{r.stderr}")
    return HERE


if __name__ == "__main__":
    print(build())
