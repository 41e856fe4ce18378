"""Builds the host-runtime harness: the library's api.hip compiled for the CPU
with g++ (AddressSanitizer and UndefinedBehaviorSanitizer on), linked with the
fake HIP runtime and checking launchers of fake_hip.cpp and the scenario
driver.  Test infrastructure only (tests/test_host_runtime.py runs it)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "looped_normalized_gpt_amd", "csrc")
OUT = os.path.join(HERE, "_build")
EXE = os.path.join(OUT, "hostsim")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         "-Wall", "-Wno-unused-parameter", "-Wno-unused-variable"]
UNITS = [("api", ["-x", "c++", os.path.join(CSRC, "api.hip")]),
         ("fake_hip", [os.path.join(HERE, "fake_hip.cpp")]),
         ("scenarios", [os.path.join(HERE, "scenarios.cpp")])]


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    procs, objs = [], []
    for name, src in UNITS:
        obj = os.path.join(OUT, name + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(["g++"] + FLAGS + ["-c"] + src + ["-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        if p.returncode:
            raise RuntimeError(out)
    subprocess.run(["g++", "-fsanitize=address,undefined", "-o", EXE] + objs, check=True)
    return EXE


if __name__ == "__main__":
    print(build())
    sys.exit(0)
