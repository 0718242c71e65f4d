"""Builds the CPU oracle (oracle.c) into liboracle.so next to this file.

Test infrastructure: the oracle is the independent double-precision
reference the HIP path is checked against.  `plant` builds a deliberately
broken variant (see ORACLE_PLANT in oracle.c) for the CPU test that checks
the oracle's pins catch such mistakes.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(out=LIB, plant=0, plant_bwd=0, plant_ch=0, plant_gated=0):
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if plant:
        cmd.insert(1, "-DORACLE_PLANT=%d" % int(plant))
    if plant_bwd:
        cmd.insert(1, "-DORACLE_PLANT_BWD=%d" % int(plant_bwd))
    if plant_ch:
        cmd.insert(1, "-DORACLE_PLANT_CH=%d" % int(plant_ch))
    if plant_gated:
        cmd.insert(1, "-DORACLE_PLANT_GATED=%d" % int(plant_gated))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
