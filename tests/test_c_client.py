"""The boundary from plain C: tests/c_client.c includes only
include/simar.h (compiled as strict C99, warnings as errors), links against
the shared library and calls its host-only entry points; every line it
prints is checked here against the algorithms' closed forms and against the
Python binding over the same library."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RING, ALLPAIRS, ONESHOT = 1, 2, 3


@pytest.fixture(scope="module")
def client_output(tmp_path_factory):
    import all_reduce_reduction_amd as sim
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(sim.LIBPATH)
    exe = str(tmp_path_factory.mktemp("c_client") / "c_client")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_client.c"),
                    "-o", exe, "-L", libdir, "-lsimar", "-Wl,-rpath," + libdir], check=True)
    env = dict(os.environ)
    env.pop("SIM_CALIB", None)
    out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=60, env=env).stdout
    lines = {}
    for line in out.splitlines():
        key, _, rest = line.partition(" ")
        lines.setdefault(key, []).append(rest)
    return lines


def test_version_and_status(client_output):
    import all_reduce_reduction_amd as sim
    assert client_output["version"] == [str(sim.sim_version())]
    assert client_output["status"] == ["ok"]


def test_schedule_shapes_follow_the_closed_forms(client_output):
    import all_reduce_reduction_amd as sim
    info = {}
    for rest in client_output["info"]:
        f = rest.split()
        if f[1] != "status":
            info[int(f[0])] = tuple(int(x) for x in f[1:])
    p = 8
    assert info[RING][0] == 2 * (p - 1) and info[RING][2] == p      # 2(p-1) steps over p chunks
    assert info[ALLPAIRS][0] == 2 and info[ALLPAIRS][2] == p        # gather-reduce, then fan-out
    assert info[ONESHOT][0] == 1                                    # both fused in one launch
    for algo, (nsteps, nxfers, nchunks) in info.items():
        assert sim.sim_schedule_info(sim.ALGO_NAMES[algo], p) == (nsteps, nxfers, nchunks)
    verified = {int(r.split()[0]): int(r.split()[1]) for r in client_output["verify"]}
    assert verified and all(st == 0 for st in verified.values())


def test_custom_schedule_checked_from_c(client_output):
    assert client_output["custom"] == ["0"]
    assert client_output["swapped"] == ["-8"]   # fan-out before gather-reduce: SIM_ERR_VERIFY


def test_tree_and_config_and_init_guard(client_output):
    # NCCL's tree over 8 nodes: node 4 hangs below the root 0, children 2 and 6
    assert client_output["tree"] == ["0 0 2 2 6"]
    st, g = client_output["config"][0].split()
    assert st == "0" and int(g) >= 1
    assert client_output["config_bad"] == ["-1"]
    assert client_output["before_init"] == ["-9"]
