"""CPU check of the chain barrier's counter arithmetic across the 32-bit wrap.

The counters of a prepared chain are cumulative over launches and compared
modulo 2^32 (csrc/chain_sync.h, the same header the kernel uses). A host
program built from that header simulates launches that start just below
the point where launch_count * workgroups wraps, and where the launch count
itself wraps, and checks that every barrier releases exactly once, on its
last arrival, and that every launch advances the generation once. The same
program, told to derive the launch count back from the wrapped target
(target / G, the arithmetic the barrier used to have), must fail there:
that shows the cases reach the wrap.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verification_gemm_amd", "csrc")
SIM = os.path.join(ROOT, "tests", "chain_counters_sim.cpp")


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("chain_sim") / "chain_counters_sim")
    subprocess.run([cxx, "-O1", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, SIM, "-o", exe],
                   check=True)
    return exe


def run(exe, G, n_lin, gen0, launches, old=False):
    args = [exe, str(G), str(n_lin), str(gen0), str(launches)] + (["old"] if old else [])
    r = subprocess.run(args, capture_output=True, text=True)
    return r.returncode, r.stdout.strip()


# workgroup counts: one per CU, two per CU, groups of unequal size, tiny grids
GRIDS = [256, 512, 1000, 7, 1]


@pytest.mark.parametrize("G", GRIDS)
def test_counters_from_zero(sim, G):
    rc, out = run(sim, G, 3, 0, 4)
    assert rc == 0 and out == "ok", out


@pytest.mark.parametrize("G", GRIDS)
def test_counters_across_target_wrap(sim, G):
    """Start a few launches before (gen + 1) * G passes 2^32."""
    gen0 = (1 << 32) // G - 3
    rc, out = run(sim, G, 3, gen0, 8)
    assert rc == 0 and out == "ok", out


@pytest.mark.parametrize("G", GRIDS)
def test_counters_across_generation_wrap(sim, G):
    """The launch count itself wraps from 2^32 - 1 to 0."""
    rc, out = run(sim, G, 2, (1 << 32) - 3, 6)
    assert rc == 0 and out == "ok", out


@pytest.mark.parametrize("G", [256, 512, 1000, 7])
def test_old_derivation_fails_at_wrap(sim, G):
    """Deriving the launch count as target / G breaks once the target has
    wrapped; the simulation catches it, so the cases above do reach the
    wrap (with one workgroup, target / G is exact and cannot fail)."""
    gen0 = (1 << 32) // G - 3
    rc, out = run(sim, G, 3, gen0, 8, old=True)
    assert rc == 1, out
