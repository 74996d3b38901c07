"""The launch planner's kernel choice and tile geometry, checked on the host.

tests/native/plan_rules.cpp links the planner's source (no kernels, no GPU)
and compares its plans with the selection rule: direct kernel for
token-major views and for gathers, head runs for scatters into head-major
views with head rows of at least one 128-byte line, the LDS transpose below
that, the direct kernel for head rows longer than one tile or one-head
groups; plus the vector width from the operands' alignment.
"""
import os
import subprocess

import __graft_entry__ as entry


def test_plan_rules():
    if not os.path.exists(entry.PLAN_TEST):
        entry.build_plan_test()
    r = subprocess.run([entry.PLAN_TEST], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan rules ok" in r.stdout
