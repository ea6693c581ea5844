"""bench.py's kernel names against the kernels the library defines (CPU only).

bench.py credits each kernel that streams a stage's data with that stage's algorithmic bytes
(its work keys, "a+b" for kernels that share one stage) and lists the kernels of every
stage. Both name kernels by their source names; a kernel renamed or added in the sources
without the same change in bench.py would silently drop out of the roofline line. Every
name bench.py uses must be a kernel of the sources, and every kernel that streams rows, keys
or values (rows, attention, walk and verification kernels) must be in some work key.
"""
from __future__ import annotations

import glob
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads.configs import CONFIG_ORDER, config_by_name  # noqa: E402

KERNEL_RE = re.compile(r"__global__\s+(?:__launch_bounds__\([^)]*\)\s+)?void\s+(\w+)\s*\(")


def source_kernels() -> set[str]:
    names = set()
    for f in glob.glob(os.path.join(ROOT, "draft_tree_verification_build_amd", "csrc", "*.hip")):
        with open(f) as fh:
            names.update(KERNEL_RE.findall(fh.read()))
    return names


class _Step:
    def __init__(self, fuse):
        self.fuse_compact = fuse


class _Wl:
    def __init__(self, cfg):
        self.cfg = cfg


def _work():
    one = {"bytes": 1.0}
    return {k: dict(one) for k in ("build", "attention", "verify", "verify_compact", "compact")}


def test_source_kernels_found():
    names = source_kernels()
    for k in ("talon_rows_bf16_kernel", "talon_select_kernel", "attn_bf16_kernel", "sample_walk_kernel",
              "verify_greedy_bf16_kernel", "opt_rows_bf16_kernel", "spine_bf16_kernel", "given_tree_kernel"):
        assert k in names, k


def test_bench_names_are_kernels():
    names = source_kernels()
    for name in CONFIG_ORDER:
        cfg = config_by_name(name)
        for fuse in (True, False):
            for key in bench.kernel_work(_Step(fuse), _Wl(cfg), _work()):
                for k in key.split("+"):
                    assert k in names, (name, key, k)
        for stage, fn in bench.STAGE_KERNELS.items():
            for k in fn(cfg):
                k = k.split(" ")[0]
                assert k in names, (name, stage, k)


def test_streaming_kernels_carry_work():
    streaming = {k for k in source_kernels()
                 if re.match(r"(talon_rows|opt_rows|opt_root|spine|attn_bf16|attn_f32|verify_greedy|sample_walk|"
                             r"given_tree|compact_kernel)", k)}
    covered = set()
    for name in CONFIG_ORDER:
        for dtype in ("bf16", "f32"):   # every configuration in both row types
            cfg = config_by_name(name, dtype=dtype)
            for fuse in (True, False):
                for key in bench.kernel_work(_Step(fuse), _Wl(cfg), _work()):
                    covered.update(key.split("+"))
    assert streaming <= covered, sorted(streaming - covered)
